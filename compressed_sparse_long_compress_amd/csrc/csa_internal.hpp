// Host-side launchers of the libcsa kernels (arguments already validated).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa {

// RoPE frequencies theta_i = base^(-2i/64), i < 32, evaluated once on the host in fp64.
struct RopeTab {
    double theta[32];
};
RopeTab rope_table(double base);

struct KvView {
    const uint8_t* nope;
    const uint16_t* rope;
    const float* scale;
    int64_t cap;
    const int32_t* pages;  // nullptr: contiguous rows seq*cap + slot
    int pshift;            // log2(slots per page) when paged
};

// Row of slot `slot` (< cap) of sequence `seq`: contiguous, or through the page table.
__host__ __device__ __forceinline__ int64_t kv_row(const int32_t* pages, int pshift, int64_t cap, int64_t seq,
                                                   int64_t slot) {
    if (!pages) return seq * cap + slot;
    const int64_t npp = cap >> pshift;
    return ((int64_t)pages[seq * npp + (slot >> pshift)] << pshift) | (slot & ((1LL << pshift) - 1));
}

// Top-k workspace of the few-long-rows path (T < kTopkMaxRows rows): the
// row summaries, summ[T][topk_groups(n_cols)], each the largest order key of
// the visible columns of one kTopkGroup-column group (0 for none).
constexpr int kTopkMaxRows = 128;
constexpr int kTopkGroup = 32;
__host__ __device__ inline int64_t topk_groups(int64_t n_cols) { return (n_cols + kTopkGroup - 1) / kTopkGroup; }

hipError_t launch_compress(const uint16_t* kv, const float* logits, int64_t tok0, int64_t n_tok, int m, int d,
                           const RopeTab& rt, int64_t seq, const KvView& out, uint8_t* nope, uint16_t* rope,
                           float* scale, hipStream_t st);
// logits [n_tok][d]: per-channel weights
hipError_t launch_compress_channel(const uint16_t* kv, const float* logits, int64_t tok0, int64_t n_tok, int m, int d,
                                   const RopeTab& rt, int64_t seq, const KvView& out, uint8_t* nope, uint16_t* rope,
                                   float* scale, hipStream_t st);
// raw bf16 index keys -> MXFP4 rows
hipError_t launch_compress_index_keys(const uint16_t* k, const float* logits, int64_t tok0, int64_t n_tok, int m,
                                      int d_i, int64_t seq, int64_t cap, const int32_t* pages, int pshift,
                                      uint8_t* data, uint8_t* kscale, hipStream_t st);

// gmax != nullptr: also write each row's summary (the largest order key of
// the visible columns of every kTopkGroup-column group) to gmax[T][groups]
hipError_t launch_index_scores(const uint8_t* q, const uint8_t* q_scale, const float* w, const int32_t* seq,
                               const int64_t* pos, int64_t T, int h_i, int d_i, const uint8_t* kdata,
                               const uint8_t* kscale, int64_t kcap, const int32_t* kpages, int kpshift, int m,
                               int64_t n_cols, float* scores, uint32_t* gmax, hipStream_t st);
// rows g*group .. g*group+group-1 share each key stream (group 1, 2 or 4; T % group == 0)
hipError_t launch_index_scores_grouped(const uint8_t* q, const uint8_t* q_scale, const float* w, const int32_t* seq,
                                       const int64_t* pos, int64_t T, int h_i, int d_i, const uint8_t* kdata,
                                       const uint8_t* kscale, int64_t kcap, const int32_t* kpages, int kpshift, int m,
                                       int64_t n_cols, int group, float* scores, uint32_t* gmax, hipStream_t st);

// fused indexer + top-k (no score row written): workspace and launch
size_t index_topk_workspace_bytes(int64_t T, int64_t n_cols, int k, int h_i);
hipError_t launch_index_topk(const uint8_t* q, const uint8_t* q_scale, const float* w, const int32_t* seq,
                             const int64_t* pos, int64_t T, int h_i, int d_i, const uint8_t* kdata,
                             const uint8_t* kscale, int64_t kcap, const int32_t* kpages, int kpshift, int m,
                             int64_t n_cols, int k, int32_t* idx, void* ws, hipStream_t st);

size_t topk_workspace_bytes(int64_t T, int64_t n_cols, int k);
// true when the top-k for this shape uses the row summaries (few long rows)
bool topk_uses_summary(int64_t T, int64_t n_cols);
// prepared: the row summaries were already written by the indexer
hipError_t launch_topk(const float* scores, int64_t T, int64_t n_cols, const int64_t* pos, int m, int k, int32_t* idx,
                       void* ws, bool prepared, hipStream_t st);
// the same selection with the library's own scratch array in place of a workspace
// (shapes needing more than topk_scratch_bytes() of it are refused by the caller)
size_t topk_scratch_bytes();
hipError_t launch_topk_noalloc(const float* scores, int64_t T, int64_t n_cols, const int64_t* pos, int m, int k,
                               int32_t* idx, hipStream_t st);



// 64-bit fixed-point gradient buffers (fx_add): clear n words; dst[i] += src[i] * 2^-40
hipError_t launch_fx_zero(unsigned long long* p, int64_t n, hipStream_t st);
hipError_t launch_fx_flush(const unsigned long long* src, float* dst, int64_t n, hipStream_t st);

// gradient of the indexer scores at the selected columns; ws: key_rows x d_i x 8 bytes
hipError_t launch_index_bwd(const uint8_t* q, const uint8_t* q_scale, const float* w, const int32_t* seq,
                            const int64_t* pos, int64_t T, int h_i, int d_i, const uint8_t* kdata,
                            const uint8_t* kscale, int64_t kcap, const int32_t* kpages, int kpshift, int m,
                            const int32_t* idx, const float* g, int n_sel, float* dq, float* dw, float* dkeys,
                            int64_t key_rows, void* ws, hipStream_t st);

size_t mqa_workspace_bytes(int64_t T, int H, int d, int64_t max_keys);
// idx == nullptr selects the dense (HCA) key set
hipError_t launch_mqa(const uint16_t* q, const int32_t* seq, const int64_t* pos, int64_t T, int H, int d,
                      const int32_t* idx, int k, int m, int64_t max_keys, KvView comp, KvView win, int window,
                      float sm_scale, const RopeTab& rt, float* out, float* lse, void* ws, hipStream_t st);
// sets *bad (device int) when an entry the attention would read for these rows holds a
// bf16 RoPE dim outside the fp16 range (64-head kernels stage those dims as fp16)
hipError_t launch_check_rope(const int32_t* seq, const int64_t* pos, int64_t T, const int32_t* idx, int k, int m,
                             KvView comp, KvView win, int window, int* bad, hipStream_t st);
// ws: (comp_rows + win_rows) x 512 x 8 bytes of fixed-point entry gradients
hipError_t launch_mqa_bwd(const uint16_t* q, const int32_t* seq, const int64_t* pos, int64_t T, int H,
                          const int32_t* idx, int k, int m, KvView comp, KvView win, int window, float sm_scale,
                          const RopeTab& rt, const float* out, const float* lse, const float* dout, float* dq,
                          float* dcomp, int64_t comp_rows, float* dwin, int64_t win_rows, void* ws, hipStream_t st);

// matrix-core throughput probe: `blocks` workgroups of kProbeThreads threads, each wave
// issuing iters x kProbeChains MFMAs (kind 0: fp16 16x16x32, kind 1: MXFP4 32x32x64);
// sink: blocks x kProbeThreads floats
constexpr int kProbeThreads = 256;
constexpr int kProbeChains = 4;
hipError_t launch_mfma_probe(int kind, int blocks, int64_t iters, float* sink, hipStream_t st);

}  // namespace csa
