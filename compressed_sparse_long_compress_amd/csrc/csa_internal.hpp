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

// Top-k workspace row block for few-long-row batches: 4096 histogram bins of
// the top 12 key bits, 4096 bins of the next 12 bits of the candidates, then
// 16 counters.  Must start zero-filled.
constexpr size_t kTopkRowBlock = 2 * 4096 * 4 + 64;

hipError_t launch_compress(const uint16_t* kv, const float* logits, int64_t tok0, int64_t n_tok, int m, int d,
                           const RopeTab& rt, int64_t row0, int64_t cap, uint8_t* nope, uint16_t* rope, float* scale,
                           hipStream_t st);

// hist_ws != nullptr: also add each row's top-12-bit key histogram into the
// top-k workspace (row blocks of kTmRowBlock bytes, histogram first)
hipError_t launch_index_scores(const uint8_t* q, const uint8_t* q_scale, const float* w, const int32_t* seq,
                               const int64_t* pos, int64_t T, int h_i, int d_i, const uint8_t* kdata,
                               const uint8_t* kscale, int64_t kcap, int m, int64_t n_cols, float* scores,
                               void* hist_ws, hipStream_t st);

size_t topk_workspace_bytes(int64_t T, int64_t n_cols, int k);
// true when the top-k for this shape uses the workspace histogram (few long rows)
bool topk_uses_hist(int64_t T, int64_t n_cols);
// hist_done: the row histograms were already accumulated by the indexer
hipError_t launch_topk(const float* scores, int64_t T, int64_t n_cols, const int64_t* pos, int m, int k, int32_t* idx,
                       void* ws, bool hist_done, hipStream_t st);

struct KvView {
    const uint8_t* nope;
    const uint16_t* rope;
    const float* scale;
    int64_t cap;
};

size_t mqa_workspace_bytes(int64_t T, int H, int d, int64_t max_keys);
// idx == nullptr selects the dense (HCA) key set
hipError_t launch_mqa(const uint16_t* q, const int32_t* seq, const int64_t* pos, int64_t T, int H, int d,
                      const int32_t* idx, int k, int m, int64_t max_keys, KvView comp, KvView win, int window,
                      float sm_scale, const RopeTab& rt, float* out, float* lse, void* ws, hipStream_t st);

}  // namespace csa
