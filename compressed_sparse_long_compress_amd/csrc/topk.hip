// csa_topk kernel: exact top-k by radix select, one workgroup per row.
//
// Scores map to order-preserving 32-bit keys.  Three histogram passes
// (12 + 12 + 8 key bits) find the k-th largest key `thr`; a final ordered
// compaction takes every key > thr and the lowest-index (k - #greater) keys
// equal to thr, writing indices in ascending order.  That is exactly the
// order (score desc, index asc) the selection is defined by.  Rows that fit
// in LDS (<= 36608 columns) are cached there; longer rows re-read global
// memory each pass.
#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {

constexpr int kTopkThreads = 512;
constexpr int kTopkCache = 36608;  // keys cached in LDS (143 KB)

// exclusive prefix sum over the block; returns the block total in `total`
__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kTopkThreads / 64; ++i) {
        int s = wsum[i];
        off += i < wave ? s : 0;
        tot += s;
    }
    __syncthreads();
    total = tot;
    return off + x - v;
}

// Find, scanning bins from the top, the bin where the running count reaches
// `need`.  Returns the bin; `above` receives the count in higher bins.
template <int NBINS>
__device__ int find_bin(const uint32_t* hist, int need, int* wsum, int* bcast, int& above) {
    constexpr int PER = NBINS / kTopkThreads > 0 ? NBINS / kTopkThreads : 1;
    const int tid = threadIdx.x;
    // thread tid owns bins counted from the top: [tid*PER, tid*PER + PER) in descending order
    int local = 0;
    if (tid * PER < NBINS)
        for (int i = 0; i < PER; ++i) local += (int)hist[NBINS - 1 - (tid * PER + i)];
    int total;
    int before = block_excl_scan(local, wsum, total);
    if (tid * PER < NBINS && before < need && before + local >= need) {
        int run = before;
        for (int i = 0; i < PER; ++i) {
            int bin = NBINS - 1 - (tid * PER + i);
            int c = (int)hist[bin];
            if (run + c >= need) {
                bcast[0] = bin;
                bcast[1] = run;
                break;
            }
            run += c;
        }
    }
    __syncthreads();
    above = bcast[1];
    int bin = bcast[0];
    __syncthreads();
    return bin;
}

__global__ __launch_bounds__(kTopkThreads) void k_topk_row(const float* __restrict__ scores, int64_t n_cols,
                                                           const int64_t* __restrict__ pos, int m, int k,
                                                           int32_t* __restrict__ idx) {
    __shared__ uint32_t hist[4096];
    __shared__ uint32_t cache[kTopkCache];
    __shared__ int wsum[kTopkThreads / 64];
    __shared__ int bcast[4];
    const int tid = threadIdx.x;
    const int64_t t = blockIdx.x;
    int64_t nv64 = (pos[t] + 1) / m;
    if (nv64 > n_cols) nv64 = n_cols;
    if (nv64 < 0) nv64 = 0;
    const int nv = (int)nv64;
    const float* row = scores + t * n_cols;
    int32_t* out = idx + t * (int64_t)k;

    if (nv <= k) {
        for (int a = tid; a < k; a += kTopkThreads) out[a] = a < nv ? a : -1;
        return;
    }
    const bool cached = nv <= kTopkCache;
    if (cached)
        for (int j = tid; j < nv; j += kTopkThreads) cache[j] = f32_order_key(row[j]);
    auto key_at = [&](int j) -> uint32_t { return cached ? cache[j] : f32_order_key(row[j]); };

    // pass 1: top 12 bits
    for (int i = tid; i < 4096; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    for (int j = tid; j < nv; j += kTopkThreads) atomicAdd(&hist[key_at(j) >> 20], 1u);
    __syncthreads();
    int above1;
    const uint32_t b1 = (uint32_t)find_bin<4096>(hist, k, wsum, bcast, above1);

    // pass 2: middle 12 bits among keys with prefix b1
    for (int i = tid; i < 4096; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    for (int j = tid; j < nv; j += kTopkThreads) {
        uint32_t key = key_at(j);
        if ((key >> 20) == b1) atomicAdd(&hist[(key >> 8) & 0xFFF], 1u);
    }
    __syncthreads();
    int above2;
    const uint32_t b2 = (uint32_t)find_bin<4096>(hist, k - above1, wsum, bcast, above2);
    const uint32_t p2 = (b1 << 12) | b2;

    // pass 3: low 8 bits among keys with prefix p2
    for (int i = tid; i < 256; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    for (int j = tid; j < nv; j += kTopkThreads) {
        uint32_t key = key_at(j);
        if ((key >> 8) == p2) atomicAdd(&hist[key & 0xFF], 1u);
    }
    __syncthreads();
    int above3;
    const uint32_t b3 = (uint32_t)find_bin<256>(hist, k - above1 - above2, wsum, bcast, above3);
    const uint32_t thr = (p2 << 8) | b3;
    const int need_eq = k - (above1 + above2 + above3);

    // pass 4: ordered compaction, 4 consecutive columns per thread per tile
    constexpr int E = 4;
    int eq_run = 0, out_run = 0;
    for (int j0 = 0; j0 < nv; j0 += kTopkThreads * E) {
        const int jb = j0 + tid * E;
        uint32_t kk[E];
        int n_eq = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            kk[e] = jb + e < nv ? key_at(jb + e) : 0u;
            n_eq += (jb + e < nv && kk[e] == thr) ? 1 : 0;
        }
        int eq_tot;
        int eq_before = block_excl_scan(n_eq, wsum, eq_tot) + eq_run;
        int sel[E], n_sel = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const bool in = jb + e < nv;
            const bool eq = in && kk[e] == thr;
            sel[e] = in && (kk[e] > thr || (eq && eq_before < need_eq));
            eq_before += eq ? 1 : 0;
            n_sel += sel[e];
        }
        int sel_tot;
        int o = block_excl_scan(n_sel, wsum, sel_tot) + out_run;
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (sel[e]) out[o++] = jb + e;
        eq_run += eq_tot;
        out_run += sel_tot;
    }
}

size_t topk_workspace_bytes(int64_t, int64_t, int) { return 0; }

hipError_t launch_topk(const float* scores, int64_t T, int64_t n_cols, const int64_t* pos, int m, int k, int32_t* idx,
                       void*, hipStream_t st) {
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(k_topk_row, dim3((unsigned)T), dim3(kTopkThreads), 0, st, scores, n_cols, pos, m, k, idx);
    return hipGetLastError();
}

}  // namespace csa
