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

// ---------------------------------------------------------------------------
// Few long rows (decode): the row is split over many workgroups.
//   k_topkm_clear    zero the row's histogram and counters
//   k_topkm_hist     per chunk, LDS histogram of the top 12 key bits, added
//                    to the row's global histogram (integer atomics)
//   k_topkm_collect  per chunk, every workgroup reads the row histogram,
//                    finds the bin b1 holding the k-th largest key, appends
//                    the indices of keys above b1 and the (key, index) pairs
//                    inside b1; the last workgroup of the row (a counter
//                    taken after a release fence) picks the remaining
//                    need = k - #above among the candidates by radix select on
//                    the composite (key, ~index), sorts the k indices and
//                    writes the row.
// ---------------------------------------------------------------------------
constexpr int kTmThreads = 256;
constexpr int kCandLds = 12288;  // candidates held in LDS by the finalising workgroup

struct TmRow {
    uint32_t* hist;  // [4096]
    uint32_t* ctr;   // [0] appended above, [1] candidates, [2] finished chunks
    int32_t* sel;    // [k]
    uint64_t* cand;  // [n_cols] composite (key << 32 | ~index)
};

__device__ __forceinline__ TmRow tm_row(void* ws, int64_t t, int64_t n_cols, int k) {
    const size_t per = 4096 * 4 + 64 + (((size_t)k * 4 + 255) / 256) * 256 + (size_t)n_cols * 8;
    char* b = (char*)ws + (size_t)t * per;
    TmRow r;
    r.hist = (uint32_t*)b;
    r.ctr = (uint32_t*)(b + 4096 * 4);
    r.sel = (int32_t*)(b + 4096 * 4 + 64);
    r.cand = (uint64_t*)(b + 4096 * 4 + 64 + (((size_t)k * 4 + 255) / 256) * 256);
    return r;
}

size_t topk_row_stride(int64_t n_cols, int k) {
    return 4096 * 4 + 64 + (((size_t)k * 4 + 255) / 256) * 256 + (size_t)n_cols * 8;
}

__global__ __launch_bounds__(kTmThreads) void k_topkm_clear(void* ws, int64_t n_cols, int k) {
    TmRow r = tm_row(ws, blockIdx.x, n_cols, k);
    for (int i = threadIdx.x; i < 4096; i += kTmThreads) r.hist[i] = 0;
    if (threadIdx.x < 16) r.ctr[threadIdx.x] = 0;
}

__device__ __forceinline__ int64_t row_visible(const int64_t* pos, int64_t t, int m, int64_t n_cols) {
    int64_t nv = (pos[t] + 1) / m;
    if (nv > n_cols) nv = n_cols;
    if (nv < 0) nv = 0;
    return nv;
}

__global__ __launch_bounds__(kTmThreads) void k_topkm_hist(const float* __restrict__ scores, int64_t n_cols,
                                                           const int64_t* __restrict__ pos, int m, int k, int64_t chunk,
                                                           void* ws) {
    __shared__ uint32_t h[4096];
    const int64_t t = blockIdx.y;
    const int64_t nv = row_visible(pos, t, m, n_cols);
    if (nv <= k) return;
    const int64_t c0 = (int64_t)blockIdx.x * chunk;
    if (c0 >= nv) return;
    const int64_t c1 = c0 + chunk < nv ? c0 + chunk : nv;
    for (int i = threadIdx.x; i < 4096; i += kTmThreads) h[i] = 0;
    __syncthreads();
    const float* row = scores + t * n_cols;
    for (int64_t j = c0 + threadIdx.x * 4; j < c1; j += kTmThreads * 4) {
        if (j + 4 <= c1 && (((uintptr_t)(row + j) & 15) == 0)) {
            float4 v = *(const float4*)(row + j);
            atomicAdd(&h[f32_order_key(v.x) >> 20], 1u);
            atomicAdd(&h[f32_order_key(v.y) >> 20], 1u);
            atomicAdd(&h[f32_order_key(v.z) >> 20], 1u);
            atomicAdd(&h[f32_order_key(v.w) >> 20], 1u);
        } else {
            for (int64_t jj = j; jj < c1 && jj < j + 4; ++jj) atomicAdd(&h[f32_order_key(row[jj]) >> 20], 1u);
        }
    }
    __syncthreads();
    TmRow r = tm_row(ws, t, n_cols, k);
    for (int i = threadIdx.x; i < 4096; i += kTmThreads)
        if (h[i]) atomicAdd(&r.hist[i], h[i]);
}

// exclusive scan over a 256-thread block
__device__ __forceinline__ int tm_scan(int v, int* wsum, int& total) {
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
    for (int i = 0; i < kTmThreads / 64; ++i) {
        off += i < wave ? wsum[i] : 0;
        tot += wsum[i];
    }
    __syncthreads();
    total = tot;
    return off + x - v;
}

// bin (scanning from the top) where the running count reaches need; 256 threads
template <int NB>
__device__ int tm_find(const uint32_t* hist, int need, int* wsum, int* bc, int& above) {
    constexpr int PER = NB / kTmThreads > 0 ? NB / kTmThreads : 1;
    const int tid = threadIdx.x;
    int local = 0;
    if (tid * PER < NB)
        for (int i = 0; i < PER; ++i) local += (int)hist[NB - 1 - (tid * PER + i)];
    int tot;
    const int before = tm_scan(local, wsum, tot);
    if (tid * PER < NB && before < need && before + local >= need) {
        int run = before;
        for (int i = 0; i < PER; ++i) {
            const int bin = NB - 1 - (tid * PER + i);
            const int c = (int)hist[bin];
            if (run + c >= need) {
                bc[0] = bin;
                bc[1] = run;
                break;
            }
            run += c;
        }
    }
    __syncthreads();
    above = bc[1];
    const int bin = bc[0];
    __syncthreads();
    return bin;
}

// wave-aggregated append: returns this lane's slot (valid when flag)
__device__ __forceinline__ uint32_t tm_append(uint32_t* ctr, bool flag) {
    const uint64_t mask = __ballot(flag);
    const int lane = threadIdx.x & 63;
    uint32_t base = 0;
    const int leader = mask ? __builtin_ctzll(mask) : 0;
    if (mask && lane == leader) base = atomicAdd(ctr, (uint32_t)__popcll(mask));
    base = __shfl(base, leader);
    return base + (uint32_t)__popcll(mask & ((1ull << lane) - 1ull));
}

__global__ __launch_bounds__(kTmThreads) void k_topkm_collect(const float* __restrict__ scores, int64_t n_cols,
                                                              const int64_t* __restrict__ pos, int m, int k,
                                                              int64_t chunk, int nchunk, void* ws,
                                                              int32_t* __restrict__ idx) {
    __shared__ uint32_t h[4096];
    __shared__ uint64_t cl[kCandLds];
    __shared__ int32_t srt[2048];
    __shared__ int wsum[kTmThreads / 64];
    __shared__ int bc[4];
    __shared__ int last;
    const int tid = threadIdx.x;
    const int64_t t = blockIdx.y;
    const int64_t nv = row_visible(pos, t, m, n_cols);
    int32_t* out = idx + t * (int64_t)k;
    if (nv <= k) {
        if (blockIdx.x == 0)
            for (int a = tid; a < k; a += kTmThreads) out[a] = a < nv ? a : -1;
        return;
    }
    TmRow r = tm_row(ws, t, n_cols, k);
    for (int i = tid; i < 4096; i += kTmThreads) h[i] = r.hist[i];
    __syncthreads();
    int above1;
    const uint32_t b1 = (uint32_t)tm_find<4096>(h, k, wsum, bc, above1);

    const int64_t c0 = (int64_t)blockIdx.x * chunk;
    const int64_t c1 = c0 + chunk < nv ? c0 + chunk : nv;
    const float* row = scores + t * n_cols;
    for (int64_t jb = c0; jb < c1; jb += kTmThreads) {
        const int64_t j = jb + tid;
        uint32_t key = 0;
        if (j < c1) key = f32_order_key(row[j]);
        const bool up = j < c1 && (key >> 20) > b1;
        const bool eq = j < c1 && (key >> 20) == b1;
        const uint32_t su = tm_append(&r.ctr[0], up);
        if (up) r.sel[su] = (int32_t)j;
        const uint32_t se = tm_append(&r.ctr[1], eq);
        if (eq) r.cand[se] = ((uint64_t)key << 32) | (uint32_t)~(uint32_t)j;
    }
    // release this chunk's appends, count finished chunks
    __threadfence();
    __syncthreads();
    if (tid == 0) last = atomicAdd(&r.ctr[2], 1u) == (uint32_t)(nchunk - 1);
    __syncthreads();
    if (!last) return;
    __threadfence();

    // ---- finalise the row: choose `need` candidates by (key desc, index asc) ----
    const int n_up = (int)__atomic_load_n(&r.ctr[0], __ATOMIC_RELAXED);
    const int n_cand = (int)__atomic_load_n(&r.ctr[1], __ATOMIC_RELAXED);
    const int need = k - n_up;
    const bool in_lds = n_cand <= kCandLds;
    if (in_lds)
        for (int i = tid; i < n_cand; i += kTmThreads) cl[i] = r.cand[i];
    __syncthreads();
    auto cand_at = [&](int i) -> uint64_t { return in_lds ? cl[i] : r.cand[i]; };
    // radix select over the 64-bit composite, 8 bits per pass, most significant first
    uint64_t prefix = 0, pmask = 0;
    int need_left = need;
    for (int shift = 56; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += kTmThreads) h[i] = 0;
        __syncthreads();
        for (int i = tid; i < n_cand; i += kTmThreads) {
            const uint64_t c = cand_at(i);
            if ((c & pmask) == prefix) atomicAdd(&h[(c >> shift) & 0xFF], 1u);
        }
        __syncthreads();
        int above;
        const uint32_t bin = (uint32_t)tm_find<256>(h, need_left, wsum, bc, above);
        need_left -= above;
        prefix |= (uint64_t)bin << shift;
        pmask |= (uint64_t)0xFF << shift;
    }
    // composites are unique: select every candidate >= prefix (exactly `need` of them)
    for (int i = tid; i < n_cand; i += kTmThreads) {
        const uint64_t c = cand_at(i);
        const bool take = c >= prefix;
        const uint32_t s = tm_append(&r.ctr[0], take);
        if (take) r.sel[s] = (int32_t)~(uint32_t)(c & 0xFFFFFFFFu);
    }
    __threadfence();
    __syncthreads();
    // ---- sort the k indices ascending (bitonic, padded to a power of two) ----
    int np = 1;
    while (np < k) np <<= 1;
    for (int i = tid; i < np; i += kTmThreads) srt[i] = i < k ? r.sel[i] : INT32_MAX;
    __syncthreads();
    for (int size = 2; size <= np; size <<= 1)
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < np / 2; i += kTmThreads) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool asc = (lo & size) == 0;
                const int a = srt[lo], b = srt[hi];
                if ((a > b) == asc) {
                    srt[lo] = b;
                    srt[hi] = a;
                }
            }
            __syncthreads();
        }
    for (int a = tid; a < k; a += kTmThreads) out[a] = srt[a];
}

static bool topk_multi(int64_t T, int64_t n_cols) { return T < 128 && n_cols > 4096; }

size_t topk_workspace_bytes(int64_t T, int64_t n_cols, int k) {
    if (!topk_multi(T, n_cols)) return 0;
    return (size_t)T * topk_row_stride(n_cols, k) + 256;
}

hipError_t launch_topk(const float* scores, int64_t T, int64_t n_cols, const int64_t* pos, int m, int k, int32_t* idx,
                       void* ws, hipStream_t st) {
    if (T == 0) return hipSuccess;
    if (!topk_multi(T, n_cols)) {
        hipLaunchKernelGGL(k_topk_row, dim3((unsigned)T), dim3(kTopkThreads), 0, st, scores, n_cols, pos, m, k, idx);
        return hipGetLastError();
    }
    int64_t chunk = (n_cols * T + 511) / 512;
    chunk = ((chunk + 2047) / 2048) * 2048;
    if (chunk < 2048) chunk = 2048;
    if (chunk > 16384) chunk = 16384;
    const int nchunk = (int)((n_cols + chunk - 1) / chunk);
    hipLaunchKernelGGL(k_topkm_clear, dim3((unsigned)T), dim3(kTmThreads), 0, st, ws, n_cols, k);
    hipLaunchKernelGGL(k_topkm_hist, dim3((unsigned)nchunk, (unsigned)T), dim3(kTmThreads), 0, st, scores, n_cols, pos,
                       m, k, chunk, ws);
    hipLaunchKernelGGL(k_topkm_collect, dim3((unsigned)nchunk, (unsigned)T), dim3(kTmThreads), 0, st, scores, n_cols,
                       pos, m, k, chunk, nchunk, ws, idx);
    return hipGetLastError();
}

}  // namespace csa
