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

constexpr int kTopkThreads = 1024;
constexpr int kTopkCache = 36608;  // keys cached in LDS (143 KB)

// exclusive prefix sum over the block; returns the block total in `total`
__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int x = wave_incl_scan(v);
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
    __shared__ __align__(16) uint32_t cache[kTopkCache];
    __shared__ int wsum[2 * (kTopkThreads / 64)];
    __shared__ int bcast[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
    auto key_at = [&](int j) -> uint32_t { return cached ? cache[j] : f32_order_key(row[j]); };
    for (int i = tid; i < 4096; i += kTopkThreads) hist[i] = 0;
    __syncthreads();

    // load the row into LDS (16-byte loads when aligned, several in flight) and histogram the top 12 bits
    if (cached && (((uintptr_t)row & 15) == 0)) {
        const int n4 = nv >> 2;
#pragma unroll 4
        for (int j4 = tid; j4 < n4; j4 += kTopkThreads) {
            const float4 v = ((const float4*)row)[j4];
            const uint4 kk = make_uint4(f32_order_key(v.x), f32_order_key(v.y), f32_order_key(v.z), f32_order_key(v.w));
            *(uint4*)&cache[4 * j4] = kk;
            atomicAdd(&hist[kk.x >> 20], 1u);
            atomicAdd(&hist[kk.y >> 20], 1u);
            atomicAdd(&hist[kk.z >> 20], 1u);
            atomicAdd(&hist[kk.w >> 20], 1u);
        }
        for (int j = 4 * n4 + tid; j < nv; j += kTopkThreads) {
            const uint32_t kk = f32_order_key(row[j]);
            cache[j] = kk;
            atomicAdd(&hist[kk >> 20], 1u);
        }
    } else {
        for (int j = tid; j < nv; j += kTopkThreads) {
            const uint32_t kk = f32_order_key(row[j]);
            if (cached) cache[j] = kk;
            atomicAdd(&hist[kk >> 20], 1u);
        }
    }
    __syncthreads();
    int above1;
    const uint32_t b1 = (uint32_t)find_bin<4096>(hist, k, wsum, bcast, above1);

    // refinement passes over the keys whose prefix matches (LDS read 4 keys at a time)
    auto refine = [&](auto match, auto bin) {
        if (cached) {
            const int n4 = nv >> 2;
            for (int j4 = tid; j4 < n4; j4 += kTopkThreads) {
                const uint4 kk = *(const uint4*)&cache[4 * j4];
                if (match(kk.x)) atomicAdd(&hist[bin(kk.x)], 1u);
                if (match(kk.y)) atomicAdd(&hist[bin(kk.y)], 1u);
                if (match(kk.z)) atomicAdd(&hist[bin(kk.z)], 1u);
                if (match(kk.w)) atomicAdd(&hist[bin(kk.w)], 1u);
            }
            for (int j = 4 * n4 + tid; j < nv; j += kTopkThreads) {
                const uint32_t kk = cache[j];
                if (match(kk)) atomicAdd(&hist[bin(kk)], 1u);
            }
        } else {
            for (int j = tid; j < nv; j += kTopkThreads) {
                const uint32_t kk = f32_order_key(row[j]);
                if (match(kk)) atomicAdd(&hist[bin(kk)], 1u);
            }
        }
    };

    // pass 2: middle 12 bits among keys with prefix b1
    for (int i = tid; i < 4096; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    refine([&](uint32_t kk) { return (kk >> 20) == b1; }, [](uint32_t kk) { return (kk >> 8) & 0xFFFu; });
    __syncthreads();
    int above2;
    const uint32_t b2 = (uint32_t)find_bin<4096>(hist, k - above1, wsum, bcast, above2);
    const uint32_t p2 = (b1 << 12) | b2;

    // pass 3: low 8 bits among keys with prefix p2
    for (int i = tid; i < 256; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    refine([&](uint32_t kk) { return (kk >> 8) == p2; }, [](uint32_t kk) { return kk & 0xFFu; });
    __syncthreads();
    int above3;
    const uint32_t b3 = (uint32_t)find_bin<256>(hist, k - above1 - above2, wsum, bcast, above3);
    const uint32_t thr = (p2 << 8) | b3;
    const int need_eq = k - (above1 + above2 + above3);

    // ordered compaction: wave w owns the contiguous columns [w seg, (w+1) seg); ranks within a
    // wave come from ballots, across waves from one exchange of (#greater, #equal) per wave
    constexpr int NW = kTopkThreads / 64;
    const int seg = (nv + NW * 64 - 1) / (NW * 64) * 64;
    const int s0 = wave * seg < nv ? wave * seg : nv;
    const int s1 = s0 + seg < nv ? s0 + seg : nv;
    const uint64_t lt = (1ull << lane) - 1ull;
    int cgt = 0, ceq = 0;
    for (int b = s0; b < s1; b += 64) {
        const int j = b + lane;
        const uint32_t kk = j < s1 ? key_at(j) : 0u;
        cgt += __popcll(__ballot(j < s1 && kk > thr));
        ceq += __popcll(__ballot(j < s1 && kk == thr));
    }
    if (lane == 0) {
        wsum[2 * wave] = cgt;
        wsum[2 * wave + 1] = ceq;
    }
    __syncthreads();
    int gtb = 0, eqb = 0;
    for (int w = 0; w < wave; ++w) {
        gtb += wsum[2 * w];
        eqb += wsum[2 * w + 1];
    }
    int eqrun = eqb, orun = gtb + (eqb < need_eq ? eqb : need_eq);
    for (int b = s0; b < s1; b += 64) {
        const int j = b + lane;
        const uint32_t kk = j < s1 ? key_at(j) : 0u;
        const bool eq = j < s1 && kk == thr;
        const uint64_t eqm = __ballot(eq);
        const bool sel = (j < s1 && kk > thr) || (eq && eqrun + __popcll(eqm & lt) < need_eq);
        const uint64_t selm = __ballot(sel);
        if (sel) out[orun + __popcll(selm & lt)] = j;
        eqrun += __popcll(eqm);
        orun += __popcll(selm);
    }
}

// ---------------------------------------------------------------------------
// Few long rows (decode): the row is split over many workgroups.
//   row summary      per kTopkGroup-column group, the largest order key of
//                    its visible columns (0 for a group with none), written
//                    by the indexer kernel next to the scores, or else by
//                    k_topkm_gmax
//   k_topkm_collect  per chunk.  tau = lower edge of the 12-bit key prefix
//                    holding the k-th largest group maximum (0 when the row
//                    has fewer than k groups).  The group maxima are keys of
//                    distinct columns, so the row's k-th largest key is
//                    >= tau and every column of the top-k (ties included)
//                    has key >= tau.  Appends (key, ~index) of the chunk's
//                    visible columns with key >= tau, one slot reservation
//                    per workgroup.
//   k_topkm_final    one workgroup per row: exact radix select over the
//                    candidates (12 + 12 + 8 key bits, equal keys to the
//                    lower index), marks the k winners in an LDS bitmap of
//                    the row, writes them in ascending order and resets the
//                    row's counters.
// The hand-overs are kernel boundaries: a per-workgroup agent-scope fence
// would write back the whole L2 (holding the freshly written scores).
// Workspace (topk_ws_* in csa_internal.hpp): 128 rows x 16 counters
// (zero-filled before first use, left zero-filled), the row summaries, then
// T x n_cols candidates.
// ---------------------------------------------------------------------------
constexpr int kTmThreads = 256;
constexpr int kTfThreads = 1024;     // the per-row finaliser
constexpr int kTmE = 8;              // consecutive columns per thread in the collect pass
constexpr int kBitmapWords = 16384;  // row bitmap of the finaliser: rows up to 524,288 columns
constexpr int kCandLds = 8192;       // candidates the finaliser stages in LDS
constexpr int kTieLds = 256;         // equal-key sets up to this size are ranked directly
static_assert(kTmThreads * kTmE % kTopkGroup == 0, "summary groups inside one collect step");

struct TmRow {
    uint32_t* ctr;   // [0] candidates
    uint32_t* gmax;  // [topk_groups(n_cols)] group maxima
    uint64_t* cand;  // [n_cols] (key << 32 | ~index)
};

__device__ __forceinline__ TmRow tm_row(void* ws, int64_t T, int64_t t, int64_t n_cols) {
    char* b = (char*)ws;
    TmRow r;
    r.ctr = (uint32_t*)(b + (size_t)t * 64);
    r.gmax = (uint32_t*)(b + topk_ws_gmax_off()) + t * topk_groups(n_cols);
    r.cand = (uint64_t*)(b + topk_ws_cand_off(T, n_cols)) + t * n_cols;
    return r;
}

__device__ __forceinline__ int64_t row_visible(const int64_t* pos, int64_t t, int m, int64_t n_cols) {
    int64_t nv = (pos[t] + 1) / m;
    if (nv > n_cols) nv = n_cols;
    if (nv < 0) nv = 0;
    return nv;
}

// Row summaries from the scores (when the indexer did not write them): 16
// threads x 8 consecutive columns per group.
__global__ __launch_bounds__(kTmThreads) void k_topkm_gmax(const float* __restrict__ scores, int64_t T,
                                                           int64_t n_cols, const int64_t* __restrict__ pos, int m,
                                                           int k, void* ws) {
    const int tid = threadIdx.x;
    const int64_t t = blockIdx.y;
    const int64_t nv = row_visible(pos, t, m, n_cols);
    if (nv <= k) return;
    const float* row = scores + t * n_cols;
    const int64_t j0 = (int64_t)blockIdx.x * (kTmThreads * 8) + tid * 8;
    uint32_t g = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (j0 + e < nv) g = max(g, f32_order_key(row[j0 + e]));
#pragma unroll
    for (int o = 1; o < kTopkGroup / 8; o <<= 1) g = max(g, (uint32_t)__shfl_xor((int)g, o));
    if ((tid & (kTopkGroup / 8 - 1)) == 0 && j0 < n_cols) tm_row(ws, T, t, n_cols).gmax[j0 / kTopkGroup] = g;
}

// Histograms handed to tm_find are stored "transposed": with PER = NB/256
// bins per thread and bins ranked from the top (r = NB-1-bin), rank r sits
// at position (r % PER) * 256 + r / PER.  Thread t then owns ranks
// t*PER .. t*PER+PER-1 and reads them at positions i*256 + t: consecutive
// threads, consecutive words, no LDS bank conflicts.
template <int NB, int NT = kTmThreads>
__device__ __forceinline__ int tm_pos(uint32_t bin) {
    constexpr int PER = NB / NT > 0 ? NB / NT : 1;
    const int r = NB - 1 - (int)bin;
    return (r % PER) * NT + r / PER;
}

// 4096-bin global histogram into the transposed LDS layout: thread t loads
// its PER = 4096/NT consecutive bins (16-byte loads, issued together) and
// scatters them.
template <int NT = kTmThreads>
__device__ __forceinline__ void tm_load_hist(uint32_t* dst, const uint32_t* src) {
    constexpr int PER = 4096 / NT, NV = PER / 4;
    const int t = threadIdx.x;
    uint4 v[NV];
    const uint4* p = (const uint4*)(src + 4096 - PER * (t + 1));  // bins 4096-PER(t+1) .. 4095-PER t
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = p[i];
    const uint32_t* w = (const uint32_t*)v;  // w[q] = bin 4096-PER(t+1)+q = rank PER t+PER-1-q
#pragma unroll
    for (int q = 0; q < PER; ++q) dst[(PER - 1 - q) * NT + t] = w[q];
}

// exclusive scan over an NT-thread block
template <int NT = kTmThreads>
__device__ __forceinline__ int tm_scan(int v, int* wsum, int& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int x = wave_incl_scan(v);
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
        off += i < wave ? wsum[i] : 0;
        tot += wsum[i];
    }
    __syncthreads();
    total = tot;
    return off + x - v;
}

// bin (scanning from the top) where the running count reaches need, on a
// transposed histogram; NT threads, one block scan.
template <int NB, int NT = kTmThreads>
__device__ int tm_find(const uint32_t* hist, int need, int* wsum, int* bc, int& above) {
    constexpr int PER = NB / NT > 0 ? NB / NT : 1;
    const int tid = threadIdx.x;
    uint32_t v[PER];
    int local = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        v[i] = tid * PER + i < NB ? hist[i * NT + tid] : 0u;
        local += (int)v[i];
    }
    int tot;
    const int before = tm_scan<NT>(local, wsum, tot);
    if (before < need && before + local >= need) {
        int run = before;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (run + (int)v[i] >= need) {
                bc[0] = NB - 1 - (tid * PER + i);
                bc[1] = run;
                break;
            }
            run += (int)v[i];
        }
    }
    __syncthreads();
    above = bc[1];
    const int bin = bc[0];
    __syncthreads();
    return bin;
}


__global__ __launch_bounds__(kTmThreads) void k_topkm_collect(const float* __restrict__ scores, int64_t T,
                                                              int64_t n_cols, const int64_t* __restrict__ pos, int m,
                                                              int k, int64_t chunk, void* ws,
                                                              int32_t* __restrict__ idx) {
    __shared__ uint32_t h[4096];
    __shared__ int wsum[kTmThreads / 64];
    __shared__ int bc[4];
    const int tid = threadIdx.x;
    const int64_t t = blockIdx.y;
    TmRow r = tm_row(ws, T, t, n_cols);
    // the row's group maxima (groups without visible columns hold 0) and this workgroup's first
    // scores are requested before anything that depends on pos, and the histogram is cleared
    // while they are in flight
    constexpr int GPT = 16;  // group maxima per thread held in registers (rows up to 524,288 columns)
    const int ng = (int)topk_groups(n_cols);
    uint32_t gv[GPT];
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
        const int gi = i * kTmThreads + tid;
        gv[i] = gi < ng ? r.gmax[gi] : 0u;
    }
    const int64_t c0 = (int64_t)blockIdx.x * chunk;
    const float* row = scores + t * n_cols;
    float pre[kTmE];
    {
        const int64_t j0 = c0 + (int64_t)tid * kTmE;
#pragma unroll
        for (int e = 0; e < kTmE; ++e) pre[e] = j0 + e < n_cols ? row[j0 + e] : 0.f;
    }
    for (int i = tid; i < 4096; i += kTmThreads) h[i] = 0;
    const int64_t nv = row_visible(pos, t, m, n_cols);
    int32_t* out = idx + t * (int64_t)k;
    if (nv <= k) {
        if (blockIdx.x == 0)
            for (int a = tid; a < k; a += kTmThreads) out[a] = a < nv ? a : -1;
        return;
    }
    const int64_t c1 = c0 + chunk < nv ? c0 + chunk : nv;

    // ---- tau: the lower edge of the 12-bit key prefix holding the k-th largest group maximum
    //      (0 when the row has fewer than k groups) ----
    uint32_t tau = 0;
    if (ng >= k) {
        const bool more = ng > GPT * kTmThreads;  // longer rows re-read the rest from global memory
        __syncthreads();
#pragma unroll
        for (int i = 0; i < GPT; ++i)
            if (i * kTmThreads + tid < ng) atomicAdd(&h[tm_pos<4096>(gv[i] >> 20)], 1u);
        if (more)
            for (int gi = GPT * kTmThreads + tid; gi < ng; gi += kTmThreads) atomicAdd(&h[tm_pos<4096>(r.gmax[gi] >> 20)], 1u);
        __syncthreads();
        int ab1;
        const uint32_t g1 = (uint32_t)tm_find<4096>(h, k, wsum, bc, ab1);
        tau = g1 << 20;
    }

    // ---- candidates of this chunk: E consecutive columns per thread, one slot reservation ----
    for (int64_t jb = c0; jb < c1; jb += (int64_t)kTmThreads * kTmE) {
        const int64_t j0 = jb + (int64_t)tid * kTmE;
        uint32_t key[kTmE];
        int n_c = 0;
#pragma unroll
        for (int e = 0; e < kTmE; ++e) {
            const int64_t j = j0 + e;
            key[e] = j < c1 ? f32_order_key(jb == c0 ? pre[e] : row[j]) : 0u;
            n_c += (j < c1 && key[e] >= tau) ? 1 : 0;
        }
        int tot;
        const int before = tm_scan(n_c, wsum, tot);
        if (tid == 0) bc[2] = tot ? (int)atomicAdd(&r.ctr[0], (uint32_t)tot) : 0;
        __syncthreads();
        uint32_t sc = (uint32_t)bc[2] + (uint32_t)before;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < kTmE; ++e) {
            const int64_t j = j0 + e;
            if (j < c1 && key[e] >= tau) r.cand[sc++] = ((uint64_t)key[e] << 32) | (uint32_t)~(uint32_t)j;
        }
    }
}

__global__ __launch_bounds__(kTfThreads) void k_topkm_final(int64_t T, int64_t n_cols, const int64_t* __restrict__ pos,
                                                            int m, int k, void* ws, int32_t* __restrict__ idx) {
    constexpr int NT = kTfThreads;
    __shared__ uint32_t h[4096];
    __shared__ uint32_t bm[kBitmapWords];  // row bitmap, or the index list to sort
    __shared__ uint64_t cl[kCandLds];      // candidates
    __shared__ uint32_t tie[kTieLds];      // indices of keys equal to the threshold
    __shared__ int wsum[NT / 64];
    __shared__ int bc[4];
    __shared__ uint32_t lctr[3];
    const int tid = threadIdx.x;
    const int64_t t = blockIdx.x;
    const int64_t nv = row_visible(pos, t, m, n_cols);
    int32_t* out = idx + t * (int64_t)k;
    if (nv <= k) return;  // written by the collect pass
    TmRow r = tm_row(ws, T, t, n_cols);
    const int n_cand = (int)r.ctr[0];
    const int64_t nwords = (nv + 31) / 32;
    const bool use_bm = nwords <= kBitmapWords;  // kBitmapWords is a multiple of NT
    // bitmap word w belongs to thread w / perw and sits at (w % perw) * NT + w / perw
    const uint32_t perw = (uint32_t)((nwords + NT - 1) / NT);
    if (use_bm)
        for (uint32_t i = tid; i < perw * NT; i += NT) bm[i] = 0;
    if (tid < 2) lctr[tid] = 0;
    for (int i = tid; i < 4096; i += NT) h[i] = 0;
    auto mark = [&](uint32_t j) {
        if (use_bm) {
            if (j < (uint64_t)nv) {
                const uint32_t wd = j >> 5;
                atomicOr(&bm[(wd % perw) * NT + wd / perw], 1u << (j & 31));
            }
        } else {
            const uint32_t o = atomicAdd(&lctr[1], 1u);
            if (o < (uint32_t)k) bm[o] = j;
        }
    };
    // candidates into LDS (batched loads), when they fit
    const bool cand_lds = n_cand <= kCandLds;
    if (cand_lds) {
        for (int i0 = 0; i0 < n_cand; i0 += NT * 4) {
            uint64_t v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + u * NT + tid;
                v[u] = i < n_cand ? r.cand[i] : 0;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + u * NT + tid;
                if (i < n_cand) cl[i] = v[u];
            }
        }
    }
    __syncthreads();
    auto cand_at = [&](int i) -> uint64_t { return cand_lds ? cl[i] : r.cand[i]; };
    // radix select of the k-th largest candidate key: 12, 12, 8 bits
    for (int i = tid; i < n_cand; i += NT) atomicAdd(&h[tm_pos<4096, NT>((uint32_t)(cand_at(i) >> 52))], 1u);
    __syncthreads();
    int above1;
    const uint32_t b1 = (uint32_t)tm_find<4096, NT>(h, k, wsum, bc, above1);
    for (int i = tid; i < 4096; i += NT) h[i] = 0;
    __syncthreads();
    for (int i = tid; i < n_cand; i += NT) {
        const uint32_t key = (uint32_t)(cand_at(i) >> 32);
        if ((key >> 20) == b1) atomicAdd(&h[tm_pos<4096, NT>((key >> 8) & 0xFFFu)], 1u);
    }
    __syncthreads();
    int above2;
    const int need = k - above1;
    const uint32_t b2 = (uint32_t)tm_find<4096, NT>(h, need, wsum, bc, above2);
    for (int i = tid; i < 256; i += NT) h[i] = 0;
    __syncthreads();
    const uint32_t p2 = (b1 << 12) | b2;
    for (int i = tid; i < n_cand; i += NT) {
        const uint32_t key = (uint32_t)(cand_at(i) >> 32);
        if ((key >> 8) == p2) atomicAdd(&h[tm_pos<256, NT>(key & 0xFFu)], 1u);
    }
    __syncthreads();
    int above3;
    const uint32_t b3 = (uint32_t)tm_find<256, NT>(h, need - above2, wsum, bc, above3);
    const uint32_t thr = (p2 << 8) | b3;
    const int need_eq = need - above2 - above3;  // >= 1 keys equal to thr, lowest indices first
    for (int i = tid; i < n_cand; i += NT) {
        const uint64_t c = cand_at(i);
        const uint32_t key = (uint32_t)(c >> 32);
        if (key > thr) mark(~(uint32_t)c);
        else if (key == thr) atomicAdd(&lctr[0], 1u);
    }
    __syncthreads();
    uint32_t idx_lim = 0xFFFFFFFFu;  // equal keys are taken up to this index
    const int n_eq = (int)lctr[0];
    if (n_eq > need_eq && n_eq <= kTieLds) {
        // few equal keys: list them, rank each by index, keep the need_eq lowest
        if (tid == 0) lctr[2] = 0;
        __syncthreads();
        for (int i = tid; i < n_cand; i += NT) {
            const uint64_t c = cand_at(i);
            if ((uint32_t)(c >> 32) == thr) tie[atomicAdd(&lctr[2], 1u)] = ~(uint32_t)c;
        }
        __syncthreads();
        for (int i = tid; i < n_eq; i += NT) {
            const uint32_t ji = tie[i];
            int rank = 0;
            for (int q = 0; q < n_eq; ++q) rank += tie[q] < ji ? 1 : 0;
            if (rank == need_eq - 1) bc[2] = (int)ji;
        }
        __syncthreads();
        idx_lim = (uint32_t)bc[2];
        __syncthreads();
    } else if (n_eq > need_eq) {
        // the need_eq-th smallest index among equal keys (31-bit indices, 3 passes of 11 bits)
        uint32_t pre = 0, pm = 0;
        int nl = need_eq;
        for (int sh = 22; sh >= 0; sh -= 11) {
            for (int i = tid; i < 2048; i += NT) h[i] = 0;
            __syncthreads();
            for (int i = tid; i < n_cand; i += NT) {
                const uint64_t c = cand_at(i);
                if ((uint32_t)(c >> 32) != thr) continue;
                const uint32_t jx = ~(uint32_t)c;
                if ((jx & pm) == pre) atomicAdd(&h[tm_pos<2048, NT>(2047 - ((jx >> sh) & 0x7FF))], 1u);  // smaller index, higher bin
            }
            __syncthreads();
            int ab;
            const uint32_t bn = 2047u - (uint32_t)tm_find<2048, NT>(h, nl, wsum, bc, ab);
            nl -= ab;
            pre |= bn << sh;
            pm |= 0x7FFu << sh;
        }
        idx_lim = pre;
    }
    for (int i = tid; i < n_cand; i += NT) {
        const uint64_t c = cand_at(i);
        if ((uint32_t)(c >> 32) == thr && ~(uint32_t)c <= idx_lim) mark(~(uint32_t)c);
    }
    __syncthreads();
    if (use_bm) {
        // thread t owns words t*perw .. t*perw+perw-1 (reads free of bank conflicts)
        int cnt = 0;
        for (uint32_t i = 0; i < perw; ++i) cnt += __popc(bm[i * NT + tid]);
        int tot;
        int o = tm_scan<NT>(cnt, wsum, tot);
        for (uint32_t i = 0; i < perw; ++i) {
            uint32_t b = bm[i * NT + tid];
            const int64_t wi = (int64_t)tid * perw + i;
            while (b) {
                const int bit = __builtin_ctz(b);
                if (o < k) out[o] = (int32_t)(wi * 32 + bit);
                ++o;
                b &= b - 1;
            }
        }
    } else {
        // bitonic sort of the k marked indices
        int np = 1;
        while (np < k) np <<= 1;
        for (int i = k + tid; i < np; i += NT) bm[i] = 0xFFFFFFFFu;
        __syncthreads();
        for (int size = 2; size <= np; size <<= 1)
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int i = tid; i < np / 2; i += NT) {
                    const int lo = 2 * i - (i & (stride - 1));
                    const int hi = lo + stride;
                    const bool asc = (lo & size) == 0;
                    const uint32_t a = bm[lo], b = bm[hi];
                    if ((a > b) == asc) {
                        bm[lo] = b;
                        bm[hi] = a;
                    }
                }
                __syncthreads();
            }
        for (int a = tid; a < k; a += NT) out[a] = (int32_t)bm[a];
    }
    // ---- leave the row's counters zero for the next call ----
    if (tid < 16) r.ctr[tid] = 0;
}

// ---------------------------------------------------------------------------
// Many rows of up to kTsMaxCols columns: one workgroup per row streams the
// row twice instead of caching it (so several rows share a CU):
//   pass A  histogram of the top 12 key bits -> bin b1 holding the k-th key
//   pass B  keys above b1 go straight into an LDS bitmap of the row; keys in
//           b1 (the boundary) go to an LDS list as (key << 32 | ~index)
//   the boundary is resolved exactly on the list (12 + 8 key bits, then the
//   lowest indices among equal keys), its winners are marked, and the
//   bitmap is written out in ascending order.
// A boundary bin larger than the list is resolved by further streamed
// passes (12 + 8 key bits, index bits for ties) that mark the bitmap.
// ---------------------------------------------------------------------------
constexpr int kTsThreads = 512;
constexpr int kTsMaxCols = 65536;  // bitmap of 2048 words
constexpr int kTsCand = 4096;      // boundary keys held in LDS

__global__ __launch_bounds__(kTsThreads) void k_topk_stream(const float* __restrict__ scores, int64_t n_cols,
                                                            const int64_t* __restrict__ pos, int m, int k,
                                                            int32_t* __restrict__ idx) {
    constexpr int NT = kTsThreads;
    __shared__ uint32_t h[4096];
    __shared__ uint32_t bm[kTsMaxCols / 32];
    __shared__ uint64_t cl[kTsCand];
    __shared__ uint32_t tie[kTieLds];
    __shared__ int wsum[NT / 64];
    __shared__ int bc[4];
    __shared__ uint32_t lctr[3];
    const int tid = threadIdx.x;
    const int64_t t = blockIdx.x;
    const int64_t nv64 = row_visible(pos, t, m, n_cols);
    const int nv = (int)nv64;
    const float* row = scores + t * n_cols;
    int32_t* out = idx + t * (int64_t)k;
    if (nv <= k) {
        for (int a = tid; a < k; a += NT) out[a] = a < nv ? a : -1;
        return;
    }
    const int nwords = (nv + 31) / 32;
    const int perw = (nwords + NT - 1) / NT;  // word w at (w % perw) * NT + w / perw (conflict-free emission)
    for (int i = tid; i < perw * NT; i += NT) bm[i] = 0;
    for (int i = tid; i < 4096; i += NT) h[i] = 0;
    if (tid < 3) lctr[tid] = 0;
    __syncthreads();
    auto mark = [&](uint32_t j) {
        const uint32_t wd = j >> 5;
        atomicOr(&bm[(wd % perw) * NT + wd / perw], 1u << (j & 31));
    };
    // visible keys of the row, 16-byte loads (several in flight) when the row is aligned
    const bool vec = (((uintptr_t)row & 15) == 0);
    auto stream = [&](auto fn) {
        int j0 = 0;
        if (vec) {
            const int n4 = nv >> 2;
#pragma unroll 4
            for (int j4 = tid; j4 < n4; j4 += NT) {
                const float4 v = ((const float4*)row)[j4];
                fn(f32_order_key(v.x), 4 * j4);
                fn(f32_order_key(v.y), 4 * j4 + 1);
                fn(f32_order_key(v.z), 4 * j4 + 2);
                fn(f32_order_key(v.w), 4 * j4 + 3);
            }
            j0 = 4 * n4;
        }
        for (int j = j0 + tid; j < nv; j += NT) fn(f32_order_key(row[j]), j);
    };

    // ---- pass A ----
    stream([&](uint32_t key, int) { atomicAdd(&h[tm_pos<4096, NT>(key >> 20)], 1u); });
    __syncthreads();
    int above1;
    const uint32_t b1 = (uint32_t)tm_find<4096, NT>(h, k, wsum, bc, above1);
    const int n_b1 = (int)h[tm_pos<4096, NT>(b1)];
    const int need = k - above1;  // >= 1 keys of bin b1
    __syncthreads();
    for (int i = tid; i < 4096; i += NT) h[i] = 0;
    __syncthreads();

    if (n_b1 <= kTsCand) {
        // ---- pass B: mark above b1, list b1 ----
        stream([&](uint32_t key, int j) {
            const uint32_t bin = key >> 20;
            if (bin > b1) mark((uint32_t)j);
            else if (bin == b1) cl[atomicAdd(&lctr[0], 1u)] = ((uint64_t)key << 32) | (uint32_t)~(uint32_t)j;
        });
        __syncthreads();
        const int n_cand = n_b1;
        for (int i = tid; i < n_cand; i += NT) {
            const uint32_t key = (uint32_t)(cl[i] >> 32);
            atomicAdd(&h[tm_pos<4096, NT>((key >> 8) & 0xFFFu)], 1u);
        }
        __syncthreads();
        int above2;
        const uint32_t b2 = (uint32_t)tm_find<4096, NT>(h, need, wsum, bc, above2);
        for (int i = tid; i < 256; i += NT) h[i] = 0;
        __syncthreads();
        const uint32_t p2 = (b1 << 12) | b2;
        for (int i = tid; i < n_cand; i += NT) {
            const uint32_t key = (uint32_t)(cl[i] >> 32);
            if ((key >> 8) == p2) atomicAdd(&h[tm_pos<256, NT>(key & 0xFFu)], 1u);
        }
        __syncthreads();
        int above3;
        const uint32_t b3 = (uint32_t)tm_find<256, NT>(h, need - above2, wsum, bc, above3);
        const uint32_t thr = (p2 << 8) | b3;
        const int need_eq = need - above2 - above3;
        for (int i = tid; i < n_cand; i += NT) {
            const uint64_t c = cl[i];
            const uint32_t key = (uint32_t)(c >> 32);
            if (key > thr) mark(~(uint32_t)c);
            else if (key == thr) atomicAdd(&lctr[1], 1u);
        }
        __syncthreads();
        uint32_t idx_lim = 0xFFFFFFFFu;  // equal keys are taken up to this index
        const int n_eq = (int)lctr[1];
        if (n_eq > need_eq && n_eq <= kTieLds) {
            for (int i = tid; i < n_cand; i += NT) {
                const uint64_t c = cl[i];
                if ((uint32_t)(c >> 32) == thr) tie[atomicAdd(&lctr[2], 1u)] = ~(uint32_t)c;
            }
            __syncthreads();
            for (int i = tid; i < n_eq; i += NT) {
                const uint32_t ji = tie[i];
                int rank = 0;
                for (int q = 0; q < n_eq; ++q) rank += tie[q] < ji ? 1 : 0;
                if (rank == need_eq - 1) bc[2] = (int)ji;
            }
            __syncthreads();
            idx_lim = (uint32_t)bc[2];
            __syncthreads();
        } else if (n_eq > need_eq) {
            uint32_t pre = 0, pm = 0;
            int nl = need_eq;
            for (int sh = 22; sh >= 0; sh -= 11) {
                for (int i = tid; i < 2048; i += NT) h[i] = 0;
                __syncthreads();
                for (int i = tid; i < n_cand; i += NT) {
                    const uint64_t c = cl[i];
                    if ((uint32_t)(c >> 32) != thr) continue;
                    const uint32_t jx = ~(uint32_t)c;
                    if ((jx & pm) == pre) atomicAdd(&h[tm_pos<2048, NT>(2047 - ((jx >> sh) & 0x7FF))], 1u);
                }
                __syncthreads();
                int ab;
                const uint32_t bn = 2047u - (uint32_t)tm_find<2048, NT>(h, nl, wsum, bc, ab);
                nl -= ab;
                pre |= bn << sh;
                pm |= 0x7FFu << sh;
            }
            idx_lim = pre;
        }
        for (int i = tid; i < n_cand; i += NT) {
            const uint64_t c = cl[i];
            if ((uint32_t)(c >> 32) == thr && ~(uint32_t)c <= idx_lim) mark(~(uint32_t)c);
        }
    } else {
        // ---- large boundary bin: streamed refinement ----
        stream([&](uint32_t key, int) {
            if ((key >> 20) == b1) atomicAdd(&h[tm_pos<4096, NT>((key >> 8) & 0xFFFu)], 1u);
        });
        __syncthreads();
        int above2;
        const uint32_t b2 = (uint32_t)tm_find<4096, NT>(h, need, wsum, bc, above2);
        for (int i = tid; i < 256; i += NT) h[i] = 0;
        __syncthreads();
        const uint32_t p2 = (b1 << 12) | b2;
        stream([&](uint32_t key, int) {
            if ((key >> 8) == p2) atomicAdd(&h[tm_pos<256, NT>(key & 0xFFu)], 1u);
        });
        __syncthreads();
        int above3;
        const uint32_t b3 = (uint32_t)tm_find<256, NT>(h, need - above2, wsum, bc, above3);
        const uint32_t thr = (p2 << 8) | b3;
        const int need_eq = need - above2 - above3;
        const int n_eq = (int)h[tm_pos<256, NT>(b3)];
        uint32_t idx_lim = 0xFFFFFFFFu;
        if (n_eq > need_eq) {
            uint32_t pre = 0, pm = 0;
            int nl = need_eq;
            for (int sh = 22; sh >= 0; sh -= 11) {
                __syncthreads();
                for (int i = tid; i < 2048; i += NT) h[i] = 0;
                __syncthreads();
                stream([&](uint32_t key, int j) {
                    const uint32_t jx = (uint32_t)j;
                    if (key == thr && (jx & pm) == pre) atomicAdd(&h[tm_pos<2048, NT>(2047 - ((jx >> sh) & 0x7FF))], 1u);
                });
                __syncthreads();
                int ab;
                const uint32_t bn = 2047u - (uint32_t)tm_find<2048, NT>(h, nl, wsum, bc, ab);
                nl -= ab;
                pre |= bn << sh;
                pm |= 0x7FFu << sh;
            }
            idx_lim = pre;
        }
        stream([&](uint32_t key, int j) {
            if (key > thr || (key == thr && (uint32_t)j <= idx_lim)) mark((uint32_t)j);
        });
    }
    __syncthreads();
    // ---- emit in ascending order: thread t owns words t*perw .. t*perw+perw-1 ----
    int cnt = 0;
    for (int i = 0; i < perw; ++i) cnt += __popc(bm[i * NT + tid]);
    int tot;
    int o = tm_scan<NT>(cnt, wsum, tot);
    for (int i = 0; i < perw; ++i) {
        uint32_t b = bm[i * NT + tid];
        const int wi = tid * perw + i;
        while (b) {
            const int bit = __builtin_ctz(b);
            if (o < k) out[o] = wi * 32 + bit;
            ++o;
            b &= b - 1;
        }
    }
}

static bool topk_multi(int64_t T, int64_t n_cols) { return T < kTopkMaxRows && n_cols > 4096; }

size_t topk_workspace_bytes(int64_t T, int64_t n_cols, int) {
    if (!topk_multi(T, n_cols)) return 0;
    return topk_ws_cand_off(T, n_cols) + (size_t)T * n_cols * 8;
}

int64_t topk_chunk(int64_t T, int64_t n_cols) {
    int64_t chunk = (n_cols * T + 511) / 512;
    chunk = ((chunk + 2047) / 2048) * 2048;
    if (chunk < 2048) chunk = 2048;
    if (chunk > 16384) chunk = 16384;
    return chunk;
}

hipError_t launch_topk(const float* scores, int64_t T, int64_t n_cols, const int64_t* pos, int m, int k, int32_t* idx,
                       void* ws, bool prepared, hipStream_t st) {
    if (T == 0) return hipSuccess;
    if (!topk_multi(T, n_cols)) {
        if (n_cols <= kTsMaxCols)
            hipLaunchKernelGGL(k_topk_stream, dim3((unsigned)T), dim3(kTsThreads), 0, st, scores, n_cols, pos, m, k, idx);
        else
            hipLaunchKernelGGL(k_topk_row, dim3((unsigned)T), dim3(kTopkThreads), 0, st, scores, n_cols, pos, m, k, idx);
        return hipGetLastError();
    }
    const int64_t chunk = topk_chunk(T, n_cols);
    const int nchunk = (int)((n_cols + chunk - 1) / chunk);
    if (!prepared)
        hipLaunchKernelGGL(k_topkm_gmax, dim3((unsigned)((n_cols + kTmThreads * 8 - 1) / (kTmThreads * 8)), (unsigned)T),
                           dim3(kTmThreads), 0, st, scores, T, n_cols, pos, m, k, ws);
    hipLaunchKernelGGL(k_topkm_collect, dim3((unsigned)nchunk, (unsigned)T), dim3(kTmThreads), 0, st, scores, T, n_cols,
                       pos, m, k, chunk, ws, idx);
    hipLaunchKernelGGL(k_topkm_final, dim3((unsigned)T), dim3(kTfThreads), 0, st, T, n_cols, pos, m, k, ws, idx);
    return hipGetLastError();
}

bool topk_uses_summary(int64_t T, int64_t n_cols) { return topk_multi(T, n_cols); }

}  // namespace csa
