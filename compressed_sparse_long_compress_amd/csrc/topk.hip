// csa_topk kernels: exact top-k per row under the order (score desc, index
// asc), written in ascending index order.  Scores map to order-preserving
// 32-bit keys (select_device.hpp).  The kernel is picked by shape: the row
// held in registers (many rows of up to 36,864 columns), streamed twice
// (up to 65,536), a whole-row radix select (longer rows, many of them), or
// a selection from the row summary (few long rows, decode).
#include <atomic>
#include <mutex>

#include "csa_device.hpp"
#include "csa_internal.hpp"
#include "select_device.hpp"

namespace csa {

__global__ __launch_bounds__(kTopkThreads) void k_topk_row(const float* __restrict__ scores, int64_t n_cols,
                                                           const int64_t* __restrict__ pos, int m, int k,
                                                           int32_t* __restrict__ idx) {
    __shared__ uint32_t hist[4096];
    __shared__ __align__(16) uint32_t cache[kTopkCache];
    __shared__ int wsum[2 * (kTopkThreads / 64)];
    __shared__ int bcast[4];
    const int64_t t = blockIdx.x;
    int64_t nv64 = (pos[t] + 1) / m;
    if (nv64 > n_cols) nv64 = n_cols;
    if (nv64 < 0) nv64 = 0;
    const int nv = (int)nv64;
    int32_t* out = idx + t * (int64_t)k;
    if (nv <= k) {
        for (int a = threadIdx.x; a < k; a += kTopkThreads) out[a] = a < nv ? a : -1;
        return;
    }
    row_select(scores + t * n_cols, nv, k, out, hist, cache, kTopkCache, wsum, bcast);
}

// ---------------------------------------------------------------------------
// Few long rows (decode): selection from the row summary, in two kernels.
//   row summary    per kTopkGroup-column group, the largest order key of its
//                  visible columns (0 for a group with none).  Written by the
//                  indexer kernel next to the scores, or else by k_topk_gmax.
//   k_topk_cand    grid (slices, rows).  Every workgroup derives the same
//                  tau from the whole summary: the lower edge of a narrow key
//                  window holding the k-th largest group maximum.  The group
//                  maxima are keys of distinct columns, so the row's k-th
//                  largest key is >= tau: every column of the top-k (ties
//                  included) has key >= tau and lies in a group whose maximum
//                  is >= tau.  The workgroup reads back only those groups of
//                  its slice of the row (about k groups per row in all) and
//                  writes their keys >= tau as (key << 32 | ~column) to its
//                  slice of the candidate buffer, with the count, tau and the
//                  row's largest key in its record.
//   k_topk_pick    one workgroup per row: gathers the candidates into LDS,
//                  finds the k-th largest by a histogram descent, ranks the
//                  few keys of its window directly (equal keys to the lower
//                  column), marks the winners in an LDS bitmap of the row and
//                  writes them in ascending order.  When a slice overflowed
//                  or the candidates exceed LDS (heavy ties), the row is
//                  selected by row_select over the whole row instead.
// The hand-overs are kernel boundaries: a per-workgroup agent-scope fence
// would write back the whole L2 (holding the freshly written scores).
// ---------------------------------------------------------------------------
constexpr int kTgThreads = 256;      // k_topk_gmax: 8 consecutive columns per thread
constexpr int kTcThreads = 1024;     // k_topk_cand
constexpr int kTcChunks = 1;         // 8-group chunks per k_topk_cand thread held in registers
constexpr int kTqCand = 8192;        // candidates k_topk_pick holds in LDS
constexpr int kMaxSlices = 32;       // k_topk_cand workgroups (slices) per row, at most
constexpr int kTpThreads = 1024;     // k_topk_pick
constexpr int kBitmapWords = 16384;  // k_topk_pick's row bitmap: rows up to 524,288 columns

__global__ __launch_bounds__(kTgThreads) void k_topk_gmax(const float* __restrict__ scores, int64_t n_cols,
                                                          const int64_t* __restrict__ pos, int m, int k,
                                                          uint32_t* __restrict__ summ) {
    constexpr int TPG = kTopkGroup / 8;  // threads per group
    const int tid = threadIdx.x;
    const int64_t t = blockIdx.y;
    const int64_t nv = row_visible(pos, t, m, n_cols);
    if (nv <= k) return;
    const float* row = scores + t * n_cols;
    const int64_t j0 = (int64_t)blockIdx.x * (kTgThreads * 8) + tid * 8;
    uint32_t g = 0;
    for (int e = 0; e < 8; ++e)
        if (j0 + e < nv) g = max(g, f32_order_key(row[j0 + e]));
#pragma unroll
    for (int o = 1; o < TPG; o <<= 1) g = max(g, (uint32_t)__shfl_xor((int)g, o));
    if ((tid & (TPG - 1)) == 0 && j0 < n_cols) summ[t * topk_groups(n_cols) + j0 / kTopkGroup] = g;
}

// j-th largest (1 <= j <= 8) of 8 values held in registers: the maximum, or a
// descending sorting network (19 compare-exchanges) and a select
__device__ __forceinline__ uint32_t jth_largest8(const uint32_t* v, int j) {
    if (j == 1) {
        uint32_t r = v[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) r = max(r, v[i]);
        return r;
    }
    uint32_t a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = v[i];
    constexpr int net[19][2] = {{0, 2}, {1, 3}, {4, 6}, {5, 7}, {0, 4}, {1, 5}, {2, 6}, {3, 7}, {0, 1}, {2, 3},
                                {4, 5}, {6, 7}, {2, 4}, {3, 5}, {1, 4}, {3, 6}, {1, 2}, {3, 4}, {5, 6}};
#pragma unroll
    for (int c = 0; c < 19; ++c) {
        const uint32_t x = a[net[c][0]], y = a[net[c][1]];
        a[net[c][0]] = max(x, y);
        a[net[c][1]] = min(x, y);
    }
    uint32_t r = a[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) r = j == i + 1 ? a[i] : r;
    return r;
}

// Keys of B 16-byte pieces (4 columns from col[b]; 0 past nv) of a row.  Aligned rows: every
// piece's load is issued before the first is used (a load per piece inside the branch that
// handles a partial piece would wait for each in turn); a piece reaching past nv loads the
// row's first 16 bytes instead and is re-read by element.
template <int B>
__device__ __forceinline__ void group_pieces(const float* __restrict__ row, int nv, bool vec, const int (&col)[B],
                                             uint32_t (&key)[B][4]) {
    if (vec) {
        float4 x[B];
#pragma unroll
        for (int b = 0; b < B; ++b) x[b] = *(const float4*)(row + (col[b] + 4 <= nv ? col[b] : 0));
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (col[b] + 4 <= nv) {
                key[b][0] = f32_order_key(x[b].x);
                key[b][1] = f32_order_key(x[b].y);
                key[b][2] = f32_order_key(x[b].z);
                key[b][3] = f32_order_key(x[b].w);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) key[b][e] = col[b] + e < nv ? f32_order_key(row[col[b] + e]) : 0u;
            }
        }
    } else {
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int e = 0; e < 4; ++e) key[b][e] = col[b] + e < nv ? f32_order_key(row[col[b] + e]) : 0u;
    }
}

struct TcRec {  // per (row, slice): candidates written (may exceed the slice), tau, the row's largest key
    uint32_t n, tau, hi, pad;
};

__global__ __launch_bounds__(kTcThreads) void k_topk_cand(const float* __restrict__ scores, int64_t n_cols,
                                                          const int64_t* __restrict__ pos, int m, int k,
                                                          const uint32_t* __restrict__ summ, int S, int cap,
                                                          TcRec* __restrict__ recs, uint64_t* __restrict__ cands) {
    constexpr int NT = kTcThreads, NW = NT / 64, CH = kTcChunks, RC = NT * CH;  // RC chunks in registers
    constexpr int GS = kTopkGroup;
    __shared__ uint32_t h[4096];
    __shared__ uint32_t glist[2048];
    __shared__ int wsum[NW];
    __shared__ uint32_t red[2 * NW];
    __shared__ int bc[4];
    __shared__ uint32_t lctr[2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t t = blockIdx.y;
    const int s = blockIdx.x;
    const float* row = scores + t * n_cols;
    const int64_t ng_all = topk_groups(n_cols);
    const uint32_t* gs = summ + t * ng_all;
    // chunk c of thread tid = groups [8 (c NT + tid), +8); the first CH chunks are requested first
    const bool gvec = (((uintptr_t)gs) & 15) == 0;
    uint32_t gv[CH][8];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int64_t g0 = (int64_t)(c * NT + tid) * 8;
        if (gvec && g0 + 8 <= ng_all) {
            const uint4 a = ((const uint4*)(gs + g0))[0], b = ((const uint4*)(gs + g0))[1];
            gv[c][0] = a.x, gv[c][1] = a.y, gv[c][2] = a.z, gv[c][3] = a.w;
            gv[c][4] = b.x, gv[c][5] = b.y, gv[c][6] = b.z, gv[c][7] = b.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) gv[c][i] = g0 + i < ng_all ? gs[g0 + i] : 0u;
        }
    }
    if (tid < 2) lctr[tid] = 0;
    for (int i = tid; i < 4096; i += NT) h[i] = 0;
    const int nv = (int)row_visible(pos, t, m, n_cols);
    if (nv <= k) return;  // written by k_topk_pick
    const int ngv = (nv + GS - 1) / GS;  // groups holding visible columns
    const int nch = (ngv + 7) / 8;
    // visit every visible group maximum: chunks held in registers, the rest re-read
    auto for_groups = [&](auto fn) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int g0 = (c * NT + tid) * 8;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (g0 + i < ngv) fn(gv[c][i]);
        }
        for (int c = RC + tid; c < nch; c += NT)
            for (int i = 0; i < 8; ++i)
                if (c * 8 + i < ngv) fn(gs[c * 8 + i]);
    };

    // ---- hi = the row's largest key; lo <= the k-th largest group maximum: over the chunks
    //      held in registers whose 8 groups are all visible, the smallest of each one's j-th
    //      largest, j = ceil(k / #chunks) (those values come from >= k distinct groups) ----
    uint32_t hi, lo;
    {
        uint32_t mx = 0;
        for_groups([&](uint32_t x) { mx = max(mx, x); });
        const int n_full = (ngv < RC * 8 ? ngv : RC * 8) / 8;
        const int j = n_full > 0 ? (k + n_full - 1) / n_full : 9;
        uint32_t mn = j > 8 ? 0u : 0xFFFFFFFFu;
        if (j <= 8) {
#pragma unroll
            for (int c = 0; c < CH; ++c)
                if (c * NT + tid < n_full) mn = min(mn, jth_largest8(gv[c], j));
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
            mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
        }
        if (lane == 0) {
            red[wave] = mx;
            red[NW + wave] = mn;
        }
        __syncthreads();
        hi = red[0];
        lo = red[NW];
#pragma unroll
        for (int w = 1; w < NW; ++w) {
            hi = max(hi, red[w]);
            lo = min(lo, red[NW + w]);
        }
    }

    // ---- tau (h was cleared before the barrier above) ----
    uint32_t tau = 0;
    if (ngv >= k) {
        int sh, ab, nb;
        hist_descend<NT>(for_groups, lo, hi, k, 64, h, wsum, bc, tau, sh, ab, nb);
    }

    // ---- this slice's groups whose maximum is >= tau (any order) ----
    const int q0 = (int)((int64_t)ngv * s / S), q1 = (int)((int64_t)ngv * (s + 1) / S);
    for (int q = q0 + tid; q < q1; q += NT) {
        const uint32_t g = gs[q];
        if (g >= tau) {
            const uint32_t o = atomicAdd(&lctr[0], 1u);
            if (o < 2048u) glist[o] = (uint32_t)q;
        }
    }
    __syncthreads();
    const int nq = (int)lctr[0];
    uint64_t* out = cands + ((int64_t)t * S + s) * cap;
    bool over = nq > 2048;
    if (!over) {
        // ---- keys >= tau of the listed groups, 8 lanes x 16 bytes per group ----
        const bool vec = ((uintptr_t)row & 15) == 0;
        constexpr int B = 4;
        for (int u0 = 0; u0 < nq * 8; u0 += B * NT) {
            uint32_t key[B][4];
            int col[B];
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const int u = u0 + b * NT + tid;
                col[b] = u < nq * 8 ? (int)glist[u >> 3] * GS + (u & 7) * 4 : nv;
            }
            group_pieces<B>(row, nv, vec, col, key);
            int c = 0;
#pragma unroll
            for (int b = 0; b < B; ++b)
#pragma unroll
                for (int e = 0; e < 4; ++e) c += (col[b] + e < nv && key[b][e] >= tau) ? 1 : 0;
            const int x = wave_incl_scan(c);
            uint32_t base = 0;
            if (lane == 63) base = atomicAdd(&lctr[1], (uint32_t)x);
            uint32_t slot = (uint32_t)__shfl((int)base, 63) + (uint32_t)(x - c);
#pragma unroll
            for (int b = 0; b < B; ++b)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (col[b] + e < nv && key[b][e] >= tau) {
                        if (slot < (uint32_t)cap) out[slot] = ((uint64_t)key[b][e] << 32) | (uint32_t)~(uint32_t)(col[b] + e);
                        ++slot;
                    }
        }
    }
    __syncthreads();
    if (tid == 0) {
        TcRec r;
        r.n = over ? 0xFFFFFFFFu : lctr[1];
        r.tau = tau;
        r.hi = hi;
        r.pad = 0;
        recs[t * S + s] = r;
    }
}

template <int NT>
__global__ __launch_bounds__(NT) void k_topk_pick(const float* __restrict__ scores, int64_t n_cols,
                                                  const int64_t* __restrict__ pos, int m, int k, int S, int cap,
                                                  const TcRec* __restrict__ recs, const uint64_t* __restrict__ cands,
                                                  int32_t* __restrict__ idx) {
    constexpr int NW = NT / 64;
    constexpr int SPW = (kMaxSlices + NW - 1) / NW;  // slices per wave
    __shared__ uint32_t h[4096];
    __shared__ __align__(16) uint32_t big[2 * kTqCand + kBitmapWords];  // candidates, then the row bitmap
    __shared__ uint64_t tie[kTieLds];
    __shared__ int wsum[2 * NW];
    __shared__ int bc[4];
    __shared__ uint32_t lctr[4];
    __shared__ uint32_t scnt[kMaxSlices];
    uint64_t* cl = (uint64_t*)big;
    uint32_t* bm = big + 2 * kTqCand;  // row bitmap, or the list of winners to sort
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t t = blockIdx.x;
    const float* row = scores + t * n_cols;
    const int nv = (int)row_visible(pos, t, m, n_cols);
    int32_t* out = idx + t * (int64_t)k;
    if (nv <= k) {
        for (int a = tid; a < k; a += NT) out[a] = a < nv ? a : -1;
        return;
    }
    // slice records and the first 128 candidates of each slice are requested together
    // (wave w: slices w + i NW, i < SPW; S <= kMaxSlices, kSliceCap >= 128)
    uint64_t pre[SPW][2];
    TcRec rr[SPW];
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int s = wave + i * NW;
        rr[i] = TcRec{0, 0, 0, 0};
        pre[i][0] = pre[i][1] = 0;
        if (s < S) {
            const uint64_t* src = cands + ((int64_t)t * S + s) * cap;
            rr[i] = recs[t * S + s];
            pre[i][0] = src[lane];
            pre[i][1] = src[64 + lane];
        }
    }
    // the LDS set-up runs while those loads are in flight
    const int nwords = (nv + 31) / 32;
    const bool use_bm = nwords <= kBitmapWords;  // kBitmapWords is a multiple of NT
    // bitmap word w belongs to thread w / perw and sits at (w % perw) * NT + w / perw
    const int perw = (nwords + NT - 1) / NT;
    if (use_bm)
        for (int i = tid; i < perw * NT; i += NT) bm[i] = 0;
    for (int i = tid; i < 4096; i += NT) h[i] = 0;
    if (tid < 2) lctr[tid] = 0;
    uint32_t rn[SPW];
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int s = wave + i * NW;
        rn[i] = rr[i].n;
        if (s < S && lane == 0) scnt[s] = rn[i];
        if (s == 0 && lane == 0) {
            lctr[2] = rr[i].tau;
            lctr[3] = rr[i].hi;
        }
    }
    __syncthreads();
    // offsets of the slices: one wave-wide scan of the counts (S <= 64)
    const uint32_t sn = lane < S ? scnt[lane] : 0u;
    const bool sbad = sn > (uint32_t)cap;
    const int sx = wave_incl_scan(sbad ? 0 : (int)sn);
    const int n_cand = __shfl(sx, 63);
    int off[SPW];
#pragma unroll
    for (int i = 0; i < SPW; ++i) off[i] = __shfl(sx - (int)sn, (wave + i * NW) & 63);
    if (__ballot(sbad) != 0 || n_cand > kTqCand) {
        row_select<NT>(row, nv, k, out, h, big, 2 * kTqCand + kBitmapWords, wsum, bc);
        return;
    }
    const uint32_t tau = lctr[2], hi = lctr[3];
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int s = wave + i * NW;
        if (s >= S) continue;
        const int n = (int)rn[i];
        if (lane < n) cl[off[i] + lane] = pre[i][0];
        if (64 + lane < n) cl[off[i] + 64 + lane] = pre[i][1];
        const uint64_t* src = cands + ((int64_t)t * S + s) * cap;
        for (int j = 128 + lane; j < n; j += 64) cl[off[i] + j] = src[j];
    }
    __syncthreads();
    pick_candidates<NT>(cl, n_cand, tau, hi, k, out, bm, use_bm, perw, h, tie, wsum, bc, lctr);
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

// ---------------------------------------------------------------------------
// Many rows of up to kTrMaxCols columns (e.g. prefill): one workgroup per row
// holds the row's visible keys in registers (NV4 float4 slots per thread), so
// the row is read once.  A lower bound lo of the k-th largest key: each thread
// keeps its two largest keys; the smallest j-th of them over the threads
// holding >= j keys, j = ceil(k / NT), bounds the k-th largest of those pairs
// (distinct columns) from below, and one histogram level over the pairs
// brings lo up to the lower edge of the bin holding their k-th largest, which
// never exceeds the row's k-th largest key.  One pass then lists the
// keys >= lo (a few k of the row) in LDS as (key << 32 | ~column), placed by a
// block scan, and the selection runs on that list: a histogram descent with
// bins scaled to [lo, hi] down to a window of at most kTieLds keys (ranked
// directly, key desc and column asc) or a single key value (its lowest columns
// by two 11-bit passes over the column index).  A list that would not fit LDS
// (heavy ties at lo) is handled the same way over the registers.  Winners go
// to an LDS bitmap of the row, written in ascending column order.
// ---------------------------------------------------------------------------
constexpr int kTrThreads = 1024;
constexpr int kTrMaxV4 = 9;                            // float4 slots per thread at most
constexpr int kTrMaxCols = kTrThreads * kTrMaxV4 * 4;  // 36,864 columns
constexpr int kTrList = 8192;                          // keys >= lo held in LDS

template <int NV4>
__global__ __launch_bounds__(kTrThreads) void k_topk_reg(const float* __restrict__ scores, int64_t n_cols,
                                                            const int64_t* __restrict__ pos, int m, int k,
                                                            int32_t* __restrict__ idx) {
    constexpr int NT = kTrThreads, NW = NT / 64;
    constexpr int NCOL = NV4 * NT * 4;
    static_assert(NCOL < (1 << 22), "columns fit two 11-bit passes");
    constexpr int BMW = (NCOL / 32 + NT - 1) / NT * NT;  // bitmap words, whole per-thread runs
    __shared__ uint32_t h[4096];
    __shared__ uint32_t bm[BMW];
    __shared__ uint64_t cl[kTrList];
    __shared__ uint64_t tie[kTieLds];
    __shared__ int wsum[NW];
    __shared__ uint32_t red[3 * NW];
    __shared__ int bc[4];
    __shared__ uint32_t lctr[1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t t = blockIdx.x;
    const int nv = (int)row_visible(pos, t, m, n_cols);
    int32_t* out = idx + t * (int64_t)k;
    if (nv <= k) {
        for (int a = tid; a < k; a += NT) out[a] = a < nv ? a : -1;
        return;
    }
    const float* row = scores + t * n_cols;

    // ---- the row in registers: slot i holds columns 4 (i NT + tid) .. +3; key 0 = not visible ----
    // (every load is issued before any is used: a conversion next to its load would make
    // each slot wait for the previous one)
    uint32_t key[NV4][4];
    {
        v4f raw[NV4];
        if (((uintptr_t)row & 15) == 0) {
#pragma unroll
            for (int i = 0; i < NV4; ++i) {
                const int c = 4 * (i * NT + tid);
                raw[i] = c + 4 <= nv ? __builtin_nontemporal_load((const v4f*)(row + c)) : v4f{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int i = 0; i < NV4; ++i) {
                const int c = 4 * (i * NT + tid);
                if (c < nv && c + 4 > nv)  // the slot holding the row's last visible columns
#pragma unroll
                    for (int e = 0; e < 4; ++e) raw[i][e] = c + e < nv ? row[c + e] : 0.f;
            }
        } else {
#pragma unroll
            for (int i = 0; i < NV4; ++i) {
                const int c = 4 * (i * NT + tid);
#pragma unroll
                for (int e = 0; e < 4; ++e) raw[i][e] = c + e < nv ? row[c + e] : 0.f;
            }
        }
#pragma unroll
        for (int i = 0; i < NV4; ++i) {
            const int c = 4 * (i * NT + tid);
#pragma unroll
            for (int e = 0; e < 4; ++e) key[i][e] = c + e < nv ? f32_order_key(raw[i][e]) : 0u;
        }
    }
    for (int i = tid; i < BMW; i += NT) bm[i] = 0;
    for (int i = tid; i < 4096; i += NT) h[i] = 0;
    if (tid == 0) lctr[0] = 0;
    auto for_cols = [&](auto fn) {
#pragma unroll
        for (int i = 0; i < NV4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) fn(key[i][e], (uint32_t)(4 * (i * NT + tid) + e));
    };
    auto for_keys = [&](auto fn) { for_cols([&](uint32_t x, uint32_t) { fn(x); }); };

    // ---- hi = the row's largest key; lo = the smallest j-th largest key of the threads holding >= j ----
    static_assert(2 * NT >= 2048, "j <= 2 for k <= 2048");
    const int j = (k + NT - 1) / NT;          // 1 or 2
    uint32_t t1 = 0, t2 = 0;                  // this thread's two largest keys
    int nk = 0;
    for_keys([&](uint32_t x) {
        t2 = max(t2, min(t1, x));
        t1 = max(t1, x);
        nk += x != 0u;
    });
    uint32_t lo, hi;
    bool tight;
    {
        const bool part = nk >= j;
        uint32_t mx = t1, mn = part ? (j == 1 ? t1 : t2) : 0xFFFFFFFFu;
        const uint32_t np = (uint32_t)__popcll(__ballot(part));
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
            mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
        }
        if (lane == 0) {
            red[wave] = mx;
            red[NW + wave] = mn;
            red[2 * NW + wave] = np;
        }
        __syncthreads();
        hi = red[0];
        lo = red[NW];
        uint32_t npart = red[2 * NW];
#pragma unroll
        for (int w = 1; w < NW; ++w) {
            hi = max(hi, red[w]);
            lo = min(lo, red[NW + w]);
            npart += red[2 * NW + w];
        }
        tight = (int64_t)npart * j >= k;
        if (!tight) lo = 1;  // too few full threads: every visible key (all > 0)
    }
    if (tight) {
        // the k-th largest of the threads' pairs (t1, t2), >= lo, is <= the row's k-th largest key:
        // 256 bins scaled to [lo, hi] over those 2 NT keys, scanned from the top by wave 0, and lo
        // moves up to the lower edge of the bin holding that k-th largest
        int s = 0;
        while ((((uint64_t)hi - lo) >> s) >= 256) ++s;
        if (t1 >= lo) atomicAdd(&h[255 - ((t1 - lo) >> s)], 1u);
        if (t2 >= lo) atomicAdd(&h[255 - ((t2 - lo) >> s)], 1u);
        __syncthreads();
        if (wave == 0) {
            // lane l holds ranks 4l .. 4l+3 from the top (bins 255-4l .. 252-4l)
            const uint4 c = *(const uint4*)&h[4 * lane];
            const int sum4 = (int)(c.x + c.y + c.z + c.w);
            const int incl = wave_incl_scan(sum4);
            const int before = incl - sum4;
            if (before < k && incl >= k) {
                int run = before, r = 4 * lane;
                const int cc[4] = {(int)c.x, (int)c.y, (int)c.z, (int)c.w};
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (run < k) {
                        run += cc[q];
                        r = 4 * lane + q;
                    }
                bc[0] = 255 - r;  // the bin whose running count from the top reaches k
            }
        }
        __syncthreads();
        lo = lo + ((uint32_t)bc[0] << s);
        if (tid < 256) h[tid] = 0;  // read by wave 0 only, before the barrier above
    }

    // ---- list the keys >= lo (block scan; no atomics) when they fit ----
    int cnt = 0;
    for_keys([&](uint32_t x) { cnt += x >= lo; });
    int n_c;
    int off = tm_scan<NT>(cnt, wsum, n_c);
    const bool listed = n_c <= kTrList;
    if (listed)
        for_cols([&](uint32_t x, uint32_t col) {
            if (x >= lo) cl[off++] = ((uint64_t)x << 32) | (uint32_t)~col;
        });
    __syncthreads();
    // visit the candidates: the list, or every key in registers
    auto for_cand = [&](auto fn) {
        if (listed) {
            for (int i = tid; i < n_c; i += NT) {
                const uint64_t c = cl[i];
                fn((uint32_t)(c >> 32), ~(uint32_t)c);
            }
        } else {
            for_cols(fn);
        }
    };

    // ---- the window holding the k-th largest key ----
    uint32_t wbase;
    int wsh, above, nb;
    hist_descend<NT>([&](auto fn) { for_cand([&](uint32_t x, uint32_t) { fn(x); }); }, lo, hi, k, kTieLds, h, wsum,
                     bc, wbase, wsh, above, nb);
    const uint64_t wtop = (uint64_t)wbase + ((uint64_t)1 << wsh);
    const int need = k - above;  // >= 1 winners inside the window
    const int nwords = (nv + 31) / 32;
    const int perw = (nwords + NT - 1) / NT;  // word w at (w % perw) * NT + w / perw (conflict-free emission)
    auto mark = [&](uint32_t col) {
        const uint32_t wd = col >> 5;
        atomicOr(&bm[(wd % perw) * NT + wd / perw], 1u << (col & 31));
    };
    for_cand([&](uint32_t x, uint32_t col) {
        if ((uint64_t)x >= wtop) mark(col);
        else if (nb <= kTieLds && x >= wbase) tie[atomicAdd(&lctr[0], 1u)] = ((uint64_t)x << 32) | (uint32_t)~col;
    });
    __syncthreads();
    if (nb <= kTieLds) {
        // (key desc, column asc) is (key << 32 | ~column) desc: rank each window entry directly
        for (int q = tid; q < nb; q += NT) {
            const uint64_t e = tie[q];
            int rank = 0;
            for (int r = 0; r < nb; ++r) rank += tie[r] > e ? 1 : 0;
            if (rank < need) mark(~(uint32_t)e);
        }
    } else {
        // one key value (wbase) held by more than kTieLds keys: the need lowest columns among them
        const uint32_t thr = wbase;
        uint32_t pre = 0, pm = 0;
        int nl = need;
        for (int sh = 11; sh >= 0; sh -= 11) {
            for (int i = tid; i < 2048; i += NT) h[i] = 0;
            __syncthreads();
            for_cand([&](uint32_t x, uint32_t col) {
                if (x == thr && (col & pm) == pre) atomicAdd(&h[tm_pos<2048, NT>(2047 - ((col >> sh) & 0x7FF))], 1u);
            });
            __syncthreads();
            int ab;
            const uint32_t bn = 2047u - (uint32_t)tm_find<2048, NT>(h, nl, wsum, bc, ab);
            nl -= ab;
            pre |= bn << sh;
            pm |= 0x7FFu << sh;
        }
        for_cand([&](uint32_t x, uint32_t col) {
            if (x == thr && col <= pre) mark(col);
        });
    }
    __syncthreads();
    // ---- emit in ascending order: thread t owns words t*perw .. t*perw+perw-1 ----
    int nm = 0;
    for (int i = 0; i < perw; ++i) nm += __popc(bm[i * NT + tid]);
    int tot;
    int o = tm_scan<NT>(nm, wsum, tot);
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

// few rows longer than k_topk_stream takes: selection from the row summary
static bool topk_summ(int64_t T, int64_t n_cols) { return T < kTopkMaxRows && n_cols > kTsMaxCols; }
// k_topk_cand workgroups per row (about 256 in all) and candidates each may write
static int topk_slices(int64_t T) { return T >= 256 ? 1 : (int)(256 / T < kMaxSlices ? 256 / T : kMaxSlices); }
constexpr int kSliceCap = 4096;  // >= 128

// workspace: summaries [T][groups], slice records [T][S], candidates [T][S][kSliceCap]
static size_t ws_recs_off(int64_t T, int64_t n_cols) { return ((size_t)T * topk_groups(n_cols) * 4 + 255) & ~(size_t)255; }
static size_t ws_cands_off(int64_t T, int64_t n_cols) {
    return (ws_recs_off(T, n_cols) + (size_t)T * topk_slices(T) * sizeof(TcRec) + 255) & ~(size_t)255;
}

size_t topk_workspace_bytes(int64_t T, int64_t n_cols, int) {
    if (!topk_summ(T, n_cols)) return 0;
    return ws_cands_off(T, n_cols) + (size_t)T * topk_slices(T) * kSliceCap * 8;
}

hipError_t launch_topk(const float* scores, int64_t T, int64_t n_cols, const int64_t* pos, int m, int k, int32_t* idx,
                       void* ws, bool prepared, hipStream_t st) {
    if (T == 0) return hipSuccess;
    if (topk_summ(T, n_cols)) {
        uint32_t* summ = (uint32_t*)ws;
        TcRec* recs = (TcRec*)((char*)ws + ws_recs_off(T, n_cols));
        uint64_t* cands = (uint64_t*)((char*)ws + ws_cands_off(T, n_cols));
        const int S = topk_slices(T);
        if (!prepared)
            hipLaunchKernelGGL(k_topk_gmax, dim3((unsigned)((n_cols + kTgThreads * 8 - 1) / (kTgThreads * 8)), (unsigned)T),
                               dim3(kTgThreads), 0, st, scores, n_cols, pos, m, k, summ);
        hipLaunchKernelGGL(k_topk_cand, dim3((unsigned)S, (unsigned)T), dim3(kTcThreads), 0, st, scores, n_cols, pos, m, k,
                           summ, S, kSliceCap, recs, cands);
        hipLaunchKernelGGL(k_topk_pick<kTpThreads>, dim3((unsigned)T), dim3(kTpThreads), 0, st, scores, n_cols, pos, m,
                           k, S, kSliceCap, recs, cands, idx);
    } else if (n_cols <= kTrMaxCols) {
        const dim3 g((unsigned)T), b(kTrThreads);
        if (n_cols <= kTrThreads * 4)
            hipLaunchKernelGGL(k_topk_reg<1>, g, b, 0, st, scores, n_cols, pos, m, k, idx);
        else if (n_cols <= kTrThreads * 8)
            hipLaunchKernelGGL(k_topk_reg<2>, g, b, 0, st, scores, n_cols, pos, m, k, idx);
        else if (n_cols <= kTrThreads * 16)
            hipLaunchKernelGGL(k_topk_reg<4>, g, b, 0, st, scores, n_cols, pos, m, k, idx);
        else
            hipLaunchKernelGGL(k_topk_reg<kTrMaxV4>, g, b, 0, st, scores, n_cols, pos, m, k, idx);
    } else if (n_cols <= kTsMaxCols) {
        hipLaunchKernelGGL(k_topk_stream, dim3((unsigned)T), dim3(kTsThreads), 0, st, scores, n_cols, pos, m, k, idx);
    } else {
        hipLaunchKernelGGL(k_topk_row, dim3((unsigned)T), dim3(kTopkThreads), 0, st, scores, n_cols, pos, m, k, idx);
    }
    return hipGetLastError();
}

bool topk_uses_summary(int64_t T, int64_t n_cols) { return topk_summ(T, n_cols); }

// ---------------------------------------------------------------------------
// Selection without a caller workspace: for shapes that select from the row
// summary, the summaries, slice records and candidates live in `scratch`, a
// device array of the library (each GPU holds its own copy, at its own
// address, until the process ends).  Host code never passes the array's name
// to a kernel: its device address is looked up once per device, with that
// device current, and kept.  Nothing in it needs to start at zero; calls that
// overlap on one GPU share it and race.
// ---------------------------------------------------------------------------
constexpr size_t kTopkScratchBytes = (size_t)12 << 20;
static __device__ __align__(256) uint8_t scratch[kTopkScratchBytes];

constexpr int kMaxDevices = 64;
static std::atomic<void*> g_scratch_addr[kMaxDevices];
static std::mutex g_scratch_mu;

static hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

size_t topk_scratch_bytes() { return kTopkScratchBytes; }

hipError_t launch_topk_noalloc(const float* scores, int64_t T, int64_t n_cols, const int64_t* pos, int m, int k,
                               int32_t* idx, hipStream_t st) {
    if (T == 0) return hipSuccess;
    void* ws = nullptr;
    if (topk_summ(T, n_cols)) {
        if (topk_workspace_bytes(T, n_cols, k) > kTopkScratchBytes) return hipErrorInvalidValue;
        const hipError_t e = scratch_address(&ws);
        if (e != hipSuccess) return e;
    }
    return launch_topk(scores, T, n_cols, pos, m, k, idx, ws, false, st);
}

}  // namespace csa
