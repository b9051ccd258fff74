// csa_index_scores kernels: lightning-indexer scores with MXFP4 scaled MFMA.
//
// score[t][j] = sum_h w[t][h] * max(0, <q[t][h], key_j>), -inf where j is not
// yet visible to t.  Both operands are E2M1 with E8M0 block-32 scales, fed
// straight to v_mfma_scale_f32_*_f8f6f4 (format 4 = E2M1 on both sides), so
// the per-block scaling happens inside the matrix core.
//
// Two kernels:
//   k_index_rows  few query rows (decode): MFMA rows = heads of one query,
//                 columns = 16 keys per 16x16x128 MFMA; the run is bound by
//                 streaming the MXFP4 keys from HBM (68 B per key at d_i=128).
//   k_index_gemm  many query rows sharing a sequence (prefill): MFMA rows =
//                 (query, head) pairs, 32 per 32x32x64 MFMA, 4 row tiles per
//                 wave so each key fragment feeds 4-8 MFMAs.
#include <math.h>

#include <type_traits>

#include "csa_device.hpp"
#include "csa_internal.hpp"
#include "select_device.hpp"

namespace csa {

// What an indexer kernel does with the scores it computes.
enum IndexMode {
    kStore = 0,   // write every score (and, for decode, the row summary)
    kSample = 1,  // write the order keys of the sample columns (0 where not visible)
    kEmit = 2     // append (key << 32 | ~column) of every visible column whose key >= tau[t]
};

// Arguments of the fused selection passes (unused by kStore).
struct ItkArgs {
    uint32_t* samp;       // [T][n_s] sample keys
    int64_t n_s;          // sample columns per row
    int64_t n_real;       // columns of the score row (the sample maps into [0, n_real))
    int D;                // columns [0, D) are all sampled
    int F;                // after D, one 32-column group in F is sampled
    const uint32_t* tau;  // [T] emission threshold (order key)
    uint32_t* cnt;        // [T][S] candidates appended per (row, segment)
    uint64_t* cand;       // [T][S][cap] candidates
    int cap;              // candidates kept per (row, segment)
};

constexpr int kItkRowSegs = 64;  // candidate segments per row of the decode (rows) kernel

// Sample column v -> score column: the prefix [0, D) whole, then the first group of every
// F groups of 32 columns.
__device__ __forceinline__ int64_t sample_col(int64_t v, int D, int F) {
    return v < D ? v : D + ((v - D) >> 5) * (32 * (int64_t)F) + ((v - D) & 31);
}

// The float t such that, for every score v, v >= t exactly when f32_order_key(v) >= key
// (-inf for a key at or below that of -inf; NaN, which nothing reaches, above that of +inf).
__device__ __forceinline__ float order_key_floor(uint32_t key) {
    if (key <= 0x007FFFFFu) return -INFINITY;
    if (key > 0xFF800000u) return __int_as_float(0x7FC00000);
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// max(x, 0) as one v_med3_f32 (median of x, 0 and FLT_MAX); fmaxf costs a canonicalising max
// first.  The argument is always a dot product accumulated from +0, which is never -0 (an exact
// zero sum rounds to +0) and is finite for finite inputs: there both forms give the same bits.
__device__ __forceinline__ float relu1(float x) { return __builtin_amdgcn_fmed3f(x, 0.f, 3.402823466e38f); }

__device__ __forceinline__ v8i frag16(const uint8_t* p) {
    v4i x = *(const v4i*)p;
    v8i r = {x[0], x[1], x[2], x[3], 0, 0, 0, 0};
    return r;
}

// ---------------------------------------------------------------------------
// decode: grid (key chunks, T), 4 waves; each wave streams tiles of 16 keys
// ---------------------------------------------------------------------------
template <int DI, int U, int MODE = kStore>
__global__ __launch_bounds__(256) void k_index_rows(const uint8_t* __restrict__ q, const uint8_t* __restrict__ q_scale,
                                                    const float* __restrict__ w, const int32_t* __restrict__ seq,
                                                    const int64_t* __restrict__ pos, int h_i,
                                                    const uint8_t* __restrict__ kdata,
                                                    const uint8_t* __restrict__ kscale, int64_t kcap,
                                                    const int32_t* __restrict__ kpages, int kpshift, int m,
                                                    int64_t n_cols, int64_t chunk, float* __restrict__ scores,
                                                    uint32_t* __restrict__ gmax, ItkArgs ia = {}) {
    // kSample: the loop runs over the n_cols = n_s sample columns, each mapped to its score column
    constexpr int KB = DI / 2;   // bytes per key
    constexpr int NB = DI / 32;  // scale blocks per key
    static_assert(16 * U == 4 * kTopkGroup, "one wave step = four summary groups");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t t = blockIdx.y;
    const int r = lane & 15, g = lane >> 4;

    v8i a = {0, 0, 0, 0, 0, 0, 0, 0};
    int sa = 127;
    if (r < h_i && g < NB) {
        a = frag16(q + (t * h_i + r) * KB + g * 16);
        sa = q_scale[(t * h_i + r) * NB + g];
    }
    float wr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int h = 4 * g + i;
        wr[i] = h < h_i ? w[t * h_i + h] : 0.f;
    }
    auto real = [&](int64_t j) -> int64_t {
        if constexpr (MODE == kSample) return sample_col(j, ia.D, ia.F);
        else return j;
    };
    int64_t nv = (pos[t] + 1) / m;
    const int64_t ncl = MODE == kSample ? ia.n_real : n_cols;
    if (nv > ncl) nv = ncl;
    const int32_t sq = seq[t];
    auto krow = [&](int64_t j) { return kv_row(kpages, kpshift, kcap, sq, j); };  // row of entry j's key
    const int64_t c0 = (int64_t)blockIdx.x * chunk;
    const int64_t c1 = c0 + chunk < n_cols ? c0 + chunk : n_cols;
    float* out = scores + t * n_cols;
    const float tauf = MODE == kEmit ? order_key_floor(ia.tau[t]) : 0.f;

    for (int64_t j0 = c0 + (int64_t)wave * 16 * U; j0 < c1; j0 += 4 * 16 * U) {
        uint32_t gm[4] = {0u, 0u, 0u, 0u};  // per summary group of this step: largest visible order key (lanes < 16)
        v4i bk[U];
        int sb[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = real(j0 + u * 16 + r);
            if (j < nv && g < NB) {
                // streamed once: nontemporal, so the keys do not displace cached lines
                const int64_t kr = krow(j);
                bk[u] = __builtin_nontemporal_load((const v4i*)(kdata + kr * KB + g * 16));
                sb[u] = kscale[kr * NB + g];
            } else {
                bk[u] = v4i{0, 0, 0, 0};
                sb[u] = 127;
            }
        }
        float pv[U];  // score of key j0 + 16 u + r (every lane, after the head-group sum)
#pragma unroll
        for (int u = 0; u < U; ++u) {
            v4f acc = {0.f, 0.f, 0.f, 0.f};
            const v8i bf = {bk[u][0], bk[u][1], bk[u][2], bk[u][3], 0, 0, 0, 0};
            acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bf, acc, 4, 4, 0, sa, 0, sb[u]);
            float p = wr[0] * relu1(acc[0]);
            p = fmaf(wr[1], relu1(acc[1]), p);
            p = fmaf(wr[2], relu1(acc[2]), p);
            p = fmaf(wr[3], relu1(acc[3]), p);
            p = rows4_sum(p);  // the four head groups (exact: every partial sum is representable)
            const int64_t j = j0 + u * 16 + r;
            pv[u] = real(j) < nv ? p : -INFINITY;
            if (MODE == kStore && lane < 16 && j < c1 && j < nv) gm[u / (U / 4)] = max(gm[u / (U / 4)], f32_order_key(p));
        }
        static_assert(U == 8, "two groups of 64 keys per step");
        // lane (r, g) owns keys j0 + 16 g + r and j0 + 64 + 16 g + r of the step
        const float v0 = g == 0 ? pv[0] : g == 1 ? pv[1] : g == 2 ? pv[2] : pv[3];
        const float v1 = g == 0 ? pv[4] : g == 1 ? pv[5] : g == 2 ? pv[6] : pv[7];
        const int64_t ja = j0 + lane, jb = j0 + 64 + lane;
        if constexpr (MODE == kSample) {
            uint32_t* so = ia.samp + t * ia.n_s;
            if (ja < c1) so[ja] = v0 == -INFINITY ? 0u : f32_order_key(v0);
            if (jb < c1) so[jb] = v1 == -INFINITY ? 0u : f32_order_key(v1);
            continue;
        } else if constexpr (MODE == kEmit) {
            // one counter update per step of the wave (few keys pass the threshold)
            const bool ea = ja < c1 && ja < nv && v0 >= tauf, eb = jb < c1 && jb < nv && v1 >= tauf;
            const uint64_t ma = __ballot(ea), mb = __ballot(eb);
            const int na = __popcll(ma), nb = __popcll(mb);
            if (na + nb > 0) {
                // segment sg of the row (one of kItkRowSegs): its counter sees a 64th of the updates
                const int64_t sg = t * kItkRowSegs + (blockIdx.x * 4 + wave) % kItkRowSegs;
                uint32_t slot0 = 0;
                if (lane == 0) slot0 = atomicAdd(&ia.cnt[sg], (uint32_t)(na + nb));
                slot0 = (uint32_t)__shfl((int)slot0, 0);
                const uint64_t lt = (1ull << lane) - 1ull;
                uint64_t* co = ia.cand + sg * (int64_t)ia.cap;
                if (ea) {
                    const uint32_t sl = slot0 + (uint32_t)__popcll(ma & lt);
                    if (sl < (uint32_t)ia.cap) co[sl] = ((uint64_t)f32_order_key(v0) << 32) | (uint32_t)~(uint32_t)ja;
                }
                if (eb) {
                    const uint32_t sl = slot0 + (uint32_t)na + (uint32_t)__popcll(mb & lt);
                    if (sl < (uint32_t)ia.cap) co[sl] = ((uint64_t)f32_order_key(v1) << 32) | (uint32_t)~(uint32_t)jb;
                }
            }
            continue;
        }
        {
            // the step's 128 scores in two full-wave stores (a quarter-wave store per tile would
            // issue four times as many)
            if (ja < c1) out[ja] = v0;
            if (jb < c1) out[jb] = v1;
        }
        if (gmax) {
            // unsigned max over lanes 0..15 of four values, spread so that lanes 4G..4G+3 end with
            // group G: exchange halves with the mirrored lane (l <-> 15-l), then with the mirrored
            // lane within each half (l <-> 7-l), then reduce each quad (xor 1, xor 2)
            const bool hi8 = (lane & 8) != 0, hi4 = (lane & 4) != 0;
            const uint32_t s0 = hi8 ? gm[0] : gm[2], s1 = hi8 ? gm[1] : gm[3];
            uint32_t k0 = hi8 ? gm[2] : gm[0], k1 = hi8 ? gm[3] : gm[1];
            k0 = max(k0, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s0, 0x140, 0xf, 0xf, false));  // row_mirror
            k1 = max(k1, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s1, 0x140, 0xf, 0xf, false));
            const uint32_t s2 = hi4 ? k0 : k1;
            uint32_t x = hi4 ? k1 : k0;
            x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s2, 0x141, 0xf, 0xf, false));  // row_half_mirror
            x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xf, 0xf, false));   // quad_perm 1,0,3,2
            x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xf, 0xf, false));   // quad_perm 2,3,0,1
            const int64_t gi = j0 / kTopkGroup + (lane >> 2);
            if (lane < 16 && (lane & 3) == 0 && gi < topk_groups(n_cols)) gmax[t * topk_groups(n_cols) + gi] = x;
        }
    }
}

// ---------------------------------------------------------------------------
// grouped decode (several query rows of one sequence per step, e.g. the draft
// tokens of multi-token prediction): grid (key chunks, T / R).  The R rows of
// a group share every key fragment: MFMA rows = (row, head) pairs, 16 per
// 16x16x128 tile, NA = ceil(R HI / 16) tiles per key tile, so the keys are
// streamed once per group.  Lane group g of tile a holds MFMA rows
// 16a + 4g .. +3: four heads of one row; with HI = 8 a row spans two lane
// groups, summed by a row swap.  Rows of a group on another sequence than
// its first row are handled in a pass of their own (their A rows zeroed in
// the other passes), so every layout gives the plain kernel's scores.
// ---------------------------------------------------------------------------
template <int DI, int R, int HI>
__global__ __launch_bounds__(256) void k_index_rows_grp(const uint8_t* __restrict__ q,
                                                        const uint8_t* __restrict__ q_scale,
                                                        const float* __restrict__ w, const int32_t* __restrict__ seq,
                                                        const int64_t* __restrict__ pos,
                                                        const uint8_t* __restrict__ kdata,
                                                        const uint8_t* __restrict__ kscale, int64_t kcap,
                                                        const int32_t* __restrict__ kpages, int kpshift, int m,
                                                        int64_t n_cols, int64_t chunk, float* __restrict__ scores,
                                                        uint32_t* __restrict__ gmax) {
    constexpr int KB = DI / 2;            // bytes per key
    constexpr int NB = DI / 32;           // scale blocks per key
    constexpr int U = 8;                  // key tiles of 16 per wave step
    constexpr int NA = (R * HI + 15) / 16;
    constexpr int GPQ = HI / 4;           // lane groups per row in a tile
    static_assert(16 * U == 4 * kTopkGroup, "one wave step = four summary groups");
    static_assert(R * HI <= 32 && (HI == 4 || HI == 8), "at most two tiles of (row, head) pairs");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int64_t t0 = (int64_t)blockIdx.y * R;
    const int64_t c0 = (int64_t)blockIdx.x * chunk;
    const int64_t c1 = c0 + chunk < n_cols ? c0 + chunk : n_cols;
    const int64_t ng = topk_groups(n_cols);

    int64_t nvr[R];
    int32_t sr[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        nvr[i] = (pos[t0 + i] + 1) / m;
        if (nvr[i] > n_cols) nvr[i] = n_cols;
        sr[i] = seq[t0 + i];
    }
    uint32_t todo = (1u << R) - 1;
    while (todo) {
        const int first = __builtin_ctz(todo);
        int32_t s = sr[0];
#pragma unroll
        for (int i = 1; i < R; ++i) s = i == first ? sr[i] : s;
        uint32_t mask = 0;
#pragma unroll
        for (int i = 0; i < R; ++i)
            if (((todo >> i) & 1u) && sr[i] == s) mask |= 1u << i;
        todo &= ~mask;

        // A of tile a: lane (r, g) = MFMA row 16a + r = (row qa, head ha), block g of its query vector
        v8i a[NA];
        int sa[NA];
        // this lane group's row in tile a (-1: none in this pass), its head weights, visible count, output
        int qrow[NA];
        float wr[NA][4];
        int64_t nvl[NA];
        float* orow[NA];
        int64_t nv_max = 0;
#pragma unroll
        for (int i = 0; i < R; ++i)
            if ((mask >> i) & 1u) nv_max = nvr[i] > nv_max ? nvr[i] : nv_max;
#pragma unroll
        for (int at = 0; at < NA; ++at) {
            const int qa = (16 * at + r) / HI, ha = (16 * at + r) % HI;
            a[at] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
            sa[at] = 127;
            if (qa < R && ((mask >> qa) & 1u) && g < NB) {
                a[at] = frag16(q + ((t0 + qa) * HI + ha) * KB + g * 16);
                sa[at] = q_scale[((t0 + qa) * HI + ha) * NB + g];
            }
            const int qg = (16 * at + 4 * g) / HI, hb = (16 * at + 4 * g) % HI;
            const bool live = qg < R && ((mask >> qg) & 1u);
            qrow[at] = live ? qg : -1;
            int64_t nv = 0;
#pragma unroll
            for (int i = 0; i < R; ++i) nv = i == qg ? nvr[i] : nv;
            nvl[at] = live ? nv : 0;
            orow[at] = scores + (t0 + (live ? qg : 0)) * n_cols;
#pragma unroll
            for (int i = 0; i < 4; ++i) wr[at][i] = live ? w[(t0 + qg) * HI + hb + i] : 0.f;
        }
        for (int64_t j0 = c0 + (int64_t)wave * 16 * U; j0 < c1; j0 += 4 * 16 * U) {
            uint32_t gm[NA][4];  // per tile and summary group of this step: the lane group's largest visible key
#pragma unroll
            for (int at = 0; at < NA; ++at) gm[at][0] = gm[at][1] = gm[at][2] = gm[at][3] = 0u;
            v4i bk[U];
            int sb[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t j = j0 + u * 16 + r;
                if (j < nv_max && g < NB) {
                    const int64_t kr = kv_row(kpages, kpshift, kcap, s, j);
                    bk[u] = __builtin_nontemporal_load((const v4i*)(kdata + kr * KB + g * 16));
                    sb[u] = kscale[kr * NB + g];
                } else {
                    bk[u] = v4i{0, 0, 0, 0};
                    sb[u] = 127;
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const v8i bf = {bk[u][0], bk[u][1], bk[u][2], bk[u][3], 0, 0, 0, 0};
                const int64_t j = j0 + u * 16 + r;
#pragma unroll
                for (int at = 0; at < NA; ++at) {
                    v4f acc = {0.f, 0.f, 0.f, 0.f};
                    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[at], bf, acc, 4, 4, 0, sa[at], 0, sb[u]);
                    float p = wr[at][0] * relu1(acc[0]);
                    p = fmaf(wr[at][1], relu1(acc[1]), p);
                    p = fmaf(wr[at][2], relu1(acc[2]), p);
                    p = fmaf(wr[at][3], relu1(acc[3]), p);
                    if (GPQ == 2) {
                        // the row's two lane groups (exact: every partial sum is representable)
                        const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(p), __float_as_uint(p), false, false);
                        p = __uint_as_float(x[0]) + __uint_as_float(x[1]);
                    }
                    if (qrow[at] >= 0 && (g % GPQ) == 0 && j < c1) {
                        orow[at][j] = j < nvl[at] ? p : -INFINITY;
                        if (j < nvl[at]) gm[at][u / (U / 4)] = max(gm[at][u / (U / 4)], f32_order_key(p));
                    }
                }
            }
            if (gmax) {
                // per lane group: unsigned max over its 16 lanes of four values, lanes 4G..4G+3 ending with
                // group G (mirror exchanges within the 16-lane row, then quad reductions)
                const bool hi8 = (lane & 8) != 0, hi4 = (lane & 4) != 0;
#pragma unroll
                for (int at = 0; at < NA; ++at) {
                    const uint32_t s0 = hi8 ? gm[at][0] : gm[at][2], s1 = hi8 ? gm[at][1] : gm[at][3];
                    uint32_t k0 = hi8 ? gm[at][2] : gm[at][0], k1 = hi8 ? gm[at][3] : gm[at][1];
                    k0 = max(k0, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s0, 0x140, 0xf, 0xf, false));  // row_mirror
                    k1 = max(k1, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s1, 0x140, 0xf, 0xf, false));
                    const uint32_t s2 = hi4 ? k0 : k1;
                    uint32_t x = hi4 ? k1 : k0;
                    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s2, 0x141, 0xf, 0xf, false));  // row_half_mirror
                    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xf, 0xf, false));   // quad_perm 1,0,3,2
                    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xf, 0xf, false));   // quad_perm 2,3,0,1
                    const int64_t gi = j0 / kTopkGroup + (r >> 2);
                    if (qrow[at] >= 0 && (g % GPQ) == 0 && (r & 3) == 0 && gi < ng)
                        gmax[(t0 + qrow[at]) * ng + gi] = x;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// prefill: grid (key chunks, query tiles).  A row tile = 32 (query, head) rows
// = 32/HI queries; each wave owns NA row tiles; keys stream 32 per step.
// Rows of a wave that belong to different sequences are processed in one pass
// per distinct sequence (a single pass when the batch is one sequence).
// ---------------------------------------------------------------------------
// kEmit: segment s = blockIdx.x of every query row collects the candidates of this column
// chunk.  A wave owns its queries, so it counts their candidates itself (ballots into
// wave-uniform counters: no atomics, a fixed order) and writes the counts to cnt[t][s].
// Row tiles per wave: four for the store code (each key fragment feeds four MFMAs); two for
// the sample and emit codes, whose smaller register set leaves room for three waves per SIMD
// to hide the latency of their longer epilogue (measured: the fused call 0.85 -> 0.80 ms;
// the store code is faster with four, 0.51 against 0.70 ms).
constexpr int gemm_row_tiles(int mode) { return mode == kStore ? 4 : 2; }
constexpr int gemm_min_blocks(int hi, int mode) { return hi == 8 ? (mode == kStore ? 2 : 3) : 1; }

template <int DI, int HI, int MODE = kStore>
__global__ __launch_bounds__(256, gemm_min_blocks(HI, MODE)) void k_index_gemm(const uint8_t* __restrict__ q, const uint8_t* __restrict__ q_scale,
                                                    const float* __restrict__ w, const int32_t* __restrict__ seq,
                                                    const int64_t* __restrict__ pos, int64_t T,
                                                    const uint8_t* __restrict__ kdata,
                                                    const uint8_t* __restrict__ kscale, int64_t kcap,
                                                    const int32_t* __restrict__ kpages, int kpshift, int m,
                                                    int64_t n_cols, int64_t chunk, float* __restrict__ scores,
                                                    ItkArgs ia = {}) {
    constexpr int KB = DI / 2, NB = DI / 32;
    constexpr int KS = DI / 64;       // 32x32x64 MFMA steps per score
    constexpr int QA = 32 / HI;       // queries per row tile
    constexpr int NA = gemm_row_tiles(MODE);  // row tiles per wave
    // The head weights come from LDS (a lane's 16 per row tile depend only on its half-wave),
    // freeing registers: for the emission's third wave per SIMD, and for the store code's
    // prefetched key tile
    constexpr bool kLdsW = MODE != kSample;
    constexpr int QW = QA * NA;       // queries per wave (at most 32)
    using NvT = int32_t;              // visible counts (n_cols < 2^31)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 31, g2 = lane >> 5;
    const int64_t tq0 = ((int64_t)blockIdx.y * 4 + wave) * QW;  // first query of this wave
    if (tq0 >= T) return;
    constexpr int NI = HI == 8 ? 2 : 4;  // stored query slots per lane and row tile
    // kEmit: candidates so far of query slot (at, i) in the lower / upper half-wave: wave-uniform
    // (ballot counts), kept in scalar registers
    uint32_t ec[NA][NI][2];
#pragma unroll
    for (int at = 0; at < NA; ++at)
#pragma unroll
        for (int i = 0; i < NI; ++i) ec[at][i][0] = ec[at][i][1] = 0u;
    const int64_t c0 = (int64_t)blockIdx.x * chunk;
    const int64_t c1 = c0 + chunk < n_cols ? c0 + chunk : n_cols;
    const int64_t ncl = MODE == kSample ? ia.n_real : n_cols;  // columns of the score row
    auto real = [&](int64_t j) -> int64_t {
        if constexpr (MODE == kSample) return sample_col(j, ia.D, ia.F);
        else return j;
    };

    uint32_t todo = 0;
    for (int i = 0; i < QW; ++i)
        if (tq0 + i < T) todo |= 1u << i;

    while (todo) {
        const int first = __builtin_ctz(todo);
        const int32_t s = seq[tq0 + first];
        uint32_t mask = 0;
        for (int i = 0; i < QW; ++i)
            if (((todo >> i) & 1u) && seq[tq0 + i] == s) mask |= 1u << i;
        todo &= ~mask;

        // A fragments (rows of other sequences zeroed) and head weights
        v8i a[NA][KS];
        int sa[NA][KS];
        float wt[kLdsW ? 1 : NA][16];
        __shared__ __align__(16) float lw[kLdsW ? 4 : 1][NA][2][16];
        NvT nvq[NA][4];      // visible count per stored query slot
        float tq[NA][4];     // kEmit: threshold per stored query slot (order_key_floor)
        int64_t nv_max = 0, nv_min = INT64_MAX;
#pragma unroll
        for (int at = 0; at < NA; ++at) {
            const int qi = at * QA + r / HI, h = r % HI;
            const int64_t t = tq0 + qi;
            const bool live = (mask >> qi) & 1u;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int blk = 2 * ks + g2;
                if (live) {
                    a[at][ks] = frag16(q + (t * HI + h) * KB + blk * 16);
                    sa[at][ks] = q_scale[(t * HI + h) * NB + blk];
                } else {
                    a[at][ks] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
                    sa[at][ks] = 127;
                }
            }
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int row = 8 * (rr / 4) + 4 * g2 + (rr % 4);
                const int qj = at * QA + row / HI;
                const float wv = ((mask >> qj) & 1u) ? w[(tq0 + qj) * HI + row % HI] : 0.f;
                if constexpr (kLdsW) {
                    if (r == 0) lw[wave][at][g2][rr] = wv;
                } else {
                    wt[at][rr] = wv;
                }
            }
            for (int i = 0; i < 4; ++i) {
                // stored query slots of this lane: HI=8 -> queries 2*g2+i' (i'<2 used), HI=4 -> 2*i+g2
                const int qj = at * QA + (HI == 8 ? (i < 2 ? 2 * g2 + i : 0) : 2 * i + g2);
                int64_t nv = -1;
                float tv = 0.f;
                if (((mask >> qj) & 1u) && (HI == 4 || i < 2)) {
                    nv = (pos[tq0 + qj] + 1) / m;
                    if (nv > ncl) nv = ncl;
                    if (MODE == kEmit) tv = order_key_floor(ia.tau[tq0 + qj]);
                }
                nvq[at][i] = (NvT)nv;
                tq[at][i] = tv;
            }
        }
        for (int i = 0; i < QW; ++i)
            if ((mask >> i) & 1u) {
                int64_t nv = (pos[tq0 + i] + 1) / m;
                if (nv > ncl) nv = ncl;
                nv_max = nv > nv_max ? nv : nv_max;
                nv_min = nv < nv_min ? nv : nv_min;
            }
        // one score (or sample key, or candidate) of query slot (at, i) at tile column j (jr: score column)
        auto put = [&](int at, int i, int64_t j, int64_t jr, float v) {
            const int qj = at * QA + (HI == 8 ? 2 * g2 + i : 2 * i + g2);
            const int64_t nv = nvq[at][i];
            if constexpr (MODE == kStore) {
                scores[(tq0 + qj) * n_cols + j] = j < nv ? v : -INFINITY;
            } else if constexpr (MODE == kSample) {
                ia.samp[(tq0 + qj) * ia.n_s + j] = jr < nv ? f32_order_key(v) : 0u;
            }
        };
        // kEmit: first candidate slot of query slot (at, i) in this workgroup's segment, split
        // into a part common to the wave (scalar registers) and the lane half's offset
        int64_t cbu[NA][NI];
#pragma unroll
        for (int at = 0; at < NA; ++at)
#pragma unroll
            for (int i = 0; i < NI; ++i)
                cbu[at][i] = ((tq0 + at * QA + (HI == 8 ? i : 2 * i)) * (int64_t)gridDim.x + blockIdx.x) * ia.cap;
        const int64_t cg2 = (HI == 8 ? 2 : 1) * (int64_t)g2 * gridDim.x * ia.cap;
        const int32_t c1_32 = (int32_t)c1;
        // kEmit: the candidates of query slot (at, i), both half-waves (every lane calls it)
        auto emit = [&](int at, int i, int64_t j, float v) {
            // (columns < 2^31: 32-bit compares; a dead slot's count is -1)
            const bool pass = (int32_t)j < c1_32 && (int32_t)j < nvq[at][i] && v >= tq[at][i];
            const uint64_t mk = __builtin_amdgcn_ballot_w64(pass);
            if (mk == 0) return;
            const uint32_t lo = (uint32_t)mk, hi = (uint32_t)(mk >> 32);
            if (pass) {
                const uint32_t sl = (g2 ? ec[at][i][1] : ec[at][i][0]) + (uint32_t)__popc((g2 ? hi : lo) & ((1u << r) - 1u));
                if (sl < (uint32_t)ia.cap)
                    ia.cand[cbu[at][i] + cg2 + sl] = ((uint64_t)f32_order_key(v) << 32) | (uint32_t)~(uint32_t)j;
            }
            ec[at][i][0] += (uint32_t)__builtin_popcount(lo);
            ec[at][i][1] += (uint32_t)__builtin_popcount(hi);
        };

        // Key tiles of 32 columns: fragments of one tile, then per row tile two MFMAs and the
        // epilogue (ReLU, weighted head sum, store / sample / emit).
        auto load_tile = [&](int64_t j0n, v8i (&bb)[KS], int (&sbb)[KS]) {
            const int64_t jrn = real(j0n + r);
            const bool kload = j0n < c1 && jrn < nv_max;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int blk = 2 * ks + g2;
                if (kload) {
                    const int64_t kr = kv_row(kpages, kpshift, kcap, s, jrn);
                    bb[ks] = frag16(kdata + kr * KB + blk * 16);
                    sbb[ks] = kscale[kr * NB + blk];
                } else {
                    bb[ks] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
                    sbb[ks] = 127;
                }
            }
        };
        auto mma = [&](int at, const v8i (&bb)[KS], const int (&sbb)[KS]) -> v16f {
            v16f acc = {};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[at][ks], bb[ks], acc, 4, 4, 0, sa[at][ks], 0,
                                                                      sbb[ks]);
            return acc;
        };
        auto epilogue = [&](int at, const v16f& acc, int64_t j, int64_t jr) {
            float part[4];
            const float* wr = kLdsW ? lw[wave][at][g2] : wt[kLdsW ? 0 : at];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float p = wr[4 * i] * relu1(acc[4 * i]);
                p = fmaf(wr[4 * i + 1], relu1(acc[4 * i + 1]), p);
                p = fmaf(wr[4 * i + 2], relu1(acc[4 * i + 2]), p);
                p = fmaf(wr[4 * i + 3], relu1(acc[4 * i + 3]), p);
                part[i] = p;
            }
            if constexpr (HI == 8) {
                // query i of the tile = regs 4i..4i+3, its heads split over the lane halves.
                // Lanes < 32 keep queries 0, 1 and lanes >= 32 queries 2, 3: one swap of the
                // halves of (part[i], part[2 + i]) hands each lane its partner's half of the
                // query it keeps, and the two results sum to it (own + partner, either order)
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[i]),
                                                                     __float_as_uint(part[2 + i]), false, false);
                    const float v = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
                    if constexpr (MODE == kEmit) emit(at, i, j, v);
                    else if (nvq[at][i] >= 0 && j < c1) put(at, i, j, jr, v);
                }
            } else {
                // query 2i+g2 complete in regs 4i..4i+3
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if constexpr (MODE == kEmit) emit(at, i, j, part[i]);
                    else if (nvq[at][i] >= 0 && j < c1) put(at, i, j, jr, part[i]);
                }
            }
        };
        auto tile = [&](int64_t j0, const v8i (&bb)[KS], const int (&sbb)[KS]) {
            const int64_t j = j0 + r;
            const int64_t jr = real(j);  // a 32-column tile maps to 32 consecutive score columns
            if (real(j0) >= nv_max) {
                // nothing visible in this tile for any live query of the pass
                if constexpr (MODE != kEmit) {
#pragma unroll
                    for (int at = 0; at < NA; ++at)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (nvq[at][i] >= 0 && j < c1) put(at, i, j, jr, -INFINITY);
                }
                return;
            }
#pragma unroll
            for (int at = 0; at < NA; ++at) epilogue(at, mma(at, bb, sbb), j, jr);
        };

        if constexpr (MODE == kStore) {
            // the next tile's fragments in flight while this one computes (two register sets)
            v8i b0[KS], b1[KS];
            int sb0[KS], sb1[KS];
            load_tile(c0, b0, sb0);
            for (int64_t j0 = c0; j0 < c1; j0 += 64) {
                load_tile(j0 + 32, b1, sb1);
                tile(j0, b0, sb0);
                if (j0 + 32 >= c1) break;
                load_tile(j0 + 64, b0, sb0);
                tile(j0 + 32, b1, sb1);
            }
        } else {
            // (the sample and emit codes keep their registers for a third wave per SIMD)
            for (int64_t j0 = c0; j0 < c1; j0 += 32) {
                v8i b0[KS];
                int sb0[KS];
                load_tile(j0, b0, sb0);
                tile(j0, b0, sb0);
            }
        }
        (void)nv_min;
    }
    if constexpr (MODE == kEmit) {
        // every query of the wave got its counts in exactly one pass (zero in the others)
        if (lane == 0)
#pragma unroll
            for (int at = 0; at < NA; ++at)
#pragma unroll
                for (int i = 0; i < NI; ++i)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int qj = at * QA + (HI == 8 ? 2 * h + i : 2 * i + h);
                        if (tq0 + qj < T) ia.cnt[(tq0 + qj) * gridDim.x + blockIdx.x] = ec[at][i][h];
                    }
    }
}

hipError_t launch_index_scores(const uint8_t* q, const uint8_t* q_scale, const float* w, const int32_t* seq,
                               const int64_t* pos, int64_t T, int h_i, int d_i, const uint8_t* kdata,
                               const uint8_t* kscale, int64_t kcap, const int32_t* kpages, int kpshift, int m,
                               int64_t n_cols, float* scores, uint32_t* gmax, hipStream_t st) {
    if (T == 0 || n_cols == 0) return hipSuccess;
    if (T <= 64 || gmax) {
        // aim for >= 2048 workgroups (one 128-key step per wave at the 1M-context decode shape);
        // each wave handles 128 keys per step
        int64_t chunk = (n_cols * T + 2047) / 2048;
        chunk = ((chunk + 511) / 512) * 512;
        if (chunk < 512) chunk = 512;
        if (chunk > 16384) chunk = 16384;
        dim3 grid((unsigned)((n_cols + chunk - 1) / chunk), (unsigned)T), block(256);
        if (d_i == 128)
            hipLaunchKernelGGL((k_index_rows<128, 8>), grid, block, 0, st, q, q_scale, w, seq, pos, h_i, kdata, kscale,
                               kcap, kpages, kpshift, m, n_cols, chunk, scores, gmax);
        else
            hipLaunchKernelGGL((k_index_rows<64, 8>), grid, block, 0, st, q, q_scale, w, seq, pos, h_i, kdata, kscale,
                               kcap, kpages, kpshift, m, n_cols, chunk, scores, gmax);
        return hipGetLastError();
    }
    const int qwg = 4 * gemm_row_tiles(kStore) * (32 / h_i);  // queries per workgroup
    const int64_t qtiles = (T + qwg - 1) / qwg;
    int64_t chunk = (n_cols * qtiles + 1023) / 1024;
    chunk = ((chunk + 31) / 32) * 32;
    if (chunk < 256) chunk = 256;
    dim3 grid((unsigned)((n_cols + chunk - 1) / chunk), (unsigned)qtiles), block(256);
#define CSA_GEMM(DI, HI)                                                                                          \
    hipLaunchKernelGGL((k_index_gemm<DI, HI>), grid, block, 0, st, q, q_scale, w, seq, pos, T, kdata, kscale, kcap, \
                       kpages, kpshift, m, n_cols, chunk, scores)
    if (d_i == 128 && h_i == 8) CSA_GEMM(128, 8);
    else if (d_i == 128 && h_i == 4) CSA_GEMM(128, 4);
    else if (d_i == 64 && h_i == 8) CSA_GEMM(64, 8);
    else CSA_GEMM(64, 4);
#undef CSA_GEMM
    return hipGetLastError();
}

hipError_t launch_index_scores_grouped(const uint8_t* q, const uint8_t* q_scale, const float* w, const int32_t* seq,
                                       const int64_t* pos, int64_t T, int h_i, int d_i, const uint8_t* kdata,
                                       const uint8_t* kscale, int64_t kcap, const int32_t* kpages, int kpshift, int m,
                                       int64_t n_cols, int group, float* scores, uint32_t* gmax, hipStream_t st) {
    if (group == 1)
        return launch_index_scores(q, q_scale, w, seq, pos, T, h_i, d_i, kdata, kscale, kcap, kpages, kpshift, m, n_cols, scores, gmax,
                                   st);
    if (T == 0 || n_cols == 0) return hipSuccess;
    const int64_t G = T / group;
    // about 2048 workgroups, one 128-key step per wave at the 1M-context shape
    int64_t chunk = (n_cols * G + 2047) / 2048;
    chunk = ((chunk + 511) / 512) * 512;
    if (chunk < 512) chunk = 512;
    if (chunk > 16384) chunk = 16384;
    const dim3 grid((unsigned)((n_cols + chunk - 1) / chunk), (unsigned)G), block(256);
#define CSA_GRP(DI, R, HI)                                                                                         \
    hipLaunchKernelGGL((k_index_rows_grp<DI, R, HI>), grid, block, 0, st, q, q_scale, w, seq, pos, kdata, kscale, \
                       kcap, kpages, kpshift, m, n_cols, chunk, scores, gmax)
    if (d_i == 128) {
        if (h_i == 8) {
            if (group == 2) CSA_GRP(128, 2, 8);
            else CSA_GRP(128, 4, 8);
        } else {
            if (group == 2) CSA_GRP(128, 2, 4);
            else CSA_GRP(128, 4, 4);
        }
    } else {
        if (h_i == 8) {
            if (group == 2) CSA_GRP(64, 2, 8);
            else CSA_GRP(64, 4, 8);
        } else {
            if (group == 2) CSA_GRP(64, 2, 4);
            else CSA_GRP(64, 4, 4);
        }
    }
#undef CSA_GRP
    return hipGetLastError();
}



// ---------------------------------------------------------------------------
// Fused indexer + top-k (no score row is written):
//   1. sample    the indexer kernel scores the sample columns of every row (the
//                prefix [0, D) and one 32-column group in F after it) and
//                stores their order keys;
//   2. tau       per row, a threshold tau from the sample: the sample keys,
//                weighted 1 in the prefix and F after it (each stands for F
//                columns there), are descended to the key where the weight
//                above reaches `target` (k when the prefix covers the row,
//                k plus a margin of several standard deviations of the
//                estimate otherwise);
//   3. emit      the indexer kernel scores every column again and appends the
//                visible columns whose key is >= tau to the row's candidate
//                segments;
//   4. pick      per row, the count is verified (at least k candidates, none
//                dropped by a full segment, all fit in LDS) and the exact top-k
//                is taken among the candidates, which hold every column whose
//                key is >= tau; a row failing the check joins a list;
//   5. fallback  each listed row is scored on the vector units (exact under
//                the same precondition as the matrix-core kernels) into a
//                scratch row and selected by the whole-row radix select.
// The result equals csa_index_scores followed by csa_topk.
// ---------------------------------------------------------------------------
constexpr int kItkF = 16;          // one 32-column group in 16 is sampled after the prefix
constexpr int kItkFbGroups = 16;   // fallback workgroups
constexpr int kItkFbCache = 32768; // fallback row keys cached in LDS

struct ItkPlan {
    bool gemm;
    int D, F;
    int64_t n_s, chunk_s, chunk_e;
    int S, cap, target_far, lcap;
    size_t off_samp, off_tau, off_cnt, off_cand, off_fb, off_fbrow, total;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static ItkPlan itk_plan(int64_t T, int64_t n_cols, int k, int h_i) {
    ItkPlan p{};
    p.gemm = T > 64;
    p.F = kItkF;
    p.D = (int)(((k > 1024 ? 2 * k : 2048) + 32 * kItkF - 1) / (32 * kItkF) * (32 * kItkF));
    p.n_s = n_cols <= p.D ? n_cols : p.D + (n_cols - p.D + 32 * p.F - 1) / (32 * p.F) * 32;
    // weighted target beyond the prefix: k plus 6 standard deviations of the estimate (the count
    // of sampled columns above the k-th largest is about binomial, sd ~ F sqrt(k / F)) and 8
    // groups' worth
    const double sd = p.F * sqrt((double)k / p.F);
    p.target_far = k + (int)ceil(6.0 * sd + 8.0 * p.F);
    if (!p.gemm) {
        auto rows_chunk = [&](int64_t n) {
            int64_t c = (n * T + 2047) / 2048;
            c = ((c + 511) / 512) * 512;
            return c < 512 ? (int64_t)512 : (c > 16384 ? (int64_t)16384 : c);
        };
        p.chunk_s = rows_chunk(p.n_s);
        p.chunk_e = rows_chunk(n_cols);
        p.S = kItkRowSegs;
        // each segment holds 4x its share of the expected candidates (at least 256)
        p.cap = (int)(4 * (int64_t)p.target_far / kItkRowSegs);
        if (p.cap < 256) p.cap = 256;
        p.lcap = 8192;
    } else {
        // queries per workgroup: 4 waves x 4 row tiles x 32 / h_i
        auto gemm_chunk = [&](int64_t n, int na) {
            const int64_t qtiles = (T + 4 * na * (32 / h_i) - 1) / (4 * na * (32 / h_i));
            int64_t c = (n * qtiles + 1023) / 1024;
            c = ((c + 31) / 32) * 32;
            return c < 256 ? (int64_t)256 : c;
        };
        p.chunk_s = gemm_chunk(p.n_s, 4);
        p.chunk_e = gemm_chunk(n_cols, 4);
        // one candidate segment per column chunk, at most 64 per row (the pick scans the
        // segment counts with one wave)
        const int64_t min_chunk = ((n_cols + 63) / 64 + 31) / 32 * 32;
        if (p.chunk_e < min_chunk) p.chunk_e = min_chunk;
        p.S = (int)((n_cols + p.chunk_e - 1) / p.chunk_e);
        // a segment holds twice its share of the expected candidates (or its whole chunk)
        int64_t c = 2 * (int64_t)p.target_far * p.chunk_e / n_cols + 512;
        if (c < 1024) c = 1024;
        if (c > p.chunk_e) c = p.chunk_e;
        p.cap = (int)c;
        // candidates held in LDS: 3,072 leaves room for three picking workgroups per CU (the
        // count sits within a few sd of target_far; a row beyond the space falls back)
        p.lcap = p.target_far + 8 * sd <= 3072 ? 3072 : (p.target_far <= 2048 ? 4096 : 8192);
    }
    const int G = (int)(T < kItkFbGroups ? T : kItkFbGroups);
    p.off_samp = 0;
    p.off_tau = align256(p.off_samp + (size_t)T * p.n_s * 4);
    p.off_cnt = align256(p.off_tau + (size_t)T * 4);
    p.off_cand = align256(p.off_cnt + (size_t)T * p.S * 4);
    p.off_fb = align256(p.off_cand + (size_t)T * p.S * p.cap * 8);
    p.off_fbrow = align256(p.off_fb + (size_t)(64 + T) * 4);
    p.total = align256(p.off_fbrow + (size_t)G * n_cols * 4);
    return p;
}

size_t index_topk_workspace_bytes(int64_t T, int64_t n_cols, int k, int h_i) {
    if (T == 0 || n_cols == 0) return 0;
    return itk_plan(T, n_cols, k, h_i).total;
}

// 2. per-row threshold from the sample (one workgroup per row; PER > 0: the row's sample keys
//    held in registers, PER sample columns per thread, else re-read at every descent level).
//    Also clears the row's candidate counters (decode layout) and, in workgroup 0, the
//    fallback list.
template <int NT, int PER>
__global__ __launch_bounds__(NT) void k_itk_tau(const uint32_t* __restrict__ samp, int64_t n_s,
                                                const int64_t* __restrict__ pos, int m, int64_t n_cols, int k, int D,
                                                int F, int target_far, uint32_t* __restrict__ tau,
                                                uint32_t* __restrict__ cnt_rows, uint32_t* __restrict__ fb) {
    constexpr int NW = NT / 64;
    __shared__ uint32_t h[4096];
    __shared__ int wsum[NW];
    __shared__ int bc[4];
    __shared__ uint32_t red[3 * NW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t t = blockIdx.x;
    if (t == 0 && tid < 2) fb[tid] = 0;  // fallback count and cursor
    if (cnt_rows && tid < kItkRowSegs) cnt_rows[t * kItkRowSegs + tid] = 0;
    const int64_t nv = row_visible(pos, t, m, n_cols);
    if (nv <= k) {
        if (tid == 0) tau[t] = 0xFFFFFFFFu;  // every visible column is taken; nothing is emitted
        return;
    }
    const uint32_t* row = samp + t * n_s;
    uint32_t kr[PER > 0 ? PER : 1];
    if constexpr (PER > 0) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int64_t v = tid + (int64_t)i * NT;
            kr[i] = v < n_s ? row[v] : 0u;
        }
    }
    // every visible sample key (nonzero) with its column, in any order
    auto for_keys = [&](auto fn) {
        if constexpr (PER > 0) {
#pragma unroll
            for (int i = 0; i < PER; ++i)
                if (kr[i]) fn(kr[i], tid + (int64_t)i * NT);
        } else {
            for (int64_t v = tid; v < n_s; v += NT) {
                const uint32_t key = row[v];
                if (key) fn(key, v);
            }
        }
    };
    auto wgt = [&](int64_t v) -> uint32_t { return v < D ? 1u : (uint32_t)F; };
    for (int i = tid; i < 4096; i += NT) h[i] = 0;
    // the descent's bins span [smallest, largest] visible sample key: a span from key 1 would
    // put nearly every key into a few bins and serialise the histogram's atomics
    uint32_t mx = 0, mn = 0xFFFFFFFFu, wt = 0;
    for_keys([&](uint32_t key, int64_t v) {
        mx = max(mx, key);
        mn = min(mn, key);
        wt += wgt(v);
    });
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
        mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
        wt += (uint32_t)__shfl_xor((int)wt, o);
    }
    if (lane == 0) {
        red[wave] = mx;
        red[NW + wave] = wt;
        red[2 * NW + wave] = mn;
    }
    __syncthreads();
    uint32_t hi = 0, W = 0, lo = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        hi = max(hi, red[i]);
        W += red[NW + i];
        lo = min(lo, red[2 * NW + i]);
    }
    const int target = nv <= D ? k : target_far;  // the prefix covers the row: the sample is the row
    uint32_t th = 1u;                             // all visible columns
    if ((int64_t)W >= target) {
        int sh, ab, nb;
        hist_descend<NT>([&](auto fn) { for_keys([&](uint32_t key, int64_t v) { fn(key, wgt(v)); }); }, lo, hi,
                         target, 16 * F, h, wsum, bc, th, sh, ab, nb);
    }
    if (tid == 0) tau[t] = th;
}

// 4. per-row exact selection among the candidates, or the row joins the fallback list.
template <int NT, int LCAP, int BMW>
__global__ __launch_bounds__(NT) void k_itk_pick(const uint32_t* __restrict__ cnt, const uint64_t* __restrict__ cand,
                                                 const uint32_t* __restrict__ tau, int S, int cap,
                                                 const int64_t* __restrict__ pos, int m, int64_t n_cols, int k,
                                                 int32_t* __restrict__ idx, uint32_t* __restrict__ fb) {
    constexpr int NW = NT / 64;
    static_assert(BMW % NT == 0 && BMW >= 2048, "bitmap in whole per-thread runs; room for 2048 winners");
    __shared__ uint32_t h[4096];
    __shared__ __align__(16) uint64_t cl[LCAP];
    __shared__ uint32_t bm[BMW];
    __shared__ uint64_t tie[kTieLds];
    __shared__ int wsum[2 * NW];
    __shared__ int bc[4];
    __shared__ uint32_t lctr[4];
    __shared__ int soff[65];
    __shared__ uint32_t red[NW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t t = blockIdx.x;
    const int nv = (int)row_visible(pos, t, m, n_cols);
    int32_t* out = idx + t * (int64_t)k;
    if (nv <= k) {
        for (int a = tid; a < k; a += NT) out[a] = a < nv ? a : -1;
        return;
    }
    // segment counts (S <= 64): offsets by one wave scan
    if (wave == 0) {
        const uint32_t c = lane < S ? cnt[t * S + lane] : 0u;
        const bool over = c > (uint32_t)cap;
        const int x = wave_incl_scan(over ? 0 : (int)c);
        if (lane < S) soff[lane] = x - (int)c;
        const bool bad = __ballot(over) != 0;
        if (lane == 63) soff[64] = bad ? -1 : x;
    }
    const int nwords = (nv + 31) / 32;
    const bool use_bm = nwords <= BMW;
    const int perw = (nwords + NT - 1) / NT;
    if (use_bm)
        for (int i = tid; i < perw * NT; i += NT) bm[i] = 0;
    for (int i = tid; i < 4096; i += NT) h[i] = 0;
    if (tid < 2) lctr[tid] = 0;
    __syncthreads();
    const int n_cand = soff[64];
    if (n_cand < k || n_cand > LCAP) {  // a segment overflowed, too few, or too many for LDS
        if (tid == 0) fb[64 + atomicAdd(&fb[0], 1u)] = (uint32_t)t;
        return;
    }
    uint32_t mx = 0;
    for (int sg = wave; sg < S; sg += NW) {
        const int n = (sg + 1 < S ? soff[sg + 1] : n_cand) - soff[sg];
        const uint64_t* src = cand + (t * S + sg) * (int64_t)cap;
        for (int j = lane; j < n; j += 64) {
            const uint64_t c = src[j];
            cl[soff[sg] + j] = c;
            mx = max(mx, (uint32_t)(c >> 32));
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    uint32_t hi = red[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) hi = max(hi, red[i]);
    pick_candidates<NT>(cl, n_cand, tau[t], hi, k, out, bm, use_bm, perw, h, tie, wsum, bc, lctr);
}

// 5. rows whose candidates failed the check: every score of the row on the vector units
//    (E2M1 x E2M1 products exact in fp32, sums exact under the indexer's precondition) into
//    this workgroup's scratch row, then the whole-row radix select.  Workgroups take listed
//    rows in turn until the list is exhausted.
__global__ __launch_bounds__(kTopkThreads) void k_itk_fallback(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ q_scale, const float* __restrict__ w,
    const int32_t* __restrict__ seq, const int64_t* __restrict__ pos, int h_i, int d_i,
    const uint8_t* __restrict__ kdata, const uint8_t* __restrict__ kscale, int64_t kcap,
    const int32_t* __restrict__ kpages, int kpshift, int m, int64_t n_cols, int k, int32_t* __restrict__ idx,
    uint32_t* __restrict__ fb, float* __restrict__ fbrow) {
    constexpr int NT = kTopkThreads;
    __shared__ uint32_t hist[4096];
    __shared__ __align__(16) uint32_t cache[kItkFbCache];
    __shared__ float qf[8 * 128];
    __shared__ float wh[8];
    __shared__ int wsum[2 * (NT / 64)];
    __shared__ int bcast[4];
    __shared__ int cur;
    const int tid = threadIdx.x;
    float* srow = fbrow + (int64_t)blockIdx.x * n_cols;
    const int KB = d_i / 2, NB = d_i / 32;
    const float e2m1[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};
    for (;;) {
        if (tid == 0) cur = (int)atomicAdd(&fb[1], 1u);
        __syncthreads();
        const int i = cur;
        if (i >= (int)fb[0]) break;
        const int64_t t = (int64_t)fb[64 + i];
        const int nv = (int)row_visible(pos, t, m, n_cols);
        for (int e = tid; e < h_i * d_i; e += NT) {
            const int hh = e / d_i, c = e % d_i;
            const uint8_t byte = q[(t * h_i + hh) * KB + c / 2];
            const uint32_t nib = (c & 1) ? (byte >> 4) : (byte & 15);
            const float v = e2m1[nib & 7] * ((nib & 8) ? -1.f : 1.f);
            qf[e] = ldexpf(v, (int)q_scale[(t * h_i + hh) * NB + c / 32] - 127);
        }
        if (tid < h_i) wh[tid] = w[t * h_i + tid];
        __syncthreads();
        const int32_t sq = seq[t];
        for (int j = tid; j < nv; j += NT) {
            const int64_t kr = kv_row(kpages, kpshift, kcap, sq, j);
            const uint8_t* kd = kdata + kr * KB;
            const uint8_t* ks = kscale + kr * NB;
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (int b = 0; b < NB; ++b) {
                const int sc = (int)ks[b] - 127;
                for (int c = 32 * b; c < 32 * b + 32; ++c) {
                    const uint32_t nib = (c & 1) ? (kd[c / 2] >> 4) : (kd[c / 2] & 15);
                    const float kv = ldexpf(e2m1[nib & 7] * ((nib & 8) ? -1.f : 1.f), sc);
#pragma unroll
                    for (int hh = 0; hh < 8; ++hh)
                        if (hh < h_i) acc[hh] = fmaf(qf[hh * d_i + c], kv, acc[hh]);
                }
            }
            float p = 0.f;
#pragma unroll
            for (int hh = 0; hh < 8; ++hh)
                if (hh < h_i) p = fmaf(wh[hh], relu1(acc[hh]), p);
            srow[j] = p;
        }
        __syncthreads();  // the scratch row is complete (and qf no longer read)
        row_select(srow, nv, k, idx + t * (int64_t)k, hist, cache, kItkFbCache, wsum, bcast);
        __syncthreads();
    }
}

hipError_t launch_index_topk(const uint8_t* q, const uint8_t* q_scale, const float* w, const int32_t* seq,
                             const int64_t* pos, int64_t T, int h_i, int d_i, const uint8_t* kdata,
                             const uint8_t* kscale, int64_t kcap, const int32_t* kpages, int kpshift, int m,
                             int64_t n_cols, int k, int32_t* idx, void* ws, hipStream_t st) {
    if (T == 0) return hipSuccess;
    const ItkPlan p = itk_plan(T, n_cols, k, h_i);
    if (p.S < 1 || p.S > 64) return hipErrorInvalidValue;  // k_itk_pick reads at most 64 segment counts
    char* wb = (char*)ws;
    ItkArgs ia;
    ia.samp = (uint32_t*)(wb + p.off_samp);
    ia.n_s = p.n_s;
    ia.n_real = n_cols;
    ia.D = p.D;
    ia.F = p.F;
    ia.tau = (const uint32_t*)(wb + p.off_tau);
    ia.cnt = (uint32_t*)(wb + p.off_cnt);
    ia.cand = (uint64_t*)(wb + p.off_cand);
    ia.cap = p.cap;
    uint32_t* tau = (uint32_t*)(wb + p.off_tau);
    uint32_t* fb = (uint32_t*)(wb + p.off_fb);
    float* fbrow = (float*)(wb + p.off_fbrow);

    // 1. sample, 3. emit: the indexer kernel of csa_index_scores for this shape
    auto indexer = [&](int mode) {
        const int64_t n = mode == kSample ? p.n_s : n_cols;
        const int64_t chunk = mode == kSample ? p.chunk_s : p.chunk_e;
        if (!p.gemm) {
            const dim3 grid((unsigned)((n + chunk - 1) / chunk), (unsigned)T), block(256);
#define CSA_ROWS(DI, MD)                                                                                              \
    hipLaunchKernelGGL((k_index_rows<DI, 8, MD>), grid, block, 0, st, q, q_scale, w, seq, pos, h_i, kdata, kscale, kcap, \
                       kpages, kpshift, m, n, chunk, nullptr, nullptr, ia)
            if (d_i == 128) {
                if (mode == kSample) CSA_ROWS(128, kSample);
                else CSA_ROWS(128, kEmit);
            } else {
                if (mode == kSample) CSA_ROWS(64, kSample);
                else CSA_ROWS(64, kEmit);
            }
#undef CSA_ROWS
        } else {
            const int qwg = 4 * gemm_row_tiles(kEmit) * (32 / h_i);  // (sample and emit alike)
            const dim3 grid((unsigned)((n + chunk - 1) / chunk), (unsigned)((T + qwg - 1) / qwg)), block(256);
#define CSA_GEMM(DI, HI, MD)                                                                                      \
    hipLaunchKernelGGL((k_index_gemm<DI, HI, MD>), grid, block, 0, st, q, q_scale, w, seq, pos, T, kdata, kscale, \
                       kcap, kpages, kpshift, m, n, chunk, nullptr, ia)
#define CSA_GEMM_M(DI, HI)                   \
    if (mode == kSample) CSA_GEMM(DI, HI, kSample); \
    else CSA_GEMM(DI, HI, kEmit)
            if (d_i == 128 && h_i == 8) { CSA_GEMM_M(128, 8); }
            else if (d_i == 128 && h_i == 4) { CSA_GEMM_M(128, 4); }
            else if (d_i == 64 && h_i == 8) { CSA_GEMM_M(64, 8); }
            else { CSA_GEMM_M(64, 4); }
#undef CSA_GEMM_M
#undef CSA_GEMM
        }
    };
    indexer(kSample);
    {
        // one workgroup per row: 256 threads for many rows, 1024 for few; sample keys in registers
        const int nt = p.gemm ? 256 : 1024;
        const int64_t per = (p.n_s + nt - 1) / nt;
        uint32_t* cr = p.gemm ? (uint32_t*)nullptr : ia.cnt;
#define CSA_TAU(NT, PER)                                                                                     \
    hipLaunchKernelGGL((k_itk_tau<NT, PER>), dim3((unsigned)T), dim3(NT), 0, st, ia.samp, p.n_s, pos, m, n_cols, \
                       k, p.D, p.F, p.target_far, tau, cr, fb)
        if (nt == 256) {
            if (per <= 8) CSA_TAU(256, 8);
            else if (per <= 16) CSA_TAU(256, 16);  // (the chunked-prefill shape: fewer registers, more waves)
            else if (per <= 24) CSA_TAU(256, 24);
            else CSA_TAU(256, 0);
        } else {
            if (per <= 8) CSA_TAU(1024, 8);
            else if (per <= 24) CSA_TAU(1024, 24);
            else CSA_TAU(1024, 0);
        }
#undef CSA_TAU
    }
    indexer(kEmit);
    if (p.lcap == 3072)
        hipLaunchKernelGGL((k_itk_pick<512, 3072, 2048>), dim3((unsigned)T), dim3(512), 0, st, ia.cnt, ia.cand, tau,
                           p.S, p.cap, pos, m, n_cols, k, idx, fb);
    else if (p.lcap == 4096)
        hipLaunchKernelGGL((k_itk_pick<512, 4096, 2048>), dim3((unsigned)T), dim3(512), 0, st, ia.cnt, ia.cand, tau,
                           p.S, p.cap, pos, m, n_cols, k, idx, fb);
    else
        hipLaunchKernelGGL((k_itk_pick<1024, 8192, 16384>), dim3((unsigned)T), dim3(1024), 0, st, ia.cnt, ia.cand, tau,
                           p.S, p.cap, pos, m, n_cols, k, idx, fb);
    const int G = (int)(T < kItkFbGroups ? T : kItkFbGroups);
    hipLaunchKernelGGL(k_itk_fallback, dim3((unsigned)G), dim3(kTopkThreads), 0, st, q, q_scale, w, seq, pos, h_i, d_i,
                       kdata, kscale, kcap, kpages, kpshift, m, n_cols, k, idx, fb, fbrow);
    return hipGetLastError();
}

}  // namespace csa
