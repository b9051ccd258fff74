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
#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {

__device__ __forceinline__ v8i frag16(const uint8_t* p) {
    v4i x = *(const v4i*)p;
    v8i r = {x[0], x[1], x[2], x[3], 0, 0, 0, 0};
    return r;
}

// ---------------------------------------------------------------------------
// decode: grid (key chunks, T), 4 waves; each wave streams tiles of 16 keys
// ---------------------------------------------------------------------------
template <int DI, int U>
__global__ __launch_bounds__(256) void k_index_rows(const uint8_t* __restrict__ q, const uint8_t* __restrict__ q_scale,
                                                    const float* __restrict__ w, const int32_t* __restrict__ seq,
                                                    const int64_t* __restrict__ pos, int h_i,
                                                    const uint8_t* __restrict__ kdata,
                                                    const uint8_t* __restrict__ kscale, int64_t kcap, int m,
                                                    int64_t n_cols, int64_t chunk, float* __restrict__ scores,
                                                    uint32_t* __restrict__ gmax) {
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
    int64_t nv = (pos[t] + 1) / m;
    if (nv > n_cols) nv = n_cols;
    const int64_t base = (int64_t)seq[t] * kcap;
    const int64_t c0 = (int64_t)blockIdx.x * chunk;
    const int64_t c1 = c0 + chunk < n_cols ? c0 + chunk : n_cols;
    float* out = scores + t * n_cols;

    for (int64_t j0 = c0 + (int64_t)wave * 16 * U; j0 < c1; j0 += 4 * 16 * U) {
        uint32_t gm[4] = {0u, 0u, 0u, 0u};  // per summary group of this step: largest visible order key (lanes < 16)
        v4i bk[U];
        int sb[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = j0 + u * 16 + r;
            if (j < nv && g < NB) {
                // streamed once: nontemporal, so the keys do not displace cached lines
                bk[u] = __builtin_nontemporal_load((const v4i*)(kdata + (base + j) * KB + g * 16));
                sb[u] = kscale[(base + j) * NB + g];
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
            float p = wr[0] * fmaxf(acc[0], 0.f);
            p = fmaf(wr[1], fmaxf(acc[1], 0.f), p);
            p = fmaf(wr[2], fmaxf(acc[2], 0.f), p);
            p = fmaf(wr[3], fmaxf(acc[3], 0.f), p);
            p = rows4_sum(p);  // the four head groups (exact: every partial sum is representable)
            const int64_t j = j0 + u * 16 + r;
            pv[u] = j < nv ? p : -INFINITY;
            if (lane < 16 && j < c1 && j < nv) gm[u / (U / 4)] = max(gm[u / (U / 4)], f32_order_key(p));
        }
        {
            // the step's 128 scores in two full-wave stores: lane (r, g) writes keys j0 + 16 g + r
            // and j0 + 64 + 16 g + r (a quarter-wave store per tile would issue four times as many)
            static_assert(U == 8, "two stores of 64 keys");
            const float v0 = g == 0 ? pv[0] : g == 1 ? pv[1] : g == 2 ? pv[2] : pv[3];
            const float v1 = g == 0 ? pv[4] : g == 1 ? pv[5] : g == 2 ? pv[6] : pv[7];
            const int64_t ja = j0 + lane, jb = j0 + 64 + lane;
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
                                                        const uint8_t* __restrict__ kscale, int64_t kcap, int m,
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
        const int64_t base = (int64_t)s * kcap;

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
                    bk[u] = __builtin_nontemporal_load((const v4i*)(kdata + (base + j) * KB + g * 16));
                    sb[u] = kscale[(base + j) * NB + g];
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
                    float p = wr[at][0] * fmaxf(acc[0], 0.f);
                    p = fmaf(wr[at][1], fmaxf(acc[1], 0.f), p);
                    p = fmaf(wr[at][2], fmaxf(acc[2], 0.f), p);
                    p = fmaf(wr[at][3], fmaxf(acc[3], 0.f), p);
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
template <int DI, int HI>
__global__ __launch_bounds__(256) void k_index_gemm(const uint8_t* __restrict__ q, const uint8_t* __restrict__ q_scale,
                                                    const float* __restrict__ w, const int32_t* __restrict__ seq,
                                                    const int64_t* __restrict__ pos, int64_t T,
                                                    const uint8_t* __restrict__ kdata,
                                                    const uint8_t* __restrict__ kscale, int64_t kcap, int m,
                                                    int64_t n_cols, int64_t chunk, float* __restrict__ scores) {
    constexpr int KB = DI / 2, NB = DI / 32;
    constexpr int KS = DI / 64;       // 32x32x64 MFMA steps per score
    constexpr int QA = 32 / HI;       // queries per row tile
    constexpr int NA = 4;             // row tiles per wave
    constexpr int QW = QA * NA;       // queries per wave (16 or 32)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 31, g2 = lane >> 5;
    const int64_t tq0 = ((int64_t)blockIdx.y * 4 + wave) * QW;  // first query of this wave
    if (tq0 >= T) return;
    const int64_t c0 = (int64_t)blockIdx.x * chunk;
    const int64_t c1 = c0 + chunk < n_cols ? c0 + chunk : n_cols;

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
        float wt[NA][16];
        int64_t nvq[NA][4];  // visible count per stored query slot
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
                wt[at][rr] = ((mask >> qj) & 1u) ? w[(tq0 + qj) * HI + row % HI] : 0.f;
            }
            for (int i = 0; i < 4; ++i) {
                // stored query slots of this lane: HI=8 -> queries 2*g2+i' (i'<2 used), HI=4 -> 2*i+g2
                const int qj = at * QA + (HI == 8 ? (i < 2 ? 2 * g2 + i : 0) : 2 * i + g2);
                int64_t nv = -1;
                if (((mask >> qj) & 1u) && (HI == 4 || i < 2)) {
                    nv = (pos[tq0 + qj] + 1) / m;
                    if (nv > n_cols) nv = n_cols;
                }
                nvq[at][i] = nv;
            }
        }
        for (int i = 0; i < QW; ++i)
            if ((mask >> i) & 1u) {
                int64_t nv = (pos[tq0 + i] + 1) / m;
                if (nv > n_cols) nv = n_cols;
                nv_max = nv > nv_max ? nv : nv_max;
                nv_min = nv < nv_min ? nv : nv_min;
            }
        const int64_t base = (int64_t)s * kcap;

        for (int64_t j0 = c0; j0 < c1; j0 += 32) {
            const int64_t j = j0 + r;
            if (j0 >= nv_max) {
                // nothing visible in this tile for any live query of the pass
#pragma unroll
                for (int at = 0; at < NA; ++at)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (nvq[at][i] >= 0 && j < c1) {
                            const int qj = at * QA + (HI == 8 ? 2 * g2 + i : 2 * i + g2);
                            scores[(tq0 + qj) * n_cols + j] = -INFINITY;
                        }
                continue;
            }
            v8i b[KS];
            int sb[KS];
            const bool kload = j < nv_max;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int blk = 2 * ks + g2;
                if (kload) {
                    b[ks] = frag16(kdata + (base + j) * KB + blk * 16);
                    sb[ks] = kscale[(base + j) * NB + blk];
                } else {
                    b[ks] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
                    sb[ks] = 127;
                }
            }
#pragma unroll
            for (int at = 0; at < NA; ++at) {
                v16f acc = {};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[at][ks], b[ks], acc, 4, 4, 0, sa[at][ks], 0,
                                                                          sb[ks]);
                float part[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float p = wt[at][4 * i] * fmaxf(acc[4 * i], 0.f);
                    p = fmaf(wt[at][4 * i + 1], fmaxf(acc[4 * i + 1], 0.f), p);
                    p = fmaf(wt[at][4 * i + 2], fmaxf(acc[4 * i + 2], 0.f), p);
                    p = fmaf(wt[at][4 * i + 3], fmaxf(acc[4 * i + 3], 0.f), p);
                    part[i] = p;
                }
                if constexpr (HI == 8) {
                    // query i of the tile = regs 4i..4i+3; heads split over lane halves
#pragma unroll
                    for (int i = 0; i < 4; ++i) part[i] += __shfl_xor(part[i], 32);
                    // lanes < 32 store queries 0,1; lanes >= 32 store queries 2,3
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const int64_t nv = nvq[at][i];
                        const float v = g2 ? part[2 + i] : part[i];
                        if (nv >= 0 && j < c1) {
                            const int qj = at * QA + 2 * g2 + i;
                            scores[(tq0 + qj) * n_cols + j] = j < nv ? v : -INFINITY;
                        }
                    }
                } else {
                    // query 2i+g2 complete in regs 4i..4i+3
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int64_t nv = nvq[at][i];
                        if (nv >= 0 && j < c1) {
                            const int qj = at * QA + 2 * i + g2;
                            scores[(tq0 + qj) * n_cols + j] = j < nv ? part[i] : -INFINITY;
                        }
                    }
                }
            }
        }
        (void)nv_min;
    }
}

hipError_t launch_index_scores(const uint8_t* q, const uint8_t* q_scale, const float* w, const int32_t* seq,
                               const int64_t* pos, int64_t T, int h_i, int d_i, const uint8_t* kdata,
                               const uint8_t* kscale, int64_t kcap, int m, int64_t n_cols, float* scores,
                               uint32_t* gmax, hipStream_t st) {
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
                               kcap, m, n_cols, chunk, scores, gmax);
        else
            hipLaunchKernelGGL((k_index_rows<64, 8>), grid, block, 0, st, q, q_scale, w, seq, pos, h_i, kdata, kscale,
                               kcap, m, n_cols, chunk, scores, gmax);
        return hipGetLastError();
    }
    const int qwg = 4 * 4 * (32 / h_i);  // queries per workgroup
    const int64_t qtiles = (T + qwg - 1) / qwg;
    int64_t chunk = (n_cols * qtiles + 1023) / 1024;
    chunk = ((chunk + 31) / 32) * 32;
    if (chunk < 256) chunk = 256;
    dim3 grid((unsigned)((n_cols + chunk - 1) / chunk), (unsigned)qtiles), block(256);
#define CSA_GEMM(DI, HI)                                                                                          \
    hipLaunchKernelGGL((k_index_gemm<DI, HI>), grid, block, 0, st, q, q_scale, w, seq, pos, T, kdata, kscale, kcap, \
                       m, n_cols, chunk, scores)
    if (d_i == 128 && h_i == 8) CSA_GEMM(128, 8);
    else if (d_i == 128 && h_i == 4) CSA_GEMM(128, 4);
    else if (d_i == 64 && h_i == 8) CSA_GEMM(64, 8);
    else CSA_GEMM(64, 4);
#undef CSA_GEMM
    return hipGetLastError();
}

hipError_t launch_index_scores_grouped(const uint8_t* q, const uint8_t* q_scale, const float* w, const int32_t* seq,
                                       const int64_t* pos, int64_t T, int h_i, int d_i, const uint8_t* kdata,
                                       const uint8_t* kscale, int64_t kcap, int m, int64_t n_cols, int group,
                                       float* scores, uint32_t* gmax, hipStream_t st) {
    if (group == 1)
        return launch_index_scores(q, q_scale, w, seq, pos, T, h_i, d_i, kdata, kscale, kcap, m, n_cols, scores, gmax,
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
                       kcap, m, n_cols, chunk, scores, gmax)
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


}  // namespace csa
