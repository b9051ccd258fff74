// csa_sparse_mqa / hca_dense_mqa kernels: multi-query attention over a key
// list (selected or all visible compressed entries, then the window tokens),
// one shared KV head, every entry both key and value.
//
// Grid: one workgroup per (row, split); a split is a contiguous range of the
// row's key list.  Per tile of 32 keys the workgroup
//   1. stages the entries into LDS twice: a row-major bf16 copy (FP8 codes
//      and bf16 RoPE dims, both exact in bf16) for QK, and a transposed fp16
//      copy (codes exact in fp16) for PV; the next tile's entries are already
//      in flight into registers while the current tile computes;
//   2. S^T = K Q^T with bf16 MFMA 16x16x32: rows = keys, columns = heads; the
//      query (RoPE applied at t in fp32) lives in registers, its 64 RoPE dims
//      split hi + lo in bf16 so they keep ~16 bits; the FP8 part's per-entry
//      scale multiplies the fp32 accumulator;
//   3. online softmax in fp32 per head (running max / sum);
//   4. O^T += V^T P^T with fp16 MFMA 16x16x32 into fp32 accumulators
//      (dims x heads).  For the FP8 dims P carries scale_j / S_tile (S_tile =
//      largest scale of the tile, so P stays within [0, 1]); the accumulators
//      are kept in units of the current S_tile and rescaled with the softmax
//      correction when it changes.
// A single split writes the normalised output (inverse RoPE on the last 64
// dims); several splits write unnormalised partials plus (max, sum), merged by
// k_mqa_combine in the fixed split order (a log-sum-exp merge).
#include <type_traits>

#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {

constexpr int KT = 32;   // keys per tile
constexpr int RB = 256;  // key-list positions resolved per batch (8 tiles)

template <int H, int D>
struct MqaSmem {
    static constexpr int DN = D - 64;
    static constexpr int KR = D + 8;    // bf16 row stride of the key copy
    static constexpr int VT = KT + 8;   // fp16 row stride of the transposed value copy
    static constexpr int SS = H + 4;    // fp32 row stride of the score tile
    static constexpr int PS = KT + 8;   // fp16 row stride of P
    __bf16 kr[KT * KR];
    _Float16 vt[D * VT];
    float s[KT * SS];
    _Float16 pn[H * PS];  // P * scale_j / S_tile (FP8 dims)
    _Float16 pr[H * PS];  // P (RoPE dims)
    float alpha[H];
    float mrun[H];
    float lrun[H];
    float cs[64];         // cos / sin of t * theta_i, i < 32
    int64_t row[RB];      // cache rows of the current batch of key-list positions: >= 0 comp, <= -2 window, -1 masked
    float scl[2][KT];     // entry scales of the tile (0 when masked)
    int valid[2][KT];
    float sfac[2];        // ratio old S_tile / new S_tile for the FP8 accumulators
};

struct RowKeys {
    int64_t n_c, n, lo;  // compressed positions, total positions, first window token
    int64_t nv;
};

__device__ __forceinline__ RowKeys row_keys(int64_t t, const int32_t* idx, int k, int m, int window) {
    RowKeys r;
    r.nv = (t + 1) / m;
    if (r.nv < 0) r.nv = 0;
    r.n_c = idx ? k : r.nv;
    r.lo = t - window + 1 < 0 ? 0 : t - window + 1;
    const int64_t n_w = window > 0 ? t - r.lo + 1 : 0;
    r.n = r.n_c + n_w;
    return r;
}

// Key-list position u of row t -> encoded cache row (comp >= 0, window <= -2, masked -1).
__device__ __forceinline__ int64_t resolve(int64_t u, int64_t t, int32_t sq, const RowKeys& rk, const int32_t* idx,
                                           int k, const KvView& comp, const KvView& win) {
    if (u < rk.n_c) {
        const int64_t j = idx ? (int64_t)idx[t * k + u] : u;
        if (j < 0 || j >= rk.nv) return -1;
        return kv_row(comp.pages, comp.pshift, comp.cap, sq, j % comp.cap);
    }
    const int64_t p = rk.lo + (u - rk.n_c);
    return -(kv_row(win.pages, win.pshift, win.cap, sq, p % win.cap) + 2);
}

// cos / sin of pos * theta: fp64 product, fp64 reduction by 2*pi (two-part
// constant), fp32 sincos of the reduced angle.
__device__ __forceinline__ void angle_cs(double pos, double theta, float& c, float& s) {
    const double a = pos * theta;
    const double k = rint(a * 0.15915494309189533577);
    double r = fma(-k, 6.28318530717958623200, a);
    r = fma(-k, 2.44929359829470635445e-16, r);
    sincosf((float)r, &s, &c);
}

template <int H, int D>
__global__ __launch_bounds__(256) void k_mqa(const uint16_t* __restrict__ q, const int32_t* __restrict__ seq,
                                             const int64_t* __restrict__ pos, const int32_t* __restrict__ idx, int k,
                                             int m, KvView comp, KvView win, int window, float sm_scale, RopeTab rt,
                                             int S, float* __restrict__ out, float* __restrict__ lse,
                                             float* __restrict__ part_o, float* __restrict__ part_ml) {
    using Sm = MqaSmem<H, D>;
    constexpr int DN = Sm::DN;
    constexpr int HT = H / 16;                  // head tiles
    constexpr int QK_KS = HT >= 4 ? 2 : 1;       // key subtiles per wave in QK
    constexpr int DSTEP = D / 32;               // 32-dim steps
    constexpr int NSTEP = DN / 32;              // steps over the FP8 dims
    constexpr int TPH = 256 / H;                // softmax threads per head
    constexpr int KPT = KT / TPH;               // keys per softmax thread
    constexpr int DW = D / 4;                   // dims per wave in PV
    constexpr int DT = DW / 16;                 // 16-dim tiles per wave in PV
    constexpr int CPK = DN / 16 + 8;            // 16-byte chunks per entry
    constexpr int NCH = (KT * CPK + 255) / 256;  // chunks per thread per tile

    __shared__ Sm sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int64_t t = blockIdx.x / S;
    const int s = blockIdx.x % S;
    const int64_t tp = pos[t];
    const int32_t sq = seq[t];
    const RowKeys rk = row_keys(tp, idx, k, m, window);
    const int64_t u0 = rk.n * s / S, u1 = rk.n * (s + 1) / S;

    // ---- resolve the first batch of positions (one index load per thread), angles ----
    static_assert(RB == 256 && RB % KT == 0, "one position per thread per batch");
    sm.row[tid] = u0 + tid < u1 ? resolve(u0 + tid, t, sq, rk, idx, k, comp, win) : -1;
    if (tid < 32) {
        float c, sn;
        angle_cs((double)tp, rt.theta[tid], c, sn);
        sm.cs[2 * tid] = c;
        sm.cs[2 * tid + 1] = sn;
    }
    __syncthreads();

    // entries of a tile go to registers: 16-byte chunks, plus the scale for part 0
    v4i pre[NCH];
    float pscl = 0.f;
    int pval = 0;
    auto issue = [&](int slot) {  // slot: first position of the tile inside the batch
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = tid + i * 256;
            pre[i] = v4i{0, 0, 0, 0};
            if (c < KT * CPK) {
                const int key = c % KT, part = c / KT;  // lanes of a wave: consecutive keys of one chunk column
                const int64_t code = sm.row[slot + key];
                if (code != -1) {
                    const bool w = code <= -2;
                    const int64_t r = w ? -code - 2 : code;
                    if (part < DN / 16) pre[i] = *(const v4i*)((w ? win.nope : comp.nope) + r * DN + part * 16);
                    else pre[i] = *(const v4i*)((w ? win.rope : comp.rope) + r * 64 + (part - DN / 16) * 8);
                    if (c < KT) pscl = (w ? win.scale : comp.scale)[r];
                }
                if (c < KT) pval = code != -1;
            }
        }
    };
    issue(0);

    // ---- query fragments (B operand of S^T = K Q^T) with RoPE at tp ----
    const int hb = HT >= 4 ? wave : wave % HT;
    const int ks0 = HT >= 4 ? 0 : wave / HT;
    const bool qk_active = HT >= 4 || ks0 < 2;
    v8bf qf[DSTEP];
    v8bf qlo[2];
    {
        const int h = hb * 16 + l16;
        const uint16_t* qrow = q + (t * H + h) * (int64_t)D;
#pragma unroll
        for (int st = 0; st < DSTEP; ++st) {
            const int d0 = 32 * st + 8 * g4;
            v4i raw = *(const v4i*)(qrow + d0);
            v8bf v = *(v8bf*)&raw;
            if (st >= NSTEP) {
                float x[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const int pi = (d0 - DN + e) >> 1;
                    const float cs = sm.cs[2 * pi], sn = sm.cs[2 * pi + 1];
                    const float x0 = x[e], x1 = x[e + 1];
                    x[e] = x0 * cs - x1 * sn;
                    x[e + 1] = x0 * sn + x1 * cs;
                }
                v8bf hi, lo;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    hi[e] = (__bf16)x[e];
                    lo[e] = (__bf16)(x[e] - (float)hi[e]);
                }
                v = hi;
                qlo[st - NSTEP] = lo;
            }
            qf[st] = v;
        }
    }

    // running softmax stats live with the softmax threads (TPH per head)
    const int sh = tid / TPH, sk = tid % TPH;
    float m_run = -INFINITY, l_run = 0.f;
    float s_ref = 0.f;  // S_tile the FP8 accumulators are expressed in (0: none yet)

    v4f acc[DT][HT];
#pragma unroll
    for (int a = 0; a < DT; ++a)
#pragma unroll
        for (int b = 0; b < HT; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};

    int buf = 0, ti = 0;
    for (int64_t ut = u0; ut < u1; ut += KT, buf ^= 1, ++ti) {
        if (tid < KT) {
            sm.scl[buf][tid] = pval ? pscl : 0.f;
            sm.valid[buf][tid] = pval;
            pscl = 0.f;
            pval = 0;
        }
        // ---- stage this tile from registers into LDS ----
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = tid + i * 256;
            if (c < KT * CPK) {
                const int key = c % KT, part = c / KT;  // lanes of a wave: consecutive keys of one chunk column
                __bf16* kr = sm.kr + key * Sm::KR;
                const v4i raw = pre[i];
                if (part < DN / 16) {
                    v8bf b0, b1;
#pragma unroll
                    for (int wd = 0; wd < 4; ++wd) {
                        const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8(raw[wd], false);
                        const v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8(raw[wd], true);
                        const float f[4] = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if (wd < 2) b0[wd * 4 + e] = (__bf16)f[e];
                            else b1[(wd - 2) * 4 + e] = (__bf16)f[e];
                            sm.vt[(part * 16 + wd * 4 + e) * Sm::VT + key] = (_Float16)f[e];
                        }
                    }
                    *(v8bf*)(kr + part * 16) = b0;
                    *(v8bf*)(kr + part * 16 + 8) = b1;
                } else {
                    const int rp = part - DN / 16;  // 8 rope dims per chunk
                    *(v4i*)(kr + DN + rp * 8) = raw;
                    const uint16_t* hv = (const uint16_t*)&raw;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        sm.vt[(DN + rp * 8 + e) * Sm::VT + key] = (_Float16)bf16_bits_to_f32(hv[e]);
                }
            }
        }
        // ---- put the next tile in flight (resolving a new batch of positions first when needed) ----
        const bool more = ut + KT < u1;
        const int nslot = ((ti + 1) % (RB / KT)) * KT;
        if (more && nslot == 0) {
            const int64_t u = ut + KT + tid;
            sm.row[tid] = u < u1 ? resolve(u, t, sq, rk, idx, k, comp, win) : -1;
        }
        __syncthreads();
        if (more) issue(nslot);
        const float* scl = sm.scl[buf];
        // ---- S^T = K Q^T ----
        if (qk_active) {
#pragma unroll
            for (int kk = 0; kk < QK_KS; ++kk) {
                const int ksub = ks0 + kk;
                const __bf16* kb = sm.kr + (ksub * 16 + l16) * Sm::KR + 8 * g4;
                v4f an = {0.f, 0.f, 0.f, 0.f}, ar = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < NSTEP; ++st)
                    an = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const v8bf*)(kb + 32 * st), qf[st], an, 0, 0, 0);
#pragma unroll
                for (int st = NSTEP; st < DSTEP; ++st) {
                    const v8bf kv = *(const v8bf*)(kb + 32 * st);
                    ar = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qf[st], ar, 0, 0, 0);
                    ar = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qlo[st - NSTEP], ar, 0, 0, 0);
                }
                // lane: head hb*16+l16, keys ksub*16 + 4*g4 + i
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = ksub * 16 + 4 * g4 + i;
                    const float sc = sm_scale * fmaf(scl[key], an[i], ar[i]);
                    sm.s[key * Sm::SS + hb * 16 + l16] = sm.valid[buf][key] ? sc : -INFINITY;
                }
            }
        }
        __syncthreads();
        // ---- online softmax: TPH threads per head, KPT keys each ----
        {
            float st_max = 0.f;
#pragma unroll 8
            for (int i = 0; i < KT; ++i) st_max = fmaxf(st_max, scl[i]);
            const float s_new = st_max > 0.f ? st_max : (s_ref > 0.f ? s_ref : 1.f);
            const float inv_s = 1.f / s_new;
            float sv[KPT];
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < KPT; ++i) {
                sv[i] = sm.s[(sk * KPT + i) * Sm::SS + sh];
                mx = fmaxf(mx, sv[i]);
            }
#pragma unroll
            for (int o = 1; o < TPH; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
            const float m_new = fmaxf(m_run, mx);
            float sum = 0.f;
#pragma unroll
            for (int i = 0; i < KPT; ++i) {
                const int key = sk * KPT + i;
                const float p = m_new == -INFINITY ? 0.f : __expf(sv[i] - m_new);
                sum += p;
                sm.pr[sh * Sm::PS + key] = (_Float16)p;
                sm.pn[sh * Sm::PS + key] = (_Float16)(p * (scl[key] * inv_s));
            }
#pragma unroll
            for (int o = 1; o < TPH; o <<= 1) sum += __shfl_xor(sum, o);
            const float alpha = m_new == -INFINITY ? 1.f : __expf(m_run - m_new);
            l_run = l_run * alpha + sum;
            m_run = m_new;
            if (sk == 0) sm.alpha[sh] = alpha;
            if (tid == 0) sm.sfac[buf] = s_ref > 0.f ? s_ref * inv_s : 1.f;
            s_ref = s_new;
        }
        __syncthreads();
        // ---- O^T += V^T P^T over this wave's dims ----
        {
            const float sf = sm.sfac[buf];
            float al[HT];
#pragma unroll
            for (int b = 0; b < HT; ++b) al[b] = sm.alpha[b * 16 + l16];
            v8h pfn[HT], pfr[HT];
#pragma unroll
            for (int b = 0; b < HT; ++b) {
                pfn[b] = *(const v8h*)(sm.pn + (b * 16 + l16) * Sm::PS + 8 * g4);
                pfr[b] = *(const v8h*)(sm.pr + (b * 16 + l16) * Sm::PS + 8 * g4);
            }
#pragma unroll
            for (int a = 0; a < DT; ++a) {
                const int d0 = wave * DW + a * 16;
                const v8h vf = *(const v8h*)(sm.vt + (d0 + l16) * Sm::VT + 8 * g4);
                const bool nope_tile = d0 < DN;
#pragma unroll
                for (int b = 0; b < HT; ++b) {
                    acc[a][b] *= nope_tile ? al[b] * sf : al[b];
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, nope_tile ? pfn[b] : pfr[b], acc[a][b], 0,
                                                                       0, 0);
                }
            }
        }
        __syncthreads();
    }

    // ---- epilogue ----
    if (sk == 0) {
        sm.mrun[sh] = m_run;
        sm.lrun[sh] = l_run;
    }
    if (tid == 0) sm.sfac[0] = s_ref > 0.f ? s_ref : 1.f;
    __syncthreads();
    const float sfin = sm.sfac[0];
    // lane holds dims wave*DW + a*16 + 4*g4 + i for head b*16 + l16
#pragma unroll
    for (int b = 0; b < HT; ++b) {
        const int h = b * 16 + l16;
        const float mh = sm.mrun[h], lh = sm.lrun[h];
#pragma unroll
        for (int a = 0; a < DT; ++a) {
            const int d0 = wave * DW + a * 16 + 4 * g4;
            float o[4];
            const float f = d0 < DN ? sfin : 1.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = acc[a][b][i] * f;
            if (S == 1) {
                const float inv = lh > 0.f ? 1.f / lh : 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] *= inv;
                if (d0 >= DN) {
#pragma unroll
                    for (int i = 0; i < 4; i += 2) {
                        const int pi = (d0 - DN + i) >> 1;
                        const float cs = sm.cs[2 * pi], sn = -sm.cs[2 * pi + 1];  // rotation by -t
                        const float x0 = o[i], x1 = o[i + 1];
                        o[i] = x0 * cs - x1 * sn;
                        o[i + 1] = x0 * sn + x1 * cs;
                    }
                }
                *(float4*)(out + (t * H + h) * (int64_t)D + d0) = make_float4(o[0], o[1], o[2], o[3]);
            } else {
                *(float4*)(part_o + ((t * S + s) * H + h) * (int64_t)D + d0) = make_float4(o[0], o[1], o[2], o[3]);
            }
        }
        if (wave == 0 && g4 == 0) {
            if (S == 1) lse[t * H + h] = lh > 0.f ? mh + __logf(lh) : -INFINITY;
            else {
                part_ml[((t * S + s) * H + h) * 2 + 0] = mh;
                part_ml[((t * S + s) * H + h) * 2 + 1] = lh;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// 64 query heads.  Each 32-key tile is staged once, as fp16 (FP8 codes and
// bf16 RoPE dims both convert exactly), row-major with rows D + 16 halves
// apart: that stride keeps the row-wise 16-byte reads of QK and the
// transposed 8-byte reads of PV free of LDS bank conflicts.
//   QK: wave w computes S^T = K Q^T for heads 16w..16w+15 over all dims.  The
//       query lives in registers as fp16, scaled per head by a power of two
//       (max |q| in [2^14, 2^15)) that is divided out of the scores exactly.
//   softmax: in registers, a head's 32 scores in one 16-lane column of the
//       accumulators.
//   PV: wave w computes O for all 64 heads over the FP8 dims
//       [w DN/4, (w+1) DN/4) and the RoPE dims [DN + 16w, DN + 16w + 16), so
//       every wave has the same mix of the two.  P (fp16) comes through LDS,
//       stored in the MFMA's K-slot order; V comes from the row-major tile
//       through ds_read_b64_tr_b16 transposed loads.
// K-slot order (both MFMAs): lane group g holds keys 4g..4g+3 and
// 16+4g..16+4g+3, exactly the keys of its QK accumulator rows.
//
// Head split (HS = 2, for grids that would leave most CUs idle): a pair of
// workgroups shares a (row, split), each taking 32 of the heads, so each
// stages the same tiles but does half the MFMA work per tile.  Wave w then
// computes S^T for the 16 heads 16 (w & 1) of its half over keys
// 16 (w >> 1)..+15 of the tile, P goes through LDS in the same K-slot order, and
// the two key halves of a head meet through LDS: their maxima at the first
// visible tile (the reference) and before a second pass, their sums at the end.
// PV is split over dims as above, for the workgroup's 32 heads.
//
// Fixed references instead of a running rescale: each head's reference max
// m_ref is the max of the first tile with visible keys, and S_ref (the FP8
// part's scale reference) is that tile's largest entry scale.  P = exp(s -
// m_ref) and P * scale_j / S_ref then stay below e^kLazy * kSRatio < 65504 as
// long as no later tile's max exceeds m_ref + kLazy and no later scale
// exceeds kSRatio * S_ref.  A tile that breaks either bound sets a flag; the
// pass still runs to its end (its output is then discarded), collecting the
// maxima of every tile, and a second pass with those as the references
// (which no tile can break) produces the output.  The output accumulators
// are thus only ever touched by MFMAs.
// ---------------------------------------------------------------------------
constexpr float kLazy = 8.f;     // e^8 ~ 2981
constexpr float kSRatio = 16.f;  // 2981 * 16 < 65504
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef short v4s __attribute__((ext_vector_type(4)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

// A masked key-list position (top-k padding, an entry not yet visible) reads
// this all-zero entry, so the tile loads need no per-lane masking.
__device__ __align__(16) uint8_t g_zero_entry[1024];

template <int D>
struct __align__(16) Mqa64Smem {
    static constexpr int KS = D + 16;  // fp16 row stride of a staged tile
    static constexpr int PS = KT + 8;  // fp16 row stride of P (80-byte rows: 16 lanes hit 16 distinct bank groups)
    _Float16 kv[3][KT * KS];           // tile t in kv[t % 3]
    _Float16 pn[64 * PS];  // [head][K slot] P * scale_j / S_ref (FP8 dims)
    _Float16 pr[64 * PS];  // [head][K slot] P (RoPE dims)
    float lfin[64];
    float hx[2][32];  // two workgroups per row: per key half, the maxima one half hands the other
    // two batches of resolved key-list positions: FP8-row and RoPE-row
    // addresses, entry scale (0 when masked) and visibility
    const uint8_t* kaddr[2][RB][2];
    float kscl[2][RB];  // entry scale, -1 for a masked position
    float cs[64];
    int restart;
};

// Loads through addresses read back from LDS: tell the compiler they are global memory.
typedef const __attribute__((address_space(1))) uint8_t* gptr_t;
template <typename T>
__device__ __forceinline__ T gload(const uint8_t* p) {
    return *(const __attribute__((address_space(1))) T*)(gptr_t)p;
}

// Workgroup barrier for hand-overs through LDS only: waits for this wave's LDS
// operations but not for its global loads in flight (the fences of
// __syncthreads would wait for those too, cutting short the prefetch of the
// next tiles).  The memory clobber keeps the compiler from moving LDS accesses
// across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ v4s lds_read_tr16(const _Float16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p));
}

// The output of 64 heads leaves in two halves of 32 heads, staged in LDS as fp32 rows of
// D + 4 floats (the lanes' 4 head groups then fall on distinct banks) and written in 16-byte
// stores: one lane per element would issue 8x the store instructions.
template <int D>
constexpr int kOutStride = D + 4;

// Lane (l16, g4) puts its normalised head values 16 hh + 4 g4 + i at dim d into the staging rows.
__device__ __forceinline__ void stage_out(float* ob, int os, int hh, int g4, int d, const float (&o)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ob[(16 * hh + 4 * g4 + i) * os + d] = o[i];
}

// Rows [h0, h0 + 32) of the staging to the row's output (S == 1; inverse RoPE on the last 64
// dims) or to the split's fp16 partial (S > 1; each head normalised by its own sum).
template <int D, int NTH>
__device__ __forceinline__ void store_out(const float* ob, const float* cs, int h0, int tid, int64_t t, int s, int S,
                                          float* __restrict__ out, _Float16* __restrict__ po) {
    constexpr int OS = kOutStride<D>, DN = D - 64, H = 64;
    if (S == 1) {
#pragma unroll
        for (int c = tid; c < 32 * D / 4; c += NTH) {
            const int r = c / (D / 4), d = (c % (D / 4)) * 4;
            float4 v = *(const float4*)(ob + r * OS + d);
            if (d >= DN) {
                const int p = (d - DN) >> 1;
                const float c0 = cs[2 * p], s0 = -cs[2 * p + 1], c1 = cs[2 * p + 2], s1 = -cs[2 * p + 3];
                v = make_float4(v.x * c0 - v.y * s0, v.x * s0 + v.y * c0, v.z * c1 - v.w * s1, v.z * s1 + v.w * c1);
            }
            // streamed past the L2: the output is not read again here, and the L2 keeps the
            // entries the other rows gather
            __builtin_nontemporal_store(v4f{v.x, v.y, v.z, v.w}, (v4f*)(out + (t * H + h0 + r) * (int64_t)D + d));
        }
    } else {
#pragma unroll
        for (int c = tid; c < 32 * D / 8; c += NTH) {
            const int r = c / (D / 8), d = (c % (D / 8)) * 8;
            const float4 a = *(const float4*)(ob + r * OS + d), b = *(const float4*)(ob + r * OS + d + 4);
            const v8h hv = {(_Float16)a.x, (_Float16)a.y, (_Float16)a.z, (_Float16)a.w,
                            (_Float16)b.x, (_Float16)b.y, (_Float16)b.z, (_Float16)b.w};
            *(v8h*)(po + ((t * S + s) * H + h0 + r) * (int64_t)D + d) = hv;
        }
    }
}

template <int D, bool PG, int HS>  // PG: a view is paged; HS: workgroups per (row, split), 1 or 2
__global__ __launch_bounds__(256) void k_mqa64(const uint16_t* __restrict__ q, const int32_t* __restrict__ seq,
                                               const int64_t* __restrict__ pos, const int32_t* __restrict__ idx, int k,
                                               int m, KvView comp, KvView win, int window, float sm_scale, RopeTab rt,
                                               int S, float* __restrict__ out, float* __restrict__ lse,
                                               float* __restrict__ part_o, float* __restrict__ part_ml) {
    constexpr int H = 64;
    static_assert(HS == 1 || HS == 2, "64 or 32 heads per workgroup");
    constexpr int NHT = 4 / HS;  // 16-head tiles of the workgroup in PV
    using Sm = Mqa64Smem<D>;
    constexpr int KS = Sm::KS;
    constexpr int DN = D - 64;
    constexpr int DSTEP = D / 32, NSTEP = DN / 32;  // QK steps of 32 dims
    constexpr int NN = DN / 64, DT = NN + 1;        // PV 16-dim tiles per wave: NN FP8 tiles, then one RoPE tile
    constexpr int CPN = DN / 16;                    // 16-byte chunks of an entry's FP8 part (RoPE part: 8)
    constexpr int NCN = KT * CPN;                   // FP8 chunks of a tile
    constexpr int NFULL = NCN / 256;                // whole FP8 chunks per thread; the other NCN % 256 go by halves
    constexpr int TPB = RB / KT;                    // tiles per batch of resolved positions
    static_assert(RB == 256 && TPB >= 6, "one resolved position per thread, a batch resolved 3+ tiles ahead");
    static_assert(KT * 8 == 256 && NCN % 256 == 128, "per thread: NFULL FP8 chunks, one RoPE chunk, one FP8 half chunk");

    __shared__ Sm sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    // HS == 2: workgroups 2p and 2p + 1 take heads [0, 32) and [32, 64) of pair p = (row, split)
    const int hh = HS == 1 ? 0 : (int)(blockIdx.x & 1);
    const unsigned pair = blockIdx.x / HS;
    const int64_t t = pair / (unsigned)S;
    const int s = (int)(pair % (unsigned)S);
    const int kh = HS == 1 ? 0 : wave >> 1;                            // HS == 2: the wave's key half
    const int hl = HS == 1 ? wave * 16 + l16 : 16 * (wave & 1) + l16;  // the lane's head in the workgroup
    // the query's loads go first: they depend on nothing but the row
    const int hq = 32 * hh + hl;
    v4i qraw[DSTEP];
    {
        const uint16_t* qrow = q + (t * H + hq) * (int64_t)D;
#pragma unroll
        for (int st = 0; st < DSTEP; ++st) qraw[st] = *(const v4i*)(qrow + 32 * st + 8 * g4);
    }
    const int64_t tp = pos[t];
    const int32_t sq = seq[t];
    const RowKeys rk = row_keys(tp, idx, k, m, window);
    const int64_t u0 = rk.n * s / S, u1 = rk.n * (s + 1) / S;
    const int nt = (int)((u1 - u0 + KT - 1) / KT);

    // key-list position u -> cache row code, given the selected index j (read from idx beforehand)
    auto fetch = [&](int64_t u) -> int64_t {
        return (u < u1 && u < rk.n_c) ? (idx ? (int64_t)idx[t * k + u] : u) : 0;
    };
    // position u (selected index j) -> FP8 / RoPE row addresses and scale pointer; false when masked
    struct Res {
        const uint8_t* an;
        const uint8_t* ar;
        const float* sp;
        bool ok;
    };
    // (the views' fields as scalars: a choice between the two views as objects would put both
    // in scratch memory)
    const uint8_t* const c_nope = comp.nope;
    const uint8_t* const w_nope = win.nope;
    const uint16_t* const c_rope = comp.rope;
    const uint16_t* const w_rope = win.rope;
    const float* const c_scale = comp.scale;
    const float* const w_scale = win.scale;
    const int64_t c_cap = comp.cap, w_cap = win.cap;
    const int32_t* const c_pages = comp.pages;
    const int32_t* const w_pages = win.pages;
    const int c_psh = comp.pshift, w_psh = win.pshift;
    auto resolve_at = [&](int64_t u, int64_t j) -> Res {
        const bool inw = u >= rk.n_c;
        if (u >= u1 || (!inw && (j < 0 || j >= rk.nv))) return Res{g_zero_entry, g_zero_entry + DN, nullptr, false};
        const uint8_t* nb = inw ? w_nope : c_nope;
        const uint16_t* rb = inw ? w_rope : c_rope;
        const float* sb = inw ? w_scale : c_scale;
        const int64_t x = inw ? rk.lo + (u - rk.n_c) : j;
        int64_t row;
        if constexpr (!PG) {
            const int64_t cap = inw ? w_cap : c_cap;
            row = (int64_t)sq * cap + (x % cap);
        } else if (inw) {  // a branch, not selects: selects of this many view fields went to scratch memory
            row = kv_row(w_pages, w_psh, w_cap, sq, x % w_cap);
        } else {
            row = kv_row(c_pages, c_psh, c_cap, sq, x % c_cap);
        }
        return Res{nb + row * DN, (const uint8_t*)(rb + row * 64), sb + row, true};
    };
    auto publish_addr = [&](int b, const Res& r) {
        sm.kaddr[b][tid][0] = r.an;
        sm.kaddr[b][tid][1] = r.ar;
    };
    auto publish_scale = [&](int b, const Res& r, float sc) { sm.kscl[b][tid] = r.ok ? sc : -1.f; };
    auto publish = [&](int b, const Res& r, float sc) {
        publish_addr(b, r);
        publish_scale(b, r, sc);
    };

    // batch 0 of the positions: row addresses now (the first tile's loads need them), the
    // entry scales in flight until the query is converted
    const Res r0 = resolve_at(u0 + tid, fetch(u0 + tid));
    if (tid < 32) {
        float c, sn;
        angle_cs((double)tp, rt.theta[tid], c, sn);
        sm.cs[2 * tid] = c;
        sm.cs[2 * tid + 1] = sn;
    }
    if (tid == 0) sm.restart = 0;
    publish_addr(0, r0);
    const float sc0 = r0.ok ? gload<float>((const uint8_t*)r0.sp) : 0.f;
    lds_barrier();

    // ---- tile loads (global -> registers) and staging (registers -> LDS) ----
    // Per thread and tile: FP8 chunks c = tid + 256 i (i < NFULL; entry c / CPN, bytes (c % CPN) * 16),
    // the RoPE chunk of entry tid / 8 (bytes (tid % 8) * 16), and 8 bytes of FP8 chunk
    // 256 NFULL + tid / 2.  Consecutive lanes read consecutive bytes of a row; no branches.
    v4i pre[NFULL > 0 ? NFULL : 1];
    v4i pre_r;
    v2u pre_h;
    auto issue = [&](int j) {
        const int b = (j / TPB) & 1, slot = (j % TPB) * KT;
#pragma unroll
        for (int i = 0; i < NFULL; ++i) {
            const int c = tid + i * 256;
            pre[i] = gload<v4i>(sm.kaddr[b][slot + c / CPN][0] + (c % CPN) * 16);
        }
        pre_r = gload<v4i>(sm.kaddr[b][slot + (tid >> 3)][1] + (tid & 7) * 16);
        const int ch = 256 * NFULL + (tid >> 1);
        pre_h = gload<v2u>(sm.kaddr[b][slot + ch / CPN][0] + (ch % CPN) * 16 + (tid & 1) * 8);
    };
    auto fp8x8_to_f16 = [](uint32_t lo, uint32_t hi) -> uint4 {
        return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.f, false)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.f, true)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.f, false)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.f, true)));
    };
    auto stage = [&](int j) {
        _Float16* kv = sm.kv[j % 3];
#pragma unroll
        for (int i = 0; i < NFULL; ++i) {
            const int c = tid + i * 256;
            const int part = c % CPN;
            const uint4 lo = fp8x8_to_f16((uint32_t)pre[i][0], (uint32_t)pre[i][1]);
            const uint4 hi = fp8x8_to_f16((uint32_t)pre[i][2], (uint32_t)pre[i][3]);
            _Float16* dst = kv + (c / CPN) * KS + part * 16;
            *(uint4*)dst = lo;
            *(uint4*)(dst + 8) = hi;
        }
        {
            uint32_t w[4];
#pragma unroll
            for (int wd = 0; wd < 4; ++wd) {
                const uint32_t u = (uint32_t)pre_r[wd];
                w[wd] = __builtin_bit_cast(
                    uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(u << 16), __uint_as_float(u & 0xFFFF0000u)));
            }
            *(uint4*)(kv + (tid >> 3) * KS + DN + (tid & 7) * 8) = make_uint4(w[0], w[1], w[2], w[3]);
        }
        {
            const int ch = 256 * NFULL + (tid >> 1);
            *(uint4*)(kv + (ch / CPN) * KS + (ch % CPN) * 16 + (tid & 1) * 8) = fp8x8_to_f16(pre_h[0], pre_h[1]);
        }
    };

    // ---- query: lane holds head wave*16 + l16, dims 32 st + 8 g4 + e; RoPE at tp; fp16 with a per-head 2^e ----
    v8h qf[DSTEP];
    float sm_q = 0.f;
    auto convert_q = [&]() {
        const v4i (&raw)[DSTEP] = qraw;
        float xr[DSTEP - NSTEP][8];
        float mx = 0.f;
#pragma unroll
        for (int st = 0; st < DSTEP; ++st) {
            const uint16_t* hv = (const uint16_t*)&raw[st];
            if (st < NSTEP) {
#pragma unroll
                for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(bf16_bits_to_f32(hv[e])));
            } else {
                const int d0 = 32 * st + 8 * g4 - DN;
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const int pi = (d0 + e) >> 1;
                    const float cs = sm.cs[2 * pi], sn = sm.cs[2 * pi + 1];
                    const float x0 = bf16_bits_to_f32(hv[e]), x1 = bf16_bits_to_f32(hv[e + 1]);
                    xr[st - NSTEP][e] = x0 * cs - x1 * sn;
                    xr[st - NSTEP][e + 1] = x0 * sn + x1 * cs;
                    mx = fmaxf(mx, fmaxf(fabsf(xr[st - NSTEP][e]), fabsf(xr[st - NSTEP][e + 1])));
                }
            }
        }
        mx = rows4_max(mx);
        int ex = 0;
        if (mx > 0.f) frexpf(mx, &ex);  // mx in [2^(ex-1), 2^ex)
        int sh = mx > 0.f ? 15 - ex : 0;
        sh = sh < -100 ? -100 : (sh > 100 ? 100 : sh);
        const float qs = ldexpf(1.f, sh);
        sm_q = sm_scale * ldexpf(1.f, -sh);
#pragma unroll
        for (int st = 0; st < DSTEP; ++st) {
            const uint16_t* hv = (const uint16_t*)&raw[st];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                qf[st][e] = (_Float16)((st < NSTEP ? bf16_bits_to_f32(hv[e]) : xr[st - NSTEP][e]) * qs);
            // keep the query in AGPRs (MFMA reads its B operand from there): the VGPRs
            // are left for K fragments in flight, softmax and the tile loads
            asm volatile("" : "+a"(qf[st]));
        }
    };

    v4f acc[NHT][DT];
    float m_ref = -INFINITY, l_run = 0.f, s_ref = 0.f;
    float m_seen = -INFINITY, s_seen = 0.f;  // maxima over every tile seen (second-pass references)
    int64_t nraw = 0;  // this thread's position in the next batch: selected index, then resolved
    Res nres{g_zero_entry, g_zero_entry + DN, nullptr, false};
    float nscl = 0.f;

    // S^T (keys x heads) of tile j for this wave's 16 heads: FP8-dim and RoPE-dim parts, over
    // NKB 16-key blocks (HS == 1: both of the tile; HS == 2: the wave's key half).
    // K fragments go in groups of QG dim steps (8 loads a group), the next group's loads issued
    // before this group's MFMAs (the scheduler is not allowed to sink them: two groups in flight).
    constexpr int NKB = 2 / HS;
    constexpr int QG = 8 / NKB < DSTEP ? 8 / NKB : DSTEP;
    static_assert(DSTEP % QG == 0, "whole groups");
    auto qk = [&](int j, v4f (&an)[NKB], v4f (&ar)[NKB]) {
        const _Float16* kb = sm.kv[j % 3] + (16 * kh + l16) * KS + 8 * g4;
#pragma unroll
        for (int b = 0; b < NKB; ++b) an[b] = ar[b] = v4f{0.f, 0.f, 0.f, 0.f};
        v8h kf[2][NKB * QG];
#pragma unroll
        for (int e = 0; e < QG; ++e)
#pragma unroll
            for (int b = 0; b < NKB; ++b) kf[0][NKB * e + b] = *(const v8h*)(kb + 16 * KS * b + 32 * e);
#pragma unroll
        for (int g = 0; g < DSTEP / QG; ++g) {
            if (g + 1 < DSTEP / QG) {
#pragma unroll
                for (int e = 0; e < QG; ++e) {
                    const int st = (g + 1) * QG + e;
#pragma unroll
                    for (int b = 0; b < NKB; ++b)
                        kf[(g + 1) & 1][NKB * e + b] = *(const v8h*)(kb + 16 * KS * b + 32 * st);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = 0; e < QG; ++e) {
                const int st = g * QG + e;
#pragma unroll
                for (int b = 0; b < NKB; ++b) {
                    if (st < NSTEP)
                        an[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[g & 1][NKB * e + b], qf[st], an[b], 0, 0, 0);
                    else
                        ar[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[g & 1][NKB * e + b], qf[st], ar[b], 0, 0, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // entry scales of tile j: lane (l16, g4) holds keys 4 g4 + i and 16 + 4 g4 + i (read before QK)
    auto tile_scales = [&](int j, float4& s0, float4& s1) {
        const float* tscl = sm.kscl[(j / TPB) & 1] + (j % TPB) * KT;
        s0 = *(const float4*)(tscl + 4 * g4);
        s1 = *(const float4*)(tscl + 16 + 4 * g4);
    };
    // scores and P of tile j for head hl; returns whether a reference is exceeded
    auto softmax = [&](const float4& s0, const float4& s1, const v4f (&an)[2], const v4f (&ar)[2]) -> bool {
        const float kscl[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        float sv[8];
        float st_max = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            sv[i] = kscl[i] >= 0.f ? sm_q * fmaf(kscl[i], an[i >> 2][i & 3], ar[i >> 2][i & 3]) : -INFINITY;
            st_max = fmaxf(st_max, kscl[i]);
        }
        st_max = rows4_max(st_max);  // over the tile's 32 keys: the same in every lane and wave
        float mx = sv[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
        mx = rows4_max(mx);
        m_seen = fmaxf(m_seen, mx);
        s_seen = fmaxf(s_seen, st_max);
        m_ref = m_ref == -INFINITY ? mx : m_ref;  // first tile with visible keys (accumulators still zero)
        s_ref = s_ref == 0.f ? st_max : s_ref;
        const bool over = mx > m_ref + kLazy || st_max > kSRatio * s_ref;
        const float inv_s = s_ref > 0.f ? 1.f / s_ref : 0.f;
        v8h pn, pr;
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p = m_ref == -INFINITY ? 0.f : __expf(sv[i] - m_ref);
            sum += p;
            pr[i] = (_Float16)p;
            pn[i] = (_Float16)(p * (kscl[i] * inv_s));
        }
        l_run += rows4_sum(sum);
        *(v8h*)(sm.pn + hl * Sm::PS + 8 * g4) = pn;
        *(v8h*)(sm.pr + hl * Sm::PS + 8 * g4) = pr;
        return over;
    };
    // HS == 2: the same over the wave's key half (keys 16 kh + 4 g4 + i of the lane); the
    // references are the maxima over both halves, which meet in LDS at the first tile with
    // visible keys (a tile-wide condition, so every wave takes that barrier or none does).
    // P goes to K slots 8 g4 + 4 kh + i, the order of HS == 1.  l_run sums the wave's half only.
    bool have_ref = false;
    auto softmax2 = [&](const float4& s0, const float4& s1, const v4f (&an)[NKB], const v4f (&ar)[NKB]) -> bool {
        const float4 sk = kh ? s1 : s0;
        const float kscl[4] = {sk.x, sk.y, sk.z, sk.w};
        // the tile's largest entry scale, -1 when no key is visible
        float smx = fmaxf(fmaxf(fmaxf(s0.x, s0.y), fmaxf(s0.z, s0.w)), fmaxf(fmaxf(s1.x, s1.y), fmaxf(s1.z, s1.w)));
        smx = rows4_max(smx);
        const float st_max = fmaxf(smx, 0.f);
        float sv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            sv[i] = kscl[i] >= 0.f ? sm_q * fmaf(kscl[i], an[0][i], ar[0][i]) : -INFINITY;
        float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
        mx = rows4_max(mx);
        m_seen = fmaxf(m_seen, mx);
        s_seen = fmaxf(s_seen, st_max);
        if (!have_ref && __builtin_amdgcn_readfirstlane(smx >= 0.f ? 1 : 0)) {
            if (g4 == 0) sm.hx[kh][hl] = mx;
            lds_barrier();
            m_ref = fmaxf(mx, sm.hx[kh ^ 1][hl]);
            have_ref = true;
        }
        s_ref = s_ref == 0.f ? st_max : s_ref;
        const bool over = mx > m_ref + kLazy || st_max > kSRatio * s_ref;
        const float inv_s = s_ref > 0.f ? 1.f / s_ref : 0.f;
        v4h pn, pr;
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float p = m_ref == -INFINITY ? 0.f : __expf(sv[i] - m_ref);
            sum += p;
            pr[i] = (_Float16)p;
            pn[i] = (_Float16)(p * (kscl[i] * inv_s));
        }
        l_run += rows4_sum(sum);
        *(v4h*)(sm.pn + hl * Sm::PS + 8 * g4 + 4 * kh) = pn;
        *(v4h*)(sm.pr + hl * Sm::PS + 8 * g4 + 4 * kh) = pr;
        return over;
    };
    // O[heads x dims] += P V (tile j) for the workgroup's heads over this wave's dims.  The B
    // fragment of lane (l16, g4) holds the keys of P's K slots 8 g4..8 g4 + 7: keys 4 g4 + r
    // and 16 + 4 g4 + r.
    auto pv = [&](int j) {
        const _Float16* vb = sm.kv[j % 3] + (4 * g4 + (l16 >> 2)) * KS + 4 * (l16 & 3);
        v8h vf[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int d0 = dt < NN ? 16 * (NN * wave + dt) : DN + 16 * wave;
            const v4s lo = lds_read_tr16(vb + d0);
            const v4s hi = lds_read_tr16(vb + 16 * KS + d0);
            const v8u16 c = {(uint16_t)lo[0], (uint16_t)lo[1], (uint16_t)lo[2], (uint16_t)lo[3],
                             (uint16_t)hi[0], (uint16_t)hi[1], (uint16_t)hi[2], (uint16_t)hi[3]};
            vf[dt] = __builtin_bit_cast(v8h, c);
        }
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
            const int hr = 16 * ht + l16;
            const v8h pnf = *(const v8h*)(sm.pn + hr * Sm::PS + 8 * g4);
            const v8h prf = *(const v8h*)(sm.pr + hr * Sm::PS + 8 * g4);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                acc[ht][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dt < NN ? pnf : prf, vf[dt], acc[ht][dt], 0, 0, 0);
        }
    };
    // Next batch of positions, one step per tile: index load (tile j % TPB == 1), row addresses
    // (end of that tile), scale load (tile 2), publish (end of tile 2; first used 5 tiles later).
    // Every load is issued at the start of a tile and consumed at its end, so no load but the
    // tile prefetch is in flight across the loop's back edge (a pending load there makes the
    // next tile wait for all of them before its first LDS read).
    auto batch_begin = [&](int j) {
        const int b1 = j / TPB + 1;
        const int64_t u = u0 + (int64_t)b1 * RB + tid;
        if (b1 * TPB < nt) {
            if (j % TPB == 1) nraw = fetch(u);
            if (j % TPB == 2) nscl = nres.ok ? gload<float>((const uint8_t*)nres.sp) : 0.f;  // global, not flat
        }
    };
    auto batch_end = [&](int j) {
        const int b1 = j / TPB + 1;
        const int64_t u = u0 + (int64_t)b1 * RB + tid;
        if (b1 * TPB < nt) {
            if (j % TPB == 1) nres = resolve_at(u, nraw);
            if (j % TPB == 2) publish(b1 & 1, nres, nscl);
        }
    };

    // One pass over the split.  Per tile, two barriers: [QK(j), softmax(j) -> P]  sync
    // [stage(j+1), load j+2, PV(j)]  sync.  Tile t lives in kv[t % 3].  Returns whether a tile
    // broke the references (the pass's output is then discarded).  The loop has a single exit,
    // so the output accumulators keep their registers and every PV MFMA runs in place.
    auto run_pass = [&](bool first) -> bool {
        if (first) {
            // batch 0's addresses are published; convert the query while tile 0 is in flight
            if (nt > 0) issue(0);
            convert_q();
            publish_scale(0, r0, sc0);
        } else {
            const Res r = resolve_at(u0 + tid, fetch(u0 + tid));
            publish(0, r, r.ok ? gload<float>((const uint8_t*)r.sp) : 0.f);
            lds_barrier();
            if (nt > 0) issue(0);
        }
#pragma unroll
        for (int a = 0; a < NHT; ++a)
#pragma unroll
            for (int b = 0; b < DT; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};
        m_ref = m_seen;
        s_ref = s_seen;
        l_run = 0.f;
        have_ref = m_ref > -INFINITY;  // (the second pass, when a tile was visible: the same in every lane)
        if (nt > 0) stage(0);
        if (nt > 1) issue(1);
        lds_barrier();
        for (int j = 0; j < nt; ++j) {
            v4f sn[NKB], sr[NKB];
            batch_begin(j);
            float4 s0, s1;
            tile_scales(j, s0, s1);
            qk(j, sn, sr);
            bool over;
            if constexpr (HS == 1) over = softmax(s0, s1, sn, sr);
            else over = softmax2(s0, s1, sn, sr);
            if (over) sm.restart = 1;
            lds_barrier();
            if (j + 1 < nt) stage(j + 1);
            if (j + 2 < nt) issue(j + 2);
            pv(j);
            batch_end(j);
            lds_barrier();
        }
        return sm.restart != 0;
    };
    if (run_pass(true)) {
        // a tile broke the references: run the split again with the maxima of every tile as the
        // references (no tile can break them); every wave has read the flag before the last barrier
        m_seen = rows4_max(m_seen);
        if constexpr (HS == 2) {  // and over both key halves
            if (g4 == 0) sm.hx[kh][hl] = m_seen;
            lds_barrier();
            m_seen = fmaxf(m_seen, sm.hx[kh ^ 1][hl]);
        }
        lds_barrier();
        if (tid == 0) sm.restart = 0;
        run_pass(false);
    }

    // ---- epilogue: lane holds heads 16 ht + 4 g4 + i at one dim of each of its dim tiles ----
    // The sum of the workgroup's head h (HS == 2: over both key halves).
    auto head_sum = [&](int h) { return HS == 1 ? sm.lfin[h] : sm.lfin[h] + sm.lfin[32 + h]; };
    if (g4 == 0) sm.lfin[HS == 1 ? hl : 32 * kh + hl] = l_run;
    lds_barrier();
    if (g4 == 0 && kh == 0) {
        const float l = head_sum(hl);
        if (S == 1) lse[t * H + hq] = l > 0.f ? m_ref + __logf(l) : -INFINITY;
        else {
            part_ml[((t * S + s) * H + hq) * 2 + 0] = m_ref;
            part_ml[((t * S + s) * H + hq) * 2 + 1] = l;
        }
    }
    const float sfin = s_ref > 0.f ? s_ref : 1.f;
    if (S > 1) {
        // the split's partial in the accumulators' own order (k_mqa_combine_sw reads it): lane
        // (l16, g4) of wave w puts heads 16 ht + 4 g4 + i, i < 4, at its dim of tile dt as 8 bytes
        // at (((w * 4 + ht) * DT + dt) * 64 + lane) * 4; each head normalised by its own sum
        _Float16* pw = (_Float16*)part_o + (t * S + s) * (int64_t)H * D;
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
            float inv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float l = head_sum(16 * ht + 4 * g4 + i);
                inv[i] = l > 0.f ? 1.f / l : 0.f;
            }
            const int htg = NHT * hh + ht;  // the head tile among the row's 64 heads
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const float f = dt < NN ? sfin : 1.f;
                const v4h o = {(_Float16)(acc[ht][dt][0] * f * inv[0]), (_Float16)(acc[ht][dt][1] * f * inv[1]),
                               (_Float16)(acc[ht][dt][2] * f * inv[2]), (_Float16)(acc[ht][dt][3] * f * inv[3])};
                // streamed past the L2 (read once, by the merge kernel): less to write back at the
                // kernel's end, which the merge would otherwise wait for
                __builtin_nontemporal_store(__builtin_bit_cast(v2u, o),
                                            (v2u*)(pw + (((wave * 4 + htg) * DT + dt) * 64 + lane) * 4));
            }
        }
        return;
    }
    float* ob = (float*)&sm.kv[0][0];  // the tiles are no longer read
    static_assert(32 * kOutStride<D> * sizeof(float) <= sizeof(sm.kv), "32 staged output rows fit the tile buffers");
#pragma unroll
    for (int half = 0; half < 2 / HS; ++half) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            const int ht = 2 * half + hb;
            float inv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float l = head_sum(16 * ht + 4 * g4 + i);
                inv[i] = l > 0.f ? 1.f / l : 0.f;
            }
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const bool nope = dt < NN;
                const int d = (nope ? 16 * (NN * wave + dt) : DN + 16 * wave) + l16;
                float o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = acc[ht][dt][i] * (nope ? sfin : 1.f) * inv[i];
                stage_out(ob, kOutStride<D>, hb, g4, d, o);
            }
        }
        lds_barrier();
        store_out<D, 256>(ob, sm.cs, HS == 1 ? 32 * half : 32 * hh, tid, t, s, S, out, (_Float16*)part_o);
        if (half + 1 < 2 / HS) lds_barrier();
    }
}

// ---------------------------------------------------------------------------
// 64 query heads, d = 512, eight waves in two roles that run one tile apart
// (two waves per SIMD, one of each role), so that the softmax and the LDS
// reads of one role overlap the MFMAs of the other:
//   waves 0-3 (scores): wave w computes S^T for heads 16w..16w+15 over all
//       dims (query fp16 in AGPRs), then the softmax of tile i against the
//       lazy references into P buffer i & 1;
//   waves 4-7 (values): gather and stage tile i+1 (and issue tile i+2),
//       then O += P V for tile i-1 over the FP8 dims [112 (w-4), +112) and
//       the RoPE dims [448 + 16 (w-4), +16), reading P buffer (i-1) & 1.
// One barrier per step; tiles, references and the second pass are those of
// k_mqa64.  Each role's loop is its own branch, so the query registers of
// one and the output accumulators of the other can share the register file.
// ---------------------------------------------------------------------------
template <int D>
struct __align__(16) MqaWsSmem {
    static constexpr int KS = D + 16;  // fp16 row stride of a staged tile
    static constexpr int PS = KT + 8;  // fp16 row stride of P
    _Float16 kv[3][KT * KS];           // tile t in kv[t % 3]
    _Float16 pn[2][64 * PS];           // [tile & 1][head][K slot] P * scale_j / S_ref (FP8 dims)
    _Float16 pr[2][64 * PS];           // [tile & 1][head][K slot] P (RoPE dims)
    float mfin[64];                    // per head: reference max and sum of the pass (scores -> values)
    float lfin[64];
    float sfin;
    const uint8_t* kaddr[2][RB][2];
    float kscl[2][RB];  // entry scale, -1 for a masked position
    float tmax[2][RB / KT];     // per tile: the largest entry scale (-1: no position visible)
    uint32_t tfull[2][RB / KT];  // per tile: every position visible
    float cs[64];
    int restart;
};

template <int D, bool PG>  // PG: a view is paged
__global__ __launch_bounds__(512) void k_mqa64ws(const uint16_t* __restrict__ q, const int32_t* __restrict__ seq,
                                                 const int64_t* __restrict__ pos, const int32_t* __restrict__ idx,
                                                 int k, int m, KvView comp, KvView win, int window, float sm_scale,
                                                 RopeTab rt, int S, float* __restrict__ out, float* __restrict__ lse,
                                                 float* __restrict__ part_o, float* __restrict__ part_ml) {
    static_assert(D == 512, "the 64-head shape of the pages");
    constexpr int H = 64;
    using Sm = MqaWsSmem<D>;
    constexpr int KS = Sm::KS;
    constexpr int DN = D - 64;
    constexpr int DSTEP = D / 32, NSTEP = DN / 32;  // QK steps of 32 dims
    constexpr int NN = DN / 64, DT = NN + 1;        // PV 16-dim tiles per wave: NN FP8 tiles, then one RoPE tile
    constexpr int CPN = DN / 16;                    // 16-byte chunks of an entry's FP8 part (RoPE part: 8)
    constexpr int NCN = KT * CPN;                   // FP8 chunks of a tile
    constexpr int NFULL = NCN / 256;                // whole FP8 chunks per value thread; the other NCN % 256 go by halves
    constexpr int TPB = RB / KT;                    // tiles per batch of resolved positions
    static_assert(RB == 256 && TPB >= 6, "one resolved position per value thread, a batch resolved 3+ tiles ahead");
    static_assert(KT * 8 == 256 && NCN % 256 == 128, "per thread: NFULL FP8 chunks, one RoPE chunk, one FP8 half chunk");

    __shared__ Sm sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool scores_role = wave < 4;
    const int rw = wave & 3;      // wave index within the role
    const int vt = tid & 255;     // thread index within the role
    const int l16 = lane & 15, g4 = lane >> 4;
    const int64_t t = blockIdx.x / S;
    const int s = blockIdx.x % S;
    const int64_t tp = pos[t];
    const int32_t sq = seq[t];
    const RowKeys rk = row_keys(tp, idx, k, m, window);
    const int64_t u0 = rk.n * s / S, u1 = rk.n * (s + 1) / S;
    const int nt = (int)((u1 - u0 + KT - 1) / KT);

    auto fetch = [&](int64_t u) -> int64_t {
        return (u < u1 && u < rk.n_c) ? (idx ? (int64_t)idx[t * k + u] : u) : 0;
    };
    struct Res {
        const uint8_t* an;
        const uint8_t* ar;
        const float* sp;
        bool ok;
    };
    // (the views' fields as scalars: a choice between the two views as objects would put both
    // in scratch memory)
    const uint8_t* const c_nope = comp.nope;
    const uint8_t* const w_nope = win.nope;
    const uint16_t* const c_rope = comp.rope;
    const uint16_t* const w_rope = win.rope;
    const float* const c_scale = comp.scale;
    const float* const w_scale = win.scale;
    const int64_t c_cap = comp.cap, w_cap = win.cap;
    const int32_t* const c_pages = comp.pages;
    const int32_t* const w_pages = win.pages;
    const int c_psh = comp.pshift, w_psh = win.pshift;
    auto resolve_at = [&](int64_t u, int64_t j) -> Res {
        const bool inw = u >= rk.n_c;
        if (u >= u1 || (!inw && (j < 0 || j >= rk.nv))) return Res{g_zero_entry, g_zero_entry + DN, nullptr, false};
        const uint8_t* nb = inw ? w_nope : c_nope;
        const uint16_t* rb = inw ? w_rope : c_rope;
        const float* sb = inw ? w_scale : c_scale;
        const int64_t x = inw ? rk.lo + (u - rk.n_c) : j;
        int64_t row;
        if constexpr (!PG) {
            const int64_t cap = inw ? w_cap : c_cap;
            row = (int64_t)sq * cap + (x % cap);
        } else if (inw) {  // a branch, not selects: selects of this many view fields went to scratch memory
            row = kv_row(w_pages, w_psh, w_cap, sq, x % w_cap);
        } else {
            row = kv_row(c_pages, c_psh, c_cap, sq, x % c_cap);
        }
        return Res{nb + row * DN, (const uint8_t*)(rb + row * 64), sb + row, true};
    };
    auto publish = [&](int b, const Res& r, float sc) {
        sm.kaddr[b][vt][0] = r.an;
        sm.kaddr[b][vt][1] = r.ar;
        const float v = r.ok ? sc : -1.f;
        sm.kscl[b][vt] = v;
        // per 32-position tile (a half of this wave): the largest entry scale (-1 when none is
        // visible) and whether every position is visible, so the scores role skips its masking
        float mx = v;
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        const uint64_t bad = __ballot(v < 0.f);
        if ((vt & 31) == 0) {
            sm.tmax[b][vt >> 5] = mx;
            sm.tfull[b][vt >> 5] = (uint32_t)(bad >> (lane & 32)) == 0u ? 1 : 0;
        }
    };

    if (tid < 32) {
        float c, sn;
        angle_cs((double)tp, rt.theta[tid], c, sn);
        sm.cs[2 * tid] = c;
        sm.cs[2 * tid + 1] = sn;
    }
    if (tid == 0) sm.restart = 0;
    __syncthreads();

    float m_seen = -INFINITY, s_seen = 0.f;  // scores role: maxima over every tile seen (second-pass references)

    // ---- tile loads (global -> registers) and staging (registers -> LDS), shared by the roles.
    // Thread vt of the values role: FP8 chunks c = vt and vt + 256 (entry c / CPN, bytes (c % CPN) * 16).
    // Thread vt of the scores role: FP8 chunk vt + 512, the RoPE chunk of entry vt / 8 (bytes
    // (vt % 8) * 16) and 8 bytes of FP8 chunk 768 + vt / 2.  Consecutive lanes read consecutive bytes.
    static_assert(NFULL == 3, "two whole FP8 chunks per values thread, one per scores thread");
    v4i pre_a, pre_b;
    v2u pre_h;
    auto issue = [&](int j) {
        const int b = (j / TPB) & 1, slot = (j % TPB) * KT;
        if (!scores_role) {
            pre_a = gload<v4i>(sm.kaddr[b][slot + vt / CPN][0] + (vt % CPN) * 16);
            const int c = vt + 256;
            pre_b = gload<v4i>(sm.kaddr[b][slot + c / CPN][0] + (c % CPN) * 16);
        } else {
            const int c = vt + 512;
            pre_a = gload<v4i>(sm.kaddr[b][slot + c / CPN][0] + (c % CPN) * 16);
            pre_b = gload<v4i>(sm.kaddr[b][slot + (vt >> 3)][1] + (vt & 7) * 16);
            const int ch = 768 + (vt >> 1);
            pre_h = gload<v2u>(sm.kaddr[b][slot + ch / CPN][0] + (ch % CPN) * 16 + (vt & 1) * 8);
        }
    };
    auto fp8x8_to_f16 = [](uint32_t lo, uint32_t hi) -> uint4 {
        return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.f, false)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.f, true)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.f, false)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.f, true)));
    };
    auto stage_chunk = [&](_Float16* kv, int c, const v4i& x) {
        _Float16* dst = kv + (c / CPN) * KS + (c % CPN) * 16;
        *(uint4*)dst = fp8x8_to_f16((uint32_t)x[0], (uint32_t)x[1]);
        *(uint4*)(dst + 8) = fp8x8_to_f16((uint32_t)x[2], (uint32_t)x[3]);
    };
    auto stage = [&](int j) {
        _Float16* kv = sm.kv[j % 3];
        if (!scores_role) {
            stage_chunk(kv, vt, pre_a);
            stage_chunk(kv, vt + 256, pre_b);
        } else {
            stage_chunk(kv, vt + 512, pre_a);
            uint32_t w[4];
#pragma unroll
            for (int wd = 0; wd < 4; ++wd) {
                const uint32_t u = (uint32_t)pre_b[wd];
                w[wd] = __builtin_bit_cast(
                    uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(u << 16), __uint_as_float(u & 0xFFFF0000u)));
            }
            *(uint4*)(kv + (vt >> 3) * KS + DN + (vt & 7) * 8) = make_uint4(w[0], w[1], w[2], w[3]);
            const int ch = 768 + (vt >> 1);
            *(uint4*)(kv + (ch / CPN) * KS + (ch % CPN) * 16 + (vt & 1) * 8) = fp8x8_to_f16(pre_h[0], pre_h[1]);
        }
    };
    Res nres{g_zero_entry, g_zero_entry + DN, nullptr, false};  // this thread's position in the next batch
    int32_t pend_i = 0;  // the tile's selected-index load
    float pend_s = 0.f;  // the tile's entry-scale load
    // next batch, one step per tile: the selected index is loaded on tile 1 of a batch, the
    // entry scale on tile 2, each used at the tile's end.  Both loads are issued on every tile
    // (from the zero entry when not needed) and waited for before the tile prefetch leaves: a
    // load issued on some paths only made the compiler wait for every load, the tile prefetch
    // included, before the first LDS read of P V.
    auto batch_begin = [&](int j) {
        const int b1 = j / TPB + 1;
        const int64_t u = u0 + (int64_t)b1 * RB + vt;
        const bool more = b1 * TPB < nt;
        const bool li = more && j % TPB == 1 && idx && u < u1 && u < rk.n_c;
        const bool ls = more && j % TPB == 2 && nres.ok;
        pend_i = gload<int32_t>(li ? (const uint8_t*)(idx + t * k + u) : g_zero_entry);
        pend_s = gload<float>(ls ? (const uint8_t*)nres.sp : g_zero_entry);
    };
    // both loads complete here, on every path: before the tile prefetch is issued, so that no
    // wait for them covers the prefetch
    auto batch_take = [&]() { asm volatile("" ::"v"(pend_i), "v"(pend_s)); };
    auto batch_end = [&](int j) {
        const int b1 = j / TPB + 1;
        const int64_t u = u0 + (int64_t)b1 * RB + vt;
        const int32_t iv = pend_i;
        const float sv = pend_s;
        if (b1 * TPB < nt) {
            if (j % TPB == 1) nres = resolve_at(u, (u < u1 && u < rk.n_c) ? (idx ? (int64_t)iv : u) : 0);
            if (j % TPB == 2) publish(b1 & 1, nres, nres.ok ? sv : 0.f);
        }
    };

    // One pass over the split (both roles); writes the output unless a tile broke the references
    // in a first pass, which it returns.
    float* ob = (float*)&sm.kv[0][0];  // output staging, once the tiles are no longer read
    static_assert(32 * kOutStride<D> * sizeof(float) <= sizeof(sm.kv), "32 staged output rows fit the tile buffers");
    auto run_pass = [&](bool second) -> bool {
        // batch 0 of the positions: row addresses published at once, the entry scales once tile
        // 0's loads are in flight; then tile 0 staged, tile 1 in flight
        Res r0{g_zero_entry, g_zero_entry + DN, nullptr, false};
        float sc0 = 0.f;
        if (!scores_role) {
            r0 = resolve_at(u0 + vt, fetch(u0 + vt));
            sm.kaddr[0][vt][0] = r0.an;
            sm.kaddr[0][vt][1] = r0.ar;
            if (r0.ok) sc0 = gload<float>((const uint8_t*)r0.sp);
        }
        lds_barrier();
        if (nt > 0) issue(0);
        if (!scores_role) publish(0, r0, sc0);
        if (nt > 0) stage(0);
        if (nt > 1) issue(1);
        lds_barrier();
        if (scores_role) {
            // ---- query: lane holds head 16 rw + l16, dims 32 st + 8 g4 + e; RoPE at tp; fp16 with a per-head 2^e ----
            const int hq = rw * 16 + l16;
            v8h qf[DSTEP];
            float sm_q;
            {
                const uint16_t* qrow = q + (t * H + hq) * (int64_t)D;
                v4i raw[DSTEP];
#pragma unroll
                for (int st = 0; st < DSTEP; ++st)  // read once: nontemporal, the L2 keeps the entries
                    raw[st] = __builtin_nontemporal_load((const v4i*)(qrow + 32 * st + 8 * g4));
                float xr[DSTEP - NSTEP][8];
                float mx = 0.f;
#pragma unroll
                for (int st = 0; st < DSTEP; ++st) {
                    const uint16_t* hv = (const uint16_t*)&raw[st];
                    if (st < NSTEP) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(bf16_bits_to_f32(hv[e])));
                    } else {
                        const int d0 = 32 * st + 8 * g4 - DN;
#pragma unroll
                        for (int e = 0; e < 8; e += 2) {
                            const int pi = (d0 + e) >> 1;
                            const float cs = sm.cs[2 * pi], sn = sm.cs[2 * pi + 1];
                            const float x0 = bf16_bits_to_f32(hv[e]), x1 = bf16_bits_to_f32(hv[e + 1]);
                            xr[st - NSTEP][e] = x0 * cs - x1 * sn;
                            xr[st - NSTEP][e + 1] = x0 * sn + x1 * cs;
                            mx = fmaxf(mx, fmaxf(fabsf(xr[st - NSTEP][e]), fabsf(xr[st - NSTEP][e + 1])));
                        }
                    }
                }
                mx = rows4_max(mx);
                int ex = 0;
                if (mx > 0.f) frexpf(mx, &ex);  // mx in [2^(ex-1), 2^ex)
                int shq = mx > 0.f ? 15 - ex : 0;
                shq = shq < -100 ? -100 : (shq > 100 ? 100 : shq);
                const float qs = ldexpf(1.f, shq);
                sm_q = sm_scale * ldexpf(1.f, -shq) * kLog2e;  // scores kept in log2 units
#pragma unroll
                for (int st = 0; st < DSTEP; ++st) {
                    const uint16_t* hv = (const uint16_t*)&raw[st];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        qf[st][e] = (_Float16)((st < NSTEP ? bf16_bits_to_f32(hv[e]) : xr[st - NSTEP][e]) * qs);
                    asm volatile("" : "+a"(qf[st]));
                }
            }
            float m_ref = m_seen, s_ref = s_seen, l_run = 0.f;
            float inv_s = s_ref > 0.f ? 1.f / s_ref : 0.f;
            constexpr int QG = 2;
            static_assert(DSTEP % QG == 0, "whole groups");
            for (int it = 0; it <= nt; ++it) {
                if (it + 1 < nt) stage(it + 1);
                if (it + 2 < nt) issue(it + 2);
                if (it < nt) {
                    const int j = it;
                    const float* tscl = sm.kscl[(j / TPB) & 1] + (j % TPB) * KT;
                    const float4 s0 = *(const float4*)(tscl + 4 * g4), s1 = *(const float4*)(tscl + 16 + 4 * g4);
                    const float st_max = fmaxf(sm.tmax[(j / TPB) & 1][j % TPB], 0.f);  // over the tile's 32 keys
                    const bool full = __builtin_amdgcn_readfirstlane(sm.tfull[(j / TPB) & 1][j % TPB]) != 0;
                    // S^T (keys x heads) of tile j for this wave's 16 heads: FP8-dim and RoPE-dim parts
                    v4f an[2], ar[2];
                    {
                        const _Float16* kb = sm.kv[j % 3] + l16 * KS + 8 * g4;
                        an[0] = an[1] = ar[0] = ar[1] = v4f{0.f, 0.f, 0.f, 0.f};
                        v8h kf[2][2 * QG];
#pragma unroll
                        for (int e = 0; e < QG; ++e) {
                            kf[0][2 * e] = *(const v8h*)(kb + 32 * e);
                            kf[0][2 * e + 1] = *(const v8h*)(kb + 16 * KS + 32 * e);
                        }
#pragma unroll
                        for (int g = 0; g < DSTEP / QG; ++g) {
                            if (g + 1 < DSTEP / QG) {
#pragma unroll
                                for (int e = 0; e < QG; ++e) {
                                    const int st = (g + 1) * QG + e;
                                    kf[(g + 1) & 1][2 * e] = *(const v8h*)(kb + 32 * st);
                                    kf[(g + 1) & 1][2 * e + 1] = *(const v8h*)(kb + 16 * KS + 32 * st);
                                }
                            }
                            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                            for (int e = 0; e < QG; ++e) {
                                const int st = g * QG + e;
                                if (st < NSTEP) {
                                    an[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[g & 1][2 * e], qf[st], an[0], 0, 0, 0);
                                    an[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[g & 1][2 * e + 1], qf[st], an[1], 0, 0, 0);
                                } else {
                                    ar[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[g & 1][2 * e], qf[st], ar[0], 0, 0, 0);
                                    ar[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[g & 1][2 * e + 1], qf[st], ar[1], 0, 0, 0);
                                }
                            }
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                    // scores and P of tile j for head hq: lane (l16, g4) holds keys 4 g4 + i and 16 + 4 g4 + i
                    const float kscl[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
                    float sv[8];
                    if (full) {
#pragma unroll
                        for (int i = 0; i < 8; ++i) sv[i] = sm_q * fmaf(kscl[i], an[i >> 2][i & 3], ar[i >> 2][i & 3]);
                    } else {
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            sv[i] = kscl[i] >= 0.f ? sm_q * fmaf(kscl[i], an[i >> 2][i & 3], ar[i >> 2][i & 3])
                                                   : -INFINITY;
                    }
                    float mx = sv[0];
#pragma unroll
                    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
                    mx = rows4_max(mx);
                    m_seen = fmaxf(m_seen, mx);
                    s_seen = fmaxf(s_seen, st_max);
                    m_ref = m_ref == -INFINITY ? mx : m_ref;  // first tile with visible keys (accumulators still zero)
                    if (s_ref == 0.f && st_max > 0.f) {     // (the same in every lane)
                        s_ref = st_max;
                        inv_s = 1.f / s_ref;
                    }
                    if (mx > m_ref + kLazy * kLog2e || st_max > kSRatio * s_ref) sm.restart = 1;
                    v8h pn, pr;
                    float sum = 0.f;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float p = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[i] - m_ref);
                        sum += p;
                        pr[i] = (_Float16)p;
                        pn[i] = (_Float16)(p * (kscl[i] * inv_s));
                    }
                    l_run += rows4_sum(sum);
                    *(v8h*)(sm.pn[j & 1] + hq * Sm::PS + 8 * g4) = pn;
                    *(v8h*)(sm.pr[j & 1] + hq * Sm::PS + 8 * g4) = pr;
                }
                lds_barrier();
            }
            // hand the head's references and sum to the values role; lse / partial statistics
            const float m_nat = m_ref * kLn2;  // back to natural units
            if (g4 == 0) {
                sm.mfin[hq] = m_nat;
                sm.lfin[hq] = l_run;
            }
            if (tid == 0) sm.sfin = s_ref > 0.f ? s_ref : 1.f;
            const bool redo = !second && sm.restart != 0;
            if (!redo && g4 == 0) {
                if (S == 1) lse[t * H + hq] = l_run > 0.f ? m_nat + __logf(l_run) : -INFINITY;
                else {
                    part_ml[((t * S + s) * H + hq) * 2 + 0] = m_nat;
                    part_ml[((t * S + s) * H + hq) * 2 + 1] = l_run;
                }
            }
            lds_barrier();
            if (!redo) {
                // the values role stages the output half by half; both roles store it
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    lds_barrier();
                    store_out<D, 512>(ob, sm.cs, 32 * half, tid, t, s, S, out, (_Float16*)part_o);
                    lds_barrier();
                }
            }
        } else {
            v4f acc[4][DT];
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < DT; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};
            for (int it = 0; it <= nt; ++it) {
                batch_begin(it);
                if (it + 1 < nt) stage(it + 1);
                batch_take();
                if (it + 2 < nt) issue(it + 2);
                __builtin_amdgcn_sched_barrier(0);  // the prefetch leaves before P V, not after it
                if (it >= 1) {
                    // O[heads x dims] += P V (tile it - 1) for all heads over this wave's dims
                    const int j = it - 1;
                    const _Float16* vb = sm.kv[j % 3] + (4 * g4 + (l16 >> 2)) * KS + 4 * (l16 & 3);
                    auto vfrag = [&](int dt) -> v8h {
                        const int d0 = dt < NN ? 16 * (NN * rw + dt) : DN + 16 * rw;
                        const v4s lo = lds_read_tr16(vb + d0);
                        const v4s hi = lds_read_tr16(vb + 16 * KS + d0);
                        const v8u16 c = {(uint16_t)lo[0], (uint16_t)lo[1], (uint16_t)lo[2], (uint16_t)lo[3],
                                         (uint16_t)hi[0], (uint16_t)hi[1], (uint16_t)hi[2], (uint16_t)hi[3]};
                        return __builtin_bit_cast(v8h, c);
                    };
                    // P of every head group, then one V fragment at a time (fewer registers live)
                    v8h pf[4];
#pragma unroll
                    for (int ht = 0; ht < 4; ++ht) pf[ht] = *(const v8h*)(sm.pn[j & 1] + (16 * ht + l16) * Sm::PS + 8 * g4);
#pragma unroll
                    for (int dt = 0; dt < NN; ++dt) {
                        const v8h vf = vfrag(dt);
#pragma unroll
                        for (int ht = 0; ht < 4; ++ht)
                            acc[ht][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf[ht], vf, acc[ht][dt], 0, 0, 0);
                    }
#pragma unroll
                    for (int ht = 0; ht < 4; ++ht) pf[ht] = *(const v8h*)(sm.pr[j & 1] + (16 * ht + l16) * Sm::PS + 8 * g4);
                    {
                        const v8h vf = vfrag(NN);
#pragma unroll
                        for (int ht = 0; ht < 4; ++ht)
                            acc[ht][NN] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf[ht], vf, acc[ht][NN], 0, 0, 0);
                    }
                }
                batch_end(it);
                lds_barrier();
            }
            lds_barrier();  // the scores role's per-head statistics
            const bool redo = !second && sm.restart != 0;
            if (!redo) {
                // ---- output: lane holds heads 16 ht + 4 g4 + i at one dim of each of its dim tiles ----
                const float sfin = sm.sfin;
#pragma unroll
                for (int half = 0; half < 2; ++half) {
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int ht = 2 * half + hh;
                        float inv[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float l = sm.lfin[16 * ht + 4 * g4 + i];
                            inv[i] = l > 0.f ? 1.f / l : 0.f;
                        }
#pragma unroll
                        for (int dt = 0; dt < DT; ++dt) {
                            const bool nope = dt < NN;
                            const int d = (nope ? 16 * (NN * rw + dt) : DN + 16 * rw) + l16;
                            float o[4];
#pragma unroll
                            for (int i = 0; i < 4; ++i) o[i] = acc[ht][dt][i] * (nope ? sfin : 1.f) * inv[i];
                            stage_out(ob, kOutStride<D>, hh, g4, d, o);
                        }
                    }
                    lds_barrier();
                    store_out<D, 512>(ob, sm.cs, 32 * half, tid, t, s, S, out, (_Float16*)part_o);
                    lds_barrier();
                }
            }
        }
        const bool redo = !second && sm.restart != 0;
        lds_barrier();  // every wave has read the flag
        return redo;
    };

    if (run_pass(false)) {
        // a tile broke the references: again, with the maxima of every tile as the references
        // (no tile can break them)
        if (tid == 0) sm.restart = 0;
        run_pass(true);
    }
}

// Merge the S split partials of one (row, head) in the fixed order s = 0 .. S-1.
template <int D>
__global__ __launch_bounds__(128) void k_mqa_combine(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                                                     const int64_t* __restrict__ pos, int H, int S, RopeTab rt,
                                                     float* __restrict__ out, float* __restrict__ lse) {
    constexpr int DN = D - 64;
    constexpr int SMAX = 64;
    __shared__ float wgt[SMAX];
    __shared__ float red[2];
    const int64_t th = blockIdx.x;  // t*H + h
    const int64_t t = th / H;
    const int h = (int)(th % H);
    const int tid = threadIdx.x;
    if (tid < 64) {
        float ms = -INFINITY, ls = 0.f;
        if (tid < S) {
            ms = part_ml[((t * S + tid) * H + h) * 2];
            ls = part_ml[((t * S + tid) * H + h) * 2 + 1];
        }
        const float M = wave_max(ms);
        const float e = ms == -INFINITY ? 0.f : __expf(ms - M);
        float L = ls * e;
        // fixed-order sum over splits: lane 0 accumulates sequentially
        float Lseq = 0.f;
        for (int i = 0; i < S; ++i) Lseq += __shfl(L, i);
        if (tid < S) wgt[tid] = Lseq > 0.f ? e / Lseq : 0.f;
        if (tid == 0) {
            red[0] = M;
            red[1] = Lseq;
        }
    }
    __syncthreads();
    for (int d0 = tid * 4; d0 < D; d0 += 128 * 4) {
        float o[4] = {0.f, 0.f, 0.f, 0.f};
        const float* base = part_o + (t * S * H + h) * (int64_t)D + d0;
        int s = 0;
        for (; s + 8 <= S; s += 8) {
            float4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = *(const float4*)(base + (int64_t)(s + u) * H * D);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float wv = wgt[s + u];
                o[0] = fmaf(wv, v[u].x, o[0]);
                o[1] = fmaf(wv, v[u].y, o[1]);
                o[2] = fmaf(wv, v[u].z, o[2]);
                o[3] = fmaf(wv, v[u].w, o[3]);
            }
        }
        for (; s < S; ++s) {
            const float4 v = *(const float4*)(base + (int64_t)s * H * D);
            const float wv = wgt[s];
            o[0] = fmaf(wv, v.x, o[0]);
            o[1] = fmaf(wv, v.y, o[1]);
            o[2] = fmaf(wv, v.z, o[2]);
            o[3] = fmaf(wv, v.w, o[3]);
        }
        if (d0 >= DN) {
            const double tp = (double)pos[t];
            for (int i = 0; i < 4; i += 2) {
                float cs, sn;
                angle_cs(tp, rt.theta[(d0 - DN + i) >> 1], cs, sn);
                sn = -sn;  // rotation by -t
                const float x0 = o[i], x1 = o[i + 1];
                o[i] = x0 * cs - x1 * sn;
                o[i + 1] = x0 * sn + x1 * cs;
            }
        }
        *(float4*)(out + th * D + d0) = make_float4(o[0], o[1], o[2], o[3]);
    }
    if (tid == 0) lse[th] = red[1] > 0.f ? red[0] + __logf(red[1]) : -INFINITY;
}

// Merge of the 64-head kernels' split partials: fp16, each normalised by its own sum l_s,
// weighted by e^(m_s - M) l_s / L, L summed in the fixed order s = 0 .. S-1.  The partial
// loads are issued first (up to kC16Reg splits held in registers), beside the splits'
// statistics, so the merge waits for one round of global loads.
constexpr int kC16Reg = 24;
template <int D>
__global__ __launch_bounds__(128) void k_mqa_combine16(const _Float16* __restrict__ part_o,
                                                       const float* __restrict__ part_ml, const int64_t* __restrict__ pos,
                                                       int H, int S, RopeTab rt, float* __restrict__ out,
                                                       float* __restrict__ lse) {
    static_assert(D <= 4 * 128, "one pass of 128 threads x 4 dims");
    constexpr int DN = D - 64;
    constexpr int SMAX = 64;
    __shared__ float ms[SMAX], ll[SMAX];
    const int64_t th = blockIdx.x;  // t*H + h
    const int64_t t = th / H;
    const int h = (int)(th % H);
    const int tid = threadIdx.x;
    const int d0 = tid * 4;
    const bool live = d0 < D;  // D = 128: 32 threads carry dims
    const _Float16* base = part_o + (t * S * H + h) * (int64_t)D + (live ? d0 : 0);
    uint2 v[kC16Reg];
#pragma unroll
    for (int s = 0; s < kC16Reg; ++s)
        if (s < S && live) v[s] = *(const uint2*)(base + (int64_t)s * H * D);
    if (tid < S) {
        ms[tid] = part_ml[((t * S + tid) * H + h) * 2];
        ll[tid] = part_ml[((t * S + tid) * H + h) * 2 + 1];
    }
    __syncthreads();
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, ms[s]);
    float Ls = 0.f;
    if (tid < S) Ls = ms[tid] == -INFINITY ? 0.f : ll[tid] * __expf(ms[tid] - M);
    __syncthreads();  // every thread has read ms and ll
    if (tid < S) ll[tid] = Ls;
    __syncthreads();
    float L = 0.f;
    for (int s = 0; s < S; ++s) L += ll[s];  // fixed order
    const float inv = L > 0.f ? 1.f / L : 0.f;
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    auto acc = [&](const uint2 x, float wv) {
        const v2h a = __builtin_bit_cast(v2h, x.x), b = __builtin_bit_cast(v2h, x.y);
        o[0] = fmaf(wv, (float)a[0], o[0]);
        o[1] = fmaf(wv, (float)a[1], o[1]);
        o[2] = fmaf(wv, (float)b[0], o[2]);
        o[3] = fmaf(wv, (float)b[1], o[3]);
    };
    if (live) {
#pragma unroll
        for (int s = 0; s < kC16Reg; ++s)
            if (s < S) acc(v[s], ll[s] * inv);
        for (int s = kC16Reg; s < S; ++s) acc(*(const uint2*)(base + (int64_t)s * H * D), ll[s] * inv);
    }
    if (live && d0 >= DN) {
        const double tp = (double)pos[t];
        for (int i = 0; i < 4; i += 2) {
            float cs, sn;
            angle_cs(tp, rt.theta[(d0 - DN + i) >> 1], cs, sn);
            sn = -sn;  // rotation by -t
            const float x0 = o[i], x1 = o[i + 1];
            o[i] = x0 * cs - x1 * sn;
            o[i + 1] = x0 * sn + x1 * cs;
        }
    }
    if (live) *(float4*)(out + th * D + d0) = make_float4(o[0], o[1], o[2], o[3]);
    if (tid == 0) lse[th] = L > 0.f ? M + __logf(L) : -INFINITY;
}

// Merge of k_mqa64's split partials, stored in its accumulators' order (see its epilogue): one
// one-wave workgroup per (row, 16-head tile ht, producer wave w, dim tile dt), a lane per 8-byte
// quad (heads 16 ht + 4 g4 + i, i < 4, at one dim), so each split's load is one 512-byte wave
// row; small workgroups spread the partials' lines over many CUs (a CU keeps only so many
// misses in flight).  The 16 heads' weights e^(m_s - M) l_s / L (L summed in a fixed order) go
// through LDS while the quads' loads are in flight.
template <int D>
__global__ __launch_bounds__(64) void k_mqa_combine_sw(const _Float16* __restrict__ part_o,
                                                       const float* __restrict__ part_ml,
                                                       const int64_t* __restrict__ pos, int S, RopeTab rt,
                                                       float* __restrict__ out, float* __restrict__ lse) {
    constexpr int H = 64, DN = D - 64, NN = DN / 64, DT = NN + 1, NTH = 64;
    constexpr int SMAX = 64;
    __shared__ float wg[16][SMAX];
    static_assert(NTH == 4 * 16, "four lanes per head for the weights");
    const int64_t t = blockIdx.x / (16 * DT);
    const int r = blockIdx.x % (16 * DT);
    const int ht = r / (4 * DT), w = (r / DT) & 3, dt = r % DT;
    const int tid = threadIdx.x;
    const int lane = tid, l16 = lane & 15, g4 = lane >> 4;
    const _Float16* base = part_o + t * (int64_t)S * H * D + (((w * 4 + ht) * DT + dt) * 64 + lane) * 4;
    v4h v[kC16Reg];
#pragma unroll
    for (int s = 0; s < kC16Reg; ++s)
        if (s < S) v[s] = *(const v4h*)(base + (int64_t)s * H * D);
    // RoPE dims: the rotation by tp, while the partials are in flight
    const int d = dt < NN ? 16 * (NN * w + dt) + l16 : DN + 16 * w + l16;
    float cs = 1.f, sn = 0.f;
    if (dt == NN) angle_cs((double)pos[t], rt.theta[(d - DN) >> 1], cs, sn);
    // the 16 heads' merge weights: lane (h = lane / 4, q = lane % 4) takes splits q, q + 4, ...
    // (every (m, l) load in flight at once); M and L over the four lanes of a head by a fixed
    // butterfly, so every lane of the quad holds the same bits
    {
        constexpr int PERL = SMAX / 4;
        const int h = tid >> 2, q = tid & 3;
        float2 ml[PERL];
#pragma unroll
        for (int i = 0; i < PERL; ++i) {
            const int sp = q + 4 * i;
            ml[i] = sp < S ? *(const float2*)(part_ml + ((t * S + sp) * H + 16 * ht + h) * 2)
                           : make_float2(-INFINITY, 0.f);
        }
        float M = -INFINITY;
#pragma unroll
        for (int i = 0; i < PERL; ++i) M = fmaxf(M, ml[i].x);
        M = fmaxf(M, __shfl_xor(M, 1));
        M = fmaxf(M, __shfl_xor(M, 2));
        float ls[PERL];
        float L = 0.f;
#pragma unroll
        for (int i = 0; i < PERL; ++i) {
            ls[i] = ml[i].x == -INFINITY ? 0.f : ml[i].y * __expf(ml[i].x - M);
            L += ls[i];
        }
        L += __shfl_xor(L, 1);
        L += __shfl_xor(L, 2);
        const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
        for (int i = 0; i < PERL; ++i)
            if (q + 4 * i < S) wg[h][q + 4 * i] = ls[i] * inv;
        if (q == 0 && w == 0 && dt == 0) lse[t * H + 16 * ht + h] = L > 0.f ? M + __logf(L) : -INFINITY;
    }
    __syncthreads();
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    auto acc = [&](const v4h x, int sp) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = fmaf(wg[4 * g4 + i][sp], (float)x[i], o[i]);
    };
#pragma unroll
    for (int s = 0; s < kC16Reg; ++s)
        if (s < S) acc(v[s], s);
    for (int s = kC16Reg; s < S; ++s) acc(*(const v4h*)(base + (int64_t)s * H * D), s);
    if (dt == NN) {
        // RoPE dims: undo the rotation by tp; the pair's other dim is in lane l16 ^ 1
        sn = -sn;
        const bool odd = (l16 & 1) != 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float p = __shfl_xor(o[i], 1);
            const float x0 = odd ? p : o[i], x1 = odd ? o[i] : p;
            o[i] = odd ? x0 * sn + x1 * cs : x0 * cs - x1 * sn;
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) out[(t * H + 16 * ht + 4 * g4 + i) * (int64_t)D + d] = o[i];
}

// Range check of the entries a call reads (debug builds of a caller's pipeline): the
// 64-head kernels stage the bf16 RoPE dims as fp16 with truncation, so a value of magnitude
// above 65504 (or a NaN / infinity) would be clamped.  One workgroup per row walks the row's
// key list like the attention kernels and sets *bad when any referenced entry holds one.
__global__ __launch_bounds__(256) void k_check_rope(const int32_t* __restrict__ seq, const int64_t* __restrict__ pos,
                                                    const int32_t* __restrict__ idx, int k, int m, KvView comp,
                                                    KvView win, int window, int* __restrict__ bad) {
    const int64_t t = blockIdx.x;
    const RowKeys rk = row_keys(pos[t], idx, k, m, window);
    const int32_t sq = seq[t];
    int found = 0;
    for (int64_t u = threadIdx.x; u < rk.n; u += 256) {
        const int64_t r = resolve(u, t, sq, rk, idx, k, comp, win);
        if (r == -1) continue;
        const uint16_t* rp = r >= 0 ? comp.rope + r * 64 : win.rope + (-r - 2) * 64;
        for (int e = 0; e < 64; ++e) {
            const uint32_t b = (uint32_t)rp[e] & 0x7FFFu;
            found |= b > 0x477Fu;  // |x| > 65504 in bf16 (0x477F = 65280; the next value 65536 is beyond)
        }
    }
    if (found) atomicOr(bad, 1);
}

hipError_t launch_check_rope(const int32_t* seq, const int64_t* pos, int64_t T, const int32_t* idx, int k, int m,
                             KvView comp, KvView win, int window, int* bad, hipStream_t st) {
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(k_check_rope, dim3((unsigned)T), dim3(256), 0, st, seq, pos, idx, k, m, comp, win, window, bad);
    return hipGetLastError();
}

// Splits per row: about one workgroup per CU in all (the 64-head kernels hold most of a
// CU's LDS, so a second round of workgroups would run after the first), at least 64 keys
// per split, at most 64 splits.
static int choose_splits(int64_t T, int64_t max_keys) {
    int64_t s = (256 + T - 1) / T;
    int64_t by_keys = (max_keys + 63) / 64;
    if (s > by_keys) s = by_keys;
    if (s > 64) s = 64;
    if (s < 1) s = 1;
    return (int)s;
}

// The 64-head kernels share a split between two workgroups of 32 heads when the grid would
// otherwise leave at least half the CUs idle: at T x S <= 128 with splits of up to 12 tiles;
// else, when half the splits would hold at most 4 tiles each and T x ceil(S/2) <= 128, with
// half the splits (measured: 8 rows at 1M context, 53.1 -> 51.0 us per decode step; longer
// halved splits were slower).  The workspace is sized for choose_splits' S, never smaller.
static void choose_partition(int64_t T, int H, int64_t max_keys, int& S, bool& hsplit) {
    S = choose_splits(T, max_keys);
    hsplit = false;
    if (H != 64) return;
    if (T * S <= 128 && (max_keys + S - 1) / S <= 12 * KT) {
        hsplit = true;
        return;
    }
    const int S2 = (S + 1) / 2;
    if (T * S2 <= 128 && (max_keys + S2 - 1) / S2 <= 4 * KT) {
        S = S2;
        hsplit = true;
    }
}

size_t mqa_workspace_bytes(int64_t T, int H, int d, int64_t max_keys) {
    const int S = choose_splits(T, max_keys);
    if (S == 1) return 0;
    return (size_t)T * S * H * ((size_t)d + 2) * sizeof(float) + 256;
}

template <int H, int D>
static void launch_mqa_t(const uint16_t* q, const int32_t* seq, const int64_t* pos, int64_t T, const int32_t* idx,
                         int k, int m, KvView comp, KvView win, int window, float sm_scale, const RopeTab& rt, int S,
                         bool hsplit, int64_t max_keys, float* out, float* lse, float* po, float* pml,
                         hipStream_t st) {
    // splits of more than a few tiles: the two-role kernel (its pipeline costs a step at either end)
    const bool long_splits = (max_keys + S - 1) / S > 12 * KT;
    const bool paged = comp.pages || win.pages;  // paged views: their own instantiation
#define CSA_MQA_LAUNCH(KERN, NTH, NWG)                                                                              \
    hipLaunchKernelGGL((KERN), dim3((unsigned)(NWG)), dim3(NTH), 0, st, q, seq, pos, idx, k, m, comp, win, window, \
                       sm_scale, rt, S, out, lse, po, pml)
    if (H == 64 && D == 512 && long_splits) {
        if (paged) CSA_MQA_LAUNCH((k_mqa64ws<512, true>), 512, T * S);
        else CSA_MQA_LAUNCH((k_mqa64ws<512, false>), 512, T * S);
    } else if constexpr (H == 64) {
        if (hsplit) {
            if (paged) CSA_MQA_LAUNCH((k_mqa64<D, true, 2>), 256, 2 * T * S);
            else CSA_MQA_LAUNCH((k_mqa64<D, false, 2>), 256, 2 * T * S);
        } else {
            if (paged) CSA_MQA_LAUNCH((k_mqa64<D, true, 1>), 256, T * S);
            else CSA_MQA_LAUNCH((k_mqa64<D, false, 1>), 256, T * S);
        }
    } else {
        CSA_MQA_LAUNCH((k_mqa<H, D>), 256, T * S);
    }
#undef CSA_MQA_LAUNCH
    if (S > 1) {
        if constexpr (H == 64) {
            // the two-role kernel writes head-major partials, k_mqa64 its accumulators' order
            if (D == 512 && long_splits)
                hipLaunchKernelGGL((k_mqa_combine16<D>), dim3((unsigned)(T * H)), dim3(128), 0, st, (const _Float16*)po,
                                   pml, pos, H, S, rt, out, lse);
            else
                hipLaunchKernelGGL((k_mqa_combine_sw<D>), dim3((unsigned)(T * 16 * (D / 64))), dim3(64), 0, st,
                                   (const _Float16*)po, pml, pos, S, rt, out, lse);
        } else {
            hipLaunchKernelGGL((k_mqa_combine<D>), dim3((unsigned)(T * H)), dim3(128), 0, st, po, pml, pos, H, S, rt,
                               out, lse);
        }
    }
}

hipError_t launch_mqa(const uint16_t* q, const int32_t* seq, const int64_t* pos, int64_t T, int H, int d,
                      const int32_t* idx, int k, int m, int64_t max_keys, KvView comp, KvView win, int window,
                      float sm_scale, const RopeTab& rt, float* out, float* lse, void* ws, hipStream_t st) {
    if (T == 0) return hipSuccess;
    int S;
    bool hsplit;
    choose_partition(T, H, max_keys, S, hsplit);
    float* po = nullptr;
    float* pml = nullptr;
    if (S > 1) {
        po = (float*)ws;
        pml = po + (size_t)T * S * H * d;
    }
#define CSA_MQA(HH, DD)                                                                                          \
    launch_mqa_t<HH, DD>(q, seq, pos, T, idx, k, m, comp, win, window, sm_scale, rt, S, hsplit, max_keys, out, lse, \
                         po, pml, st)
    if (d == 512) {
        if (H == 64) CSA_MQA(64, 512);
        else if (H == 32) CSA_MQA(32, 512);
        else CSA_MQA(16, 512);
    } else {
        if (H == 64) CSA_MQA(64, 128);
        else if (H == 32) CSA_MQA(32, 128);
        else CSA_MQA(16, 128);
    }
#undef CSA_MQA
    return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Backward of the attention step (training side): the gradient of sum(g * out)
// with respect to the pre-RoPE query and to the dequantised entries, for the
// forward above (keys and values are the same entry, RoPE on the last 64 dims,
// reverse RoPE on the output).  With q~ = R(tp) q, g~ = R(tp) g, the forward's
// lse and out, D = <g, out>:
//   p_u = exp(c <q~, e_u> - lse),  ds_u = p_u (<g~, e_u> - D)
//   dq  = R(-tp) (c sum_u ds_u e_u),  de_u += c ds_u q~ + p_u g~.
// One workgroup per query row, one wave per 16 heads, the row's key list in
// tiles of 16 entries (the next tile's loads in flight during this one):
//   S, dP    per wave: keys x its heads (MFMA 16x16x32 f16) on the entries as
//            staged, dequantised to fp16 (the entry scale folded in keeps ds and
//            the keys clear of fp16's subnormal range)
//   dq      per wave: its heads x 512 dims += ds K, the ds values straight from
//            the S layout as the A operand of 16x16x16 MFMAs; kept in registers
//   de      per wave: the tile's keys x its share of the dims, summed over all
//            heads in the MFMA ([ds | p] x [c q~ ; g~] from the LDS copies),
//            then one fp32 atomic per (key, dim): an entry is shared by many
//            rows, so the summation order varies.
// g is scaled by a power of two per row (|g~ s_g| <= 1 for every head) so that
// it and ds fit fp16 whatever the loss scale; the scale is divided out exactly.
// ---------------------------------------------------------------------------
constexpr int kBwdKT = 16;   // keys per tile
constexpr int kBwdRB = 256;  // keys resolved per batch (one per thread of a 4-wave workgroup)

template <int NW>
struct __align__(16) MqaBwdSmem {
    static constexpr int QS = 512 + 8;  // fp16 row stride of the [head][dim] copies
    static constexpr int KS = 512 + 16;
    static constexpr int PS = kBwdKT + 8;
    _Float16 qs[16 * NW * QS];   // c * q~, [head][dim]
    _Float16 gs[16 * NW * QS];   // s_g * g~
    _Float16 kt[kBwdKT * KS];    // the tile, dequantised: FP8 dims * entry scale, RoPE dims
    _Float16 dsr[16 * NW * PS];  // [head][key] ds * s_g
    _Float16 pp[16 * NW * PS];   // [head][key] p
    int64_t krow[3][kBwdKT];     // resolved row code per key of tile j in [j % 3] (-1 masked)
    float kscl[3][kBwdKT];       // entry scale, -1 for a masked key
    float cs[64];
    float g2w[NW];
};

template <int NW>
__global__ __launch_bounds__(64 * NW) void k_mqa_bwd(const uint16_t* __restrict__ q, const int32_t* __restrict__ seq,
                                                     const int64_t* __restrict__ pos, const int32_t* __restrict__ idx,
                                                     int k, int m, KvView comp, KvView win, int window,
                                                     float sm_scale, RopeTab rt, const float* __restrict__ out,
                                                     const float* __restrict__ lse, const float* __restrict__ dout,
                                                     float* __restrict__ dq, unsigned long long* __restrict__ dcomp,
                                                     unsigned long long* __restrict__ dwin) {
    constexpr int D = 512, DN = 448, NT = 64 * NW, H = 16 * NW;
    constexpr int DTW = D / NW / 16;                           // 16-dim tiles of de per wave
    constexpr int NCH = (kBwdKT * 36 + NT - 1) / NT;           // staged 16-byte chunks per thread
    constexpr int TPB = kBwdRB / kBwdKT;                       // tiles per resolved batch
    static_assert(NT <= kBwdRB && kBwdRB % NT == 0, "threads resolve whole batches");
    constexpr int RPT = kBwdRB / NT;                           // keys resolved per thread and batch
    using Sm = MqaBwdSmem<NW>;
    __shared__ Sm sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    const int64_t t = blockIdx.x;
    const int64_t tp = pos[t];
    const int32_t sq = seq[t];
    const RowKeys rk = row_keys(tp, idx, k, m, window);
    const int64_t n = rk.n;
    const int64_t hrow = t * H + 16 * wave + l16;  // this lane's head (row of q, g, out)

    if (tid < 32) {
        float c, sn;
        angle_cs((double)tp, rt.theta[tid], c, sn);
        sm.cs[2 * tid] = c;
        sm.cs[2 * tid + 1] = sn;
    }
    // ---- D = <g, out> and |g|^2 per head (rotation-free), then one power-of-two scale per row ----
    float dsum = 0.f, g2 = 0.f;
    v4f gk[D / 16];  // this lane's 128 elements of g, read once
    {
        const float* gr = dout + hrow * D + 8 * g4;
        const float* orow = out + hrow * D + 8 * g4;
#pragma unroll
        for (int st = 0; st < D / 32; ++st) {
            gk[2 * st] = *(const v4f*)(gr + 32 * st);
            gk[2 * st + 1] = *(const v4f*)(gr + 32 * st + 4);
            const v4f a0 = gk[2 * st], a1 = gk[2 * st + 1];
            const v4f o0 = *(const v4f*)(orow + 32 * st), o1 = *(const v4f*)(orow + 32 * st + 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dsum = fmaf(a0[i], o0[i], fmaf(a1[i], o1[i], dsum));
                g2 = fmaf(a0[i], a0[i], fmaf(a1[i], a1[i], g2));
            }
        }
    }
    dsum += __shfl_xor(dsum, 16);
    dsum += __shfl_xor(dsum, 32);
    g2 += __shfl_xor(g2, 16);
    g2 += __shfl_xor(g2, 32);
    float g2max = g2;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) g2max = fmaxf(g2max, __shfl_xor(g2max, o));
    if (lane == 0) sm.g2w[wave] = g2max;
    __syncthreads();  // cs, g2w
#pragma unroll
    for (int w = 0; w < NW; ++w) g2max = fmaxf(g2max, sm.g2w[w]);
    int ex = 0;
    if (g2max > 0.f) (void)frexpf(sqrtf(g2max), &ex);  // |g_h| < 2^ex for every head of the row
    ex = ex < -120 ? -120 : (ex > 120 ? 120 : ex);
    const float sg = ldexpf(1.f, -ex), inv_sg = ldexpf(1.f, ex);
    const float dh = dsum * sg;  // D * s_g of head l16
    const float lse_h = lse[hrow];

    // ---- q~ and s_g g~ in fp16: B operands of S / dP in registers, [head][dim] copies in LDS ----
    v8h qf[D / 32], gf[D / 32];
    {
        const uint16_t* qr = q + hrow * D + 8 * g4;
        _Float16* qrow = sm.qs + (16 * wave + l16) * Sm::QS + 8 * g4;
        _Float16* grow = sm.gs + (16 * wave + l16) * Sm::QS + 8 * g4;
#pragma unroll
        for (int st = 0; st < D / 32; ++st) {
            const v4i raw = *(const v4i*)(qr + 32 * st);
            const v4f a0 = gk[2 * st], a1 = gk[2 * st + 1];
            float xq[8], xg[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                xq[2 * i] = __uint_as_float((uint32_t)raw[i] << 16);
                xq[2 * i + 1] = __uint_as_float((uint32_t)raw[i] & 0xFFFF0000u);
                xg[i] = a0[i] * sg;
                xg[4 + i] = a1[i] * sg;
            }
            if (32 * st >= DN) {  // RoPE pairs (2p, 2p + 1) of the last 64 dims, at +tp
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int pr = (32 * st + 8 * g4 - DN) / 2 + i;
                    const float c = sm.cs[2 * pr], sn = sm.cs[2 * pr + 1];
                    const float q0 = xq[2 * i], q1 = xq[2 * i + 1], a = xg[2 * i], bb = xg[2 * i + 1];
                    xq[2 * i] = q0 * c - q1 * sn;
                    xq[2 * i + 1] = q0 * sn + q1 * c;
                    xg[2 * i] = a * c - bb * sn;
                    xg[2 * i + 1] = a * sn + bb * c;
                }
            }
            v8h hq, hgv, hqs;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                hq[i] = (_Float16)xq[i];
                hgv[i] = (_Float16)xg[i];
                hqs[i] = (_Float16)(xq[i] * sm_scale);
            }
            qf[st] = hq;
            gf[st] = hgv;
            *(v8h*)(qrow + 32 * st) = hqs;
            *(v8h*)(grow + 32 * st) = hgv;
        }
    }

    // ---- the key list: resolved a batch of 256 keys ahead (RPT keys per thread, in registers),
    //      handed to LDS one tile ahead, staged one tile ahead ----
    int64_t cur_code[RPT], nxt_code[RPT];
    float cur_scl[RPT], nxt_scl[RPT];
    auto resolve_batch = [&](int64_t bt, int64_t (&code)[RPT], float (&scl)[RPT]) {
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const int64_t u = bt * kBwdRB + r * NT + tid;
            code[r] = u < n ? resolve(u, t, sq, rk, idx, k, comp, win) : -1;
            scl[r] = code[r] == -1 ? -1.f : (code[r] >= 0 ? comp.scale[code[r]] : win.scale[-code[r] - 2]);
        }
    };
    // tile j's keys are keys 16 (j % 16) .. + 15 of batch j / 16: held by threads (and slots r) whose
    // batch index r NT + tid falls there
    auto publish = [&](int64_t j) {
        const int first = (int)(j % TPB) * kBwdKT;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const int bi = r * NT + tid;
            if (bi >= first && bi < first + kBwdKT) {
                sm.krow[j % 3][bi - first] = cur_code[r];
                sm.kscl[j % 3][bi - first] = cur_scl[r];
            }
        }
    };
    // Every thread issues NCH loads and every lane of the tile loop one atomic per (key, dim), masked
    // or not: with a fixed count of memory operations in flight, the wait for a tile's loads can
    // leave the previous tile's atomics in flight (a variable count makes the compiler wait for all).
    v4i raw[NCH];
    auto issue = [&](int b) {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = (tid + NT * i) % (kBwdKT * 36);  // (the overhang re-reads a chunk; not staged)
            const int kk = c / 36, part = c % 36;
            const int64_t code = sm.krow[b][kk];
            const uint8_t* src;
            if (code == -1) src = g_zero_entry;
            else if (part < 28) src = (code >= 0 ? comp.nope + code * DN : win.nope + (-code - 2) * DN) + 16 * part;
            else src = (const uint8_t*)(code >= 0 ? comp.rope + code * 64 : win.rope + (-code - 2) * 64) + 16 * (part - 28);
            raw[i] = gload<v4i>(src);
        }
    };
    auto stage = [&](int b) {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = tid + NT * i;
            if (c < kBwdKT * 36) {
                const int kk = c / 36, part = c % 36;
                _Float16* dst = sm.kt + kk * Sm::KS;
                if (part < 28) {
                    const float sc = sm.kscl[b][kk] > 0.f ? sm.kscl[b][kk] : 0.f;
                    v8h lo8, hi8;
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)raw[i][w], 1.f, false);
                        const v2h bb = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)raw[i][w], 1.f, true);
                        const _Float16 x0 = (_Float16)((float)a[0] * sc), x1 = (_Float16)((float)a[1] * sc);
                        const _Float16 x2 = (_Float16)((float)bb[0] * sc), x3 = (_Float16)((float)bb[1] * sc);
                        if (w < 2) {
                            lo8[4 * w] = x0, lo8[4 * w + 1] = x1, lo8[4 * w + 2] = x2, lo8[4 * w + 3] = x3;
                        } else {
                            hi8[4 * w - 8] = x0, hi8[4 * w - 7] = x1, hi8[4 * w - 6] = x2, hi8[4 * w - 5] = x3;
                        }
                    }
                    *(v8h*)(dst + 16 * part) = lo8;
                    *(v8h*)(dst + 16 * part + 8) = hi8;
                } else {
                    v8h r8;
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        r8[2 * w] = (_Float16)__uint_as_float((uint32_t)raw[i][w] << 16);
                        r8[2 * w + 1] = (_Float16)__uint_as_float((uint32_t)raw[i][w] & 0xFFFF0000u);
                    }
                    *(v8h*)(dst + DN + 8 * (part - 28)) = r8;
                }
            }
        }
    };

    v4f accq[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) accq[dt] = v4f{0.f, 0.f, 0.f, 0.f};

    // Tile j: its keys published (LDS ring slot j % 3) at the end of tile j - 2, its loads issued
    // at the start of tile j - 1 and staged at that tile's end, after its atomics: loads, then
    // atomics, then the wait for the loads, on one path, so the wait leaves the atomics in flight.
    // Past the last tile the keys resolve to masked ones: the extra tile's loads read the zero
    // entry and its staging is never read.
    const int64_t ntile = (n + kBwdKT - 1) / kBwdKT;
    auto next_keys = [&](int64_t jn) {  // publish tile jn's keys (batch switch on its first tile)
        if (jn % TPB == 0 && jn > 0) {
#pragma unroll
            for (int r = 0; r < RPT; ++r) cur_code[r] = nxt_code[r], cur_scl[r] = nxt_scl[r];
            resolve_batch(jn / TPB + 1, nxt_code, nxt_scl);
        }
        publish(jn);
    };
    if (ntile > 0) {
        resolve_batch(0, cur_code, cur_scl);
        resolve_batch(1, nxt_code, nxt_scl);
        publish(0);
        publish(1);
    }
    __syncthreads();  // the [head][dim] copies, the keys of tiles 0 and 1
    if (ntile > 0) {
        issue(0);
        stage(0);
    }
    for (int64_t j = 0; j < ntile; ++j) {
        const int b = (int)(j % 3);
        lds_barrier();  // tile j staged by every thread, tile j + 1's keys published
        issue((b + 1) % 3);

        // ---- S and dP: keys x this wave's heads ----
        v4f sa = {0.f, 0.f, 0.f, 0.f}, ga = sa;
        {
            const _Float16* kb = sm.kt + l16 * Sm::KS + 8 * g4;
#pragma unroll
            for (int st = 0; st < D / 32; ++st) {
                const v8h kv = *(const v8h*)(kb + 32 * st);
                sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv, qf[st], sa, 0, 0, 0);
                ga = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv, gf[st], ga, 0, 0, 0);
            }
        }
        v4h hr, hp;  // lane: keys 4 g4 + i of head l16
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = sm.kscl[b][4 * g4 + i] >= 0.f;
            const float p = ok ? __expf(sm_scale * sa[i] - lse_h) : 0.f;
            const float ds = ok ? p * (ga[i] - dh) : 0.f;
            hr[i] = (_Float16)ds;
            hp[i] = (_Float16)p;
        }
        *(v4h*)(sm.dsr + (16 * wave + l16) * Sm::PS + 4 * g4) = hr;
        *(v4h*)(sm.pp + (16 * wave + l16) * Sm::PS + 4 * g4) = hp;

        // ---- dq[its heads x 512 dims] += ds K: the S layout is the A operand of 16x16x16 ----
        {
            const _Float16* vb = sm.kt + (4 * g4 + (l16 >> 2)) * Sm::KS + 4 * (l16 & 3);
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                const v4s kv = lds_read_tr16(vb + 16 * dt);  // keys 4 g4 + i at dim 16 dt + l16
                accq[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(hr, __builtin_bit_cast(v4h, kv), accq[dt], 0, 0, 0);
            }
        }
        lds_barrier();  // every head's ds and p

        // ---- de[keys x this wave's dims] = sum over heads of [ds | p] x [c q~ ; s_g g~] ----
        auto de_phase = [&](auto last_t) {
            constexpr bool last = decltype(last_t)::value;
            v8h a[NW];  // k step hb: 4 heads 16 hb + 4 g4 + i of ds, then of p, at key l16
#pragma unroll
            for (int hb = 0; hb < NW; ++hb) {
                const int off = (16 * hb + 4 * g4 + (l16 >> 2)) * Sm::PS + 4 * (l16 & 3);
                const v4s lo = lds_read_tr16(sm.dsr + off), hi = lds_read_tr16(sm.pp + off);
                const v8u16 c = {(uint16_t)lo[0], (uint16_t)lo[1], (uint16_t)lo[2], (uint16_t)lo[3],
                                 (uint16_t)hi[0], (uint16_t)hi[1], (uint16_t)hi[2], (uint16_t)hi[3]};
                a[hb] = __builtin_bit_cast(v8h, c);
            }
            // A masked key adds zero to the row of a valid key of the same lane (else row 0), so
            // every lane issues its atomics without sending many rows' zeros to one hot row; the
            // last tile (ragged; no wait follows it) skips them instead.
            unsigned long long* dst[4];
            float mul[4];
            unsigned long long* alt = dcomp;
#pragma unroll
            for (int i = 3; i >= 0; --i) {
                const int64_t code = sm.krow[b][4 * g4 + i];
                dst[i] = code == -1 ? nullptr : (code >= 0 ? dcomp + code * D : dwin + (-code - 2) * D);
                mul[i] = code == -1 ? 0.f : inv_sg;
                if (dst[i]) alt = dst[i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[i] = dst[i] ? dst[i] : alt;
#pragma unroll
            for (int dt = 0; dt < DTW; ++dt) {
                const int d0 = (D / NW) * wave + 16 * dt;
                v4f e = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int hb = 0; hb < NW; ++hb) {
                    const int off = (16 * hb + 4 * g4 + (l16 >> 2)) * Sm::QS + 4 * (l16 & 3) + d0;
                    const v4s lo = lds_read_tr16(sm.qs + off), hi = lds_read_tr16(sm.gs + off);
                    const v8u16 c = {(uint16_t)lo[0], (uint16_t)lo[1], (uint16_t)lo[2], (uint16_t)lo[3],
                                     (uint16_t)hi[0], (uint16_t)hi[1], (uint16_t)hi[2], (uint16_t)hi[3]};
                    e = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[hb], __builtin_bit_cast(v8h, c), e, 0, 0, 0);
                }
                if constexpr (!last) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) fx_add(dst[i] + d0 + l16, e[i] * mul[i]);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (mul[i] != 0.f) fx_add(dst[i] + d0 + l16, e[i] * mul[i]);
                }
            }
        };
        // the path into the next tile's staging runs straight from this tile's loads through its
        // atomics (the wait then leaves them in flight); the last tile needs no staging
        if (j + 1 < ntile) {
            de_phase(std::false_type{});
            stage((b + 1) % 3);  // tile j + 1 (every wave is past this tile's reads of kt)
            next_keys(j + 2);     // slot (j + 2) % 3 held tile j - 1, which every wave finished before this tile
        } else {
            de_phase(std::true_type{});
        }
    }

    // ---- dq = R(-tp) (c / s_g) acc: lane holds heads 16 wave + 4 g4 + i at dim 16 dt + l16 ----
    const float fq = sm_scale * inv_sg;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
        const int dim = 16 * dt + l16;
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = accq[dt][i] * fq;
        if (16 * dt >= DN) {  // RoPE dims: the pair's other dim is in lane l16 ^ 1
            const int pr = (dim - DN) >> 1;
            const float c = sm.cs[2 * pr], sn = sm.cs[2 * pr + 1];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float other = __shfl_xor(v[i], 1);
                v[i] = (l16 & 1) ? fmaf(-other, sn, v[i] * c) : fmaf(other, sn, v[i] * c);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) dq[(t * H + 16 * wave + 4 * g4 + i) * D + dim] = v[i];
    }
}

hipError_t launch_mqa_bwd(const uint16_t* q, const int32_t* seq, const int64_t* pos, int64_t T, int H,
                          const int32_t* idx, int k, int m, KvView comp, KvView win, int window, float sm_scale,
                          const RopeTab& rt, const float* out, const float* lse, const float* dout, float* dq,
                          float* dcomp, int64_t comp_rows, float* dwin, int64_t win_rows, void* ws, hipStream_t st) {
    if (T == 0) return hipSuccess;
    // entry gradients in 64-bit fixed point (order-independent sums), then added to dcomp / dwin
    constexpr int D = 512;
    unsigned long long* fc = (unsigned long long*)ws;
    unsigned long long* fw = fc + comp_rows * D;
    const int64_t nw = window > 0 ? win_rows * D : 0;
    hipError_t e = launch_fx_zero(fc, comp_rows * D, st);
    if (e == hipSuccess) e = launch_fx_zero(fw, nw, st);
    if (e != hipSuccess) return e;
#define CSA_BWD(NW)                                                                                                    \
    hipLaunchKernelGGL(k_mqa_bwd<NW>, dim3((unsigned)T), dim3(64 * (NW)), 0, st, q, seq, pos, idx, k, m, comp, win,  \
                       window, sm_scale, rt, out, lse, dout, dq, fc, fw)
    if (H == 64) CSA_BWD(4);
    else if (H == 32) CSA_BWD(2);
    else CSA_BWD(1);
#undef CSA_BWD
    e = hipGetLastError();
    if (e == hipSuccess) e = launch_fx_flush(fc, dcomp, comp_rows * D, st);
    if (e == hipSuccess && nw > 0) e = launch_fx_flush(fw, dwin, nw, st);
    return e;
}

}  // namespace csa
