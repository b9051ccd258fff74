// csa_sparse_mqa / hca_dense_mqa kernels: multi-query attention over a key
// list (selected or all visible compressed entries, then the window tokens),
// one shared KV head, every entry both key and value.
//
// Grid: one workgroup per (row, split); a split is a contiguous range of the
// row's key list.  Per tile of 32 keys the workgroup
//   1. gathers the entries into LDS twice: a row-major bf16 copy (FP8 codes
//      and bf16 RoPE dims, both exact in bf16) for QK, and a transposed fp16
//      copy scaled by scale_j / S (S = largest scale in the split) for PV;
//   2. QK^T with bf16 MFMA 16x16x32: rows = keys, columns = heads; the query
//      (RoPE applied at t in fp32) lives in registers; its 64 RoPE dims are
//      split hi + lo in bf16 so they keep ~16 bits; the FP8 part's scale is
//      applied per key to the fp32 accumulator;
//   3. online softmax in fp32 per head (running max / sum);
//   4. P V with fp16 MFMA 16x16x32 into fp32 accumulators (dims x heads).
// A single split writes the normalised output (with the inverse RoPE on the
// last 64 dims); several splits write unnormalised partials plus (max, sum),
// merged by k_mqa_combine in a fixed order (log-sum-exp merge).
#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {

constexpr int KT = 32;  // keys per tile

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
    _Float16 p[H * PS];
    float alpha[H];
    float mrun[H];
    float lrun[H];
    int64_t row[KT];
    float scl[KT];
    int valid[KT];
    float red[8];
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

// Resolve key-list position u of row t to a cache row (-1 when masked) and its scale.
__device__ __forceinline__ int64_t resolve(int64_t u, int64_t t, int32_t sq, const RowKeys& rk, const int32_t* idx,
                                           int k, const KvView& comp, const KvView& win, bool& is_win) {
    if (u < rk.n_c) {
        is_win = false;
        int64_t j = idx ? (int64_t)idx[t * k + u] : u;
        if (j < 0 || j >= rk.nv) return -1;
        return (int64_t)sq * comp.cap + (j % comp.cap);
    }
    is_win = true;
    const int64_t p = rk.lo + (u - rk.n_c);
    return (int64_t)sq * win.cap + (p % win.cap);
}

template <int H, int D>
__global__ __launch_bounds__(256) void k_mqa(const uint16_t* __restrict__ q, const int32_t* __restrict__ seq,
                                             const int64_t* __restrict__ pos, const int32_t* __restrict__ idx, int k,
                                             int m, KvView comp, KvView win, int window, float sm_scale, double base,
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

    __shared__ Sm sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int64_t t = blockIdx.x / S;
    const int s = blockIdx.x % S;
    const int64_t tp = pos[t];
    const int32_t sq = seq[t];
    const RowKeys rk = row_keys(tp, idx, k, m, window);
    const int64_t u0 = rk.n * s / S, u1 = rk.n * (s + 1) / S;

    // ---- split-wide scale reference: largest entry scale of the split ----
    float smax = 0.f;
    for (int64_t u = u0 + tid; u < u1; u += 256) {
        bool w;
        int64_t r = resolve(u, t, sq, rk, idx, k, comp, win, w);
        if (r >= 0) smax = fmaxf(smax, w ? win.scale[r] : comp.scale[r]);
    }
    smax = wave_max(smax);
    if (lane == 0) sm.red[wave] = smax;
    __syncthreads();
    float sref = fmaxf(fmaxf(sm.red[0], sm.red[1]), fmaxf(sm.red[2], sm.red[3]));
    if (!(sref > 0.f)) sref = 1.f;
    const float inv_sref = 1.f / sref;

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
                    float cs, sn;
                    rope_cs((double)tp, base, (d0 - DN + e) >> 1, cs, sn);
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

    v4f acc[DT][HT];
#pragma unroll
    for (int a = 0; a < DT; ++a)
#pragma unroll
        for (int b = 0; b < HT; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int64_t ut = u0; ut < u1; ut += KT) {
        // ---- resolve the tile's keys ----
        if (tid < KT) {
            const int64_t u = ut + tid;
            int64_t r = -1;
            bool w = false;
            if (u < u1) r = resolve(u, t, sq, rk, idx, k, comp, win, w);
            sm.row[tid] = r >= 0 ? (w ? -(r + 2) : r) : -1;  // window rows encoded as -(r+2)
            sm.valid[tid] = r >= 0;
            sm.scl[tid] = r >= 0 ? (w ? win.scale[r] : comp.scale[r]) : 0.f;
        }
        __syncthreads();
        // ---- gather into LDS ----
        for (int c = tid; c < KT * CPK; c += 256) {
            const int key = c / CPK, part = c % CPK;
            const int64_t code = sm.row[key];
            const bool w = code <= -2;
            const int64_t r = w ? -code - 2 : code;
            const uint8_t* nope = w ? win.nope : comp.nope;
            const uint16_t* rope = w ? win.rope : comp.rope;
            __bf16* kr = sm.kr + key * Sm::KR;
            if (part < DN / 16) {
                v4i raw = {0, 0, 0, 0};
                if (code != -1) raw = *(const v4i*)(nope + r * DN + part * 16);
                const float fs = sm.scl[key] * inv_sref;
                v8bf b0, b1;
#pragma unroll
                for (int wd = 0; wd < 4; ++wd) {
                    v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8(raw[wd], false);
                    v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8(raw[wd], true);
                    float f[4] = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int dd = part * 16 + wd * 4 + e;
                        if (wd < 2) b0[wd * 4 + e] = (__bf16)f[e];
                        else b1[(wd - 2) * 4 + e] = (__bf16)f[e];
                        sm.vt[dd * Sm::VT + key] = (_Float16)(f[e] * fs);
                    }
                }
                *(v8bf*)(kr + part * 16) = b0;
                *(v8bf*)(kr + part * 16 + 8) = b1;
            } else {
                const int rp = part - DN / 16;  // 8 rope dims per chunk
                v4i raw = {0, 0, 0, 0};
                if (code != -1) raw = *(const v4i*)(rope + r * 64 + rp * 8);
                *(v4i*)(kr + DN + rp * 8) = raw;
                const uint16_t* hv = (const uint16_t*)&raw;
#pragma unroll
                for (int e = 0; e < 8; ++e) sm.vt[(DN + rp * 8 + e) * Sm::VT + key] = (_Float16)bf16_bits_to_f32(hv[e]);
            }
        }
        __syncthreads();
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
                    const float sc = sm_scale * fmaf(sm.scl[key], an[i], ar[i]);
                    sm.s[key * Sm::SS + hb * 16 + l16] = sm.valid[key] ? sc : -INFINITY;
                }
            }
        }
        __syncthreads();
        // ---- online softmax: TPH threads per head, KPT keys each ----
        {
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
                const float p = m_new == -INFINITY ? 0.f : __expf(sv[i] - m_new);
                sum += p;
                sm.p[sh * Sm::PS + sk * KPT + i] = (_Float16)p;
            }
#pragma unroll
            for (int o = 1; o < TPH; o <<= 1) sum += __shfl_xor(sum, o);
            const float alpha = m_new == -INFINITY ? 1.f : __expf(m_run - m_new);
            l_run = l_run * alpha + sum;
            m_run = m_new;
            if (sk == 0) sm.alpha[sh] = alpha;
        }
        __syncthreads();
        // ---- O^T += V^T P^T over this wave's dims ----
        {
            float al[HT];
#pragma unroll
            for (int b = 0; b < HT; ++b) al[b] = sm.alpha[b * 16 + l16];
            v8h pf[HT];
#pragma unroll
            for (int b = 0; b < HT; ++b) pf[b] = *(const v8h*)(sm.p + (b * 16 + l16) * Sm::PS + 8 * g4);
#pragma unroll
            for (int a = 0; a < DT; ++a) {
                const int dim = wave * DW + a * 16 + l16;
                const v8h vf = *(const v8h*)(sm.vt + dim * Sm::VT + 8 * g4);
#pragma unroll
                for (int b = 0; b < HT; ++b) {
                    acc[a][b] *= al[b];
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[b], acc[a][b], 0, 0, 0);
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
    __syncthreads();
    // lane holds dims wave*DW + a*16 + 4*g4 + i for head b*16 + l16
#pragma unroll
    for (int b = 0; b < HT; ++b) {
        const int h = b * 16 + l16;
        const float mh = sm.mrun[h], lh = sm.lrun[h];
#pragma unroll
        for (int a = 0; a < DT; ++a) {
            const int d0 = wave * DW + a * 16 + 4 * g4;
            float o[4];
            const float f = d0 < DN ? sref : 1.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = acc[a][b][i] * f;
            if (S == 1) {
                const float inv = lh > 0.f ? 1.f / lh : 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] *= inv;
                if (d0 >= DN) {
#pragma unroll
                    for (int i = 0; i < 4; i += 2) {
                        float cs, sn;
                        rope_cs(-(double)tp, base, (d0 - DN + i) >> 1, cs, sn);
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

// merge S split partials of one (row, head): fixed order s = 0 .. S-1
template <int D>
__global__ __launch_bounds__(128) void k_mqa_combine(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                                                     const int64_t* __restrict__ pos, int H, int S, double base,
                                                     float* __restrict__ out, float* __restrict__ lse) {
    constexpr int DN = D - 64;
    const int64_t th = blockIdx.x;  // t*H + h
    const int64_t t = th / H;
    const int h = (int)(th % H);
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, part_ml[((t * S + s) * H + h) * 2]);
    float L = 0.f;
    for (int s = 0; s < S; ++s) {
        const float ms = part_ml[((t * S + s) * H + h) * 2], ls = part_ml[((t * S + s) * H + h) * 2 + 1];
        L += ms == -INFINITY ? 0.f : ls * __expf(ms - M);
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    for (int d0 = threadIdx.x * 4; d0 < D; d0 += 128 * 4) {
        float o[4] = {0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < S; ++s) {
            const float ms = part_ml[((t * S + s) * H + h) * 2];
            if (ms == -INFINITY) continue;
            const float wgt = __expf(ms - M) * inv;
            const float4 v = *(const float4*)(part_o + ((t * S + s) * H + h) * (int64_t)D + d0);
            o[0] = fmaf(wgt, v.x, o[0]);
            o[1] = fmaf(wgt, v.y, o[1]);
            o[2] = fmaf(wgt, v.z, o[2]);
            o[3] = fmaf(wgt, v.w, o[3]);
        }
        if (d0 >= DN) {
            const double tp = (double)pos[t];
            for (int i = 0; i < 4; i += 2) {
                float cs, sn;
                rope_cs(-tp, base, (d0 - DN + i) >> 1, cs, sn);
                const float x0 = o[i], x1 = o[i + 1];
                o[i] = x0 * cs - x1 * sn;
                o[i + 1] = x0 * sn + x1 * cs;
            }
        }
        *(float4*)(out + th * D + d0) = make_float4(o[0], o[1], o[2], o[3]);
    }
    if (threadIdx.x == 0) lse[th] = L > 0.f ? M + __logf(L) : -INFINITY;
}

static int choose_splits(int64_t T, int64_t max_keys) {
    int64_t s = (512 + T - 1) / T;
    int64_t by_keys = (max_keys + 63) / 64;
    if (s > by_keys) s = by_keys;
    if (s > 64) s = 64;
    if (s < 1) s = 1;
    return (int)s;
}

size_t mqa_workspace_bytes(int64_t T, int H, int d, int64_t max_keys) {
    const int S = choose_splits(T, max_keys);
    if (S == 1) return 0;
    return (size_t)T * S * H * ((size_t)d + 2) * sizeof(float) + 256;
}

template <int H, int D>
static void launch_mqa_t(const uint16_t* q, const int32_t* seq, const int64_t* pos, int64_t T, const int32_t* idx,
                         int k, int m, KvView comp, KvView win, int window, float sm_scale, double base, int S,
                         float* out, float* lse, float* po, float* pml, hipStream_t st) {
    hipLaunchKernelGGL((k_mqa<H, D>), dim3((unsigned)(T * S)), dim3(256), 0, st, q, seq, pos, idx, k, m, comp, win,
                       window, sm_scale, base, S, out, lse, po, pml);
    if (S > 1)
        hipLaunchKernelGGL((k_mqa_combine<D>), dim3((unsigned)(T * H)), dim3(128), 0, st, po, pml, pos, H, S, base, out,
                           lse);
}

hipError_t launch_mqa(const uint16_t* q, const int32_t* seq, const int64_t* pos, int64_t T, int H, int d,
                      const int32_t* idx, int k, int m, int64_t max_keys, KvView comp, KvView win, int window,
                      float sm_scale, double base, float* out, float* lse, void* ws, hipStream_t st) {
    if (T == 0) return hipSuccess;
    const int S = choose_splits(T, max_keys);
    float* po = nullptr;
    float* pml = nullptr;
    if (S > 1) {
        po = (float*)ws;
        pml = po + (size_t)T * S * H * d;
    }
#define CSA_MQA(HH, DD) launch_mqa_t<HH, DD>(q, seq, pos, T, idx, k, m, comp, win, window, sm_scale, base, S, out, lse, po, pml, st)
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

}  // namespace csa
