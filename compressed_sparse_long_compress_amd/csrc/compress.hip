// csa_compress kernel: weighted merge of m-token blocks into mixed-precision
// entries.  One wave per entry; every lane owns D/64 consecutive dims, so a
// token row is read as one coalesced 64-lane load (16 B per lane at D = 512).
//
// The merge, RoPE and scale run in fp64 and the FP8 / bf16 roundings are
// taken from the fp64 values (round-to-odd into fp32, then the hardware
// nearest-even conversion).  With bf16 tokens, value / (amax/448) lands on
// an E4M3 rounding midpoint up to the last fp32 bit surprisingly often, so
// an fp32 quotient would round those ties the wrong way.  The kernel is
// bound by HBM traffic, so the fp64 arithmetic costs nothing measurable.
#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {

constexpr int kMaxM = 1024;

// fp64 -> fp32 rounding to odd: a later round-to-nearest-even to any format
// with at most 22 significant bits then equals rounding the fp64 value
// directly (no double-rounding ties).
__device__ __forceinline__ float f64_to_f32_odd(double d) {
    float f = (float)d;
    if ((double)f != d && f != 0.f) {
        uint32_t b = __float_as_uint(f);
        if ((b & 1u) == 0) b += fabs((double)f) < fabs(d) ? 1 : -1;
        f = __uint_as_float(b);
    }
    return f;
}

// UN: token rows in flight per lane (8, or 32 for long blocks, whose merge would otherwise
// wait on one memory round trip per 8 tokens).  Short blocks (m < 32) keep a small weight
// buffer, so that LDS does not cap the waves per CU on the streaming shapes (m = 1, 4).
template <int D, int UN>
__global__ __launch_bounds__(256) void k_compress(const uint16_t* __restrict__ kv, const float* __restrict__ logits,
                                                  int64_t tok0, int64_t n_blk, int m, RopeTab rt, int64_t seq,
                                                  int64_t cap, const int32_t* __restrict__ pages, int pshift,
                                                  uint8_t* __restrict__ nope, uint16_t* __restrict__ rope,
                                                  float* __restrict__ scale) {
    constexpr int DN = D - 64;
    constexpr int PER = D / 64;  // dims per lane (2 or 8)
    constexpr int MAXM = UN >= 32 ? kMaxM : 32;
    __shared__ double wbuf[4][MAXM];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t b = (int64_t)blockIdx.x * 4 + wv;
    if (b >= n_blk) return;
    const float* lg = logits + b * m;
    const uint16_t* x = kv + b * m * (int64_t)D + lane * PER;
    double* wb = wbuf[wv];

    // token rows i0 .. i0+UN-1 of the block into v (rows past the block's end load its last
    // row, unused: no branch, so the loads stay in flight across what follows)
    auto load_rows = [&](int i0, uint16_t (&v)[UN][PER]) {
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int64_t i = i0 + u < m ? i0 + u : m - 1;
            if constexpr (PER == 8) {
                *(v4i*)v[u] = *(const v4i*)(x + i * D);
            } else {
                uint32_t raw = *(const uint32_t*)(x + i * D);
                v[u][0] = (uint16_t)raw;
                v[u][1] = (uint16_t)(raw >> 16);
            }
        }
    };
    // the lane's first logit, then the first token rows, are requested before the weights are
    // computed, so the two memory round trips overlap (loads return in order: the logit first)
    const float lg0 = lg[lane < m ? lane : m - 1];
    uint16_t v[UN][PER];
    load_rows(0, v);

    // block softmax weights in fp64: exp terms by lanes, their sum in token order
    double mx = lane < m ? (double)lg0 : -INFINITY;  // (a maximum: any order gives the same value)
    if constexpr (UN >= 32)  // m < 32 otherwise
        for (int i = lane + 64; i < m; i += 64) mx = fmax(mx, (double)lg[i]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o));
    if (lane < m) wb[lane] = exp((double)lg0 - mx);
    if constexpr (UN >= 32)
        for (int i = lane + 64; i < m; i += 64) wb[i] = exp((double)lg[i] - mx);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    double z = 0.0;
    for (int i = 0; i < m; ++i) z = __dadd_rn(z, wb[i]);
    // the normalised weights, each divided once (by the lane that owns it) instead of per lane
    __builtin_amdgcn_wave_barrier();
    for (int i = lane; i < m; i += 64) wb[i] = wb[i] / z;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

    // weighted merge in fp64, tokens in order, no fused multiply-add
    double c[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) c[e] = 0.0;
    for (int i0 = 0; i0 < m; i0 += UN) {
        if (i0 > 0) load_rows(i0, v);
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            if (i0 + u < m) {
                const double wi = wb[i0 + u];
#pragma unroll
                for (int e = 0; e < PER; ++e)
                    c[e] = __dadd_rn(c[e], __dmul_rn(wi, (double)bf16_bits_to_f32(v[u][e])));
            }
        }
    }

    const int64_t J = tok0 / m + b;
    const int dim0 = lane * PER;
    const bool is_rope = dim0 >= DN;

    // RoPE on the last 64 dims at the last covered token, fp64.  Lane i < 32 evaluates the
    // cosine and sine of frequency pair i (one fp64 sin / cos per lane, in parallel); the
    // lanes holding the RoPE dims take theirs by shuffles.
    {
        const double p = (double)((J + 1) * (int64_t)m - 1);
        double cs_i = 1.0, sn_i = 0.0;
        if (lane < 32) sincos(__dmul_rn(p, rt.theta[lane]), &sn_i, &cs_i);  // one shared range reduction
#pragma unroll
        for (int e = 0; e < PER; e += 2) {
            const int pair = is_rope ? (dim0 - DN + e) >> 1 : 0;
            const double cs = __shfl(cs_i, pair), sn = __shfl(sn_i, pair);
            if (is_rope) {
                const double x0 = c[e], x1 = c[e + 1];
                c[e] = __dsub_rn(__dmul_rn(x0, cs), __dmul_rn(x1, sn));
                c[e + 1] = __dadd_rn(__dmul_rn(x0, sn), __dmul_rn(x1, cs));
            }
        }
    }

    // per-entry FP8 scale over the non-RoPE dims
    double am = 0.0;
    if (!is_rope) {
#pragma unroll
        for (int e = 0; e < PER; ++e) am = fmax(am, fabs(c[e]));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) am = fmax(am, __shfl_xor(am, o));
    const float s = am > 0.0 ? (float)(am / 448.0) : 1.0f;

    const int64_t row = kv_row(pages, pshift, cap, seq, J % cap);
    if (is_rope) {
        uint16_t r[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) r[e] = f32_to_bf16_bits(f64_to_f32_odd(c[e]));
        uint16_t* dst = rope + row * 64 + (dim0 - DN);
        if constexpr (PER == 8) *(v4i*)dst = *(const v4i*)r;
        else *(uint32_t*)dst = (uint32_t)r[0] | ((uint32_t)r[1] << 16);
    } else {
        uint16_t half[PER / 2];
#pragma unroll
        for (int e = 0; e < PER; e += 2) {
            float a0 = fminf(fmaxf(f64_to_f32_odd(c[e] / (double)s), -448.f), 448.f);
            float a1 = fminf(fmaxf(f64_to_f32_odd(c[e + 1] / (double)s), -448.f), 448.f);
            half[e / 2] = (uint16_t)__builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
        }
        uint8_t* dst = nope + row * DN + dim0;
        if constexpr (PER == 8) {
            *(uint2*)dst = make_uint2((uint32_t)half[0] | ((uint32_t)half[1] << 16),
                                      (uint32_t)half[2] | ((uint32_t)half[3] << 16));
        } else {
            *(uint16_t*)dst = half[0];
        }
    }
    if (lane == 0) scale[row] = s;
}

// ---------------------------------------------------------------------------
// Per-channel weights: channel e of block b merges its m tokens with weights
// softmax over logits[bm+i][e].  Same layout, RoPE and storage as
// k_compress; per dim three passes over the block's logits (max, the sum of
// exponentials in token order, the weighted merge), all in fp64.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_compress_ch(const uint16_t* __restrict__ kv, const float* __restrict__ logits,
                                                     int64_t tok0, int64_t n_blk, int m, RopeTab rt, int64_t seq,
                                                     int64_t cap, const int32_t* __restrict__ pages, int pshift,
                                                     uint8_t* __restrict__ nope, uint16_t* __restrict__ rope,
                                                     float* __restrict__ scale) {
    constexpr int DN = D - 64;
    constexpr int PER = D / 64;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t b = (int64_t)blockIdx.x * 4 + wv;
    if (b >= n_blk) return;
    const int dim0 = lane * PER;
    const float* lg = logits + b * m * (int64_t)D + dim0;
    const uint16_t* x = kv + b * m * (int64_t)D + dim0;

    double mx[PER], z[PER], c[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        mx[e] = -INFINITY;
        z[e] = 0.0;
        c[e] = 0.0;
    }
    for (int i = 0; i < m; ++i)
#pragma unroll
        for (int e = 0; e < PER; ++e) mx[e] = fmax(mx[e], (double)lg[(int64_t)i * D + e]);
    for (int i = 0; i < m; ++i)
#pragma unroll
        for (int e = 0; e < PER; ++e) z[e] = __dadd_rn(z[e], exp((double)lg[(int64_t)i * D + e] - mx[e]));
    for (int i = 0; i < m; ++i) {
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const double wi = exp((double)lg[(int64_t)i * D + e] - mx[e]) / z[e];
            c[e] = __dadd_rn(c[e], __dmul_rn(wi, (double)bf16_bits_to_f32(x[(int64_t)i * D + e])));
        }
    }

    const int64_t J = tok0 / m + b;
    const bool is_rope = dim0 >= DN;
    {
        // one frequency pair's fp64 sincos per lane below 32; the RoPE lanes take theirs by shuffles
        const double p = (double)((J + 1) * (int64_t)m - 1);
        double cs_i = 1.0, sn_i = 0.0;
        if (lane < 32) sincos(__dmul_rn(p, rt.theta[lane]), &sn_i, &cs_i);
#pragma unroll
        for (int e = 0; e < PER; e += 2) {
            const int pair = is_rope ? (dim0 - DN + e) >> 1 : 0;
            const double cs = __shfl(cs_i, pair), sn = __shfl(sn_i, pair);
            if (is_rope) {
                const double x0 = c[e], x1 = c[e + 1];
                c[e] = __dsub_rn(__dmul_rn(x0, cs), __dmul_rn(x1, sn));
                c[e + 1] = __dadd_rn(__dmul_rn(x0, sn), __dmul_rn(x1, cs));
            }
        }
    }
    double am = 0.0;
    if (!is_rope) {
#pragma unroll
        for (int e = 0; e < PER; ++e) am = fmax(am, fabs(c[e]));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) am = fmax(am, __shfl_xor(am, o));
    const float s = am > 0.0 ? (float)(am / 448.0) : 1.0f;
    const int64_t row = kv_row(pages, pshift, cap, seq, J % cap);
    if (is_rope) {
#pragma unroll
        for (int e = 0; e < PER; ++e) rope[row * 64 + (dim0 - DN) + e] = f32_to_bf16_bits(f64_to_f32_odd(c[e]));
    } else {
#pragma unroll
        for (int e = 0; e < PER; e += 2) {
            const float a0 = fminf(fmaxf(f64_to_f32_odd(c[e] / (double)s), -448.f), 448.f);
            const float a1 = fminf(fmaxf(f64_to_f32_odd(c[e + 1] / (double)s), -448.f), 448.f);
            *(uint16_t*)(nope + row * DN + dim0 + e) = (uint16_t)__builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
        }
    }
    if (lane == 0) scale[row] = s;
}

// ---------------------------------------------------------------------------
// Index keys: the softmax-weighted merge of every m raw key tokens (fp64, no
// RoPE), then MXFP4: per 32 elements the E8M0 scale 2^(floor(log2 amax) - 2)
// and E2M1 codes of value / scale, nearest with ties to the even mantissa,
// saturating at 6, zero stored as +0.  One wave per entry, lane l holds
// elements 2l, 2l+1 (its packed byte); a block is 16 lanes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e2m1_code(double v) {
    // magnitude code = midpoints of the E2M1 grid (0 .5 1 1.5 2 3 4 6) passed by |v|;
    // at a midpoint itself, toward the even code
    const double a = fabs(v);
    uint32_t c = 0;
    c += a > 0.25;
    c += a >= 0.75;
    c += a > 1.25;
    c += a >= 1.75;
    c += a > 2.5;
    c += a >= 3.5;
    c += a > 5.0;
    return (v < 0.0 && c != 0 ? 8u : 0u) | c;
}

template <int DI>
__global__ __launch_bounds__(256) void k_compress_ikey(const uint16_t* __restrict__ k, const float* __restrict__ logits,
                                                       int64_t tok0, int64_t n_blk, int m, int64_t seq, int64_t cap,
                                                       const int32_t* __restrict__ pages, int pshift,
                                                       uint8_t* __restrict__ data, uint8_t* __restrict__ kscale) {
    static_assert(DI == 64 || DI == 128, "two elements per lane");
    __shared__ double wbuf[4][kMaxM];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t b = (int64_t)blockIdx.x * 4 + wv;
    if (b >= n_blk) return;
    const float* lg = logits + b * m;
    double* wb = wbuf[wv];
    double mx = -INFINITY;  // (a maximum: any order gives the same value)
    for (int i = lane; i < m; i += 64) mx = fmax(mx, (double)lg[i]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o));
    for (int i = lane; i < m; i += 64) wb[i] = exp((double)lg[i] - mx);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    double z = 0.0;
    for (int i = 0; i < m; ++i) z = __dadd_rn(z, wb[i]);
    // the normalised weights, each divided once (by the lane that owns it)
    __builtin_amdgcn_wave_barrier();
    for (int i = lane; i < m; i += 64) wb[i] = wb[i] / z;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

    const bool live = 2 * lane < DI;
    double c0 = 0.0, c1 = 0.0;
    if (live) {
        const uint16_t* x = k + b * m * (int64_t)DI + 2 * lane;
        for (int i = 0; i < m; ++i) {
            const uint32_t raw = *(const uint32_t*)(x + (int64_t)i * DI);
            const double wi = wb[i];
            c0 = __dadd_rn(c0, __dmul_rn(wi, (double)bf16_bits_to_f32((uint16_t)raw)));
            c1 = __dadd_rn(c1, __dmul_rn(wi, (double)bf16_bits_to_f32((uint16_t)(raw >> 16))));
        }
    }
    // block amax over its 16 lanes
    double am = fmax(fabs(c0), fabs(c1));
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) am = fmax(am, __shfl_xor(am, o));
    int sb = 127;
    if (am > 0.0) {
        int ex;
        frexp(am, &ex);  // am in [2^(ex-1), 2^ex)
        sb = ex - 1 - 2 + 127;
        sb = sb < 0 ? 0 : (sb > 254 ? 254 : sb);
    }
    const double inv = ldexp(1.0, 127 - sb);  // exact power of two
    const int64_t row = kv_row(pages, pshift, cap, seq, (tok0 / m + b) % cap);
    if (live) {
        const uint32_t lo = am > 0.0 ? e2m1_code(c0 * inv) : 0u, hi = am > 0.0 ? e2m1_code(c1 * inv) : 0u;
        data[row * (DI / 2) + lane] = (uint8_t)(lo | (hi << 4));
        if ((lane & 15) == 0) kscale[row * (DI / 32) + (lane >> 4)] = (uint8_t)sb;
    }
}

hipError_t launch_compress_channel(const uint16_t* kv, const float* logits, int64_t tok0, int64_t n_tok, int m, int d,
                                   const RopeTab& rt, int64_t seq, const KvView& out, uint8_t* nope, uint16_t* rope,
                                   float* scale, hipStream_t st) {
    const int64_t n_blk = n_tok / m;
    if (n_blk == 0) return hipSuccess;
    dim3 grid((unsigned)((n_blk + 3) / 4)), block(256);
    if (d == 512)
        hipLaunchKernelGGL(k_compress_ch<512>, grid, block, 0, st, kv, logits, tok0, n_blk, m, rt, seq, out.cap, out.pages, out.pshift, nope,
                           rope, scale);
    else
        hipLaunchKernelGGL(k_compress_ch<128>, grid, block, 0, st, kv, logits, tok0, n_blk, m, rt, seq, out.cap, out.pages, out.pshift, nope,
                           rope, scale);
    return hipGetLastError();
}

hipError_t launch_compress_index_keys(const uint16_t* k, const float* logits, int64_t tok0, int64_t n_tok, int m,
                                      int d_i, int64_t seq, int64_t cap, const int32_t* pages, int pshift,
                                      uint8_t* data, uint8_t* kscale,
                                      hipStream_t st) {
    const int64_t n_blk = n_tok / m;
    if (n_blk == 0) return hipSuccess;
    dim3 grid((unsigned)((n_blk + 3) / 4)), block(256);
    if (d_i == 128)
        hipLaunchKernelGGL(k_compress_ikey<128>, grid, block, 0, st, k, logits, tok0, n_blk, m, seq, cap, pages, pshift, data,
                           kscale);
    else
        hipLaunchKernelGGL(k_compress_ikey<64>, grid, block, 0, st, k, logits, tok0, n_blk, m, seq, cap, pages, pshift, data,
                           kscale);
    return hipGetLastError();
}

hipError_t launch_compress(const uint16_t* kv, const float* logits, int64_t tok0, int64_t n_tok, int m, int d,
                           const RopeTab& rt, int64_t seq, const KvView& out, uint8_t* nope, uint16_t* rope,
                           float* scale, hipStream_t st) {
    const int64_t n_blk = n_tok / m;
    if (n_blk == 0) return hipSuccess;
    dim3 grid((unsigned)((n_blk + 3) / 4)), block(256);
#define CSA_COMPRESS(D, UN)                                                                                         \
    hipLaunchKernelGGL((k_compress<D, UN>), grid, block, 0, st, kv, logits, tok0, n_blk, m, rt, seq, out.cap, out.pages, \
                       out.pshift, nope, rope, scale)
    if (d == 512) {
        if (m >= 32) CSA_COMPRESS(512, 32);
        else CSA_COMPRESS(512, 8);
    } else {
        if (m >= 32) CSA_COMPRESS(128, 32);
        else CSA_COMPRESS(128, 8);
    }
#undef CSA_COMPRESS
    return hipGetLastError();
}

}  // namespace csa
