// csa_index_bwd: gradient of the lightning-indexer scores (training side: the
// pages warm the indexer up and train its QK path in FP4, [xmsumi] § 预训练 and
// [hortopato]'s training section; the gradient itself is the plain derivative
// of score = sum_h w_h ReLU(<q_h, k_j>) over MXFP4-dequantised vectors).
//
// One workgroup per query row, its selected columns in chunks held in LDS:
//   A  per selected column: the head dot products (exact in fp32: E2M1 x E2M1
//      products are multiples of 1/4), coef_h = G w_h [dot_h > 0] and the
//      row's dw partials (thread-local, summed in a fixed order at the end);
//   B  dq[h][c] = sum over the chunk's columns, in column order, of
//      coef_h k_j[c]: every (head, element) owned by one thread;
//   C  dk_j[c] += sum_h coef_h q_h[c] into the 64-bit fixed-point buffer
//      (rows share keys; the sum does not depend on their order).
// Fixed-point buffers are cleared and flushed by the kernels at the end of
// this file (shared with the attention backward).
#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {

constexpr int kIbThreads = 256;
constexpr int kIbChunk = 1024;  // selected columns per chunk

__device__ __forceinline__ float e2m1_value(uint32_t nib) {
    const float mag[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};
    const float v = mag[nib & 7];
    return (nib & 8) ? -v : v;
}

// element c of MXFP4 row r
template <int DI>
__device__ __forceinline__ float mx_elem(const uint8_t* data, const uint8_t* scl, int64_t r, int c) {
    const uint8_t byte = data[r * (DI / 2) + c / 2];
    return ldexpf(e2m1_value((c & 1) ? (byte >> 4) : (byte & 15)), (int)scl[r * (DI / 32) + c / 32] - 127);
}

template <int DI>
__global__ __launch_bounds__(kIbThreads) void k_index_bwd(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ q_scale, const float* __restrict__ w,
    const int32_t* __restrict__ seq, const int64_t* __restrict__ pos, int h_i, const uint8_t* __restrict__ kdata,
    const uint8_t* __restrict__ kscale, int64_t kcap, const int32_t* __restrict__ kpages, int kpshift, int m,
    const int32_t* __restrict__ idx,
    const float* __restrict__ gsel, int n_sel, float* __restrict__ dq, float* __restrict__ dw,
    unsigned long long* __restrict__ dk_fx) {
    constexpr int NT = kIbThreads;
    constexpr int TPC = NT / DI;       // threads per element index
    constexpr int HPT = 8 / TPC;       // heads per thread in B (h_i <= 8)
    __shared__ float qs[8][DI];
    __shared__ float wsh[8];
    __shared__ float coef[8][kIbChunk];
    __shared__ int64_t jrow[kIbChunk];
    __shared__ float red[8][NT];
    const int tid = threadIdx.x;
    const int64_t t = blockIdx.x;
    const int64_t nv = (pos[t] + 1) / m;
    const int32_t sq = seq[t];
    for (int e = tid; e < 8 * DI; e += NT) {
        const int h = e / DI, c = e % DI;
        qs[h][c] = h < h_i ? mx_elem<DI>(q, q_scale, t * h_i + h, c) : 0.f;
    }
    if (tid < 8) wsh[tid] = tid < h_i ? w[t * h_i + tid] : 0.f;
    __syncthreads();

    const int cb = tid % DI, h0 = tid / DI;  // B: element cb, heads h0 + TPC i
    float acc[HPT];
#pragma unroll
    for (int i = 0; i < HPT; ++i) acc[i] = 0.f;
    float dwl[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

    for (int a0 = 0; a0 < n_sel; a0 += kIbChunk) {
        const int n = n_sel - a0 < kIbChunk ? n_sel - a0 : kIbChunk;
        // ---- A: dot products, coefficients, dw partials ----
        for (int a = tid; a < n; a += NT) {
            const int64_t j = idx[t * (int64_t)n_sel + a0 + a];
            if (j < 0 || j >= nv) {
                jrow[a] = -1;
#pragma unroll
                for (int h = 0; h < 8; ++h) coef[h][a] = 0.f;
                continue;
            }
            const int64_t r = kv_row(kpages, kpshift, kcap, sq, j);
            const float gv = gsel[t * (int64_t)n_sel + a0 + a];
            float dot[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (int c = 0; c < DI; ++c) {
                const float kv = mx_elem<DI>(kdata, kscale, r, c);
#pragma unroll
                for (int h = 0; h < 8; ++h) dot[h] = fmaf(qs[h][c], kv, dot[h]);
            }
#pragma unroll
            for (int h = 0; h < 8; ++h) {
                const bool on = h < h_i && dot[h] > 0.f;
                coef[h][a] = on ? gv * wsh[h] : 0.f;
                dwl[h] += on ? gv * dot[h] : 0.f;
            }
            jrow[a] = r;
        }
        __syncthreads();
        // ---- B: dq, columns of the chunk in order ----
        for (int a = 0; a < n; ++a) {
            const int64_t r = jrow[a];
            if (r < 0) continue;
            const float kv = mx_elem<DI>(kdata, kscale, r, cb);
#pragma unroll
            for (int i = 0; i < HPT; ++i) acc[i] = fmaf(coef[h0 + TPC * i][a], kv, acc[i]);
        }
        // ---- C: key gradients (consecutive threads: consecutive elements of one key) ----
        for (int a = tid / DI; a < n; a += TPC) {
            const int64_t r = jrow[a];
            if (r < 0) continue;
            float v = 0.f;
#pragma unroll
            for (int h = 0; h < 8; ++h) v = fmaf(coef[h][a], qs[h][cb], v);
            fx_add(dk_fx + r * DI + cb, v);
        }
        __syncthreads();  // the chunk's coef / jrow are read before the next chunk writes them
    }
#pragma unroll
    for (int i = 0; i < HPT; ++i) {
        const int h = h0 + TPC * i;
        if (h < h_i) dq[(t * h_i + h) * (int64_t)DI + cb] = acc[i];
    }
    // dw: each thread's partials, summed over the threads in thread order
#pragma unroll
    for (int h = 0; h < 8; ++h) red[h][tid] = dwl[h];
    __syncthreads();
    if (tid < h_i) {
        float s = 0.f;
        for (int i = 0; i < NT; ++i) s += red[tid][i];
        dw[t * h_i + tid] = s;
    }
}

hipError_t launch_index_bwd(const uint8_t* q, const uint8_t* q_scale, const float* w, const int32_t* seq,
                            const int64_t* pos, int64_t T, int h_i, int d_i, const uint8_t* kdata,
                            const uint8_t* kscale, int64_t kcap, const int32_t* kpages, int kpshift, int m,
                            const int32_t* idx, const float* g, int n_sel, float* dq, float* dw, float* dkeys,
                            int64_t key_rows, void* ws, hipStream_t st) {
    if (T == 0) return hipSuccess;
    unsigned long long* fx = (unsigned long long*)ws;
    const int64_t n_fx = key_rows * d_i;
    hipError_t e = launch_fx_zero(fx, n_fx, st);
    if (e != hipSuccess) return e;
    if (d_i == 128)
        hipLaunchKernelGGL(k_index_bwd<128>, dim3((unsigned)T), dim3(kIbThreads), 0, st, q, q_scale, w, seq, pos, h_i,
                           kdata, kscale, kcap, kpages, kpshift, m, idx, g, n_sel, dq, dw, fx);
    else
        hipLaunchKernelGGL(k_index_bwd<64>, dim3((unsigned)T), dim3(kIbThreads), 0, st, q, q_scale, w, seq, pos, h_i,
                           kdata, kscale, kcap, kpages, kpshift, m, idx, g, n_sel, dq, dw, fx);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_fx_flush(fx, dkeys, n_fx, st);
}

// ---------------------------------------------------------------------------
// 64-bit fixed-point gradient buffers (see fx_add): clear before, flush after.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_fx_zero(unsigned long long* __restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0ull;
}

// dst[i] += src[i] * 2^-40 (one fp32 rounding of the exact sum)
__global__ __launch_bounds__(256) void k_fx_flush(const unsigned long long* __restrict__ src, float* __restrict__ dst,
                                                  int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const long long v = (long long)src[i];
        if (v != 0) dst[i] += (float)((double)v / kFxUnit);
    }
}

static unsigned fx_blocks(int64_t n) {
    const int64_t b = (n + 255) / 256;
    return (unsigned)(b < 8192 ? (b > 0 ? b : 1) : 8192);
}

hipError_t launch_fx_zero(unsigned long long* p, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fx_zero, dim3(fx_blocks(n)), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

hipError_t launch_fx_flush(const unsigned long long* src, float* dst, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fx_flush, dim3(fx_blocks(n)), dim3(256), 0, st, src, dst, n);
    return hipGetLastError();
}

}  // namespace csa
