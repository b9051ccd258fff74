// Exact top-k selection building blocks shared by the selection kernels and the
// fused indexer + selection: block scans, histogram searches over order keys
// (keys from f32_order_key: a larger score has a larger key), the histogram
// descent that narrows a key window around the need-th largest key, and the
// whole-row radix select.
#pragma once
#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {

constexpr int kTopkThreads = 1024;
constexpr int kTopkCache = 36608;  // keys cached in LDS (143 KB)

// exclusive prefix sum over the block (NT threads); returns the block total in `total`
template <int NT = kTopkThreads>
__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int x = wave_incl_scan(v);
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
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
template <int NBINS, int NT = kTopkThreads>
__device__ int find_bin(const uint32_t* hist, int need, int* wsum, int* bcast, int& above) {
    constexpr int PER = NBINS / NT > 0 ? NBINS / NT : 1;
    const int tid = threadIdx.x;
    // thread tid owns bins counted from the top: [tid*PER, tid*PER + PER) in descending order
    int local = 0;
    if (tid * PER < NBINS)
        for (int i = 0; i < PER; ++i) local += (int)hist[NBINS - 1 - (tid * PER + i)];
    int total;
    int before = block_excl_scan<NT>(local, wsum, total);
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

// Exact top-k of one row (nv > k visible columns) by one NT-thread workgroup.
// The keys are cached in `cache` when the row fits (`cap` keys); otherwise
// every pass re-reads global memory.  hist: 4096 words; wsum: 2 * NT / 64
// ints; bcast: 4 ints.
template <int NT = kTopkThreads>
__device__ void row_select(const float* __restrict__ row, int nv, int k, int32_t* __restrict__ out, uint32_t* hist,
                           uint32_t* cache, int cap, int* wsum, int* bcast) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool cached = nv <= cap;
    auto key_at = [&](int j) -> uint32_t { return cached ? cache[j] : f32_order_key(row[j]); };
    for (int i = tid; i < 4096; i += NT) hist[i] = 0;
    __syncthreads();

    // load the row into LDS (16-byte loads when aligned, several in flight) and histogram the top 12 bits
    if (cached && (((uintptr_t)row & 15) == 0)) {
        const int n4 = nv >> 2;
#pragma unroll 4
        for (int j4 = tid; j4 < n4; j4 += NT) {
            const float4 v = ((const float4*)row)[j4];
            const uint4 kk = make_uint4(f32_order_key(v.x), f32_order_key(v.y), f32_order_key(v.z), f32_order_key(v.w));
            *(uint4*)&cache[4 * j4] = kk;
            atomicAdd(&hist[kk.x >> 20], 1u);
            atomicAdd(&hist[kk.y >> 20], 1u);
            atomicAdd(&hist[kk.z >> 20], 1u);
            atomicAdd(&hist[kk.w >> 20], 1u);
        }
        for (int j = 4 * n4 + tid; j < nv; j += NT) {
            const uint32_t kk = f32_order_key(row[j]);
            cache[j] = kk;
            atomicAdd(&hist[kk >> 20], 1u);
        }
    } else {
        for (int j = tid; j < nv; j += NT) {
            const uint32_t kk = f32_order_key(row[j]);
            if (cached) cache[j] = kk;
            atomicAdd(&hist[kk >> 20], 1u);
        }
    }
    __syncthreads();
    int above1;
    const uint32_t b1 = (uint32_t)find_bin<4096, NT>(hist, k, wsum, bcast, above1);

    // refinement passes over the keys whose prefix matches (LDS read 4 keys at a time)
    auto refine = [&](auto match, auto bin) {
        if (cached) {
            const int n4 = nv >> 2;
            for (int j4 = tid; j4 < n4; j4 += NT) {
                const uint4 kk = *(const uint4*)&cache[4 * j4];
                if (match(kk.x)) atomicAdd(&hist[bin(kk.x)], 1u);
                if (match(kk.y)) atomicAdd(&hist[bin(kk.y)], 1u);
                if (match(kk.z)) atomicAdd(&hist[bin(kk.z)], 1u);
                if (match(kk.w)) atomicAdd(&hist[bin(kk.w)], 1u);
            }
            for (int j = 4 * n4 + tid; j < nv; j += NT) {
                const uint32_t kk = cache[j];
                if (match(kk)) atomicAdd(&hist[bin(kk)], 1u);
            }
        } else {
            for (int j = tid; j < nv; j += NT) {
                const uint32_t kk = f32_order_key(row[j]);
                if (match(kk)) atomicAdd(&hist[bin(kk)], 1u);
            }
        }
    };

    // pass 2: middle 12 bits among keys with prefix b1
    for (int i = tid; i < 4096; i += NT) hist[i] = 0;
    __syncthreads();
    refine([&](uint32_t kk) { return (kk >> 20) == b1; }, [](uint32_t kk) { return (kk >> 8) & 0xFFFu; });
    __syncthreads();
    int above2;
    const uint32_t b2 = (uint32_t)find_bin<4096, NT>(hist, k - above1, wsum, bcast, above2);
    const uint32_t p2 = (b1 << 12) | b2;

    // pass 3: low 8 bits among keys with prefix p2
    for (int i = tid; i < 256; i += NT) hist[i] = 0;
    __syncthreads();
    refine([&](uint32_t kk) { return (kk >> 8) == p2; }, [](uint32_t kk) { return kk & 0xFFu; });
    __syncthreads();
    int above3;
    const uint32_t b3 = (uint32_t)find_bin<256, NT>(hist, k - above1 - above2, wsum, bcast, above3);
    const uint32_t thr = (p2 << 8) | b3;
    const int need_eq = k - (above1 + above2 + above3);

    // ordered compaction: wave w owns the contiguous columns [w seg, (w+1) seg); ranks within a
    // wave come from ballots, across waves from one exchange of (#greater, #equal) per wave
    constexpr int NW = NT / 64;
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


constexpr int kTieLds = 256;  // equal-key sets up to this size are ranked directly

__device__ __forceinline__ int64_t row_visible(const int64_t* pos, int64_t t, int m, int64_t n_cols) {
    int64_t nv = (pos[t] + 1) / m;
    if (nv > n_cols) nv = n_cols;
    if (nv < 0) nv = 0;
    return nv;
}

// Histograms handed to tm_find are stored "transposed": with PER = NB/NT
// bins per thread and bins ranked from the top (r = NB-1-bin), rank r sits
// at position (r % PER) * NT + r / PER.  Thread t then owns ranks
// t*PER .. t*PER+PER-1 and reads them at positions i*NT + t: consecutive
// threads, consecutive words, no LDS bank conflicts.
template <int NB, int NT>
__device__ __forceinline__ int tm_pos(uint32_t bin) {
    constexpr int PER = NB / NT > 0 ? NB / NT : 1;
    const int r = NB - 1 - (int)bin;
    return (r % PER) * NT + r / PER;
}

// exclusive scan over an NT-thread block
template <int NT>
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
template <int NB, int NT>
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


// tm_find with two barriers: the caller must not write wsum or bc again before
// its next barrier (and then only through another tm_find / tm_scan call).
template <int NB, int NT>
__device__ __forceinline__ int tm_find2(const uint32_t* hist, int need, int* wsum, int* bc, int& above) {
    constexpr int PER = NB / NT > 0 ? NB / NT : 1;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t v[PER];
    int local = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        v[i] = tid * PER + i < NB ? hist[i * NT + tid] : 0u;
        local += (int)v[i];
    }
    const int x = wave_incl_scan(local);
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int before = x - local;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) before += i < wave ? wsum[i] : 0;
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
    return bc[0];
}

// Histogram descent over a set of keys (visited by for_each): finds a window
// [base, base + 2^sh) holding the need-th largest key, with `above` keys
// above the window and `inbin` keys inside it.  Each level histograms the
// current window into 4096 bins and keeps the bin of the need-th largest,
// until that bin holds at most `stop` keys or a single key value (sh == 0).
// A level's window never reaches past the bin the previous level kept: when
// the shift drops from s < 12 to 0, 4096 unit bins would cover more than that
// 2^s-wide bin, and keys above it (already counted in `above`) would be
// counted a second time.
// Requires lo <= the need-th largest key and every key <= hi; keys below lo
// are ignored.  h: 4096 LDS words, zero on entry (and visible to all
// threads); on return it holds the last level's counts, and the caller
// passes a barrier before writing h, wsum or bc again.
template <int NT, class ForEach>
__device__ void hist_descend(ForEach for_each, uint32_t lo, uint32_t hi, int need, int stop, uint32_t* h, int* wsum,
                             int* bc, uint32_t& base, int& sh, int& above, int& inbin) {
    const int tid = threadIdx.x;
    const uint64_t span = (uint64_t)hi - lo;
    int s = 0;
    while ((span >> s) >= 4096) ++s;
    uint32_t b0 = lo;
    int ab_tot = 0;
    uint64_t ptop = (uint64_t)lo + ((uint64_t)4096 << s);  // end of the bin kept by the previous level
    for (;;) {
        uint64_t top = (uint64_t)b0 + ((uint64_t)4096 << s);
        if (top > ptop) top = ptop;
        const uint32_t wb = b0;
        const int ws = s;
        // for_each may pass a weight with each key (a key standing for several): counts are sums of weights
        for_each([&](uint32_t key, uint32_t wt = 1u) {
            if (key >= wb && (uint64_t)key < top) atomicAdd(&h[tm_pos<4096, NT>((key - wb) >> ws)], wt);
        });
        __syncthreads();
        int ab;
        const uint32_t b = (uint32_t)tm_find2<4096, NT>(h, need - ab_tot, wsum, bc, ab);
        const int nb = (int)h[tm_pos<4096, NT>(b)];
        ab_tot += ab;
        b0 += b << s;
        ptop = (uint64_t)b0 + ((uint64_t)1 << s);
        if (nb <= stop || s == 0) {
            base = b0;
            sh = s;
            above = ab_tot;
            inbin = nb;
            break;
        }
        s = s > 12 ? s - 12 : 0;
        __syncthreads();  // h has been read before it is cleared
        for (int i = tid; i < 4096; i += NT) h[i] = 0;
        __syncthreads();
    }
}

// Exact top-k of a row from a candidate list: cl[0 .. n_cand) in LDS holds
// (key << 32 | ~column) for every visible column of the row whose key is >= lo
// (n_cand >= k, every key <= hi).  Finds the k-th largest by a histogram
// descent, ranks the few keys of its window directly (equal keys to the lower
// column) or, for one key value held by many, takes its lowest columns by
// column passes; marks the winners and writes them to out[0 .. k) in
// ascending column order.  bm: with use_bm, the row bitmap (word w at
// (w % perw) * NT + w / perw, cleared), else room for the k winners rounded
// up to a power of two (sorted by a bitonic network).  h: 4096 words, zero;
// lctr[0..1] zero; tie: kTieLds entries; a barrier passed since all were set.
template <int NT>
__device__ __forceinline__ void pick_candidates(const uint64_t* cl, int n_cand, uint32_t lo, uint32_t hi, int k, int32_t* out,
                                uint32_t* bm, bool use_bm, int perw, uint32_t* h, uint64_t* tie, int* wsum, int* bc,
                                uint32_t* lctr) {
    const int tid = threadIdx.x;
    auto mark = [&](uint32_t j) {
        if (use_bm) {
            const uint32_t wd = j >> 5;
            atomicOr(&bm[(wd % perw) * NT + wd / perw], 1u << (j & 31));
        } else {
            const uint32_t o = atomicAdd(&lctr[1], 1u);
            if (o < (uint32_t)k) bm[o] = j;
        }
    };

    // ---- the k-th largest candidate: a window holding it, then rank inside the window ----
    uint32_t wbase;
    int wsh, above, nb;
    hist_descend<NT>([&](auto fn) { for (int i = tid; i < n_cand; i += NT) fn((uint32_t)(cl[i] >> 32)); }, lo, hi, k,
                     kTieLds, h, wsum, bc, wbase, wsh, above, nb);
    const uint64_t wtop = (uint64_t)wbase + ((uint64_t)1 << wsh);
    const int need = k - above;  // >= 1 winners inside the window
    for (int i = tid; i < n_cand; i += NT) {
        const uint64_t c = cl[i];
        const uint32_t key = (uint32_t)(c >> 32);
        if ((uint64_t)key >= wtop) mark(~(uint32_t)c);
        else if (key >= wbase && nb <= kTieLds) tie[atomicAdd(&lctr[0], 1u)] = c;
    }
    __syncthreads();
    if (nb <= kTieLds) {
        // (key desc, column asc) is (key << 32 | ~column) desc: rank each window entry directly
        for (int i = tid; i < nb; i += NT) {
            const uint64_t e = tie[i];
            int rank = 0;
            for (int q = 0; q < nb; ++q) rank += tie[q] > e ? 1 : 0;
            if (rank < need) mark(~(uint32_t)e);
        }
    } else {
        // a single key value (wbase) held by more than kTieLds candidates: the need lowest
        // columns among them (3 passes of 11 bits)
        const uint32_t thr = wbase;
        uint32_t pre = 0, pm = 0;
        int nl = need;
        for (int sh = 22; sh >= 0; sh -= 11) {
            for (int i = tid; i < 2048; i += NT) h[i] = 0;
            __syncthreads();
            for (int i = tid; i < n_cand; i += NT) {
                const uint64_t c = cl[i];
                if ((uint32_t)(c >> 32) != thr) continue;
                const uint32_t jx = ~(uint32_t)c;
                if ((jx & pm) == pre) atomicAdd(&h[tm_pos<2048, NT>(2047 - ((jx >> sh) & 0x7FF))], 1u);  // lower, higher bin
            }
            __syncthreads();
            int ab;
            const uint32_t bn = 2047u - (uint32_t)tm_find<2048, NT>(h, nl, wsum, bc, ab);
            nl -= ab;
            pre |= bn << sh;
            pm |= 0x7FFu << sh;
        }
        for (int i = tid; i < n_cand; i += NT) {
            const uint64_t c = cl[i];
            if ((uint32_t)(c >> 32) == thr && ~(uint32_t)c <= pre) mark(~(uint32_t)c);
        }
    }
    __syncthreads();

    if (use_bm) {
        // thread t owns words t*perw .. t*perw+perw-1 (reads free of bank conflicts)
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
    } else {
        // bitonic sort of the k marked columns
        int np = 1;
        while (np < k) np <<= 1;
        for (int i = k + tid; i < np; i += NT) bm[i] = 0xFFFFFFFFu;
        __syncthreads();
        for (int size = 2; size <= np; size <<= 1)
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int i = tid; i < np / 2; i += NT) {
                    const int lo2 = 2 * i - (i & (stride - 1));
                    const int hi2 = lo2 + stride;
                    const bool asc = (lo2 & size) == 0;
                    const uint32_t a = bm[lo2], b = bm[hi2];
                    if ((a > b) == asc) {
                        bm[lo2] = b;
                        bm[hi2] = a;
                    }
                }
                __syncthreads();
            }
        for (int a = tid; a < k; a += NT) out[a] = (int32_t)bm[a];
    }
}

}  // namespace csa
