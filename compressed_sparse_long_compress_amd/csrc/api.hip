// libcsa C ABI: argument validation, launch selection and error reporting.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../include/csa.h"
#include "csa_internal.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return CSA_OK;
}

int hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(CSA_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_kv(const csa_kv_t& kv, int d, const char* what, const char* fn) {
    if (!kv.nope || !kv.rope || !kv.scale) return fail(CSA_EINVAL, "%s: %s has a null array", fn, what);
    if (kv.cap <= 0) return fail(CSA_EINVAL, "%s: %s.cap must be positive", fn, what);
    if (!aligned16(kv.nope) || !aligned16(kv.rope))
        return fail(CSA_EINVAL, "%s: %s.nope / %s.rope must be 16-byte aligned", fn, what, what);
    if (((uintptr_t)kv.scale & 3u) != 0) return fail(CSA_EINVAL, "%s: %s.scale must be 4-byte aligned", fn, what);
    if (kv.pages) {
        if (kv.page < 1 || (kv.page & (kv.page - 1)) != 0)
            return fail(CSA_EINVAL, "%s: %s.page (%d) must be a power of two", fn, what, kv.page);
        if (kv.cap % kv.page != 0)
            return fail(CSA_EINVAL, "%s: %s.page (%d) must divide %s.cap (%lld)", fn, what, kv.page, what,
                        (long long)kv.cap);
    }
    (void)d;
    return CSA_OK;
}

int check_keys_pages(const csa_index_keys_t& keys, const char* fn) {
    if (!keys.pages) return CSA_OK;
    if (keys.page < 1 || (keys.page & (keys.page - 1)) != 0)
        return fail(CSA_EINVAL, "%s: keys.page (%d) must be a power of two", fn, keys.page);
    if (keys.cap % keys.page != 0)
        return fail(CSA_EINVAL, "%s: keys.page (%d) must divide keys.cap (%lld)", fn, keys.page, (long long)keys.cap);
    return CSA_OK;
}

int page_shift(const int32_t* pages, int32_t page) {
    int sh = 0;
    if (pages)
        while ((1 << sh) < page) ++sh;
    return sh;
}

csa::KvView view(const csa_kv_t& kv) {
    int sh = 0;
    if (kv.pages)
        while ((1 << sh) < kv.page) ++sh;
    return csa::KvView{kv.nope, kv.rope, kv.scale, kv.cap, kv.pages, sh};
}

int check_mqa_common(const char* fn, const uint16_t* q, const int32_t* seq, const int64_t* pos, int64_t T, int32_t H,
                     int32_t d, int32_t m, const csa_kv_t& comp, const csa_kv_t& win, int32_t window, float* out,
                     float* lse) {
    if (T < 0) return fail(CSA_EINVAL, "%s: T must be >= 0", fn);
    if (T > 0 && (!q || !seq || !pos || !out || !lse)) return fail(CSA_EINVAL, "%s: null pointer argument", fn);
    if (d != 128 && d != 512) return fail(CSA_EUNSUPPORTED, "%s: d=%d unsupported (128 or 512)", fn, d);
    if (H != 16 && H != 32 && H != 64) return fail(CSA_EUNSUPPORTED, "%s: H=%d unsupported (16, 32, 64)", fn, H);
    if (m < 1) return fail(CSA_EINVAL, "%s: m must be >= 1", fn);
    if (window < 0 || window > 1024) return fail(CSA_EUNSUPPORTED, "%s: window=%d outside 0..1024", fn, window);
    if (!aligned16(q) || !aligned16(out)) return fail(CSA_EINVAL, "%s: q and out must be 16-byte aligned", fn);
    if (int rc = check_kv(comp, d, "comp", fn)) return rc;
    if (window > 0) {
        if (int rc = check_kv(win, d, "win", fn)) return rc;
        if (win.cap < window) return fail(CSA_EINVAL, "%s: win.cap (%lld) < window (%d)", fn, (long long)win.cap, window);
    }
    return CSA_OK;
}

// Debug checks (environment variable CSA_DEBUG_CHECKS set and not "0"): the attention calls
// first scan the entries they will read for RoPE dims outside the fp16 range and fail with
// CSA_EINVAL.  The check synchronises the caller's stream (not for graph capture).
static __device__ int g_rope_bad;

bool debug_checks() {
    const char* e = getenv("CSA_DEBUG_CHECKS");
    return e && e[0] && !(e[0] == '0' && e[1] == 0);
}

int check_rope_range(const char* fn, const int32_t* seq, const int64_t* pos, int64_t T, const int32_t* idx, int k,
                     int m, const csa::KvView& comp, const csa::KvView& win, int window, hipStream_t st) {
    void* flag = nullptr;
    hipError_t e = hipGetSymbolAddress(&flag, HIP_SYMBOL(g_rope_bad));
    if (e == hipSuccess) e = hipMemsetAsync(flag, 0, sizeof(int), st);
    if (e == hipSuccess) e = csa::launch_check_rope(seq, pos, T, idx, k, m, comp, win, window, (int*)flag, st);
    int bad = 0;
    if (e == hipSuccess) e = hipMemcpyAsync(&bad, flag, sizeof(int), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(CSA_EHIP, "%s: debug range check failed: %s", fn, hipGetErrorString(e));
    if (bad)
        return fail(CSA_EINVAL, "%s: an entry read by this call has a RoPE dim of magnitude above 65504 (or not "
                    "finite); the attention kernels stage those dims in fp16", fn);
    return CSA_OK;
}

}  // namespace

namespace csa {
RopeTab rope_table(double base) {
    RopeTab rt;
    for (int i = 0; i < 32; ++i) rt.theta[i] = pow(base, -2.0 * (double)i / 64.0);
    return rt;
}
}  // namespace csa

extern "C" {

const char* csa_last_error(void) { return g_err; }

int csa_version(void) { return CSA_VERSION; }

int csa_compress(const uint16_t* kv, const float* logits, int64_t tok0, int64_t n_tok, int32_t m, int32_t d,
                 float rope_base, int32_t seq, csa_kv_t out, csa_stream_t stream) {
    const char* fn = "csa_compress";
    if (m < 1 || m > 1024) return fail(CSA_EUNSUPPORTED, "%s: m=%d outside 1..1024", fn, m);
    if (d != 128 && d != 512) return fail(CSA_EUNSUPPORTED, "%s: d=%d unsupported (128 or 512)", fn, d);
    if (tok0 < 0 || n_tok < 0) return fail(CSA_EINVAL, "%s: tok0 and n_tok must be >= 0", fn);
    if (tok0 % m != 0 || n_tok % m != 0)
        return fail(CSA_EINVAL, "%s: tok0 (%lld) and n_tok (%lld) must be multiples of m (%d): only complete blocks "
                    "are compressed", fn, (long long)tok0, (long long)n_tok, m);
    if (seq < 0) return fail(CSA_EINVAL, "%s: seq must be >= 0", fn);
    if (!(rope_base > 0.f)) return fail(CSA_EINVAL, "%s: rope_base must be positive", fn);
    if (n_tok == 0) return ok();
    if (!kv || !logits) return fail(CSA_EINVAL, "%s: null kv or logits", fn);
    if (!aligned16(kv)) return fail(CSA_EINVAL, "%s: kv must be 16-byte aligned", fn);
    if (int rc = check_kv(out, d, "out", fn)) return rc;
    if (n_tok / m > out.cap)
        return fail(CSA_EINVAL, "%s: %lld new entries exceed out.cap (%lld): slots would collide", fn,
                    (long long)(n_tok / m), (long long)out.cap);
    hipError_t e = csa::launch_compress(kv, logits, tok0, n_tok, m, d, csa::rope_table((double)rope_base), seq,
                                        view(out), out.nope, out.rope, out.scale, (hipStream_t)stream);
    return hip_status(e, fn);
}

int csa_compress_channel(const uint16_t* kv, const float* logits, int64_t tok0, int64_t n_tok, int32_t m, int32_t d,
                         float rope_base, int32_t seq, csa_kv_t out, csa_stream_t stream) {
    const char* fn = "csa_compress_channel";
    if (m < 1 || m > 1024) return fail(CSA_EUNSUPPORTED, "%s: m=%d outside 1..1024", fn, m);
    if (d != 128 && d != 512) return fail(CSA_EUNSUPPORTED, "%s: d=%d unsupported (128 or 512)", fn, d);
    if (tok0 < 0 || n_tok < 0) return fail(CSA_EINVAL, "%s: tok0 and n_tok must be >= 0", fn);
    if (tok0 % m != 0 || n_tok % m != 0)
        return fail(CSA_EINVAL, "%s: tok0 (%lld) and n_tok (%lld) must be multiples of m (%d): only complete blocks "
                    "are compressed", fn, (long long)tok0, (long long)n_tok, m);
    if (seq < 0) return fail(CSA_EINVAL, "%s: seq must be >= 0", fn);
    if (!(rope_base > 0.f)) return fail(CSA_EINVAL, "%s: rope_base must be positive", fn);
    if (n_tok == 0) return ok();
    if (!kv || !logits) return fail(CSA_EINVAL, "%s: null kv or logits", fn);
    if (!aligned16(kv) || !aligned16(logits)) return fail(CSA_EINVAL, "%s: kv and logits must be 16-byte aligned", fn);
    if (int rc = check_kv(out, d, "out", fn)) return rc;
    if (n_tok / m > out.cap)
        return fail(CSA_EINVAL, "%s: %lld new entries exceed out.cap (%lld): slots would collide", fn,
                    (long long)(n_tok / m), (long long)out.cap);
    hipError_t e = csa::launch_compress_channel(kv, logits, tok0, n_tok, m, d, csa::rope_table((double)rope_base),
                                                seq, view(out), out.nope, out.rope, out.scale, (hipStream_t)stream);
    return hip_status(e, fn);
}

int csa_compress_index_keys(const uint16_t* k, const float* logits, int64_t tok0, int64_t n_tok, int32_t m,
                            int32_t d_i, int32_t seq, csa_index_keys_t out, csa_stream_t stream) {
    const char* fn = "csa_compress_index_keys";
    if (m < 1 || m > 1024) return fail(CSA_EUNSUPPORTED, "%s: m=%d outside 1..1024", fn, m);
    if (d_i != 64 && d_i != 128) return fail(CSA_EUNSUPPORTED, "%s: d_i=%d unsupported (64 or 128)", fn, d_i);
    if (tok0 < 0 || n_tok < 0) return fail(CSA_EINVAL, "%s: tok0 and n_tok must be >= 0", fn);
    if (tok0 % m != 0 || n_tok % m != 0)
        return fail(CSA_EINVAL, "%s: tok0 (%lld) and n_tok (%lld) must be multiples of m (%d): only complete blocks "
                    "are compressed", fn, (long long)tok0, (long long)n_tok, m);
    if (seq < 0) return fail(CSA_EINVAL, "%s: seq must be >= 0", fn);
    if (n_tok == 0) return ok();
    if (!k || !logits || !out.data || !out.scale) return fail(CSA_EINVAL, "%s: null array", fn);
    if (((uintptr_t)k & 3u) != 0) return fail(CSA_EINVAL, "%s: k must be 4-byte aligned", fn);
    if (out.cap < 1) return fail(CSA_EINVAL, "%s: out.cap must be >= 1", fn);
    if (n_tok / m > out.cap)
        return fail(CSA_EINVAL, "%s: %lld new entries exceed out.cap (%lld): slots would collide", fn,
                    (long long)(n_tok / m), (long long)out.cap);
    if (int rc = check_keys_pages(out, fn)) return rc;
    hipError_t e = csa::launch_compress_index_keys(k, logits, tok0, n_tok, m, d_i, seq, out.cap, out.pages,
                                                   page_shift(out.pages, out.page), out.data, out.scale,
                                                   (hipStream_t)stream);
    return hip_status(e, fn);
}

// shared by the two indexer entry points: argument checks and the row-summary destination
static int index_args(const char* fn, const uint8_t* q, const uint8_t* q_scale, const float* w, const int32_t* seq,
                      const int64_t* pos, int64_t T, int32_t h_i, int32_t d_i, const csa_index_keys_t& keys, int32_t m,
                      int64_t n_cols, const float* scores, void* topk_ws, size_t topk_ws_bytes, uint32_t** gmax,
                      bool* nothing) {
    *gmax = nullptr;
    *nothing = false;
    if (T < 0 || n_cols < 0) return fail(CSA_EINVAL, "%s: T and n_cols must be >= 0", fn);
    if (n_cols >= ((int64_t)1 << 31)) return fail(CSA_EUNSUPPORTED, "%s: n_cols must be < 2^31", fn);
    if (h_i != 4 && h_i != 8) return fail(CSA_EUNSUPPORTED, "%s: h_i=%d unsupported (4 or 8)", fn, h_i);
    if (d_i != 64 && d_i != 128) return fail(CSA_EUNSUPPORTED, "%s: d_i=%d unsupported (64 or 128)", fn, d_i);
    if (m < 1) return fail(CSA_EINVAL, "%s: m must be >= 1", fn);
    if (T == 0 || n_cols == 0) {
        *nothing = true;
        return ok();
    }
    if (!q || !q_scale || !w || !seq || !pos || !keys.data || !keys.scale || !scores)
        return fail(CSA_EINVAL, "%s: null pointer argument", fn);
    if (keys.cap < n_cols) return fail(CSA_EINVAL, "%s: n_cols (%lld) > keys.cap (%lld)", fn, (long long)n_cols,
                                       (long long)keys.cap);
    if (!aligned16(q) || !aligned16(keys.data)) return fail(CSA_EINVAL, "%s: q and keys.data must be 16-byte aligned", fn);
    if (int rc = check_keys_pages(keys, fn)) return rc;
    if (topk_ws && csa::topk_uses_summary(T, n_cols)) {
        // the row summaries are the top-k workspace
        if (topk_ws_bytes < csa::topk_workspace_bytes(T, n_cols, 1))
            return fail(CSA_EWORKSPACE, "%s: top-k workspace too small for the row summaries", fn);
        if (((uintptr_t)topk_ws & 255u) != 0) return fail(CSA_EINVAL, "%s: workspace must be 256-byte aligned", fn);
        *gmax = (uint32_t*)topk_ws;
    }
    return ok();
}

int csa_index_scores(const uint8_t* q, const uint8_t* q_scale, const float* w, const int32_t* seq,
                     const int64_t* pos, int64_t T, int32_t h_i, int32_t d_i, csa_index_keys_t keys, int32_t m,
                     int64_t n_cols, float* scores, void* topk_ws, size_t topk_ws_bytes, csa_stream_t stream) {
    const char* fn = "csa_index_scores";
    uint32_t* gmax;
    bool nothing;
    const int rc = index_args(fn, q, q_scale, w, seq, pos, T, h_i, d_i, keys, m, n_cols, scores, topk_ws,
                              topk_ws_bytes, &gmax, &nothing);
    if (rc != CSA_OK || nothing) return rc;
    hipError_t e = csa::launch_index_scores(q, q_scale, w, seq, pos, T, h_i, d_i, keys.data, keys.scale, keys.cap,
                                            keys.pages, page_shift(keys.pages, keys.page), m,
                                            n_cols, scores, gmax, (hipStream_t)stream);
    return hip_status(e, fn);
}

int csa_index_scores_grouped(const uint8_t* q, const uint8_t* q_scale, const float* w, const int32_t* seq,
                             const int64_t* pos, int64_t T, int32_t h_i, int32_t d_i, csa_index_keys_t keys,
                             int32_t m, int64_t n_cols, int32_t group, float* scores, void* topk_ws,
                             size_t topk_ws_bytes, csa_stream_t stream) {
    const char* fn = "csa_index_scores_grouped";
    if (group != 1 && group != 2 && group != 4)
        return fail(CSA_EUNSUPPORTED, "%s: group=%d unsupported (1, 2 or 4)", fn, group);
    if (T > 0 && T % group != 0) return fail(CSA_EINVAL, "%s: T (%lld) must be a multiple of group", fn, (long long)T);
    uint32_t* gmax;
    bool nothing;
    const int rc = index_args(fn, q, q_scale, w, seq, pos, T, h_i, d_i, keys, m, n_cols, scores, topk_ws,
                              topk_ws_bytes, &gmax, &nothing);
    if (rc != CSA_OK || nothing) return rc;
    hipError_t e = csa::launch_index_scores_grouped(q, q_scale, w, seq, pos, T, h_i, d_i, keys.data, keys.scale,
                                                    keys.cap, keys.pages, page_shift(keys.pages, keys.page), m, n_cols,
                                                    group, scores, gmax, (hipStream_t)stream);
    return hip_status(e, fn);
}

size_t csa_index_topk_workspace(int64_t T, int64_t n_cols, int32_t k, int32_t h_i) {
    if (T <= 0 || n_cols <= 0 || k < 1 || k > 2048 || (h_i != 4 && h_i != 8)) return 0;
    return csa::index_topk_workspace_bytes(T, n_cols, k, h_i);
}

int csa_index_topk(const uint8_t* q, const uint8_t* q_scale, const float* w, const int32_t* seq, const int64_t* pos,
                   int64_t T, int32_t h_i, int32_t d_i, csa_index_keys_t keys, int32_t m, int64_t n_cols, int32_t k,
                   int32_t* idx, void* ws, size_t ws_bytes, csa_stream_t stream) {
    const char* fn = "csa_index_topk";
    uint32_t* gmax;
    bool nothing;
    if (k < 1 || k > 2048) return fail(CSA_EUNSUPPORTED, "%s: k=%d outside 1..2048", fn, k);
    if (n_cols >= ((int64_t)1 << 31)) return fail(CSA_EUNSUPPORTED, "%s: n_cols must be < 2^31", fn);
    // same argument rules as csa_index_scores (no score row: a non-null dummy stands for it)
    const int rc = index_args(fn, q, q_scale, w, seq, pos, T, h_i, d_i, keys, m, n_cols, (const float*)idx, nullptr, 0,
                              &gmax, &nothing);
    if (rc != CSA_OK) return rc;
    if (T == 0) return ok();
    if (!idx) return fail(CSA_EINVAL, "%s: null idx", fn);
    if (n_cols == 0) {
        // nothing visible: every row is padding (a tiny launch of the selection does it)
        return fail(CSA_EINVAL, "%s: n_cols must be >= 1", fn);
    }
    const size_t need = csa::index_topk_workspace_bytes(T, n_cols, k, h_i);
    if (ws_bytes < need || !ws)
        return fail(CSA_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws_bytes);
    if (((uintptr_t)ws & 255u) != 0) return fail(CSA_EINVAL, "%s: workspace must be 256-byte aligned", fn);
    hipError_t e = csa::launch_index_topk(q, q_scale, w, seq, pos, T, h_i, d_i, keys.data, keys.scale, keys.cap,
                                          keys.pages, page_shift(keys.pages, keys.page), m,
                                          n_cols, k, idx, ws, (hipStream_t)stream);
    return hip_status(e, fn);
}

size_t csa_index_bwd_workspace(int64_t key_rows, int32_t d_i) {
    if (key_rows <= 0 || (d_i != 64 && d_i != 128)) return 0;
    return (size_t)key_rows * d_i * 8;
}

int csa_index_bwd(const uint8_t* q, const uint8_t* q_scale, const float* w, const int32_t* seq, const int64_t* pos,
                  int64_t T, int32_t h_i, int32_t d_i, csa_index_keys_t keys, int32_t m, const int32_t* idx,
                  const float* g, int32_t n_sel, float* dq, float* dw, float* dkeys, int64_t key_rows, void* ws,
                  size_t ws_bytes, csa_stream_t stream) {
    const char* fn = "csa_index_bwd";
    if (T < 0) return fail(CSA_EINVAL, "%s: T must be >= 0", fn);
    if (h_i != 4 && h_i != 8) return fail(CSA_EUNSUPPORTED, "%s: h_i=%d unsupported (4 or 8)", fn, h_i);
    if (d_i != 64 && d_i != 128) return fail(CSA_EUNSUPPORTED, "%s: d_i=%d unsupported (64 or 128)", fn, d_i);
    if (m < 1) return fail(CSA_EINVAL, "%s: m must be >= 1", fn);
    if (n_sel < 1) return fail(CSA_EINVAL, "%s: n_sel must be >= 1", fn);
    if (key_rows < 1) return fail(CSA_EINVAL, "%s: key_rows must be >= 1", fn);
    if (T == 0) return ok();
    if (!q || !q_scale || !w || !seq || !pos || !keys.data || !keys.scale || !idx || !g || !dq || !dw || !dkeys)
        return fail(CSA_EINVAL, "%s: null pointer argument", fn);
    if (keys.cap < 1) return fail(CSA_EINVAL, "%s: keys.cap must be >= 1", fn);
    if (int rc = check_keys_pages(keys, fn)) return rc;
    const size_t need = csa_index_bwd_workspace(key_rows, d_i);
    if (ws_bytes < need || !ws)
        return fail(CSA_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws_bytes);
    if (((uintptr_t)ws & 7u) != 0) return fail(CSA_EINVAL, "%s: workspace must be 8-byte aligned", fn);
    hipError_t e = csa::launch_index_bwd(q, q_scale, w, seq, pos, T, h_i, d_i, keys.data, keys.scale, keys.cap,
                                         keys.pages, page_shift(keys.pages, keys.page), m, idx,
                                         g, n_sel, dq, dw, dkeys, key_rows, ws, (hipStream_t)stream);
    return hip_status(e, fn);
}

size_t csa_pages_bytes(int32_t page, int32_t d, int32_t d_i) {
    if (page < 1 || (d != 128 && d != 512) || (d_i != 0 && d_i != 64 && d_i != 128)) return 0;
    return (size_t)page * ((size_t)(d - 64) + 64 * 2 + 4 + (size_t)d_i / 2 + (size_t)d_i / 32);
}

// one page's arrays in the host layout, in order: nope, rope, scale, key data, key scales
static int pages_copy(const char* fn, const csa_kv_t& kv, const csa_index_keys_t& keys, int32_t d, int32_t d_i,
                      const int32_t* pages, int32_t n_pages, char* host, size_t host_bytes, bool to_host,
                      hipStream_t st) {
    if (d != 128 && d != 512) return fail(CSA_EUNSUPPORTED, "%s: d=%d unsupported (128 or 512)", fn, d);
    if (d_i != 0 && d_i != 64 && d_i != 128) return fail(CSA_EUNSUPPORTED, "%s: d_i=%d unsupported (0, 64, 128)", fn, d_i);
    if (n_pages < 0) return fail(CSA_EINVAL, "%s: n_pages must be >= 0", fn);
    if (n_pages == 0) return ok();
    const int32_t page = kv.page;
    if (page < 1 || (page & (page - 1)) != 0)
        return fail(CSA_EINVAL, "%s: kv.page (%d) must be a power of two (rows per page)", fn, page);
    if (!kv.nope || !kv.rope || !kv.scale || !pages || !host) return fail(CSA_EINVAL, "%s: null pointer argument", fn);
    if (d_i > 0) {
        if (!keys.data || !keys.scale) return fail(CSA_EINVAL, "%s: null key arrays", fn);
        if (keys.page != page) return fail(CSA_EINVAL, "%s: keys.page (%d) must equal kv.page (%d)", fn, keys.page, page);
    }
    const size_t per = csa_pages_bytes(page, d, d_i);
    if (host_bytes < per * (size_t)n_pages)
        return fail(CSA_EWORKSPACE, "%s: host buffer of %zu bytes needed, %zu given", fn, per * (size_t)n_pages, host_bytes);
    const size_t dn = (size_t)(d - 64);
    struct Arr {
        char* dev;
        size_t row;
    } arrs[5] = {{(char*)kv.nope, dn}, {(char*)kv.rope, 128}, {(char*)kv.scale, 4},
                 {(char*)keys.data, (size_t)d_i / 2}, {(char*)keys.scale, (size_t)d_i / 32}};
    const int na = d_i > 0 ? 5 : 3;
    // every page number checked before the first copy, so a bad list enqueues nothing
    for (int32_t i = 0; i < n_pages; ++i)
        if (pages[i] < 0) return fail(CSA_EINVAL, "%s: negative page number at %d", fn, i);
    for (int32_t i = 0; i < n_pages; ++i) {
        char* h = host + per * (size_t)i;
        for (int a = 0; a < na; ++a) {
            const size_t bytes = arrs[a].row * (size_t)page;
            char* dv = arrs[a].dev + (size_t)pages[i] * bytes;
            const hipError_t e = to_host ? hipMemcpyAsync(h, dv, bytes, hipMemcpyDeviceToHost, st)
                                         : hipMemcpyAsync(dv, h, bytes, hipMemcpyHostToDevice, st);
            if (e != hipSuccess) return fail(CSA_EHIP, "%s: copy failed: %s", fn, hipGetErrorString(e));
            h += bytes;
        }
    }
    return ok();
}

int csa_pages_store(csa_kv_t kv, csa_index_keys_t keys, int32_t d, int32_t d_i, const int32_t* pages,
                    int32_t n_pages, void* host, size_t host_bytes, csa_stream_t stream) {
    return pages_copy("csa_pages_store", kv, keys, d, d_i, pages, n_pages, (char*)host, host_bytes, true,
                      (hipStream_t)stream);
}

int csa_pages_load(csa_kv_t kv, csa_index_keys_t keys, int32_t d, int32_t d_i, const int32_t* pages,
                   int32_t n_pages, const void* host, size_t host_bytes, csa_stream_t stream) {
    return pages_copy("csa_pages_load", kv, keys, d, d_i, pages, n_pages, (char*)host, host_bytes, false,
                      (hipStream_t)stream);
}

size_t csa_topk_workspace(int64_t T, int64_t n_cols, int32_t k) { return csa::topk_workspace_bytes(T, n_cols, k); }

int csa_topk(const float* scores, int64_t T, int64_t n_cols, const int64_t* pos, int32_t m, int32_t k, int32_t* idx,
             void* ws, size_t ws_bytes, uint32_t flags, csa_stream_t stream) {
    const char* fn = "csa_topk";
    if (T < 0 || n_cols < 0) return fail(CSA_EINVAL, "%s: T and n_cols must be >= 0", fn);
    if (k < 1 || k > 2048) return fail(CSA_EUNSUPPORTED, "%s: k=%d outside 1..2048", fn, k);
    if (n_cols >= ((int64_t)1 << 31)) return fail(CSA_EUNSUPPORTED, "%s: n_cols must be < 2^31", fn);
    if (m < 1) return fail(CSA_EINVAL, "%s: m must be >= 1", fn);
    if (T == 0) return ok();
    if (!scores || !pos || !idx) return fail(CSA_EINVAL, "%s: null pointer argument", fn);
    const size_t need = csa::topk_workspace_bytes(T, n_cols, k);
    if (ws_bytes < need || (need > 0 && !ws))
        return fail(CSA_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws_bytes);
    if (need > 0 && ((uintptr_t)ws & 255u) != 0) return fail(CSA_EINVAL, "%s: workspace must be 256-byte aligned", fn);
    if (flags & ~(uint32_t)CSA_TOPK_PREPARED) return fail(CSA_EINVAL, "%s: unknown flags 0x%x", fn, flags);
    const bool ready = (flags & CSA_TOPK_PREPARED) && csa::topk_uses_summary(T, n_cols);
    hipError_t e = csa::launch_topk(scores, T, n_cols, pos, m, k, idx, ws, ready, (hipStream_t)stream);
    return hip_status(e, fn);
}

int csa_topk_noalloc(const float* scores, int64_t T, int64_t n_cols, const int64_t* pos, int32_t m, int32_t k,
                     int32_t* idx, csa_stream_t stream) {
    const char* fn = "csa_topk_noalloc";
    if (T < 0 || n_cols < 0) return fail(CSA_EINVAL, "%s: T and n_cols must be >= 0", fn);
    if (k < 1 || k > 2048) return fail(CSA_EUNSUPPORTED, "%s: k=%d outside 1..2048", fn, k);
    if (n_cols >= ((int64_t)1 << 31)) return fail(CSA_EUNSUPPORTED, "%s: n_cols must be < 2^31", fn);
    if (m < 1) return fail(CSA_EINVAL, "%s: m must be >= 1", fn);
    if (T == 0) return ok();
    if (!scores || !pos || !idx) return fail(CSA_EINVAL, "%s: null pointer argument", fn);
    const size_t need = csa::topk_workspace_bytes(T, n_cols, k);
    if (need > csa::topk_scratch_bytes())
        return fail(CSA_EUNSUPPORTED, "%s: T=%lld x n_cols=%lld needs %zu bytes of scratch, more than the library's "
                    "%zu-byte array; call csa_topk with a workspace", fn, (long long)T, (long long)n_cols, need,
                    csa::topk_scratch_bytes());
    hipError_t e = csa::launch_topk_noalloc(scores, T, n_cols, pos, m, k, idx, (hipStream_t)stream);
    return hip_status(e, fn);
}

int64_t csa_mfma_probe_flops(int32_t kind, int32_t blocks, int64_t iters) {
    if ((kind != 0 && kind != 1) || blocks < 1 || iters < 1 || iters % 4 != 0) return -1;
    const int64_t per = kind == 0 ? 16 * 16 * 32 * 2 : 32 * 32 * 64 * 2;
    return per * csa::kProbeChains * iters * (int64_t)blocks * (csa::kProbeThreads / 64);
}

int csa_mfma_probe(int32_t kind, int32_t blocks, int64_t iters, float* sink, int64_t sink_len, csa_stream_t stream) {
    const char* fn = "csa_mfma_probe";
    if (kind != 0 && kind != 1) return fail(CSA_EUNSUPPORTED, "%s: kind=%d (0: fp16, 1: MXFP4)", fn, kind);
    if (blocks < 1 || iters < 1 || iters % 4 != 0)
        return fail(CSA_EINVAL, "%s: blocks must be >= 1 and iters a positive multiple of 4", fn);
    if (!sink || sink_len < (int64_t)blocks * csa::kProbeThreads)
        return fail(CSA_EINVAL, "%s: sink must hold blocks x %d floats", fn, csa::kProbeThreads);
    return hip_status(csa::launch_mfma_probe(kind, blocks, iters, sink, (hipStream_t)stream), fn);
}

size_t csa_mqa_workspace(int64_t T, int32_t H, int32_t d, int64_t max_keys) {
    return csa::mqa_workspace_bytes(T, H, d, max_keys);
}

int csa_sparse_mqa(const uint16_t* q, const int32_t* seq, const int64_t* pos, int64_t T, int32_t H, int32_t d,
                   const int32_t* idx, int32_t k, int32_t m, csa_kv_t comp, csa_kv_t win, int32_t window,
                   float sm_scale, float rope_base, float* out, float* lse, void* ws, size_t ws_bytes,
                   csa_stream_t stream) {
    const char* fn = "csa_sparse_mqa";
    if (int rc = check_mqa_common(fn, q, seq, pos, T, H, d, m, comp, win, window, out, lse)) return rc;
    if (k < 1 || k > 2048) return fail(CSA_EUNSUPPORTED, "%s: k=%d outside 1..2048", fn, k);
    if (T > 0 && !idx) return fail(CSA_EINVAL, "%s: null idx", fn);
    if (!(rope_base > 0.f)) return fail(CSA_EINVAL, "%s: rope_base must be positive", fn);
    if (T == 0) return ok();
    const int64_t max_keys = (int64_t)k + window;
    const size_t need = csa::mqa_workspace_bytes(T, H, d, max_keys);
    if (ws_bytes < need || (need > 0 && !ws))
        return fail(CSA_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws_bytes);
    if (need > 0 && !aligned16(ws)) return fail(CSA_EINVAL, "%s: workspace must be 16-byte aligned", fn);
    if (debug_checks())
        if (int rc = check_rope_range(fn, seq, pos, T, idx, k, m, view(comp), view(win), window, (hipStream_t)stream))
            return rc;
    hipError_t e = csa::launch_mqa(q, seq, pos, T, H, d, idx, k, m, max_keys, view(comp), view(win), window, sm_scale,
                                   csa::rope_table((double)rope_base), out, lse, ws, (hipStream_t)stream);
    return hip_status(e, fn);
}

size_t csa_mqa_bwd_workspace(int64_t comp_rows, int64_t win_rows, int32_t d) {
    if (comp_rows < 0 || win_rows < 0 || d != 512) return 0;
    return (size_t)(comp_rows + win_rows) * d * 8;
}

int csa_mqa_bwd(const uint16_t* q, const int32_t* seq, const int64_t* pos, int64_t T, int32_t H, int32_t d,
                const int32_t* idx, int32_t k, int32_t m, csa_kv_t comp, csa_kv_t win, int32_t window, float sm_scale,
                float rope_base, const float* out, const float* lse, const float* dout, float* dq, float* dcomp,
                int64_t comp_rows, float* dwin, int64_t win_rows, void* ws, size_t ws_bytes, csa_stream_t stream) {
    const char* fn = "csa_mqa_bwd";
    if (int rc = check_mqa_common(fn, q, seq, pos, T, H, d, m, comp, win, window, dq, (float*)lse)) return rc;
    if (d != 512) return fail(CSA_EUNSUPPORTED, "%s: d=%d unsupported (512)", fn, d);
    if (T > 0 && (!out || !dout || !dcomp || (window > 0 && !dwin)))
        return fail(CSA_EINVAL, "%s: null pointer argument", fn);
    if (T > 0 && (!aligned16(out) || !aligned16(dout))) return fail(CSA_EINVAL, "%s: out and dout must be 16-byte aligned", fn);
    if (idx && (k < 1 || k > 2048)) return fail(CSA_EUNSUPPORTED, "%s: k=%d outside 1..2048", fn, k);
    if (!(rope_base > 0.f)) return fail(CSA_EINVAL, "%s: rope_base must be positive", fn);
    if (comp_rows < 1 || (window > 0 && win_rows < 1))
        return fail(CSA_EINVAL, "%s: comp_rows (and win_rows when window > 0) must be >= 1", fn);
    if (T == 0) return ok();
    const int64_t wr = window > 0 ? win_rows : 0;
    const size_t need = csa_mqa_bwd_workspace(comp_rows, wr, d);
    if (ws_bytes < need || !ws)
        return fail(CSA_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws_bytes);
    if (((uintptr_t)ws & 7u) != 0) return fail(CSA_EINVAL, "%s: workspace must be 8-byte aligned", fn);
    hipError_t e = csa::launch_mqa_bwd(q, seq, pos, T, H, idx, idx ? k : 0, m, view(comp), view(win), window, sm_scale,
                                       csa::rope_table((double)rope_base), out, lse, dout, dq, dcomp, comp_rows, dwin,
                                       wr, ws, (hipStream_t)stream);
    return hip_status(e, fn);
}

int hca_dense_mqa(const uint16_t* q, const int32_t* seq, const int64_t* pos, int64_t T, int32_t H, int32_t d,
                  int32_t m, int64_t max_vis, csa_kv_t comp, csa_kv_t win, int32_t window, float sm_scale,
                  float rope_base, float* out, float* lse, void* ws, size_t ws_bytes, csa_stream_t stream) {
    const char* fn = "hca_dense_mqa";
    if (int rc = check_mqa_common(fn, q, seq, pos, T, H, d, m, comp, win, window, out, lse)) return rc;
    if (max_vis < 1) return fail(CSA_EINVAL, "%s: max_vis must be >= 1", fn);
    if (!(rope_base > 0.f)) return fail(CSA_EINVAL, "%s: rope_base must be positive", fn);
    if (T == 0) return ok();
    const int64_t max_keys = max_vis + window;
    const size_t need = csa::mqa_workspace_bytes(T, H, d, max_keys);
    if (ws_bytes < need || (need > 0 && !ws))
        return fail(CSA_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws_bytes);
    if (need > 0 && !aligned16(ws)) return fail(CSA_EINVAL, "%s: workspace must be 16-byte aligned", fn);
    if (debug_checks())
        if (int rc = check_rope_range(fn, seq, pos, T, nullptr, 0, m, view(comp), view(win), window,
                                      (hipStream_t)stream))
            return rc;
    hipError_t e = csa::launch_mqa(q, seq, pos, T, H, d, nullptr, 0, m, max_keys, view(comp), view(win), window,
                                   sm_scale, csa::rope_table((double)rope_base), out, lse, ws, (hipStream_t)stream);
    return hip_status(e, fn);
}

}  // extern "C"
