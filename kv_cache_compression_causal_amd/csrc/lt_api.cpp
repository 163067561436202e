// C-ABI shim: argument validation, launch configuration and status codes.
// Every check runs before the first launch, so a failing call writes nothing
// unless the runtime refuses a launch after an earlier one of the same call.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "lt.h"
#include "lt_internal.h"
#include "lt_probe.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return LT_OK;
}

int hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(LT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// The launchers report a launch's status through hipGetLastError, which also
// returns (and clears) an error left in this thread's HIP state by earlier,
// unrelated work.  Called once validation has passed, right before a call's
// first launch, so that only this call's launches are reported.
void clear_stale_error() { (void)hipGetLastError(); }

int elem_size(int dtype) { return dtype == LT_BF16 ? 2 : dtype == LT_F32 ? 4 : 0; }

// A shape for the log (a thread-local buffer, valid until the next call).
const char *shape_str(const lt_shape *s) {
    thread_local char buf[128];
    if (s == nullptr) return "shape=NULL";
    snprintf(buf, sizeof(buf), "B=%d N=%d Hq=%d Hkv=%d D=%d dtype=%d scale=%g", s->B, s->N, s->Hq, s->Hkv, s->D,
             s->dtype, (double)s->scale);
    return buf;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int64_t kMaxRowStride = (int64_t)1 << 25;

// Sink + recent window: S + R and i - R stay far inside int.
bool window_ok(int S, int R) { return (int64_t)S + R <= ((int64_t)1 << 30); }

// A [B, H, rows, D] view: pointer, alignment and stride checks.
int check_view(const lt_view &v, const char *name, int dtype) {
    if (v.data == nullptr) return fail(LT_ERR_NULL, "%s.data is NULL", name);
    if (!aligned16(v.data)) return fail(LT_ERR_LAYOUT, "%s.data is not 16-byte aligned", name);
    const int64_t m = dtype == LT_BF16 ? 8 : 4;
    if (v.sb < 0 || v.sh < 0 || v.sn < 0 || v.sb % m || v.sh % m || v.sn % m)
        return fail(LT_ERR_LAYOUT, "%s strides (%lld, %lld, %lld) must be non-negative multiples of %lld",
                    name, (long long)v.sb, (long long)v.sh, (long long)v.sn, (long long)m);
    // A lane's byte offset into a K/V tile (up to 64 rows) is kept in 32 bits.
    if (v.sn > kMaxRowStride)
        return fail(LT_ERR_LAYOUT, "%s row stride %lld exceeds %lld elements", name, (long long)v.sn,
                    (long long)kMaxRowStride);
    return LT_OK;
}

int check_shape(const lt_shape *s) {
    if (s == nullptr) return fail(LT_ERR_NULL, "shape is NULL");
    if (s->dtype != LT_F32 && s->dtype != LT_BF16) return fail(LT_ERR_DTYPE, "dtype %d unsupported", s->dtype);
    if (s->D != 64 && s->D != 128) return fail(LT_ERR_DTYPE, "head dim %d unsupported (64 or 128)", s->D);
    if (s->B < 1 || s->N < 1 || s->Hq < 1 || s->Hkv < 1)
        return fail(LT_ERR_SHAPE, "B, N, Hq, Hkv must be >= 1 (got %d, %d, %d, %d)", s->B, s->N, s->Hq, s->Hkv);
    if (s->Hq % s->Hkv != 0) return fail(LT_ERR_SHAPE, "Hq %d is not a multiple of Hkv %d", s->Hq, s->Hkv);
    if ((int64_t)s->N * 64 > INT32_MAX) return fail(LT_ERR_SHAPE, "N %d too large", s->N);
    // Flattened rows (position * group size + head) are int, and so is the
    // workgroup count (about B * Hq * N / 384).
    if ((int64_t)s->N * (s->Hq / s->Hkv) > INT32_MAX - 4096 || (int64_t)s->B * s->Hq * s->N > ((int64_t)1 << 38))
        return fail(LT_ERR_SHAPE, "N * Hq/Hkv or B * Hq * N too large (B=%d, N=%d, Hq=%d, Hkv=%d)", s->B, s->N,
                    s->Hq, s->Hkv);
    if (!(s->scale == s->scale) || isinf(s->scale)) return fail(LT_ERR_VALUE, "scale is not finite");
    return LT_OK;
}

lt::AttnArgs make_args(const lt_shape *s, const lt_view &q, const lt_view &k, const lt_view &v,
                       const lt_view &out, float *lse, int S, int R, int W, float *lazy_rows) {
    lt::AttnArgs a{};
    a.q = q.data; a.k = k.data; a.v = v.data; a.o = out.data;
    a.lse = lse; a.lazy_rows = lazy_rows;
    a.q_sb = q.sb; a.q_sh = q.sh; a.q_sn = q.sn;
    a.k_sb = k.sb; a.k_sh = k.sh; a.k_sn = k.sn;
    a.v_sb = v.sb; a.v_sh = v.sh; a.v_sn = v.sn;
    a.o_sb = out.sb; a.o_sh = out.sh; a.o_sn = out.sn;
    a.B = s->B; a.N = s->N; a.Hq = s->Hq; a.Hkv = s->Hkv; a.G = s->Hq / s->Hkv;
    a.n_qtiles = 1;
    a.scale = s->scale > 0.f ? s->scale : 1.f / sqrtf((float)s->D);
    a.c = a.scale * 1.4426950408889634f;
    a.S = S; a.R = R; a.W = W;
    a.seq_len = nullptr;
    a.st = lt::StreamOut{};
    return a;
}

// The calls below with and without per-sequence lengths share these bodies;
// `lens` is a device array of B lengths or nullptr.

int prefill(const lt_shape *shape, const int32_t *lens, lt_view q, lt_view k, lt_view v, lt_view out,
            float *lse, int S, int R, int W, float *lazy_rows, float *lazy_ratio, hipStream_t stream,
            const lt_view *k_st = nullptr, const lt_view *v_st = nullptr) {
    int e = check_shape(shape);
    if (e) return e;
    if ((e = check_view(q, "q", shape->dtype)) || (e = check_view(k, "k", shape->dtype)) ||
        (e = check_view(v, "v", shape->dtype)) || (e = check_view(out, "out", shape->dtype)))
        return e;
    if (lse == nullptr) return fail(LT_ERR_NULL, "lse is NULL");
    if (S < 0 || R < 1 || !window_ok(S, R))
        return fail(LT_ERR_SHAPE, "need S >= 0, R >= 1, S + R <= 2^30 (got S=%d, R=%d)", S, R);
    if (W < 0 || W > shape->N) return fail(LT_ERR_SHAPE, "W %d outside [0, N=%d]", W, shape->N);
    if (W > 0 && (lazy_rows == nullptr || lazy_ratio == nullptr))
        return fail(LT_ERR_NULL, "W > 0 needs lazy_rows and lazy_ratio");
    if (k_st != nullptr && ((e = check_view(*k_st, "k_stream", shape->dtype)) ||
                            (e = check_view(*v_st, "v_stream", shape->dtype))))
        return e;
    lt::AttnArgs a = make_args(shape, q, k, v, out, lse, S, R, W, lazy_rows);
    a.seq_len = lens;
    if (k_st != nullptr)
        a.st = lt::StreamOut{k_st->data, v_st->data, k_st->sb, k_st->sh, k_st->sn, v_st->sb, v_st->sh, v_st->sn};
    const int mode = W > 0 ? lt::MODE_FULL_LAZY : lt::MODE_FULL;
    clear_stale_error();
    hipError_t he = shape->dtype == LT_BF16 ? lt::launch_attn_bf16(a, shape->D, mode, stream)
                                            : lt::launch_attn_f32(a, shape->D, mode, stream);
    if (he != hipSuccess) return hip_status(he, "prefill launch");
    if (W > 0) {
        he = lt::launch_lazy_reduce(lazy_rows, lazy_ratio, shape->B * shape->Hq, W, lens, shape->Hq, shape->N,
                                    stream);
        if (he != hipSuccess) return hip_status(he, "lazy reduce launch");
    }
    return ok();
}

int streaming(const lt_shape *shape, const int32_t *lens, lt_view q, lt_view k, lt_view v, lt_view out,
              float *lse, int S, int R, hipStream_t stream) {
    int e = check_shape(shape);
    if (e) return e;
    if ((e = check_view(q, "q", shape->dtype)) || (e = check_view(k, "k", shape->dtype)) ||
        (e = check_view(v, "v", shape->dtype)) || (e = check_view(out, "out", shape->dtype)))
        return e;
    if (S < 0 || R < 1 || !window_ok(S, R))
        return fail(LT_ERR_SHAPE, "need S >= 0, R >= 1, S + R <= 2^30 (got S=%d, R=%d)", S, R);
    lt::AttnArgs a = make_args(shape, q, k, v, out, lse, S, R, 0, nullptr);
    a.seq_len = lens;
    clear_stale_error();
    hipError_t he = shape->dtype == LT_BF16 ? lt::launch_attn_bf16(a, shape->D, lt::MODE_STREAM, stream)
                                            : lt::launch_attn_f32(a, shape->D, lt::MODE_STREAM, stream);
    if (he != hipSuccess) return hip_status(he, "streaming launch");
    return ok();
}

// Workspace of a decode call at these sizes: enough for either layout (per-
// sequence splits for uniform contexts, equal parts for per-sequence ones),
// so one workspace serves both calls.
size_t decode_ws_need(int B, int Hq, int Hkv, int D, int64_t kv_len) {
    const size_t uni = lt::decode_ws_bytes(B, Hq, D, B * lt::decode_num_splits(B, Hkv, kv_len));
    const size_t var = lt::decode_ws_bytes(B, Hq, D, lt::decode_num_parts(B, Hkv, kv_len));
    return uni > var ? uni : var;
}

// A paged cache: k_cache / v_cache are page pools (sb = the stride between
// pages) and key j of sequence b is row j % page_size of pool page
// block_table[b * max_pages + j / page_size].
struct PagedCache {
    const int32_t *block_table;
    int page_size, max_pages, num_pages;
};

// ws == nullptr with noalloc: the partial states go to the library's fixed
// per-GPU scratch array instead of a caller's workspace.  pc != nullptr: the
// cache is paged (kv_lens required, kv_len = max_pages * page_size).
int decode(int B, int Hq, int Hkv, int D, int dtype, float scale, const void *q, lt_view k_cache,
           lt_view v_cache, int64_t kv_len, const int32_t *kv_lens, void *out, float *lse, void *ws,
           size_t ws_bytes, hipStream_t stream, bool noalloc = false, const PagedCache *pc = nullptr) {
    if (dtype != LT_F32 && dtype != LT_BF16) return fail(LT_ERR_DTYPE, "dtype %d unsupported", dtype);
    if (D != 64 && D != 128) return fail(LT_ERR_DTYPE, "head dim %d unsupported (64 or 128)", D);
    if (B < 1 || Hq < 1 || Hkv < 1 || kv_len < 1 || Hq % Hkv)
        return fail(LT_ERR_SHAPE, "bad decode sizes (B=%d Hq=%d Hkv=%d kv_len=%lld)", B, Hq, Hkv, (long long)kv_len);
    if (kv_len > ((int64_t)1 << 40)) return fail(LT_ERR_SHAPE, "kv_len too large");
    if (!(scale == scale) || isinf(scale)) return fail(LT_ERR_VALUE, "scale is not finite");
    if (q == nullptr || out == nullptr) return fail(LT_ERR_NULL, "q/out is NULL");
    if (!aligned16(q) || !aligned16(out)) return fail(LT_ERR_LAYOUT, "q/out not 16-byte aligned");
    int e;
    if ((e = check_view(k_cache, "k_cache", dtype)) || (e = check_view(v_cache, "v_cache", dtype))) return e;
    if (pc != nullptr) {
        if (kv_lens == nullptr) return fail(LT_ERR_NULL, "kv_lens is NULL");
        if (pc->block_table == nullptr) return fail(LT_ERR_NULL, "block_table is NULL");
        if (((uintptr_t)pc->block_table & 3) || ((uintptr_t)kv_lens & 3))
            return fail(LT_ERR_LAYOUT, "block_table / kv_lens not 4-byte aligned");
        const int P = pc->page_size;
        if (P < 16 || P > (1 << 20) || (P & (P - 1)))
            return fail(LT_ERR_SHAPE, "page_size %d must be a power of two in [16, 2^20]", P);
        if (pc->max_pages < 1 || pc->num_pages < 1)
            return fail(LT_ERR_SHAPE, "max_pages (%d) and num_pages (%d) must be >= 1", pc->max_pages, pc->num_pages);
    }
    const size_t need = decode_ws_need(B, Hq, Hkv, D, kv_len);
    if (noalloc) {
        if (need > LT_DECODE_NOALLOC_SCRATCH_BYTES)
            return fail(LT_ERR_WORKSPACE, "these sizes need %zu bytes of scratch, more than the %zu the library holds",
                        need, (size_t)LT_DECODE_NOALLOC_SCRATCH_BYTES);
        const hipError_t he = lt::decode_scratch(&ws);
        if (he != hipSuccess) return hip_status(he, "decode scratch lookup");
        ws_bytes = LT_DECODE_NOALLOC_SCRATCH_BYTES;
    }
    if (ws == nullptr) return fail(LT_ERR_NULL, "workspace is NULL");
    if (!aligned16(ws)) return fail(LT_ERR_LAYOUT, "workspace not 16-byte aligned");
    if (ws_bytes < need) return fail(LT_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    lt::DecodeArgs a{};
    a.q = q; a.k = k_cache.data; a.v = v_cache.data;
    a.k_sb = k_cache.sb; a.k_sh = k_cache.sh; a.k_sn = k_cache.sn;
    a.v_sb = v_cache.sb; a.v_sh = v_cache.sh; a.v_sn = v_cache.sn;
    a.o = out; a.lse = lse; a.ws = (float *)ws;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv; a.D = D;
    a.kv_len = kv_len; a.kv_lens = kv_lens;
    if (kv_lens == nullptr) {  // every context kv_len long: per-sequence splits
        a.splits = lt::decode_num_splits(B, Hkv, kv_len);
        a.part_keys = lt::decode_split_keys(kv_len, a.splits);
        a.n_parts = B * a.splits;
    } else {                   // per-sequence contexts: equal parts of the batch
        a.splits = 0;
        a.part_keys = 0;
        a.n_parts = lt::decode_num_parts(B, Hkv, kv_len);
    }
    a.scale = scale > 0.f ? scale : 1.f / sqrtf((float)D);
    a.c = a.scale * 1.4426950408889634f;
    if (pc != nullptr) {
        a.block_table = pc->block_table;
        a.page = pc->page_size;
        a.page_shift = __builtin_ctz((unsigned)pc->page_size);
        a.max_pages = pc->max_pages;
        a.num_pages = pc->num_pages;
    }
    clear_stale_error();
    return hip_status(lt::launch_decode(a, dtype, stream), "decode launch");
}

int compact(lt_view k_full, lt_view v_full, lt_view k_stream, lt_view v_stream, int B, int Hkv, int N, int D,
            int dtype, int S, int R, const int32_t *lens, hipStream_t stream) {
    if (dtype != LT_F32 && dtype != LT_BF16) return fail(LT_ERR_DTYPE, "dtype %d unsupported", dtype);
    if (D != 64 && D != 128) return fail(LT_ERR_DTYPE, "head dim %d unsupported (64 or 128)", D);
    if (B < 1 || Hkv < 1 || N < 1) return fail(LT_ERR_SHAPE, "B, Hkv, N must be >= 1");
    if (S < 0 || R < 1 || !window_ok(S, R)) return fail(LT_ERR_SHAPE, "need S >= 0, R >= 1, S + R <= 2^30");
    int e;
    if ((e = check_view(k_full, "k_full", dtype)) || (e = check_view(v_full, "v_full", dtype)) ||
        (e = check_view(k_stream, "k_stream", dtype)) || (e = check_view(v_stream, "v_stream", dtype)))
        return e;
    lt::CompactArgs a{};
    a.kf = k_full.data; a.vf = v_full.data; a.ks = k_stream.data; a.vs = v_stream.data;
    a.kf_sb = k_full.sb; a.kf_sh = k_full.sh; a.kf_sn = k_full.sn;
    a.vf_sb = v_full.sb; a.vf_sh = v_full.sh; a.vf_sn = v_full.sn;
    a.ks_sb = k_stream.sb; a.ks_sh = k_stream.sh; a.ks_sn = k_stream.sn;
    a.vs_sb = v_stream.sb; a.vs_sh = v_stream.sh; a.vs_sn = v_stream.sn;
    a.B = B; a.Hkv = Hkv; a.N = N; a.D = D; a.elem = elem_size(dtype); a.S = S; a.R = R;
    a.rows_out = N <= S + R ? N : S + R;
    a.seq_len = lens;
    clear_stale_error();
    return hip_status(lt::launch_compact(a, stream), "compaction launch");
}

int append(lt_view k_stream, lt_view v_stream, const void *k_new, const void *v_new, int B, int Hkv, int D,
           int dtype, int S, int R, int64_t pos, const int32_t *pos_dev, hipStream_t stream) {
    if (dtype != LT_F32 && dtype != LT_BF16) return fail(LT_ERR_DTYPE, "dtype %d unsupported", dtype);
    if (D != 64 && D != 128) return fail(LT_ERR_DTYPE, "head dim %d unsupported (64 or 128)", D);
    if (B < 1 || Hkv < 1) return fail(LT_ERR_SHAPE, "B and Hkv must be >= 1");
    if (S < 0 || R < 1 || pos < 0 || !window_ok(S, R))
        return fail(LT_ERR_SHAPE, "need S >= 0, R >= 1, S + R <= 2^30, pos >= 0");
    if (k_new == nullptr || v_new == nullptr) return fail(LT_ERR_NULL, "k_new/v_new is NULL");
    if (!aligned16(k_new) || !aligned16(v_new)) return fail(LT_ERR_LAYOUT, "k_new/v_new not 16-byte aligned");
    int e;
    if ((e = check_view(k_stream, "k_stream", dtype)) || (e = check_view(v_stream, "v_stream", dtype))) return e;
    lt::AppendArgs a{};
    a.kn = k_new; a.vn = v_new; a.ks = k_stream.data; a.vs = v_stream.data;
    a.ks_sb = k_stream.sb; a.ks_sh = k_stream.sh; a.ks_sn = k_stream.sn;
    a.vs_sb = v_stream.sb; a.vs_sh = v_stream.sh; a.vs_sn = v_stream.sn;
    a.B = B; a.Hkv = Hkv; a.D = D; a.elem = elem_size(dtype);
    a.slot = pos < S ? pos : S + (pos - S) % R;
    a.S = S; a.R = R; a.pos = pos_dev;
    clear_stale_error();
    return hip_status(lt::launch_append(a, stream), "append launch");
}

}  // namespace

namespace lt_detail {
void set_error(const char *msg) { snprintf(g_err, sizeof(g_err), "%s", msg); }
}  // namespace lt_detail

namespace lt {
bool log_enabled() {
    static const bool on = [] {
        const char *e = getenv("LT_LOG");
        return e != nullptr && e[0] != '\0' && strcmp(e, "0") != 0;
    }();
    return on;
}

void log_printf(const char *fmt, ...) {
    if (!log_enabled()) return;
    char line[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(line, sizeof(line), fmt, ap);
    va_end(ap);
    fprintf(stderr, "[lt] %s\n", line);  // one write per line
}
}  // namespace lt

namespace {
// The outcome of a C-ABI call, when logging is on.
int logged(int status, const char *call, const char *fmt, ...) __attribute__((format(printf, 3, 4)));
int logged(int status, const char *call, const char *fmt, ...) {
    if (!lt::log_enabled()) return status;
    char args[320];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(args, sizeof(args), fmt, ap);
    va_end(ap);
    if (status == LT_OK)
        lt::log_printf("%s(%s) -> LT_OK", call, args);
    else
        lt::log_printf("%s(%s) -> %s: %s", call, args, lt_status_str(status), g_err);
    return status;
}
}  // namespace

extern "C" {

const char *lt_status_str(int status) {
    switch (status) {
    case LT_OK: return "LT_OK";
    case LT_ERR_NULL: return "LT_ERR_NULL";
    case LT_ERR_SHAPE: return "LT_ERR_SHAPE";
    case LT_ERR_DTYPE: return "LT_ERR_DTYPE";
    case LT_ERR_LAYOUT: return "LT_ERR_LAYOUT";
    case LT_ERR_WORKSPACE: return "LT_ERR_WORKSPACE";
    case LT_ERR_HIP: return "LT_ERR_HIP";
    case LT_ERR_VALUE: return "LT_ERR_VALUE";
    default: return "LT_ERR_UNKNOWN";
    }
}

const char *lt_last_error(void) { return g_err; }

int lt_prefill_attn_lse_lazy(const lt_shape *shape, lt_view q, lt_view k, lt_view v, lt_view out,
                             float *lse, int S, int R, int W, float *lazy_rows, float *lazy_ratio,
                             hipStream_t stream) {
    return logged(prefill(shape, nullptr, q, k, v, out, lse, S, R, W, lazy_rows, lazy_ratio, stream),
                  "lt_prefill_attn_lse_lazy", "%s S=%d R=%d W=%d stream=%p", shape_str(shape), S, R, W, (void *)stream);
}

int lt_prefill_attn_lse_lazy_varlen(const lt_shape *shape, const int32_t *seq_lens, lt_view q, lt_view k,
                                    lt_view v, lt_view out, float *lse, int S, int R, int W,
                                    float *lazy_rows, float *lazy_ratio, hipStream_t stream) {
    const int rc = seq_lens == nullptr ? fail(LT_ERR_NULL, "seq_lens is NULL")
                                       : prefill(shape, seq_lens, q, k, v, out, lse, S, R, W, lazy_rows, lazy_ratio,
                                                 stream);
    return logged(rc, "lt_prefill_attn_lse_lazy_varlen", "%s S=%d R=%d W=%d stream=%p", shape_str(shape), S, R, W,
                  (void *)stream);
}

int lt_prefill_attn_lse_lazy_emit(const lt_shape *shape, const int32_t *seq_lens, lt_view q, lt_view k,
                                  lt_view v, lt_view out, float *lse, int S, int R, int W, float *lazy_rows,
                                  float *lazy_ratio, lt_view k_stream, lt_view v_stream, hipStream_t stream) {
    return logged(prefill(shape, seq_lens, q, k, v, out, lse, S, R, W, lazy_rows, lazy_ratio, stream, &k_stream,
                          &v_stream),
                  "lt_prefill_attn_lse_lazy_emit", "%s S=%d R=%d W=%d lens=%s stream=%p", shape_str(shape), S, R, W,
                  seq_lens ? "device" : "none", (void *)stream);
}

int lt_streaming_attn(const lt_shape *shape, lt_view q, lt_view k, lt_view v, lt_view out,
                      float *lse, int S, int R, hipStream_t stream) {
    return logged(streaming(shape, nullptr, q, k, v, out, lse, S, R, stream), "lt_streaming_attn",
                  "%s S=%d R=%d stream=%p", shape_str(shape), S, R, (void *)stream);
}

int lt_streaming_attn_varlen(const lt_shape *shape, const int32_t *seq_lens, lt_view q, lt_view k, lt_view v,
                             lt_view out, float *lse, int S, int R, hipStream_t stream) {
    const int rc = seq_lens == nullptr ? fail(LT_ERR_NULL, "seq_lens is NULL")
                                       : streaming(shape, seq_lens, q, k, v, out, lse, S, R, stream);
    return logged(rc, "lt_streaming_attn_varlen", "%s S=%d R=%d stream=%p", shape_str(shape), S, R, (void *)stream);
}

int lt_hybrid_decode_workspace_bytes(int B, int Hq, int Hkv, int D, int64_t kv_len, size_t *bytes) {
    if (bytes == nullptr) return fail(LT_ERR_NULL, "bytes is NULL");
    if (B < 1 || Hq < 1 || Hkv < 1 || kv_len < 1 || Hq % Hkv)
        return fail(LT_ERR_SHAPE, "bad decode sizes");
    if (D != 64 && D != 128) return fail(LT_ERR_DTYPE, "head dim %d unsupported (64 or 128)", D);
    *bytes = decode_ws_need(B, Hq, Hkv, D, kv_len);
    return ok();
}

int lt_hybrid_decode_attn(int B, int Hq, int Hkv, int D, int dtype, float scale, const void *q,
                          lt_view k_cache, lt_view v_cache, int64_t kv_len, void *out, float *lse,
                          void *ws, size_t ws_bytes, hipStream_t stream) {
    return logged(decode(B, Hq, Hkv, D, dtype, scale, q, k_cache, v_cache, kv_len, nullptr, out, lse, ws, ws_bytes,
                         stream),
                  "lt_hybrid_decode_attn", "B=%d Hq=%d Hkv=%d D=%d dtype=%d kv_len=%lld ws_bytes=%zu stream=%p", B, Hq,
                  Hkv, D, dtype, (long long)kv_len, ws_bytes, (void *)stream);
}

int lt_hybrid_decode_attn_noalloc(int B, int Hq, int Hkv, int D, int dtype, float scale, const void *q,
                                  lt_view k_cache, lt_view v_cache, int64_t kv_len, void *out, float *lse,
                                  hipStream_t stream) {
    return logged(decode(B, Hq, Hkv, D, dtype, scale, q, k_cache, v_cache, kv_len, nullptr, out, lse, nullptr, 0,
                         stream, true),
                  "lt_hybrid_decode_attn_noalloc", "B=%d Hq=%d Hkv=%d D=%d dtype=%d kv_len=%lld stream=%p", B, Hq, Hkv,
                  D, dtype, (long long)kv_len, (void *)stream);
}

int lt_hybrid_decode_attn_varlen(int B, int Hq, int Hkv, int D, int dtype, float scale, const void *q,
                                 lt_view k_cache, lt_view v_cache, const int32_t *kv_lens, int64_t max_kv_len,
                                 void *out, float *lse, void *ws, size_t ws_bytes, hipStream_t stream) {
    const int rc = kv_lens == nullptr ? fail(LT_ERR_NULL, "kv_lens is NULL")
                                      : decode(B, Hq, Hkv, D, dtype, scale, q, k_cache, v_cache, max_kv_len, kv_lens,
                                               out, lse, ws, ws_bytes, stream);
    return logged(rc, "lt_hybrid_decode_attn_varlen",
                  "B=%d Hq=%d Hkv=%d D=%d dtype=%d max_kv_len=%lld ws_bytes=%zu stream=%p", B, Hq, Hkv, D, dtype,
                  (long long)max_kv_len, ws_bytes, (void *)stream);
}

int lt_hybrid_decode_attn_paged(int B, int Hq, int Hkv, int D, int dtype, float scale, const void *q,
                                lt_view k_pool, lt_view v_pool, int page_size, int num_pages,
                                const int32_t *block_table, int max_pages, const int32_t *kv_lens, void *out,
                                float *lse, void *ws, size_t ws_bytes, hipStream_t stream) {
    const PagedCache pc{block_table, page_size, max_pages, num_pages};
    const int64_t kv_len = (int64_t)max_pages * page_size;
    const int rc = max_pages < 1 || page_size < 1
                       ? fail(LT_ERR_SHAPE, "max_pages (%d) and page_size (%d) must be >= 1", max_pages, page_size)
                       : decode(B, Hq, Hkv, D, dtype, scale, q, k_pool, v_pool, kv_len, kv_lens, out, lse, ws,
                                ws_bytes, stream, false, &pc);
    return logged(rc, "lt_hybrid_decode_attn_paged",
                  "B=%d Hq=%d Hkv=%d D=%d dtype=%d page_size=%d num_pages=%d max_pages=%d ws_bytes=%zu stream=%p", B,
                  Hq, Hkv, D, dtype, page_size, num_pages, max_pages, ws_bytes, (void *)stream);
}

int lt_compact_kv_streaming(lt_view k_full, lt_view v_full, lt_view k_stream, lt_view v_stream, int B,
                            int Hkv, int N, int D, int dtype, int S, int R, hipStream_t stream) {
    return logged(compact(k_full, v_full, k_stream, v_stream, B, Hkv, N, D, dtype, S, R, nullptr, stream),
                  "lt_compact_kv_streaming", "B=%d Hkv=%d N=%d D=%d dtype=%d S=%d R=%d stream=%p", B, Hkv, N, D,
                  dtype, S, R, (void *)stream);
}

int lt_compact_kv_streaming_varlen(lt_view k_full, lt_view v_full, lt_view k_stream, lt_view v_stream,
                                   int B, int Hkv, int N, int D, int dtype, int S, int R,
                                   const int32_t *seq_lens, hipStream_t stream) {
    const int rc = seq_lens == nullptr ? fail(LT_ERR_NULL, "seq_lens is NULL")
                                       : compact(k_full, v_full, k_stream, v_stream, B, Hkv, N, D, dtype, S, R,
                                                 seq_lens, stream);
    return logged(rc, "lt_compact_kv_streaming_varlen", "B=%d Hkv=%d N=%d D=%d dtype=%d S=%d R=%d stream=%p", B,
                  Hkv, N, D, dtype, S, R, (void *)stream);
}

int lt_stream_cache_append(lt_view k_stream, lt_view v_stream, const void *k_new, const void *v_new,
                           int B, int Hkv, int D, int dtype, int S, int R, int64_t pos,
                           hipStream_t stream) {
    return logged(append(k_stream, v_stream, k_new, v_new, B, Hkv, D, dtype, S, R, pos, nullptr, stream),
                  "lt_stream_cache_append", "B=%d Hkv=%d D=%d dtype=%d S=%d R=%d pos=%lld stream=%p", B, Hkv, D,
                  dtype, S, R, (long long)pos, (void *)stream);
}

int lt_stream_cache_append_varlen(lt_view k_stream, lt_view v_stream, const void *k_new, const void *v_new,
                                  int B, int Hkv, int D, int dtype, int S, int R, const int32_t *pos,
                                  hipStream_t stream) {
    const int rc = pos == nullptr ? fail(LT_ERR_NULL, "pos is NULL")
                                  : append(k_stream, v_stream, k_new, v_new, B, Hkv, D, dtype, S, R, 0, pos, stream);
    return logged(rc, "lt_stream_cache_append_varlen", "B=%d Hkv=%d D=%d dtype=%d S=%d R=%d stream=%p", B, Hkv, D,
                  dtype, S, R, (void *)stream);
}

int lt_kv_bytes(int B, int Hkv, int64_t N, int D, int dtype, int S, int R, int64_t *full_bytes,
                int64_t *stream_bytes) {
    if (full_bytes == nullptr || stream_bytes == nullptr) return fail(LT_ERR_NULL, "output is NULL");
    const int e = elem_size(dtype);
    if (e == 0) return fail(LT_ERR_DTYPE, "dtype %d unsupported", dtype);
    if (B < 1 || Hkv < 1 || N < 1 || D < 1 || S < 0 || R < 0) return fail(LT_ERR_SHAPE, "bad sizes");
    const int64_t rows = N < (int64_t)S + R ? N : (int64_t)S + R;
    *full_bytes = 2 * (int64_t)B * Hkv * N * D * e;
    *stream_bytes = 2 * (int64_t)B * Hkv * rows * D * e;
    return ok();
}

int lt_probe_mfma_bf16(int blocks, int iters, float *sink, hipStream_t stream) {
    if (sink == nullptr) return fail(LT_ERR_NULL, "sink is NULL");
    if (blocks < 1 || iters < 1) return fail(LT_ERR_SHAPE, "blocks and iters must be >= 1");
    clear_stale_error();
    return hip_status(lt::launch_mfma_probe(blocks, iters, sink, stream), "mfma probe launch");
}

int lt_probe_read(const void *buf, size_t bytes, int blocks, unsigned *sink, hipStream_t stream) {
    if (buf == nullptr || sink == nullptr) return fail(LT_ERR_NULL, "buf/sink is NULL");
    if (blocks < 1 || bytes == 0 || bytes % 16) return fail(LT_ERR_SHAPE, "bad probe sizes");
    if (!aligned16(buf)) return fail(LT_ERR_LAYOUT, "buf not 16-byte aligned");
    clear_stale_error();
    return hip_status(lt::launch_read_probe(buf, bytes, blocks, sink, stream), "read probe launch");
}

}  // extern "C"
