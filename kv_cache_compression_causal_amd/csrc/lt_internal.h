// Internal declarations shared by the kernels and the C-ABI shim (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "lt.h"

namespace lt {

// Library-side logging: with the environment variable LT_LOG set (to
// anything but "0"), every C-ABI call prints one line to stderr (call,
// sizes, status) and every kernel launch its kernel and launch shape.
bool log_enabled();
void log_printf(const char *fmt, ...) __attribute__((format(printf, 1, 2)));

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

// Attention kernel variants.
enum Mode : int {
    MODE_FULL = 0,       // causal attention + LSE
    MODE_FULL_LAZY = 1,  // causal attention + LSE + lazy-ratio epilogue
    MODE_STREAM = 2      // sink + recent attention (+ optional LSE)
};

// Destination of a layer's streaming slice (see AttnArgs::st).
struct StreamOut {
    void *k, *v;  // [B, Hkv, >= min(n, S+R), D], or k == nullptr: not written
    int64_t ks_sb, ks_sh, ks_sn, vs_sb, vs_sh, vs_sn;
};

struct AttnArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;        // [B,Hq,N] or nullptr (streaming only)
    float *lazy_rows;  // [B,Hq,W] (lazy mode)
    int64_t q_sb, q_sh, q_sn;
    int64_t k_sb, k_sh, k_sn;
    int64_t v_sb, v_sh, v_sn;
    int64_t o_sb, o_sh, o_sn;
    int B, N, Hq, Hkv, G;
    int n_qtiles;   // query tiles per (b, kv head, chunk)
    float scale;    // softmax scale
    float c;        // scale * log2(e)
    int S, R, W;
    // Per-sequence lengths (device [B]) of a padded variable-length batch, or
    // nullptr when every sequence has N rows.  Read on the device: values are
    // clamped to [0, N].  Rows at or past a sequence's length are neither
    // read nor written; the LSE keeps its padded [B, Hq, N] layout.
    const int *seq_len;
    // Streaming slice written by the full-attention modes: the K/V rows of
    // positions [0, S) and [n-R, n) of each (batch, KV head), in ring slot
    // order.  Read with kernel_arg_late (below), not as a.st.
    StreamOut st;
};

// A field of the kernel's first argument, read at this point of the kernel.
// Kernel-argument loads are normally all issued at the entry and kept in
// scalar registers; a field used only after the main loop then occupies
// registers through it (and pushes others into spills).  The segment
// pointer is made opaque here, so the load cannot move above this point.
// Explicit arguments start at offset 0 of the kernel-argument segment.
template <typename T>
__device__ __forceinline__ T kernel_arg_late(size_t offset) {
    const __attribute__((address_space(4))) char *p =
        (const __attribute__((address_space(4))) char *)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(p));
    return *(const __attribute__((address_space(4))) T *)(p + offset);
}

// The streaming-slice destination of the kernel's AttnArgs, read late
// field by field (a struct copy out of the argument address space has no
// constructor to use).
__device__ __forceinline__ StreamOut stream_out_late() {
    constexpr size_t o = offsetof(AttnArgs, st);
    StreamOut so;
    so.k = kernel_arg_late<void *>(o + offsetof(StreamOut, k));
    so.v = kernel_arg_late<void *>(o + offsetof(StreamOut, v));
    so.ks_sb = kernel_arg_late<int64_t>(o + offsetof(StreamOut, ks_sb));
    so.ks_sh = kernel_arg_late<int64_t>(o + offsetof(StreamOut, ks_sh));
    so.ks_sn = kernel_arg_late<int64_t>(o + offsetof(StreamOut, ks_sn));
    so.vs_sb = kernel_arg_late<int64_t>(o + offsetof(StreamOut, vs_sb));
    so.vs_sh = kernel_arg_late<int64_t>(o + offsetof(StreamOut, vs_sh));
    so.vs_sn = kernel_arg_late<int64_t>(o + offsetof(StreamOut, vs_sn));
    return so;
}

// Ring slot of position p in the streaming cache of a sequence of n rows:
// every row in order when n <= S + R; otherwise sinks in their own slots and
// the recent rows on a ring of R slots.
__device__ __forceinline__ int stream_slot(int p, int n, int S, int R) {
    return (n <= S + R || p < S) ? p : S + (p - S) % R;
}

// Copy the streaming-slice rows among positions [p_lo, p_hi) of one
// (sequence b, KV head hk) -- K rows at kbase + p*k_sn, V rows at
// vbase + p*v_sn (elements of `elem` bytes, rows of `row_bytes`) -- into
// their slots; the NT threads of the calling block share the 16-byte chunks.
// (The caller passes the head's base pointers it already holds, so that no
// other argument stays live through its main loop for this.)
template <int NT>
__device__ __forceinline__ void emit_stream_rows(const char *kbase, const char *vbase, int64_t k_sn, int64_t v_sn,
                                                 const StreamOut &so, int b, int hk, int n, int S, int R, int p_lo,
                                                 int p_hi, int elem, int row_bytes, int tid) {
    const int cpr = row_bytes / 16;
    const int total = (p_hi - p_lo) * 2 * cpr;
    for (int idx = tid; idx < total; idx += NT) {
        const int p = p_lo + idx / (2 * cpr);
        if (p >= S && p < n - R) continue;  // neither a sink nor a recent row
        const int which = (idx / cpr) & 1, ch = idx % cpr;
        const int64_t slot = stream_slot(p, n, S, R);
        const char *src = which == 0 ? kbase + (int64_t)p * k_sn * elem : vbase + (int64_t)p * v_sn * elem;
        char *dst = which == 0
            ? (char *)so.k + ((int64_t)b * so.ks_sb + (int64_t)hk * so.ks_sh + slot * so.ks_sn) * elem
            : (char *)so.v + ((int64_t)b * so.vs_sb + (int64_t)hk * so.vs_sh + slot * so.vs_sn) * elem;
        *(uint4 *)(dst + ch * 16) = *(const uint4 *)(src + ch * 16);
    }
}

// Debug builds (compiled with LT_POISON_LDS, liblt_debug.so): a kernel fills
// its LDS with all-ones words -- NaN as bf16 and as fp32 -- before first use,
// so that a read of LDS the kernel never wrote shows up in its outputs; the
// debug library's results must equal the release library's bit for bit.
// NT threads of the workgroup take part; bytes is a multiple of 16.
template <int NT>
__device__ __forceinline__ void poison_lds(void *lds, int bytes, int tid) {
#ifdef LT_POISON_LDS
    for (int i = tid * 16; i < bytes; i += NT * 16) *(uint4 *)((char *)lds + i) = make_uint4(~0u, ~0u, ~0u, ~0u);
    __syncthreads();
#else
    (void)lds, (void)bytes, (void)tid;
#endif
}

// Length of sequence b: N, or seq_len[b] clamped to [0, N].
__device__ __forceinline__ int seq_length(const int *seq_len, int b, int N) {
    if (seq_len == nullptr) return N;
    const int x = seq_len[b];
    return x < 0 ? 0 : (x > N ? N : x);
}

// Launchers (return hipError_t of the launch).
hipError_t launch_attn_bf16(const AttnArgs &a, int D, int mode, hipStream_t st);
hipError_t launch_attn_f32(const AttnArgs &a, int D, int mode, hipStream_t st);
// Per-head mean of the W lazy rows.  With seq_len (device [B], Hq heads per
// sequence) a sequence of n < W rows averages its n rows, the W - n slots of
// rows before its start are set to NaN, and an empty sequence's ratio is NaN.
hipError_t launch_lazy_reduce(float *lazy_rows, float *lazy_ratio, int BH, int W, const int *seq_len,
                              int Hq, int N, hipStream_t st);

struct DecodeArgs {
    const void *q;  // [B,Hq,D]
    const void *k, *v;
    int64_t k_sb, k_sh, k_sn, v_sb, v_sh, v_sn;
    void *o;        // [B,Hq,D]
    float *lse;     // [B,Hq] or nullptr
    float *ws;      // partials
    int B, Hq, Hkv, G, D;
    int64_t kv_len;        // every context's length, or the bound of kv_lens
    const int *kv_lens;    // per-sequence context (device [B], clamped to [0, kv_len]) or nullptr
    // Uniform contexts (kv_lens == nullptr): `splits` splits of part_keys keys
    // per sequence.  Per-sequence contexts: n_parts equal parts of the batch's
    // keys per KV head (one workgroup each).
    int splits;
    int64_t part_keys;
    int n_parts;
    float scale, c;
    // Paged caches (page > 0, a power of two >= 16; kv_lens is then set): k
    // and v are page pools, k_sb / v_sb the stride between pages, k_sh / v_sh
    // between KV heads within a page, k_sn / v_sn between a page's rows.  Key
    // j of sequence b sits in row j % page of pool page
    // block_table[b * max_pages + j / page], clamped to [0, num_pages).
    // kv_len is max_pages * page.
    const int *block_table;
    int page, page_shift, max_pages, num_pages;
};
int decode_num_splits(int B, int Hkv, int64_t kv_len);
int64_t decode_split_keys(int64_t kv_len, int splits);
int decode_num_parts(int B, int Hkv, int64_t kv_len);
size_t decode_ws_bytes(int B, int Hq, int D, int n_parts);
hipError_t launch_decode(const DecodeArgs &a, int dtype, hipStream_t st);
// Device address of the current GPU's fixed decode scratch array
// (LT_DECODE_NOALLOC_SCRATCH_BYTES), looked up on the first call per GPU.
hipError_t decode_scratch(void **ptr);

struct CompactArgs {
    const void *kf, *vf;
    void *ks, *vs;
    int64_t kf_sb, kf_sh, kf_sn, vf_sb, vf_sh, vf_sn;
    int64_t ks_sb, ks_sh, ks_sn, vs_sb, vs_sh, vs_sn;
    int B, Hkv, N, D, elem, S, R, rows_out;
    const int *seq_len;  // per-sequence N (device [B], clamped to [0, N]) or nullptr
};
hipError_t launch_compact(const CompactArgs &a, hipStream_t st);

struct AppendArgs {
    const void *kn, *vn;  // [B,Hkv,D] contiguous
    void *ks, *vs;
    int64_t ks_sb, ks_sh, ks_sn, vs_sb, vs_sh, vs_sn;
    int B, Hkv, D, elem;
    int64_t slot;
    int S, R;
    const int *pos;  // per-sequence position (device [B]; negative: no write) or nullptr: slot
};
hipError_t launch_append(const AppendArgs &a, hipStream_t st);
hipError_t launch_mfma_probe(int blocks, int iters, float *sink, hipStream_t st);
hipError_t launch_read_probe(const void *buf, size_t bytes, int blocks, unsigned *sink, hipStream_t st);

}  // namespace lt
