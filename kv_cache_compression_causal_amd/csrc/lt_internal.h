// Internal declarations shared by the kernels and the C-ABI shim (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lt.h"

namespace lt {

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
    int n_chunks;   // query heads of a group are split into n_chunks chunks
    int n_qtiles;   // query tiles per (b, kv head, chunk)
    float scale;    // softmax scale
    float c;        // scale * log2(e)
    int S, R, W;
    // Per-sequence lengths (device [B]) of a padded variable-length batch, or
    // nullptr when every sequence has N rows.  Read on the device: values are
    // clamped to [0, N].  Rows at or past a sequence's length are neither
    // read nor written; the LSE keeps its padded [B, Hq, N] layout.
    const int *seq_len;
};

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
    int n_parts;           // equal parts of the batch's keys per KV head (one workgroup each)
    int64_t part_keys;     // keys per part, ceil(B * kv_len / n_parts), when kv_lens is nullptr
    float scale, c;
};
int decode_num_parts(int B, int Hkv, int64_t kv_len);
size_t decode_ws_bytes(int B, int Hq, int D, int n_parts);
hipError_t launch_decode(const DecodeArgs &a, int dtype, hipStream_t st);

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
