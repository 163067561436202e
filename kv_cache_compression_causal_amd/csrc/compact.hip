// Switch one layer's KV cache to its streaming version (LightTransfer pages:
// Chinese write-up, "solution 2"; project page, Figure 2 caption): keep the
// S sink rows and the R most recent rows of every (batch, KV head), i.e. the
// sink + recent key set of the last query, and drop the rest.  A byte copy
// in 16-byte chunks.  Slot r < S holds position r; the recent positions sit
// on a ring of R slots, position p in slot S + (p - S) mod R, so that the
// decode steps that follow can write each new token over the oldest recent
// one (append_kernel); with N <= S + R all N rows are copied in order.
// Attention does not depend on the slot order.
#include "lt_internal.h"

namespace lt {
namespace {

__global__ __launch_bounds__(256) void compact_kernel(CompactArgs a) {
    const int row_bytes = a.D * a.elem;
    const int chunks_per_row = row_bytes / 16;
    const int64_t per_head = (int64_t)a.rows_out * chunks_per_row;
    const int64_t total = (int64_t)a.B * a.Hkv * per_head * 2;
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int which = (int)(idx / (total / 2));  // 0 = K, 1 = V
        int64_t rem = idx % (total / 2);
        const int bh = (int)(rem / per_head);
        rem %= per_head;
        const int r = (int)(rem / chunks_per_row);
        const int ch = (int)(rem % chunks_per_row);
        const int b = bh / a.Hkv, h = bh % a.Hkv;
        // this sequence's length: rows_out = min(n, S + R) rows are kept
        const int n = seq_length(a.seq_len, b, a.N);
        if (r >= (n < a.S + a.R ? n : a.S + a.R)) continue;
        int src_row = r;
        if (n > a.S + a.R && r >= a.S) {
            // the recent position p in [n-R, n) whose ring slot is r
            const int base = n - a.R;
            int m = (r - base) % a.R;
            if (m < 0) m += a.R;
            src_row = base + m;
        }
        const char *src;
        char *dst;
        if (which == 0) {
            src = (const char *)a.kf + ((int64_t)b * a.kf_sb + (int64_t)h * a.kf_sh + (int64_t)src_row * a.kf_sn) * a.elem;
            dst = (char *)a.ks + ((int64_t)b * a.ks_sb + (int64_t)h * a.ks_sh + (int64_t)r * a.ks_sn) * a.elem;
        } else {
            src = (const char *)a.vf + ((int64_t)b * a.vf_sb + (int64_t)h * a.vf_sh + (int64_t)src_row * a.vf_sn) * a.elem;
            dst = (char *)a.vs + ((int64_t)b * a.vs_sb + (int64_t)h * a.vs_sh + (int64_t)r * a.vs_sn) * a.elem;
        }
        *(uint4 *)(dst + ch * 16) = *(const uint4 *)(src + ch * 16);
    }
}

// Write the new token's K and V rows (k_new, v_new [B, Hkv, D] contiguous)
// into slot `slot` of every (batch, KV head) of the streaming cache.
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
    const int chunks_per_row = a.D * a.elem / 16;
    const int64_t total = (int64_t)a.B * a.Hkv * chunks_per_row * 2;
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int which = (int)(idx / (total / 2));  // 0 = K, 1 = V
        const int64_t rem = idx % (total / 2);
        const int bh = (int)(rem / chunks_per_row), ch = (int)(rem % chunks_per_row);
        const int b = bh / a.Hkv, h = bh % a.Hkv;
        int64_t slot = a.slot;
        if (a.pos != nullptr) {  // this sequence's own position and its ring slot
            const int p = a.pos[b];
            if (p < 0) continue;
            slot = p < a.S ? p : a.S + (p - a.S) % a.R;
        }
        const char *src = (const char *)(which == 0 ? a.kn : a.vn) + ((int64_t)bh * a.D) * a.elem;
        char *dst = which == 0
                        ? (char *)a.ks + ((int64_t)b * a.ks_sb + (int64_t)h * a.ks_sh + slot * a.ks_sn) * a.elem
                        : (char *)a.vs + ((int64_t)b * a.vs_sb + (int64_t)h * a.vs_sh + slot * a.vs_sn) * a.elem;
        *(uint4 *)(dst + ch * 16) = *(const uint4 *)(src + ch * 16);
    }
}

}  // namespace

hipError_t launch_append(const AppendArgs &a, hipStream_t st) {
    const int64_t total = (int64_t)a.B * a.Hkv * (a.D * a.elem / 16) * 2;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    if (log_enabled()) log_printf("  launch append_kernel grid %lld x 256 threads", (long long)blocks);
    hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_compact(const CompactArgs &a, hipStream_t st) {
    const int64_t total = (int64_t)a.B * a.Hkv * a.rows_out * (a.D * a.elem / 16) * 2;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    if (log_enabled()) log_printf("  launch compact_kernel grid %lld x 256 threads", (long long)blocks);
    hipLaunchKernelGGL(compact_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace lt
