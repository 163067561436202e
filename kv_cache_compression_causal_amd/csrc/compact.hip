// Switch one layer's KV cache to its streaming version (LightTransfer pages:
// Chinese write-up, "solution 2"; project page, Figure 2 caption): keep the
// S sink rows and the R most recent rows of every (batch, KV head), i.e. the
// sink + recent key set of the last query, and drop the rest.  A byte copy
// in 16-byte chunks: output row r < S comes from row r, row r >= S from row
// N - R + (r - S); with N <= S + R all N rows are copied in order.
#include "lt_internal.h"

namespace lt {
namespace {

__global__ __launch_bounds__(256) void compact_kernel(CompactArgs a) {
    const int row_bytes = a.D * a.elem;
    const int chunks_per_row = row_bytes / 16;
    const int64_t per_head = (int64_t)a.rows_out * chunks_per_row;
    const int64_t total = (int64_t)a.B * a.Hkv * per_head * 2;
    const bool all_rows = a.N <= a.S + a.R;
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int which = (int)(idx / (total / 2));  // 0 = K, 1 = V
        int64_t rem = idx % (total / 2);
        const int bh = (int)(rem / per_head);
        rem %= per_head;
        const int r = (int)(rem / chunks_per_row);
        const int ch = (int)(rem % chunks_per_row);
        const int b = bh / a.Hkv, h = bh % a.Hkv;
        const int src_row = (all_rows || r < a.S) ? r : a.N - a.R + (r - a.S);
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

}  // namespace

hipError_t launch_compact(const CompactArgs &a, hipStream_t st) {
    const int64_t total = (int64_t)a.B * a.Hkv * a.rows_out * (a.D * a.elem / 16) * 2;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(compact_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace lt
