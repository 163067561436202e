// Decode-step attention over one layer's KV cache (full or streaming): the
// halved KV cache the LightTransfer pages report (Chinese write-up, training
// paragraph; press-release page, results) is what this step reads, so it is
// bound by HBM bandwidth.
//
// Split-KV: workgroup (split, b*Hkv + kv head) streams keys
// [split*kps, (split+1)*kps) once and serves all G query heads of the group
// from each K/V row, keeping one online-softmax state per head.  A second
// kernel merges the per-split states with their log-sum-exps.
//
// bf16 path (matrix cores, v_mfma 16x16x32 for Q.K, 16x16x16 for P.V):
//   S^T (16 keys x 16 columns) = K Q^T, where column c < G is query head
//   hk*G + c and the rest are zero padding; the column layout keeps each
//   head's softmax state in the lanes that own its column.  O^T += V^T P^T
//   takes P^T straight from the S^T registers and V^T from the row-major V
//   tile through ds_read_b64_tr_b16.  Each 64-key tile is loaded with
//   coalesced 128-bit global loads into LDS; wave w handles 16 of its keys.
// fp32 path (vector ALUs): lane = pair of head dims, one key at a time.
#include "lt_internal.h"

namespace lt {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kTile = 64;  // keys per workgroup iteration (bf16 path)

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;

__device__ __forceinline__ bf16x4 lds_read_tr(const bf16 *p) {
    i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4 *)(p));
    return __builtin_bit_cast(bf16x4, r);
}

// Partial state layout: ws[(bh * n_splits + split) * (D + 2) + {0..D-1: o/l, D: m (log2), D+1: l}]
template <int D>
__global__ __launch_bounds__(256) void decode_bf16_kernel(DecodeArgs a) {
    constexpr int KS = D / 32;
    constexpr int DB = D / 16;
    constexpr int STR = D + 16;
    constexpr int CH = kTile * D / 8;
    // The K/V tiles and, after the key loop, the cross-wave merge buffer share LDS.
    constexpr int TILE_BYTES = 2 * kTile * STR * (int)sizeof(bf16);
    constexpr int RED_BYTES = 4 * 16 * (D + 1) * (int)sizeof(float);
    __shared__ __attribute__((aligned(16))) char smem[TILE_BYTES > RED_BYTES ? TILE_BYTES : RED_BYTES];
    __shared__ float red_m[4][16], red_l[4][16];
    bf16 *const Ks = (bf16 *)smem;
    bf16 *const Vs = Ks + kTile * STR;
    float (*const red_o)[16][D + 1] = (float (*)[16][D + 1])smem;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int split = blockIdx.x;
    const int bhk = blockIdx.y;
    const int b = bhk / a.Hkv, hk = bhk % a.Hkv;
    const int G = a.G;
    const int64_t kbeg = (int64_t)split * a.keys_per_split;
    const int64_t kend = kbeg + a.keys_per_split < a.kv_len ? kbeg + a.keys_per_split : a.kv_len;
    const float c = a.c;

    const bf16 *kbase = (const bf16 *)a.k + b * a.k_sb + (int64_t)hk * a.k_sh;
    const bf16 *vbase = (const bf16 *)a.v + b * a.v_sb + (int64_t)hk * a.v_sh;

    bf16x8 qreg[KS];
    {
        const bool col_ok = c16 < G;
        const bf16 *qp = (const bf16 *)a.q + ((int64_t)b * a.Hq + hk * G + (col_ok ? c16 : 0)) * D + g * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            bf16x8 v = *(const bf16x8 *)(qp + ks * 32);
            if (!col_ok) v = bf16x8{};
            qreg[ks] = v;
        }
    }

    f32x4 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = kNegInf, l = 0.f;

    for (int64_t t0 = kbeg; t0 < kend; t0 += kTile) {
        __syncthreads();
#pragma unroll
        for (int it = 0; it < CH / 256; ++it) {
            const int cidx = it * 256 + tid;
            const int r = cidx / (D / 8), c8 = cidx % (D / 8);
            const int64_t key = t0 + r;
            bf16x8 kv = bf16x8{}, vv = bf16x8{};
            if (key < kend) {
                kv = *(const bf16x8 *)(kbase + key * a.k_sn + c8 * 8);
                vv = *(const bf16x8 *)(vbase + key * a.v_sn + c8 * 8);
            }
            *(bf16x8 *)(Ks + r * STR + c8 * 8) = kv;
            *(bf16x8 *)(Vs + r * STR + c8 * 8) = vv;
        }
        __syncthreads();
        const int64_t wkey0 = t0 + 16 * wave;
        if (wkey0 >= kend) continue;
        f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 A = *(const bf16x8 *)(Ks + (16 * wave + c16) * STR + ks * 32 + g * 8);
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, qreg[ks], s, 0, 0, 0);
        }
        float mx = kNegInf;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (wkey0 + 4 * g + r >= kend) s[r] = kNegInf;
            mx = fmaxf(mx, s[r]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(m, mx * c);
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);
        m = mnew;
        bf16x4 p4;
        float rs = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -mnew));
            rs += p;
            p4[r] = (bf16)p;
        }
        l = l * alpha + rs;
        const bf16 *vrow = Vs + (16 * wave + 4 * g + (c16 >> 2)) * STR + 4 * (c16 & 3);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            o[db] *= alpha;
            const bf16x4 A = lds_read_tr(vrow + db * 16);
            o[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, p4, o[db], 0, 0, 0);
        }
    }

    // Merge the four waves' states for each column, then store the split's partial.
    __syncthreads();  // every wave is done reading the K/V tiles
    float lt = l + __shfl_xor(l, 16);
    lt += __shfl_xor(lt, 32);
    if (g == 0) {
        red_m[wave][c16] = m;
        red_l[wave][c16] = lt;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) red_o[wave][c16][db * 16 + 4 * g + r] = o[db][r];
    __syncthreads();
    for (int e = tid; e < G * D; e += 256) {
        const int col = e / D, d = e % D;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, red_m[w][col]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float f = red_m[w][col] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(red_m[w][col] - M);
            L += f * red_l[w][col];
            O += f * red_o[w][col][d];
        }
        float *dst = a.ws + (((int64_t)b * a.Hq + hk * G + col) * a.n_splits + split) * (D + 2);
        dst[d] = O / L;
        if (d == 0) {
            dst[D] = M;
            dst[D + 1] = L;
        }
    }
}

// fp32: block of 64 lanes per (split, b*Hq + h); lane owns dims lane, lane+64.
template <int D>
__global__ __launch_bounds__(64) void decode_f32_kernel(DecodeArgs a) {
    constexpr int PER = D / 64;
    const int lane = threadIdx.x;
    const int split = blockIdx.x;
    const int bh = blockIdx.y;
    const int b = bh / a.Hq, h = bh % a.Hq, hk = h / a.G;
    const int64_t kbeg = (int64_t)split * a.keys_per_split;
    const int64_t kend = kbeg + a.keys_per_split < a.kv_len ? kbeg + a.keys_per_split : a.kv_len;
    const float *kbase = (const float *)a.k + b * a.k_sb + (int64_t)hk * a.k_sh;
    const float *vbase = (const float *)a.v + b * a.v_sb + (int64_t)hk * a.v_sh;
    float q[PER], o[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        q[u] = ((const float *)a.q)[(int64_t)bh * D + lane + 64 * u];
        o[u] = 0.f;
    }
    float m = kNegInf, l = 0.f;
    for (int64_t j = kbeg; j < kend; ++j) {
        float part = 0.f;
#pragma unroll
        for (int u = 0; u < PER; ++u) part = __builtin_fmaf(q[u], kbase[j * a.k_sn + lane + 64 * u], part);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
        const float s = part * a.c;
        const float mnew = fmaxf(m, s);
        const float alpha = exp2f(m - mnew);
        const float p = exp2f(s - mnew);
        m = mnew;
        l = l * alpha + p;
#pragma unroll
        for (int u = 0; u < PER; ++u) o[u] = __builtin_fmaf(p, vbase[j * a.v_sn + lane + 64 * u], o[u] * alpha);
    }
    float *dst = a.ws + ((int64_t)bh * a.n_splits + split) * (D + 2);
#pragma unroll
    for (int u = 0; u < PER; ++u) dst[lane + 64 * u] = o[u] / l;
    if (lane == 0) {
        dst[D] = m;
        dst[D + 1] = l;
    }
}

// Merge split partials: out = sum_s w_s o_s / sum_s w_s, w_s = l_s 2^(m_s - M);
// lse = (M + log2 sum_s w_s) ln 2.
template <int D, typename T>
__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeArgs a) {
    const int bh = blockIdx.x;
    const int d = threadIdx.x;
    const float *src = a.ws + (int64_t)bh * a.n_splits * (D + 2);
    float M = kNegInf;
    for (int s = 0; s < a.n_splits; ++s) M = fmaxf(M, src[s * (D + 2) + D]);
    float L = 0.f, O = 0.f;
    for (int s = 0; s < a.n_splits; ++s) {
        const float w = src[s * (D + 2) + D + 1] * __builtin_amdgcn_exp2f(src[s * (D + 2) + D] - M);
        L += w;
        if (d < D) O += w * src[s * (D + 2) + d];
    }
    if (d < D) ((T *)a.o)[(int64_t)bh * D + d] = (T)(O / L);
    if (d == 0 && a.lse != nullptr) a.lse[bh] = (M + log2f(L)) * kLn2;
}

}  // namespace

int decode_num_splits(int B, int Hkv, int64_t kv_len) {
    // Aim for about 1024 workgroups (4 per CU) so that enough 64-key tiles are
    // in flight to cover HBM latency; never fewer than one tile per split.
    const int64_t units = (int64_t)B * Hkv;
    int64_t want = (1024 + units - 1) / units;
    const int64_t max_splits = (kv_len + kTile - 1) / kTile;
    if (want > max_splits) want = max_splits;
    if (want < 1) want = 1;
    int64_t kps = (kv_len + want - 1) / want;
    kps = (kps + kTile - 1) / kTile * kTile;
    return (int)((kv_len + kps - 1) / kps);
}

size_t decode_ws_bytes(int B, int Hq, int D, int n_splits) {
    return (size_t)B * Hq * n_splits * (D + 2) * sizeof(float);
}

hipError_t launch_decode(const DecodeArgs &a, int dtype, hipStream_t st) {
    if (dtype == LT_BF16) {
        dim3 grid((unsigned)a.n_splits, (unsigned)(a.B * a.Hkv));
        if (a.D == 64) {
            hipLaunchKernelGGL(decode_bf16_kernel<64>, grid, dim3(256), 0, st, a);
            hipLaunchKernelGGL((decode_combine_kernel<64, bf16>), dim3(a.B * a.Hq), dim3(128), 0, st, a);
        } else {
            hipLaunchKernelGGL(decode_bf16_kernel<128>, grid, dim3(256), 0, st, a);
            hipLaunchKernelGGL((decode_combine_kernel<128, bf16>), dim3(a.B * a.Hq), dim3(128), 0, st, a);
        }
    } else {
        dim3 grid((unsigned)a.n_splits, (unsigned)(a.B * a.Hq));
        if (a.D == 64) {
            hipLaunchKernelGGL(decode_f32_kernel<64>, grid, dim3(64), 0, st, a);
            hipLaunchKernelGGL((decode_combine_kernel<64, float>), dim3(a.B * a.Hq), dim3(128), 0, st, a);
        } else {
            hipLaunchKernelGGL(decode_f32_kernel<128>, grid, dim3(64), 0, st, a);
            hipLaunchKernelGGL((decode_combine_kernel<128, float>), dim3(a.B * a.Hq), dim3(128), 0, st, a);
        }
    }
    return hipGetLastError();
}

}  // namespace lt
