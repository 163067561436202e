// fp32 causal GQA attention on the vector ALUs: full prefill with LSE, the
// lazy-ratio epilogue, and streaming attention.  Same method and outputs as
// the bf16 matrix-core kernel (see attn_bf16.hip); this variant keeps every
// product and sum in fp32 for fp32 inputs, where bf16 operands would cost
// the accuracy the caller asked for.
//
// One wave per 64 / (D/64) consecutive queries of one (batch, query head).
// K/V tiles of 32 keys are staged in LDS and read by broadcast; each lane
// keeps its share of the query and output, the running max and the running
// sum in registers.
#include "lt_internal.h"

namespace lt {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kBN = 32;

// One block of 64 lanes covers ROWS = 64 / (D/64) query rows of one (b, h):
// the D dims of a row are split over D/64 lanes (lane = half * ROWS + row),
// each holding 64 dims of the query and of the output; a dot product is the
// lane's partial sum plus its partner's (one xor shuffle).
template <int D, int MODE>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
    constexpr int SPLIT = D / 64;
    constexpr int ROWS = 64 / SPLIT;
    constexpr int CHUNK = 8;
    __shared__ __attribute__((aligned(16))) float Ks[kBN * D];
    __shared__ __attribute__((aligned(16))) float Vs[kBN * D];
    const int lane = threadIdx.x;
    const int row = lane % ROWS, half = lane / ROWS;
    const int bh = blockIdx.y;
    const int b = bh / a.Hq, h = bh % a.Hq, hk = h / a.G;
    const int N = seq_length(a.seq_len, b, a.N);
    const int q0 = blockIdx.x * ROWS;
    if (q0 >= N) return;  // past this sequence's end (whole block, before any barrier)
    const int i = q0 + row;
    const bool row_ok = i < N;
    const float c = a.c;
    const int d0 = half * 64;

    const float *kbase = (const float *)a.k + b * a.k_sb + (int64_t)hk * a.k_sh;
    const float *vbase = (const float *)a.v + b * a.v_sb + (int64_t)hk * a.v_sh;

    float q[64], o[64];
    const float *qp = (const float *)a.q + b * a.q_sb + (int64_t)h * a.q_sh +
                      (int64_t)(row_ok ? i : 0) * a.q_sn + d0;
#pragma unroll
    for (int d = 0; d < 64; d += 4) {
        float4 v = *(const float4 *)(qp + d);
        q[d] = row_ok ? v.x : 0.f;
        q[d + 1] = row_ok ? v.y : 0.f;
        q[d + 2] = row_ok ? v.z : 0.f;
        q[d + 3] = row_ok ? v.w : 0.f;
        o[d] = o[d + 1] = o[d + 2] = o[d + 3] = 0.f;
    }
    float m = kNegInf, l = 0.f;

    auto visible = [&](int j) -> bool {
        if (MODE == MODE_STREAM) return (j <= i) & ((j < a.S) | (j > i - a.R));
        return j <= i;
    };
    auto dot = [&](const float *kr) -> float {
        float acc = 0.f;
#pragma unroll
        for (int d = 0; d < 64; ++d) acc = __builtin_fmaf(q[d], kr[d0 + d], acc);
        if (SPLIT == 2) acc += __shfl_xor(acc, 32);
        return acc;
    };

    const int last_row = (q0 + ROWS < N ? q0 + ROWS : N) - 1;
    const int nt = last_row / kBN + 1;
    const int ns = a.S > 0 ? ((a.S - 1) / kBN + 1 < nt ? (a.S - 1) / kBN + 1 : nt) : 0;
    int band0 = q0 - a.R + 1;
    band0 = band0 < 0 ? 0 : band0 / kBN;
    if (band0 < ns) band0 = ns;
    const int n_iter = (MODE == MODE_STREAM) ? ns + (nt - band0) : nt;

    for (int it = 0; it < n_iter; ++it) {
        const int t = (MODE == MODE_STREAM) ? (it < ns ? it : band0 + (it - ns)) : it;
        const int key0 = t * kBN;
        __syncthreads();
        for (int e = lane * 4; e < kBN * D; e += 64 * 4) {
            const int r = e / D, d = e % D;
            const int key = key0 + r;
            float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
            if (key < N) {
                kv = *(const float4 *)(kbase + (int64_t)key * a.k_sn + d);
                vv = *(const float4 *)(vbase + (int64_t)key * a.v_sn + d);
            }
            *(float4 *)(Ks + e) = kv;
            *(float4 *)(Vs + e) = vv;
        }
        __syncthreads();
#pragma unroll 1
        for (int r0 = 0; r0 < kBN; r0 += CHUNK) {
            float s[CHUNK];
            float mx = kNegInf;
#pragma unroll
            for (int r = 0; r < CHUNK; ++r) {
                const float acc = dot(Ks + (r0 + r) * D);
                s[r] = visible(key0 + r0 + r) ? acc * c : kNegInf;
                mx = fmaxf(mx, s[r]);
            }
            const float mnew = fmaxf(m, mx);
            const float mref = (mnew == kNegInf) ? 0.f : mnew;
            const float alpha = exp2f(m - mref);
            m = mnew;
            l *= alpha;
#pragma unroll
            for (int d = 0; d < 64; ++d) o[d] *= alpha;
#pragma unroll
            for (int r = 0; r < CHUNK; ++r) {
                const float p = exp2f(s[r] - mref);
                l += p;
                const float *vr = Vs + (r0 + r) * D + d0;
#pragma unroll
                for (int d = 0; d < 64; ++d) o[d] = __builtin_fmaf(p, vr[d], o[d]);
            }
        }
    }

    const float lse2 = m + log2f(l);
    if (row_ok) {
        const float inv = 1.f / l;
        float *op = (float *)a.o + b * a.o_sb + (int64_t)h * a.o_sh + (int64_t)i * a.o_sn + d0;
#pragma unroll
        for (int d = 0; d < 64; d += 4)
            *(float4 *)(op + d) = make_float4(o[d] * inv, o[d + 1] * inv, o[d + 2] * inv,
                                              o[d + 3] * inv);
        if (a.lse != nullptr && half == 0) a.lse[((int64_t)b * a.Hq + h) * a.N + i] = lse2 * kLn2;
    }

    // Lazy-ratio epilogue: sum exp2(s_ij*c - lse2_i) over the sink keys and
    // the recent keys only (keys read straight from global memory).  Both
    // lanes of a row walk the same keys, so the xor shuffle stays paired.
    if (MODE == MODE_FULL_LAZY && q0 + ROWS > N - a.W) {
        const bool obs = row_ok && i >= N - a.W;
        float acc = 0.f;
        // Uniform loop bounds across the block's observed rows keep the
        // shuffle partners together; rows outside their own set add nothing.
        const int ilo = (q0 > N - a.W ? q0 : N - a.W);
        const int ihi = last_row;
        const int sink_end = a.S < ihi + 1 ? a.S : ihi + 1;
        int rec0 = ilo - a.R + 1;
        if (rec0 < sink_end) rec0 = sink_end;
        for (int pass = 0; pass < 2; ++pass) {
            const int j0 = pass == 0 ? 0 : rec0;
            const int j1 = pass == 0 ? sink_end : ihi + 1;
            for (int j = j0; j < j1; ++j) {
                const float sc = dot(kbase + (int64_t)j * a.k_sn);
                const bool in_set = obs & (j <= i) & ((j < a.S) | (j > i - a.R));
                const float e = exp2f(sc * c - lse2);
                acc += in_set ? e : 0.f;
            }
        }
        if (obs && half == 0) a.lazy_rows[((int64_t)b * a.Hq + h) * a.W + (i - (N - a.W))] = acc;
    }

    // Streaming slice (full attention, when asked for): the blocks of the
    // group's first query head copy their positions' K/V rows.
    if (MODE != MODE_STREAM && h % a.G == 0) {
        const StreamOut so = stream_out_late();
        if (so.k != nullptr)
            emit_stream_rows<64>((const char *)kbase, (const char *)vbase, a.k_sn, a.v_sn, so, b, hk, N, a.S, a.R, q0,
                                 q0 + ROWS < N ? q0 + ROWS : N, 4, D * 4, lane);
    }
}

template <int D>
hipError_t launch_d(const AttnArgs &a, int mode, hipStream_t st) {
    constexpr int ROWS = 64 / (D / 64);
    dim3 grid((unsigned)((a.N + ROWS - 1) / ROWS), (unsigned)(a.B * a.Hq));
    dim3 block(64);
    switch (mode) {
    case MODE_FULL:
        hipLaunchKernelGGL((attn_f32_kernel<D, MODE_FULL>), grid, block, 0, st, a);
        break;
    case MODE_FULL_LAZY:
        hipLaunchKernelGGL((attn_f32_kernel<D, MODE_FULL_LAZY>), grid, block, 0, st, a);
        break;
    default:
        hipLaunchKernelGGL((attn_f32_kernel<D, MODE_STREAM>), grid, block, 0, st, a);
        break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs &a, int D, int mode, hipStream_t st) {
    if (D == 64) return launch_d<64>(a, mode, st);
    return launch_d<128>(a, mode, st);
}

}  // namespace lt
