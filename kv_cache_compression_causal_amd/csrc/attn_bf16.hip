// bf16 causal GQA attention on the gfx950 matrix cores: full prefill with LSE,
// the fused lazy-ratio epilogue, and streaming (sink + recent) attention.
//
// Method (LightTransfer pages): Chinese write-up, "solution 1" -- the LSE that
// Flash Attention produces is the lazy ratio's denominator, the numerator
// only needs the sink and recent keys; press-release page, "LightTransfer
// method" -- the ratio is the attention mass on the initial and recent keys;
// project page, "Introduction" -- converted layers run streaming attention.
//
// Work decomposition (one workgroup = 4 waves = 256 threads):
//   a workgroup owns one (batch, KV head, chunk of GC query heads of that
//   group) and BM = 64*PB consecutive query positions.  Wave w owns 16*PB of
//   those positions for all GC heads: RB = GC*PB row blocks of 16 queries.
//   Every K/V tile of BN keys is staged once in LDS and read by all four
//   waves, so the GQA group shares each tile; inside a wave each K fragment
//   read from LDS feeds RB matrix-core ops.
//
// Matrix-core formulation (v_mfma_f32_16x16x32_bf16, 64 lanes, lane l:
// c = l%16, g = l/16):
//   S^T = K Q^T  -- A = K rows (key c, dims 8g..8g+7 of a 32-dim step) read
//                   with one 128-bit LDS load; B = Q^T held in registers.
//                   The result gives lane l query column c and keys 4g..4g+3
//                   of the 16-key block, so all softmax state of a query
//                   stays in the lanes that own its column.
//   O^T += V^T P^T -- B = P^T straight from the S^T registers (two 16-key
//                   blocks make one 32-key step); A = V^T read from the
//                   row-major V tile with two ds_read_b64_tr_b16 transposing
//                   loads.  Both operands enumerate the 32 keys of a step in
//                   the same (g, element) order, which is all the product
//                   needs.
//   Row statistics: max over a lane's own 4*BN/16 values, then across the
//   four lane groups (xor 16, xor 32); the running sum stays per lane and is
//   reduced once at the end.  Scores are kept in log2 units (scale*log2 e
//   folded into one fma before exp2).
//
// Launch order: blockIdx.x % U picks the (batch, KV head, chunk) unit so that
// with B*Hkv*chunks a multiple of 8 each XCD (dispatch is round-robin over
// the 8 XCDs) keeps one KV head's K/V in its own L2; blockIdx.x / U walks the
// query tiles longest-first to even out the causal triangle.
#include "lt_internal.h"

namespace lt {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x4 lds_read_tr(const bf16 *p) {
    i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4 *)(p));
    return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 concat(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int D, int GC, int PB, int BN, int MODE>
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnArgs a) {
    constexpr int RB = GC * PB;   // 16-query row blocks per wave
    constexpr int BM = 64 * PB;   // query positions per workgroup
    constexpr int KS = D / 32;    // 32-dim steps of Q.K
    constexpr int DB = D / 16;    // 16-dim blocks of O
    constexpr int NKB = BN / 16;  // 16-key blocks per tile
    constexpr int NT2 = BN / 32;  // 32-key steps of P.V per tile
    constexpr int STR = D + 16;   // LDS row stride (elements): rows shift by 32 B
    constexpr int TILE = BN * STR;
    constexpr int CH = BN * D / 8;  // 16-byte chunks per tile
    static_assert(CH % 256 == 0, "tile must split evenly over 256 threads");
    __shared__ __attribute__((aligned(16))) bf16 lds[2 * TILE];
    bf16 *const Ks = lds;
    bf16 *const Vs = lds + TILE;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int U = a.B * a.Hkv * a.n_chunks;
    const int unit = (int)(blockIdx.x % U);
    const int qt = a.n_qtiles - 1 - (int)(blockIdx.x / U);
    const int chunk = unit % a.n_chunks;
    const int bhk = unit / a.n_chunks;
    const int hk = bhk % a.Hkv, b = bhk / a.Hkv;
    const int N = a.N;
    const int q0 = qt * BM;
    const int wpos0 = q0 + wave * 16 * PB;
    const int h0 = hk * a.G + chunk * GC;
    const float c = a.c;

    const bf16 *kbase = (const bf16 *)a.k + b * a.k_sb + hk * a.k_sh;
    const bf16 *vbase = (const bf16 *)a.v + b * a.v_sb + hk * a.v_sh;

    // Q^T operand: lane holds query column c16 of each row block, dims 8g.. of each step.
    bf16x8 qreg[RB][KS];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int pos = wpos0 + (rb % PB) * 16 + c16;
        const bf16 *qp = (const bf16 *)a.q + b * a.q_sb + (int64_t)(h0 + rb / PB) * a.q_sh +
                         (int64_t)(pos < N ? pos : 0) * a.q_sn + g * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            bf16x8 v = *(const bf16x8 *)(qp + ks * 32);
            if (pos >= N) v = bf16x8{};
            qreg[rb][ks] = v;
        }
    }

    // Stage keys [t*BN, t*BN+BN) of K (and V) into LDS; rows past N are zero.
    auto load_tile = [&](int t, bool with_v) {
        const int key0 = t * BN;
#pragma unroll
        for (int it = 0; it < CH / 256; ++it) {
            const int cidx = it * 256 + tid;
            const int r = cidx / (D / 8), c8 = cidx % (D / 8);
            const int key = key0 + r;
            bf16x8 kv = bf16x8{}, vv = bf16x8{};
            if (key < N) {
                kv = *(const bf16x8 *)(kbase + (int64_t)key * a.k_sn + c8 * 8);
                if (with_v) vv = *(const bf16x8 *)(vbase + (int64_t)key * a.v_sn + c8 * 8);
            }
            *(bf16x8 *)(Ks + r * STR + c8 * 8) = kv;
            if (with_v) *(bf16x8 *)(Vs + r * STR + c8 * 8) = vv;
        }
    };

    // S^T for the staged tile: s[kb][rb] holds keys kb*16+4g+r, query column c16.
    auto qk = [&](f32x4 (&s)[NKB][RB]) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) s[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const bf16x8 A = *(const bf16x8 *)(Ks + (kb * 16 + c16) * STR + ks * 32 + g * 8);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    s[kb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, qreg[rb][ks],
                                                                        s[kb][rb], 0, 0, 0);
            }
        }
    };

    // Visible-key test of the attention variant.  Written with non-short-
    // circuit & and | so that masking stays a per-lane select: the
    // short-circuit form became exec-mask branches around the accumulator
    // registers, and the compiler dropped one of those branches' writes.
    auto visible = [&](int j, int i) -> bool {
        if (MODE == MODE_STREAM) return (j <= i) & ((j < a.S) | (j > i - a.R));
        return j <= i;
    };

    // Key tiles to visit: full attention sees tiles 0..nt-1; streaming sees
    // the sink tiles and the band (q0-R, last query] of this workgroup.
    const int last_row = (q0 + BM < N ? q0 + BM : N) - 1;
    const int nt = last_row / BN + 1;
    const int ns = a.S > 0 ? ((a.S - 1) / BN + 1 < nt ? (a.S - 1) / BN + 1 : nt) : 0;
    int band0 = q0 - a.R + 1;
    band0 = band0 < 0 ? 0 : band0 / BN;
    if (band0 < ns) band0 = ns;
    const int n_iter_sparse = ns + (nt - band0);
    auto sparse_tile = [&](int it) { return it < ns ? it : band0 + (it - ns); };

    f32x4 o[RB][DB];
    float m[RB], l[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        m[rb] = kNegInf;
        l[rb] = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int n_iter = (MODE == MODE_STREAM) ? n_iter_sparse : nt;
    const int wlast = wpos0 + 16 * PB - 1;  // last query position of this wave
    for (int it = 0; it < n_iter; ++it) {
        const int t = (MODE == MODE_STREAM) ? sparse_tile(it) : it;
        const int key0 = t * BN;
        __syncthreads();
        load_tile(t, true);
        __syncthreads();
        if (key0 > wlast) continue;  // every key of the tile is in this wave's future

        f32x4 s[NKB][RB];
        qk(s);

        const bool need_mask = (MODE == MODE_STREAM) || (key0 + BN - 1 > wpos0);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = key0 + kb * 16 + 4 * g + r;
                        const int i = wpos0 + (rb % PB) * 16 + c16;
                        s[kb][rb][r] = visible(j, i) ? s[kb][rb][r] : kNegInf;
                    }
        }

        // Online softmax (log2 units) and P^T packing.
        bf16x8 pk[NT2][RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            float mx = kNegInf;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][rb][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mnew = fmaxf(m[rb], mx * c);
            const float mref = (mnew == kNegInf) ? 0.f : mnew;
            const float alpha = exp2_fast(m[rb] - mref);
            m[rb] = mnew;
            float rs = 0.f;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p = exp2_fast(__builtin_fmaf(s[kb][rb][r], c, -mref));
                    s[kb][rb][r] = p;
                    rs += p;
                }
            l[rb] = l[rb] * alpha + rs;
#pragma unroll
            for (int db = 0; db < DB; ++db) o[rb][db] *= alpha;
#pragma unroll
            for (int t2 = 0; t2 < NT2; ++t2) {
                bf16x8 p8;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    p8[e] = (bf16)s[2 * t2][rb][e];
                    p8[e + 4] = (bf16)s[2 * t2 + 1][rb][e];
                }
                pk[t2][rb] = p8;
            }
        }

        // O^T += V^T P^T
#pragma unroll
        for (int t2 = 0; t2 < NT2; ++t2) {
            const bf16 *vrow = Vs + (32 * t2 + 4 * g + (c16 >> 2)) * STR + 4 * (c16 & 3);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const bf16x8 A = concat(lds_read_tr(vrow + db * 16), lds_read_tr(vrow + 16 * STR + db * 16));
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    o[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, pk[t2][rb], o[rb][db],
                                                                        0, 0, 0);
            }
        }
    }

    // Finalize: O / l, LSE = (m + log2 l) * ln 2.
    float lse2[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        float lt = l[rb] + __shfl_xor(l[rb], 16);
        lt += __shfl_xor(lt, 32);
        const float inv = 1.f / lt;
        lse2[rb] = m[rb] + __log2f(lt);
        const int pos = wpos0 + (rb % PB) * 16 + c16;
        const int h = h0 + rb / PB;
        if (pos < N) {
            bf16 *op = (bf16 *)a.o + b * a.o_sb + (int64_t)h * a.o_sh + (int64_t)pos * a.o_sn + 4 * g;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                bf16x4 w;
#pragma unroll
                for (int r = 0; r < 4; ++r) w[r] = (bf16)(o[rb][db][r] * inv);
                *(bf16x4 *)(op + db * 16) = w;
            }
            if (a.lse != nullptr && g == 0)
                a.lse[((int64_t)b * a.Hq + h) * N + pos] = lse2[rb] * kLn2;
        }
    }

    // Lazy-ratio epilogue: only workgroups holding some of the last W queries.
    // Numerator: recompute s_ij over the sink and recent key tiles only and
    // sum exp2(s_ij*c - lse2_i) over j < S or i-R < j <= i; the denominator
    // is the LSE just produced.
    if (MODE == MODE_FULL_LAZY && q0 + BM > N - a.W) {
        float acc[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[rb] = 0.f;
        for (int it = 0; it < n_iter_sparse; ++it) {
            const int t = sparse_tile(it);
            const int key0 = t * BN;
            __syncthreads();
            load_tile(t, false);
            __syncthreads();
            if (wlast < N - a.W || key0 > wlast) continue;
            f32x4 s[NKB][RB];
            qk(s);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = key0 + kb * 16 + 4 * g + r;
                        const int i = wpos0 + (rb % PB) * 16 + c16;
                        const bool in_set = (j <= i) & ((j < a.S) | (j > i - a.R));
                        const float e = exp2_fast(__builtin_fmaf(s[kb][rb][r], c, -lse2[rb]));
                        acc[rb] += in_set ? e : 0.f;
                    }
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            float tot = acc[rb] + __shfl_xor(acc[rb], 16);
            tot += __shfl_xor(tot, 32);
            const int pos = wpos0 + (rb % PB) * 16 + c16;
            const int h = h0 + rb / PB;
            if (g == 0 && pos < N && pos >= N - a.W)
                a.lazy_rows[((int64_t)b * a.Hq + h) * a.W + (pos - (N - a.W))] = tot;
        }
    }
}

// Per-head lazy ratio: mean of the W per-row values, summed in row order.
__global__ void lazy_reduce_kernel(const float *rows, float *ratio, int BH, int W) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= BH) return;
    const float *r = rows + (int64_t)i * W;
    float acc = 0.f;
    for (int w = 0; w < W; ++w) acc += r[w];
    ratio[i] = acc / (float)W;
}

template <int D, int GC, int PB, int BN>
hipError_t launch_mode(const AttnArgs &a, int mode, hipStream_t st) {
    dim3 grid((unsigned)(a.n_qtiles * a.B * a.Hkv * a.n_chunks));
    dim3 block(256);
    switch (mode) {
    case MODE_FULL:
        hipLaunchKernelGGL((attn_bf16_kernel<D, GC, PB, BN, MODE_FULL>), grid, block, 0, st, a);
        break;
    case MODE_FULL_LAZY:
        hipLaunchKernelGGL((attn_bf16_kernel<D, GC, PB, BN, MODE_FULL_LAZY>), grid, block, 0, st, a);
        break;
    default:
        hipLaunchKernelGGL((attn_bf16_kernel<D, GC, PB, BN, MODE_STREAM>), grid, block, 0, st, a);
        break;
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(AttnArgs a, int mode, hipStream_t st) {
    // Heads of a GQA group per workgroup (GC) and position blocks per wave
    // (PB): up to 5 heads share each K/V tile; small groups take more
    // positions per wave so each wave still owns 4-5 row blocks.
    int gc = 1;
    for (int cand = 5; cand >= 1; --cand)
        if (a.G % cand == 0) { gc = cand; break; }
    a.n_chunks = a.G / gc;
    const int pb = gc == 1 ? 4 : gc == 2 ? 2 : 1;
    const int bm = 64 * pb;
    a.n_qtiles = (a.N + bm - 1) / bm;
    // Key tile: 64 keys at D = 64; 32 at D = 128 so that O (RB*D/16 x 4),
    // S^T (RB*BN/16 x 4) and Q^T (RB*D/16 x 2) fit the 512-register budget.
    constexpr int BN = D == 64 ? 64 : 32;
    switch (gc) {
    case 1: return launch_mode<D, 1, 4, BN>(a, mode, st);
    case 2: return launch_mode<D, 2, 2, BN>(a, mode, st);
    case 3: return launch_mode<D, 3, 1, BN>(a, mode, st);
    case 4: return launch_mode<D, 4, 1, BN>(a, mode, st);
    default: return launch_mode<D, 5, 1, BN>(a, mode, st);
    }
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs &a, int D, int mode, hipStream_t st) {
    if (D == 64) return launch_d<64>(a, mode, st);
    return launch_d<128>(a, mode, st);
}

hipError_t launch_lazy_reduce(const float *lazy_rows, float *lazy_ratio, int BH, int W,
                              hipStream_t st) {
    hipLaunchKernelGGL(lazy_reduce_kernel, dim3((BH + 255) / 256), dim3(256), 0, st, lazy_rows,
                       lazy_ratio, BH, W);
    return hipGetLastError();
}

}  // namespace lt
