// fp32 causal GQA attention on the vector ALUs: full prefill with LSE, the
// lazy ratio summed in the same pass, and streaming attention.  Same method
// and outputs as the bf16 matrix-core kernel (attn_bf16.hip); this variant
// keeps every product and sum in fp32 for fp32 inputs, where bf16 operands
// would cost the accuracy the caller asked for.
//
// Method (LightTransfer pages): Chinese write-up, "solution 1" -- the LSE is
// the lazy ratio's denominator and the numerator only needs the sink and
// recent keys; project page, "Introduction" -- converted layers run streaming
// attention.
//
// Work decomposition.  A workgroup of NW waves owns ROWS = 16 consecutive
// query rows of one (sequence, query head); each row is spread over LPR = 4
// lanes of a wave holding D/4 dims of its query and output each, so a dot
// product is four partial sums joined by two quad permutes.  The NW waves
// take every NW-th key tile of the rows' key range (split-K): each stages
// its tiles in an LDS region of its own and keeps its own running max, sum
// and lazy-ratio numerator, and the NW partial states are merged through
// LDS at the end.  Workgroups and key work are both small and many, so a
// layer of a few hundred rows (latency-bound) spreads over the whole chip.
// Full attention takes 16 waves (4 KiB K and V tiles per wave, one
// workgroup per CU, four waves per SIMD): a row's keys grow with its
// position, and the longest rows bound the launch.  Streaming attention,
// whose rows see at most S + R keys, takes 4 waves (8 KiB tiles); with 16,
// most waves of a band workgroup had no tile.  (At 512 tokens 16 waves ran
// the prefill in 21 against 37 us, at 8K tokens 3.4 against 4.6 ms; 4 waves
// kept streaming at 186 against 253 us.)
#include "lt_internal.h"

namespace lt {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kLPR = 4;               // lanes per query row
constexpr int kRows = 64 / kLPR;      // query rows per workgroup (and per wave)
constexpr int kChunk = 8;             // keys per online-softmax update

// Sum over the four lanes of a quad (the lanes of one query row): DPP quad
// permutes [1,0,3,2] and [2,3,0,1], plain vector ALU instructions rather
// than a trip through the LDS crossbar.
__device__ __forceinline__ float quad_sum(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
    return x;
}

// Waves per workgroup of each mode (see above).
constexpr int waves_of(int mode) { return mode == MODE_STREAM ? 4 : 16; }

template <int D, int MODE>
__global__ __launch_bounds__(64 * waves_of(MODE)) void attn_f32_kernel(AttnArgs a) {
    constexpr int kWaves = waves_of(MODE);
    constexpr int DPL = D / kLPR;         // dims per lane
    constexpr int TK = (kWaves > 4 ? 1024 : 2048) / D;  // keys per tile (4 or 8 KiB of K, the same of V)
    constexpr int TILE = TK * D;
    constexpr bool LAZY = MODE == MODE_FULL_LAZY;
    // Per wave: its K and V tile; after the key loop, the merge buffers (each
    // wave's partial outputs, then each row's m, l and lazy numerator per
    // wave), which at 16 waves and D = 128 need more than the tiles.
    constexpr int TILES = kWaves * 2 * TILE;
    constexpr int MERGE = kWaves * 64 * DPL + kWaves * kRows * 3;
    __shared__ __attribute__((aligned(16))) float smem[TILES > MERGE ? TILES : MERGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rl = lane / kLPR, part = lane % kLPR;
    const int bh = blockIdx.y;
    const int b = bh / a.Hq, h = bh % a.Hq, hk = h / a.G;
    const int N = seq_length(a.seq_len, b, a.N);
    const int q0 = blockIdx.x * kRows;
    if (q0 >= N) return;  // past this sequence's end (whole workgroup, before any barrier)
    poison_lds<64 * kWaves>(smem, (int)sizeof(smem), tid);
    const int i = q0 + rl;
    const bool row_ok = i < N;
    const int last_row = (q0 + kRows < N ? q0 + kRows : N) - 1;
    const float c = a.c;
    const int d0 = part * DPL;

    const float *kbase = (const float *)a.k + b * a.k_sb + (int64_t)hk * a.k_sh;
    const float *vbase = (const float *)a.v + b * a.v_sb + (int64_t)hk * a.v_sh;

    float q[DPL], o[DPL];
    {
        const float *qp = (const float *)a.q + b * a.q_sb + (int64_t)h * a.q_sh +
                          (int64_t)(row_ok ? i : 0) * a.q_sn + d0;
#pragma unroll
        for (int d = 0; d < DPL; d += 4) {
            const float4 v = *(const float4 *)(qp + d);
            q[d] = row_ok ? v.x : 0.f;
            q[d + 1] = row_ok ? v.y : 0.f;
            q[d + 2] = row_ok ? v.z : 0.f;
            q[d + 3] = row_ok ? v.w : 0.f;
        }
#pragma unroll
        for (int d = 0; d < DPL; ++d) o[d] = 0.f;
    }
    float m = kNegInf, l = 0.f, lz = 0.f;
    // This row is one of the last W (its sink + recent mass is the lazy row).
    const bool obs = LAZY && row_ok && i >= N - a.W;

    auto in_set = [&](int j) -> bool { return (j <= i) & ((j < a.S) | (j > i - a.R)); };
    auto visible = [&](int j) -> bool {
        if (MODE == MODE_STREAM) return in_set(j);
        return j <= i;
    };

    // Key tiles: full attention sees tiles 0..nt-1; streaming the sink tiles
    // and the band (first row - R, last row].  Wave w takes every fourth.
    const int nt = last_row / TK + 1;
    const int ns = a.S > 0 ? ((a.S - 1) / TK + 1 < nt ? (a.S - 1) / TK + 1 : nt) : 0;
    int band0 = q0 - a.R + 1;
    band0 = band0 < 0 ? 0 : band0 / TK;
    if (band0 < ns) band0 = ns;
    const int n_iter = (MODE == MODE_STREAM) ? ns + (nt - band0) : nt;

    float *const Kt = smem + wave * 2 * TILE;
    float *const Vt = Kt + TILE;
    for (int it = wave; it < n_iter; it += kWaves) {
        const int t = (MODE == MODE_STREAM) ? (it < ns ? it : band0 + (it - ns)) : it;
        const int key0 = t * TK;
        // Stage the tile (keys past the sequence read as zero: never visible).
        // The wave's previous tile was last read by its own lanes, whose LDS
        // accesses run in order.
#pragma unroll
        for (int u = 0; u < TILE / 4 / 64; ++u) {
            const int e = (lane + 64 * u) * 4;
            const int key = key0 + e / D, d = e % D;
            float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
            if (key < N) {
                kv = *(const float4 *)(kbase + (int64_t)key * a.k_sn + d);
                vv = *(const float4 *)(vbase + (int64_t)key * a.v_sn + d);
            }
            *(float4 *)(Kt + e) = kv;
            *(float4 *)(Vt + e) = vv;
        }
        asm volatile("" ::: "memory");  // lanes read what other lanes wrote
#pragma unroll
        for (int r0 = 0; r0 < TK; r0 += kChunk) {
            float s[kChunk];
            float mx = kNegInf;
#pragma unroll
            for (int r = 0; r < kChunk; ++r) {
                const float *kr = Kt + (r0 + r) * D + d0;
                float acc = 0.f;
#pragma unroll
                for (int d = 0; d < DPL; ++d) acc = __builtin_fmaf(q[d], kr[d], acc);
                acc = quad_sum(acc);
                s[r] = visible(key0 + r0 + r) ? acc * c : kNegInf;
                mx = fmaxf(mx, s[r]);
            }
            // Online softmax in log2 units; a row that has seen no visible
            // key yet keeps m = -inf and takes 0 as its reference.
            const float mnew = fmaxf(m, mx);
            const float mref = (mnew == kNegInf) ? 0.f : mnew;
            const float alpha = exp2f(m - mref);
            m = mnew;
            l *= alpha;
            if (LAZY) lz *= alpha;
#pragma unroll
            for (int d = 0; d < DPL; ++d) o[d] *= alpha;
#pragma unroll
            for (int r = 0; r < kChunk; ++r) {
                const float p = exp2f(s[r] - mref);
                l += p;
                // lazy-ratio numerator: the sink and recent keys of an observed row
                if (LAZY) lz += (obs & in_set(key0 + r0 + r)) ? p : 0.f;
                const float *vr = Vt + (r0 + r) * D + d0;
#pragma unroll
                for (int d = 0; d < DPL; ++d) o[d] = __builtin_fmaf(p, vr[d], o[d]);
            }
        }
        asm volatile("" ::: "memory");  // this tile's reads stay above the next tile's writes
    }

    // Merge the four waves' partial states: out = sum_w 2^(m_w - M) o_w /
    // sum_w 2^(m_w - M) l_w, and the same weights for the lazy numerator.
    __syncthreads();  // every wave is done with its tile buffers
    float *const mo = smem;                              // [waves][64 lanes][DPL]
    float *const ms = smem + kWaves * 64 * DPL;          // [waves][rows][3]: m, l, lz
    {
        float *dst = mo + (wave * 64 + lane) * DPL;
#pragma unroll
        for (int d = 0; d < DPL; d += 4) *(float4 *)(dst + d) = make_float4(o[d], o[d + 1], o[d + 2], o[d + 3]);
        if (part == 0) {
            ms[(wave * kRows + rl) * 3 + 0] = m;
            ms[(wave * kRows + rl) * 3 + 1] = l;
            ms[(wave * kRows + rl) * 3 + 2] = lz;
        }
    }
    __syncthreads();
    if (wave == 0) {
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, ms[(w * kRows + rl) * 3]);
        float L = 0.f, LZ = 0.f, O[DPL];
#pragma unroll
        for (int d = 0; d < DPL; ++d) O[d] = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = ms[(w * kRows + rl) * 3];
            const float f = mw == kNegInf ? 0.f : exp2f(mw - M);
            L += f * ms[(w * kRows + rl) * 3 + 1];
            if (LAZY) LZ += f * ms[(w * kRows + rl) * 3 + 2];
            const float *src = mo + (w * 64 + lane) * DPL;
#pragma unroll
            for (int d = 0; d < DPL; ++d) O[d] = __builtin_fmaf(f, src[d], O[d]);
        }
        if (row_ok) {
            const float inv = 1.f / L;
            float *op = (float *)a.o + b * a.o_sb + (int64_t)h * a.o_sh + (int64_t)i * a.o_sn + d0;
#pragma unroll
            for (int d = 0; d < DPL; d += 4)
                *(float4 *)(op + d) = make_float4(O[d] * inv, O[d + 1] * inv, O[d + 2] * inv, O[d + 3] * inv);
            if (a.lse != nullptr && part == 0) a.lse[((int64_t)b * a.Hq + h) * a.N + i] = (M + log2f(L)) * kLn2;
            if (obs && part == 0) a.lazy_rows[((int64_t)b * a.Hq + h) * a.W + (i - (N - a.W))] = LZ * inv;
        }
    }

    // Streaming slice (full attention, when asked for): the workgroups of the
    // group's first query head copy their positions' K/V rows.
    if (MODE != MODE_STREAM && h % a.G == 0) {
        const StreamOut so = stream_out_late();
        if (so.k != nullptr)
            emit_stream_rows<64 * kWaves>((const char *)kbase, (const char *)vbase, a.k_sn, a.v_sn, so, b, hk, N, a.S,
                                          a.R, q0, last_row + 1, 4, D * 4, tid);
    }
}

template <int D>
hipError_t launch_d(const AttnArgs &a, int mode, hipStream_t st) {
    dim3 grid((unsigned)((a.N + kRows - 1) / kRows), (unsigned)(a.B * a.Hq));
    dim3 block(64 * waves_of(mode));
    if (log_enabled())
        log_printf("  launch attn_f32_kernel<D=%d, mode=%s> grid %u x %u x %u threads", D,
                   mode == MODE_FULL ? "full" : mode == MODE_FULL_LAZY ? "full+lazy" : "stream", grid.x, grid.y,
                   block.x);
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
