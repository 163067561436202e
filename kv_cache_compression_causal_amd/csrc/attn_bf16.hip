// bf16 causal GQA attention on the gfx950 matrix cores: full prefill with LSE,
// the lazy ratio computed in the same pass, and streaming (sink + recent)
// attention.
//
// Method (LightTransfer pages): Chinese write-up, "solution 1" -- the LSE that
// Flash Attention produces is the lazy ratio's denominator, the numerator
// only needs the sink and recent keys; press-release page, "LightTransfer
// method" -- the ratio is the attention mass on the initial and recent keys;
// project page, "Introduction" -- converted layers run streaming attention.
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
//   Row statistics: max over a lane's own 8 values of a 32-key step, then
//   across the four lane groups (permlane swaps, xor 16 and xor 32); the
//   running sum stays per lane and is reduced once at the end.  Scores are
//   kept in log2 units (scale*log2 e folded into one fma before exp2).
//
// Launch order: sequence by sequence; within a sequence blockIdx.x % Hkv
// picks the KV head, so that with Hkv a multiple of 8 each XCD (dispatch is
// round-robin over the 8 XCDs) keeps one KV head's K/V in its own L2, and the
// row tiles run longest-first to even out the causal triangle.  Keeping one
// sequence's workgroups together keeps its K/V in the shared caches; with
// sequences of different lengths, interleaving them (most of the first
// workgroups then exit at once) ran at half the rate.

#include <atomic>
#include <type_traits>

#include "lt_internal.h"

namespace lt {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();
// Initial running max (log2 units): finite, so exp2(s - m) needs no -inf
// guard, and far below any score, so the first visible key always resets it.
constexpr float kMInit = -1e30f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Direct global -> LDS load (global_load_lds_dwordx4): lane i of the wave
// fetches 16 bytes from gptr into LDS at lds_base + 16 i (lds_base uniform,
// passed in M0).  Written in asm so that the compiler's wait bookkeeping does
// not see it: while a builtin one is in flight the compiler waits for every
// outstanding LDS read at each use (a full lgkmcnt(0)).  The instruction
// writes no registers; its completion is waited for explicitly (s_waitcnt
// 0) before the barrier that publishes the tile, and an extra outstanding
// load only makes the compiler's own vmcnt waits stricter.  M0 is saved and
// restored around it (the compiler does not track M0 through asm); the
// s_nops are the wait states between writing M0 and the instructions that
// read it.
__device__ __forceinline__ void lds_dma16(const void *gptr, uint32_t lds_base) {
    unsigned saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(gptr), "s"(lds_base)
        : "memory");
}
// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(size_t)(const __attribute__((address_space(3))) void *)p;
}

__device__ __forceinline__ bf16x4 lds_read_tr(const bf16 *__restrict__ p) {
    i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4 *)(p));
    return __builtin_bit_cast(bf16x4, r);
}

// Reductions across the four 16-lane groups holding one query column.
// v_permlane16_swap / v_permlane32_swap exchange halves of two registers;
// swapping a value with a copy of itself leaves, in each lane, its own
// value and the value of lane l^16 (resp. l^32), in an order that depends
// on the lane -- max and + do not care.  The swap is written in asm with
// both registers as read-write operands: through the compiler builtin the
// second result was dropped and the first read twice.  The s_nop on each
// side gives the VALU -> permlane -> VALU wait states.
__device__ __forceinline__ void permlane16_swap(unsigned &a, unsigned &b) {
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void permlane32_swap(unsigned &a, unsigned &b) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float max_xor16(float x) {
    unsigned a = __builtin_bit_cast(unsigned, x), b = a;
    permlane16_swap(a, b);
    return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float max_xor32(float x) {
    unsigned a = __builtin_bit_cast(unsigned, x), b = a;
    permlane32_swap(a, b);
    return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float sum_xor16(float x) {
    unsigned a = __builtin_bit_cast(unsigned, x), b = a;
    permlane16_swap(a, b);
    return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}
__device__ __forceinline__ float sum_xor32(float x) {
    unsigned a = __builtin_bit_cast(unsigned, x), b = a;
    permlane32_swap(a, b);
    return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}
// The row max / sum of a query column over the four lane groups.
__device__ __forceinline__ float group_max(float x) { return max_xor32(max_xor16(x)); }
__device__ __forceinline__ float group_sum(float x) { return sum_xor32(sum_xor16(x)); }

__device__ __forceinline__ bf16x8 concat(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// LDS tiles are unpadded rows of D bf16, permuted in 16-byte chunks so that
// the reads below are bank-conflict free: the 16 rows one 128-bit K read
// touches, and the four 32-byte row pieces of each transposing V read, land
// in distinct bank groups.  XOR makes each map its own inverse.
template <int D>
__device__ __forceinline__ int swz_k(int row, int chunk) {
    return D == 128 ? chunk ^ (row & 15) : chunk ^ ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int row, int chunk) {
    return D == 128 ? chunk ^ (2 * (row & 7)) : chunk ^ (2 * ((row >> 1) & 3));
}

// Work decomposition: the queries of one (batch, KV head) are flattened
// position-major over the G query heads of the group, r = position * G +
// head-in-group.  A workgroup of NW waves (8 for full attention, one
// workgroup and two waves per SIMD; 4 for streaming, two workgroups per CU)
// owns NW*16*RB consecutive rows r; each wave owns RB row blocks of 16.  K/V
// tiles of BT keys are staged in LDS once per workgroup and read by every
// wave, so the whole GQA group shares each tile; inside a wave each K fragment
// read from LDS feeds RB matrix-core ops.  The causal mask uses each lane's own
// position, so rows of different heads and positions mix freely inside a
// row block.  While one wave of a SIMD runs its softmax or waits on LDS, the
// other wave's matrix-core products run.
//
// The lazy-ratio numerator is accumulated in the same pass: on the key tiles
// that hold sink or recent keys of an observed row (the last W queries), the
// weights of the keys in that row's sink + recent set are summed next to the
// full sum l, with the same running max and the same rescaling, so
// r_i = lz_i / l_i = exp(ln lz_i + m_i - LSE_i) uses the LSE's own
// denominator and costs O(S+R) extra work per observed query; no key tile is
// read a second time.
template <int D, int RB, int BT, int MODE, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bf16_kernel(AttnArgs a) {
    constexpr int WROWS = 16 * RB;   // flattened query rows per wave
    constexpr int BROWS = NW * WROWS;
    constexpr int KS = D / 32;       // 32-dim steps of Q.K
    constexpr int DB = D / 16;       // 16-dim blocks of O
    constexpr int BN = 32;           // keys per softmax step (half a tile at BT = 64)
    constexpr int NH = BT / BN;      // softmax steps per LDS tile
    constexpr int NKB = BN / 16;     // 16-key blocks per step
    constexpr int CPR = D / 8;       // 16-byte chunks per LDS row
    constexpr int RPI = 64 / CPR;    // rows one wave fills per direct load
    constexpr int NINST = BT / RPI;  // direct loads per tile (over all waves)
    constexpr int NI = (NINST + NW - 1) / NW;
    constexpr int TILE = BT * D;
    static_assert(BT % RPI == 0, "tile rows must fill whole direct loads");
    static_assert(MODE != MODE_STREAM || NW * 16 * RB * D <= 4 * TILE,
                  "streaming stages every wave's output rows in the tile buffers");
    constexpr bool LAZY = MODE == MODE_FULL_LAZY;
    __shared__ __attribute__((aligned(16))) bf16 lds[4 * TILE];  // K0 K1 V0 V1

    const int tid = threadIdx.x;
    // The wave index is uniform; readfirstlane lets the compiler see that, so
    // every per-wave test below is a scalar branch, not an exec-mask one.
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c16 = lane & 15;
    const int per_b = a.n_qtiles * a.Hkv;
    const int b = (int)(blockIdx.x / per_b);
    const int rem = (int)(blockIdx.x % per_b);
    const int hk = rem % a.Hkv;
    const int qt = a.n_qtiles - 1 - rem / a.Hkv;
    const int N = seq_length(a.seq_len, b, a.N), G = a.G;
    const float c = a.c;
    const int r0 = qt * BROWS;
    if (r0 >= N * G) return;  // past this sequence's end (whole workgroup, before any barrier)
    poison_lds<64 * NW>(lds, (int)sizeof(lds), tid);
    const int rw0 = r0 + wave * WROWS;
    const int nrows = N * G;
    const int wg_last = ((r0 + BROWS < nrows ? r0 + BROWS : nrows) - 1) / G;  // last position
    const int wg_first = r0 / G;
    const int w_first = rw0 / G;               // first position of this wave
    const int w_last = (rw0 + WROWS - 1) / G;  // last position of this wave

    int pos[RB];   // query position of this lane's column in each row block
    int head[RB];  // its query head
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int r = rw0 + rb * 16 + c16;
        pos[rb] = r / G;
        head[rb] = hk * G + (r - pos[rb] * G);
    }
    const bf16 *kbase = (const bf16 *)a.k + b * a.k_sb + hk * a.k_sh;
    const bf16 *vbase = (const bf16 *)a.v + b * a.v_sb + hk * a.v_sh;

    // Q^T operand: lane holds query column c16 of each row block, dims 8g.. of each step.
    bf16x8 qreg[RB][KS];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const bool ok = pos[rb] < N;
        const bf16 *qp = (const bf16 *)a.q + b * a.q_sb + (int64_t)(ok ? head[rb] : 0) * a.q_sh +
                         (int64_t)(ok ? pos[rb] : 0) * a.q_sn + g * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            bf16x8 v = *(const bf16x8 *)(qp + ks * 32);
            qreg[rb][ks] = ok ? v : bf16x8{};
        }
    }

    // Direct global -> LDS loads (global_load_lds_dwordx4): lane i of a wave
    // writes 16 bytes at dst + 16 i, so each lane fetches the global chunk
    // that belongs at its swizzled LDS slot.  The lane's byte offset within
    // a tile is fixed; only the tile's base address (uniform) moves.  In a
    // tile that runs past N, rows past N are read from row N-1: their keys
    // are never visible and their values meet zero weights.
    // A wave's loads of a tile cover rows RPI*(wave + NW j) + lane/CPR; the
    // swizzle only depends on the row modulo 16, which is the same for every
    // j, so load j of a lane sits a uniform RPI*NW rows after load 0.
    const int row_l = RPI * wave + lane / CPR, ph_l = lane % CPR;
    const uint32_t koff = (uint32_t)(((int64_t)row_l * a.k_sn + swz_k<D>(row_l, ph_l) * 8) * 2);
    const uint32_t voff = (uint32_t)(((int64_t)row_l * a.v_sn + swz_v<D>(row_l, ph_l) * 8) * 2);
    static_assert((RPI * NW) % 16 == 0, "a wave's loads must share their swizzle");
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));
    auto load_tile = [&](int t, bf16 *Kd, bf16 *Vd) {
        const int key0 = t * BT;
        const uint32_t kd = lds0 + (uint32_t)(Kd - lds) * 2, vd = lds0 + (uint32_t)(Vd - lds) * 2;
        if (key0 + BT <= N) {
            const char *kb = (const char *)(kbase + (int64_t)key0 * a.k_sn);
            const char *vb = (const char *)(vbase + (int64_t)key0 * a.v_sn);
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                if (NINST % NW != 0 && wave + NW * j >= NINST) break;
                const int row0 = RPI * (wave + NW * j);
                const int64_t jr = (int64_t)RPI * NW * j;  // rows between load 0 and load j
                lds_dma16(kb + jr * a.k_sn * 2 + koff, kd + row0 * D * 2);
                lds_dma16(vb + jr * a.v_sn * 2 + voff, vd + row0 * D * 2);
            }
        } else {
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                if (NINST % NW != 0 && wave + NW * j >= NINST) break;
                const int row0 = RPI * (wave + NW * j);
                const int row = row0 + lane / CPR, ph = lane % CPR;
                const int key = key0 + row < N ? key0 + row : N - 1;
                const bf16 *kp = kbase + (int64_t)key * a.k_sn + swz_k<D>(row, ph) * 8;
                const bf16 *vp = vbase + (int64_t)key * a.v_sn + swz_v<D>(row, ph) * 8;
                lds_dma16(kp, kd + row0 * D * 2);
                lds_dma16(vp, vd + row0 * D * 2);
            }
        }
    };
    // Every wave's direct loads have landed and are visible to the workgroup.
    auto loads_done = [&]() {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };

    // S^T for keys [32h, 32h+32) of a staged tile: s[kb][rb] holds keys
    // kb*16+4g+r of the step, query column c16.  The K fragments of 32-dim
    // step ks+2 are read while the products of step ks run (the scheduling
    // groups fix that order).
    auto qk = [&](const bf16 *Kb, int h, f32x4 (&s)[NKB][RB]) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) s[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
        bf16x8 A[KS][NKB];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const int row = BN * h + kb * 16 + c16;
                A[ks][kb] = *(const bf16x8 *)(Kb + row * D + swz_k<D>(row, ks * 4 + g) * 8);
            }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    s[kb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[ks][kb], qreg[rb][ks],
                                                                        s[kb][rb], 0, 0, 0);
        // Scheduling groups (0x100: LDS reads, 0x008: matrix-core ops).
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * NKB, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 2 < KS) __builtin_amdgcn_sched_group_barrier(0x100, NKB, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, NKB * RB, 0);
        }
    };
    // O^T += V^T P^T for keys [32h, 32h+32) of a staged V tile; the V^T
    // fragments of block db+3 are read while the products of block db run.
    // Streaming: the swizzled chunk of 16-dim block db is chunk(0) ^ 2db, so
    // the lane's V^T offsets are one base XOR a per-block constant.
    const int vt_row = 4 * g + (c16 >> 2);
    const int vt_base = vt_row * D + swz_v<D>(vt_row, (c16 & 3) >> 1) * 8 + (c16 & 1) * 4;
    auto pv = [&](const bf16 *Vb, int h, const bf16x8 (&pk)[RB], f32x4 (&o)[RB][DB]) {
        const int row1 = BN * h + 4 * g + (c16 >> 2), row2 = row1 + 16;
        const int half = (c16 & 1) * 4;
        bf16x8 A[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            if (MODE == MODE_STREAM) {
                const int off = (vt_base ^ (16 * db)) + BN * h * D;
                A[db] = concat(lds_read_tr(Vb + off), lds_read_tr(Vb + off + 16 * D));
            } else {
                const int lch = 2 * db + ((c16 & 3) >> 1);
                A[db] = concat(lds_read_tr(Vb + row1 * D + swz_v<D>(row1, lch) * 8 + half),
                               lds_read_tr(Vb + row2 * D + swz_v<D>(row2, lch) * 8 + half));
            }
        }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                o[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[db], pk[rb], o[rb][db], 0, 0, 0);
        constexpr int AHEAD = 3;  // 16-dim blocks whose V^T reads are in flight
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * AHEAD, 0);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            if (db + AHEAD < DB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, RB, 0);
        }
    };
    // Visible-key test of the attention variant and the sink + recent set.
    // Written with non-short-circuit & and | so that masking stays a per-lane
    // select: the short-circuit form became exec-mask branches around the
    // accumulator registers, and the compiler dropped one of those branches'
    // writes.
    auto in_set = [&](int j, int i) -> bool { return (j <= i) & ((j < a.S) | (j > i - a.R)); };
    auto visible = [&](int j, int i) -> bool {
        if (MODE == MODE_STREAM) return in_set(j, i);
        return j <= i;
    };
    // Scores of keys a row does not see become -inf.
    auto mask = [&](f32x4 (&s)[NKB][RB], int key0) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = key0 + kb * 16 + 4 * g + r;
                    s[kb][rb][r] = visible(j, pos[rb]) ? s[kb][rb][r] : kNegInf;
                }
    };

    // Key tiles to visit: full attention sees tiles 0..nt-1; streaming sees
    // the sink tiles and the band (first position - R, last position].
    const int nt = wg_last / BT + 1;
    const int ns = a.S > 0 ? ((a.S - 1) / BT + 1 < nt ? (a.S - 1) / BT + 1 : nt) : 0;
    int band0 = wg_first - a.R + 1;
    band0 = band0 < 0 ? 0 : band0 / BT;
    if (band0 < ns) band0 = ns;
    const int n_iter = (MODE == MODE_STREAM) ? ns + (nt - band0) : nt;
    auto tile_of = [&](int it) {
        if (MODE == MODE_STREAM) return it < ns ? it : band0 + (it - ns);
        return it;
    };
    // Observed rows of this wave (lazy ratio): positions >= N - W.
    const int obs_lo = (w_first > N - a.W ? w_first : N - a.W);
    const bool wave_obs = LAZY && w_last >= N - a.W;

    f32x4 o[RB][DB];
    float m[RB], l[RB], lz[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        m[rb] = kMInit;
        l[rb] = 0.f;
        lz[rb] = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // One key tile: prefetch the next tile into the other buffer, then the
    // tile's 32-key steps.  BUF is a compile-time constant so that every LDS
    // address of the steps is a fixed offset; FIRST marks the wave's first
    // tile, whose first step streaming attention runs without the lagging
    // max.
    auto run_tile = [&](int it, auto buf_c, auto first_c) {
        constexpr int BUF = decltype(buf_c)::value;
        constexpr bool FIRST = decltype(first_c)::value;
        bf16 *const Kb = lds + BUF * TILE;
        bf16 *const Vb = lds + (2 + BUF) * TILE;
        if (it + 1 < n_iter) load_tile(tile_of(it + 1), lds + (BUF ^ 1) * TILE, lds + (2 + (BUF ^ 1)) * TILE);
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            const int key0 = tile_of(it) * BT + BN * h;
            if (key0 > w_last) continue;  // every key of the step is in this wave's future
            // Streaming: a step of non-sink keys below every row's window adds
            // nothing (its weights would all be zero) and is skipped.
            if (MODE == MODE_STREAM && key0 >= a.S && key0 + BN - 1 <= w_first - a.R) continue;
            f32x4 s[NKB][RB];
            qk(Kb, h, s);
            // Steps whose every key every row sees run unmasked: under the
            // diagonal and, for streaming, all sinks or all inside the window
            // of the wave's last row (hence of every row).
            const bool masked = (MODE == MODE_STREAM)
                ? !((key0 + BN - 1 <= w_first) & ((key0 + BN - 1 < a.S) | (key0 > w_last - a.R)))
                : (key0 + BN - 1 > w_first);
            if (masked) mask(s, key0);
            // Online softmax in log2 units.  Weights are taken against the
            // running reference max m of each row, which is allowed to lag the
            // true max by up to a factor 2^8: a lane's 8 weights of the step
            // sum to at most 256 while no row outgrew m by more than that, and
            // O, l, lz then keep their scale.  Only when some lane's sum
            // exceeds 256 (always on a row block's first visible keys, since m
            // starts far below any score) is the row max taken across the
            // four lane groups, the block rescaled and the weights redone.
            // Full attention writes the weights over the scores (registers
            // are short) and on that rare path computes the step's scores
            // again from the staged K tile; streaming attention, whose band
            // rows take that path more often, keeps the scores instead.
            __builtin_amdgcn_s_setprio(0);
            constexpr bool INPLACE = MODE != MODE_STREAM;
            float w[INPLACE ? 1 : RB][NKB][4];
            float rs[RB];
            auto weights = [&]() {
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float p0 = exp2_fast(__builtin_fmaf(s[0][rb][e], c, -m[rb]));
                        const float p1 = exp2_fast(__builtin_fmaf(s[1][rb][e], c, -m[rb]));
                        if (INPLACE) {
                            s[0][rb][e] = p0;
                            s[1][rb][e] = p1;
                        } else {
                            w[INPLACE ? 0 : rb][0][e] = p0;
                            w[INPLACE ? 0 : rb][1][e] = p1;
                        }
                        rs[rb] = e == 0 ? p0 + p1 : rs[rb] + (p0 + p1);
                    }
            };
            if (MODE == MODE_STREAM && FIRST && h == 0) {
                // The wave's first step: O, l and lz are still zero, so the
                // exact row max is taken at once and nothing is rescaled (the
                // general path would reach the same values after a rescale
                // by exp2(kMInit - max) = 0).
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    float mx = kNegInf;
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][rb][r]);
                    m[rb] = fmaxf(m[rb], group_max(mx) * c);
                }
                weights();
            } else {
            weights();
            bool outgrown = false;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) outgrown |= rs[rb] > 256.f;
            if (__any(outgrown)) {
                if (INPLACE) {
                    qk(Kb, h, s);
                    if (masked) mask(s, key0);
                }
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    float mx = kNegInf;
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][rb][r]);
                    const float mnew = fmaxf(m[rb], group_max(mx) * c);
                    const float alpha = exp2_fast(m[rb] - mnew);
                    m[rb] = mnew;
                    l[rb] *= alpha;
                    if (LAZY) lz[rb] *= alpha;
#pragma unroll
                    for (int db = 0; db < DB; ++db) o[rb][db] *= alpha;
                }
                weights();
            }
            }
            if (!INPLACE) {
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        s[0][rb][e] = w[INPLACE ? 0 : rb][0][e];
                        s[1][rb][e] = w[INPLACE ? 0 : rb][1][e];
                    }
            }
            bf16x8 pk[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pk[rb][e] = (bf16)s[0][rb][e];
                    pk[rb][e + 4] = (bf16)s[1][rb][e];
                }
                l[rb] += rs[rb];
            }
            // Lazy-ratio numerator on steps holding sink or recent keys of an
            // observed row of this wave.
            if (wave_obs && ((key0 < a.S) | (key0 + BN - 1 > obs_lo - a.R))) {
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int j = key0 + kb * 16 + 4 * g + r;
                            lz[rb] += in_set(j, pos[rb]) ? s[kb][rb][r] : 0.f;
                        }
            }
            __builtin_amdgcn_s_setprio(1);
            pv(Vb, h, pk, o);
        }
        loads_done();
    };

    load_tile(tile_of(0), lds, lds + 2 * TILE);
    loads_done();
    if (MODE == MODE_STREAM) {
        // n_iter >= 1: the band holds at least the tile of the last row.
        run_tile(0, std::integral_constant<int, 0>{}, std::true_type{});
        int it = 1;
        for (; it + 1 < n_iter; it += 2) {
            run_tile(it, std::integral_constant<int, 1>{}, std::false_type{});
            run_tile(it + 1, std::integral_constant<int, 0>{}, std::false_type{});
        }
        if (it < n_iter) run_tile(it, std::integral_constant<int, 1>{}, std::false_type{});
    } else {
        int it = 0;
        for (; it + 1 < n_iter; it += 2) {
            run_tile(it, std::integral_constant<int, 0>{}, std::false_type{});
            run_tile(it + 1, std::integral_constant<int, 1>{}, std::false_type{});
        }
        if (it < n_iter) run_tile(it, std::integral_constant<int, 0>{}, std::false_type{});
    }

    // Finalize: O / l, LSE = (m + log2 l) * ln 2, lazy row = lz / l.
    // Streaming goes through the (now idle) LDS tile buffers: each wave
    // writes its 16*RB normalized rows into a region of its own and stores
    // them back 16 bytes per lane, every wave-wide store covering whole rows
    // (stored straight from the matrix-core layout, each store instruction
    // writes 8-byte pieces of 16 rows, which costs a short streaming window a
    // few per cent).
    bf16 *const ostage = lds + wave * WROWS * D;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const float lt = group_sum(l[rb]);
        const float inv = 1.f / lt;
        if (MODE == MODE_STREAM) {
            const int row = rb * 16 + c16;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                bf16x4 w;
#pragma unroll
                for (int r = 0; r < 4; ++r) w[r] = (bf16)(o[rb][db][r] * inv);
                const int ch = (2 * db + (g >> 1)) ^ (row & (CPR - 1));
                *(bf16x4 *)(ostage + row * D + ch * 8 + (g & 1) * 4) = w;
            }
            if (a.lse != nullptr && g == 0 && pos[rb] < N)
                a.lse[((int64_t)b * a.Hq + head[rb]) * a.N + pos[rb]] = (m[rb] + __log2f(lt)) * kLn2;
        } else if (pos[rb] < N) {
            bf16 *op = (bf16 *)a.o + b * a.o_sb + (int64_t)head[rb] * a.o_sh +
                       (int64_t)pos[rb] * a.o_sn + 4 * g;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                bf16x4 w;
#pragma unroll
                for (int r = 0; r < 4; ++r) w[r] = (bf16)(o[rb][db][r] * inv);
                *(bf16x4 *)(op + db * 16) = w;
            }
            if (a.lse != nullptr && g == 0)
                a.lse[((int64_t)b * a.Hq + head[rb]) * a.N + pos[rb]] = (m[rb] + __log2f(lt)) * kLn2;
        }
        if (LAZY) {
            const float zt = group_sum(lz[rb]);
            if (g == 0 && pos[rb] < N && pos[rb] >= N - a.W)
                a.lazy_rows[((int64_t)b * a.Hq + head[rb]) * a.W + (pos[rb] - (N - a.W))] = zt * inv;
        }
    }

    if (MODE == MODE_STREAM) {
        // Read back whole rows: lane l takes chunk l % CPR of row
        // RPI * u + l / CPR; row r of the wave is query position r / G,
        // head r % G (positions advance by carrying the head index).  The
        // region is the wave's own and a wave's LDS accesses run in order;
        // lanes read what other lanes wrote, so the reads must stay below
        // the writes.
        asm volatile("" ::: "memory");
        const int ch = lane % CPR;
        const int r = rw0 + lane / CPR;
        int p = r / G, hh = r - p * G;
#pragma unroll
        for (int u = 0; u < WROWS / RPI; ++u) {
            const int row = RPI * u + lane / CPR;
            const bf16x8 v = *(const bf16x8 *)(ostage + row * D + (ch ^ (row & (CPR - 1))) * 8);
            if (p < N)
                *(bf16x8 *)((bf16 *)a.o + b * a.o_sb + (int64_t)(hk * G + hh) * a.o_sh + (int64_t)p * a.o_sn +
                            ch * 8) = v;
            hh += RPI;
            while (hh >= G) {
                hh -= G;
                ++p;
            }
        }
    }

    // Streaming slice of this layer's KV (full attention, when asked for):
    // the workgroup holding flattened row p*G copies position p, so every
    // position has exactly one writer.  The workgroups of the last positions
    // run first (longest-first order), so this stays off the kernel's tail.
    if (MODE != MODE_STREAM) {
        const StreamOut so = stream_out_late();
        if (so.k != nullptr) {
            const int p_lo = (r0 + G - 1) / G;
            const int p_end = (r0 + BROWS + G - 1) / G;
            emit_stream_rows<64 * NW>((const char *)kbase, (const char *)vbase, a.k_sn, a.v_sn, so, b, hk, N, a.S,
                                      a.R, p_lo, p_end < N ? p_end : N, 2, D * 2, tid);
        }
    }
}

// Per-head lazy ratio: mean of the observed rows, summed in row order.  A
// sequence observes its last min(W, n) rows; slot k holds row n - W + k, so
// the slots of rows before position 0 (n < W) are set to NaN.  One wave per
// (batch, head): the wave stages the rows in LDS, 16 per lane in one
// coalesced round per chunk, and lane 0 adds them in row order.  (One thread
// per head reading its rows from memory one after the other took about
// 12 us for W = 128, a few per cent of an 8K-token layer.)
constexpr int kReduceChunk = 1024;
__global__ __launch_bounds__(64) void lazy_reduce_kernel(float *rows, float *ratio, int BH, int W,
                                                         const int *seq_len, int Hq, int N) {
    __shared__ float sh[kReduceChunk];
    const int i = blockIdx.x, lane = threadIdx.x;
    if (i >= BH) return;
    poison_lds<64>(sh, (int)sizeof(sh), lane);
    const int n = seq_length(seq_len, i / Hq, N);
    const int cnt = n < W ? n : W;
    float *r = rows + (int64_t)i * W;
    for (int w = lane; w < W - cnt; w += 64) r[w] = __builtin_nanf("");
    float acc = 0.f;
    for (int c0 = W - cnt; c0 < W; c0 += kReduceChunk) {
        const int len = W - c0 < kReduceChunk ? W - c0 : kReduceChunk;
        for (int w = lane; w < len; w += 64) sh[w] = r[c0 + w];
        __syncthreads();
        if (lane == 0)
            for (int w = 0; w < len; ++w) acc += sh[w];
        __syncthreads();
    }
    if (lane == 0) ratio[i] = cnt > 0 ? acc / (float)cnt : __builtin_nanf("");
}

// MODES: bit mask of the modes this configuration is built for.
template <int D, int RB, int BT, int NW, int MODES>
hipError_t launch_cfg(AttnArgs a, int mode, hipStream_t st) {
    const int64_t rows = (int64_t)a.N * a.G;
    const int brows = NW * 16 * RB;
    a.n_qtiles = (int)((rows + brows - 1) / brows);
    dim3 grid((unsigned)(a.n_qtiles * a.B * a.Hkv));
    dim3 block(64 * NW);
    if (log_enabled())
        log_printf("  launch attn_bf16_kernel<D=%d, RB=%d, BT=%d, mode=%s, NW=%d> grid %u x %u threads", D, RB, BT,
                   mode == MODE_FULL ? "full" : mode == MODE_FULL_LAZY ? "full+lazy" : "stream", NW, grid.x, block.x);
    if constexpr ((MODES & (1 << MODE_FULL)) != 0) {
        if (mode == MODE_FULL) {
            hipLaunchKernelGGL((attn_bf16_kernel<D, RB, BT, MODE_FULL, NW>), grid, block, 0, st, a);
            return hipGetLastError();
        }
    }
    if constexpr ((MODES & (1 << MODE_FULL_LAZY)) != 0) {
        if (mode == MODE_FULL_LAZY) {
            hipLaunchKernelGGL((attn_bf16_kernel<D, RB, BT, MODE_FULL_LAZY, NW>), grid, block, 0, st, a);
            return hipGetLastError();
        }
    }
    if constexpr ((MODES & (1 << MODE_STREAM)) != 0) {
        if (mode == MODE_STREAM) {
            hipLaunchKernelGGL((attn_bf16_kernel<D, RB, BT, MODE_STREAM, NW>), grid, block, 0, st, a);
            return hipGetLastError();
        }
    }
    return hipErrorInvalidValue;
}

// Compute units of the current device (cached per device).
int cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

template <int D>
hipError_t launch_d(AttnArgs a, int mode, hipStream_t st) {
    // 3 row blocks per wave: O (3*D/16 x 4), S^T (3 x 8), Q^T (3*D/16 x 2)
    // and the rest fit 256 registers for two waves per SIMD.  Full attention
    // takes 128-key tiles (half the workgroup barriers per key) in 8-wave
    // workgroups, one per CU.  Streaming, which keeps its raw scores, stays at
    // 64 keys to fit its registers, in 4-wave workgroups: a window of about
    // S + R keys is short work next to the workgroup's own Q loads and O
    // stores, and with two workgroups per CU one computes while the other
    // waits on memory.  Full attention over a grid of fewer than four 8-wave
    // workgroups per CU (an 8K-token layer: 688 on 256 CUs) takes the
    // 4-wave, 64-key shape too: twice the workgroups even out the causal
    // triangle's tail (2-3% faster there; at 32K tokens the 8-wave shape is).
    if (mode == MODE_STREAM) return launch_cfg<D, 3, 64, 4, 1 << MODE_STREAM>(a, mode, st);
    const int64_t items8 = ((int64_t)a.N * a.G + 383) / 384 * a.B * a.Hkv;
    if (items8 < 4 * cu_count())
        return launch_cfg<D, 3, 64, 4, (1 << MODE_FULL) | (1 << MODE_FULL_LAZY)>(a, mode, st);
    return launch_cfg<D, 3, 128, 8, (1 << MODE_FULL) | (1 << MODE_FULL_LAZY)>(a, mode, st);
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs &a, int D, int mode, hipStream_t st) {
    if (D == 64) return launch_d<64>(a, mode, st);
    return launch_d<128>(a, mode, st);
}

hipError_t launch_lazy_reduce(float *lazy_rows, float *lazy_ratio, int BH, int W, const int *seq_len,
                              int Hq, int N, hipStream_t st) {
    if (log_enabled()) log_printf("  launch lazy_reduce_kernel grid %d x 64 threads", BH);
    hipLaunchKernelGGL(lazy_reduce_kernel, dim3(BH), dim3(64), 0, st, lazy_rows, lazy_ratio, BH, W, seq_len, Hq,
                       N);
    return hipGetLastError();
}

}  // namespace lt
