// Decode-step attention over one layer's KV cache (full or streaming): the
// halved KV cache the LightTransfer pages report (Chinese write-up, training
// paragraph; press-release page, results) is what this step reads, so it is
// bound by HBM bandwidth.
//
// Split-KV.  Every workgroup streams a stretch of one KV head's keys once
// and serves all G query heads of the group from each K/V row, keeping one
// online-softmax state per head and writing one partial state per segment;
// a second kernel merges each sequence's partial states with their
// log-sum-exps.  Two ways of cutting the keys:
//   * every context kv_len long: each sequence's keys are cut into `splits`
//     splits of a multiple of 64 keys, one workgroup per (split, sequence,
//     KV head) -- no partition arithmetic in the kernel;
//   * per-sequence contexts (kv_lens, on the device): for each KV head the B
//     contexts are laid end to end (T keys in all) and cut into P equal parts
//     of Q = ceil(T/P) keys, one workgroup per (part, KV head), a part being
//     a segment of one sequence or the end of one and the start of the next.
//     Every workgroup gets the same number of keys whatever the length mix
//     is; the partition is computed by every workgroup from the lengths.
// Both write the partial of (sequence b, split or part p) to slot p + b (p
// counted over the batch), so one merge kernel serves both.
//
// bf16 path (matrix cores, v_mfma_f32_16x16x32_bf16 for Q.K and P.V):
//   S^T (16 keys x 16 columns) = K Q^T, where column c < G is query head
//   hk*G + c and the rest are zero padding; the column layout keeps each
//   head's softmax state in the lanes that own its column.  O^T += V^T P^T
//   takes P^T straight from the S^T registers and V^T from the row-major V
//   rows through ds_read_b64_tr_b16.  Each wave streams its own 32-key steps
//   with coalesced 128-bit loads, one step ahead.
// fp32 path (vector ALUs): lane = pair of head dims, one key at a time.
#include <mutex>
#include <type_traits>

#include "lt_internal.h"

namespace lt {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kTile = 64;  // split granularity in keys

__device__ __forceinline__ bf16x4 lds_read_tr(const bf16 *__restrict__ p) {
    i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4 *)(p));
    return __builtin_bit_cast(bf16x4, r);
}

// A 16-byte load of the V stream, marked nontemporal: every cache byte is
// read once per call, and such loads sustain a higher HBM read rate on this
// chip (a read kernel whose wave-wide loads cover 1 KiB in one piece holds
// about 6.3 TB/s with plain loads and 7.2 with nontemporal ones).  V rows are
// loaded that way, four full rows per wave-wide load.  The K loads (16 bytes
// per lane at a 64-byte stride inside each row, the matrix-core operand
// layout) stay plain: marked nontemporal, each row's lines were fetched
// piecemeal and the kernel ran 15% slower.
__device__ __forceinline__ bf16x8 load_stream(const bf16 *p) {
    return __builtin_nontemporal_load((const bf16x8 *)p);
}

// V tiles in LDS use the same 16-byte-chunk swizzle as the prefill kernel,
// so the transposing reads of a 32-key step are bank-conflict free.
__device__ __forceinline__ int swz_v128(int row, int chunk) { return chunk ^ (2 * (row & 7)); }
__device__ __forceinline__ int swz_v64(int row, int chunk) { return chunk ^ (2 * ((row >> 1) & 3)); }

// Max over the four 16-lane groups of a column: v_permlane16/32_swap of a
// value with a copy of itself leaves each lane its own value and that of
// lane l^16 (l^32).  Issued in asm with both registers read-write (through
// the compiler builtin one result was dropped); s_nop gives the wait states.
__device__ __forceinline__ float group_max(float x) {
    unsigned a0 = __builtin_bit_cast(unsigned, x), b0 = a0;
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a0), "+v"(b0));
    const float y = fmaxf(__builtin_bit_cast(float, a0), __builtin_bit_cast(float, b0));
    unsigned a1 = __builtin_bit_cast(unsigned, y), b1 = a1;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a1), "+v"(b1));
    return fmaxf(__builtin_bit_cast(float, a1), __builtin_bit_cast(float, b1));
}

// Makes a uniform value available at this point: the kernel-argument reads
// the decode kernel needs are all placed at its entry this way, so they are
// issued together instead of in dependent rounds after the partition's
// branches (each round trip to argument memory is microseconds that a short
// layer pays in full).
template <typename T>
__device__ __forceinline__ void read_now(const T &x) {
    asm volatile("" ::"s"(x));
}

// Context length of sequence b (the uniform kv_len, or kv_lens[b] clamped
// to [0, kv_len]); uniform across the workgroup.
__device__ __forceinline__ int64_t ctx_len(const DecodeArgs &a, int b) {
    if (a.kv_lens == nullptr) return a.kv_len;
    const int x = __builtin_amdgcn_readfirstlane(a.kv_lens[b]);
    return x < 0 ? 0 : (x > a.kv_len ? a.kv_len : (int64_t)x);
}

// x / y for x >= 0, y > 0 (uniform values).  A 64-bit division expands to
// hundreds of vector instructions, which a short layer's workgroups would
// wait on before their first load; 32-bit operands (every realistic size)
// take the short path.
__device__ __forceinline__ int64_t div_nonneg(int64_t x, int64_t y) {
    // The hardware has no scalar divide: the quotient comes out of vector
    // registers and is moved back to a scalar one, so that nothing derived
    // from it occupies vector registers (they decide the occupancy).
    if (((x | y) >> 31) == 0) return (int64_t)__builtin_amdgcn_readfirstlane((uint32_t)x / (uint32_t)y);
    const int64_t q = x / y;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)q);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(q >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Keys sequence b takes in the end-to-end order of the per-sequence
// partition: its context, rounded up to whole pages for a paged cache, so
// that with parts of a whole number of pages every segment starts on a page
// (and every 16-key half of a 32-key step lies inside one page).
template <bool PAGED>
__device__ __forceinline__ int64_t ctx_span(const DecodeArgs &a, int b) {
    const int64_t n = ctx_len(a, b);
    if constexpr (PAGED) return (n + a.page - 1) >> a.page_shift << a.page_shift;
    return n;
}

// Per-sequence contexts (kv_lens): total keys T of one head over the batch
// and the part size Q = ceil(T/P) (rounded up to whole pages when paged).
struct Partition {
    int64_t T, Q;
};
template <bool PAGED>
__device__ __forceinline__ Partition partition(const DecodeArgs &a) {
    int64_t T = 0;
    for (int b = 0; b < a.B; ++b) T += ctx_span<PAGED>(a, b);
    int64_t Q = T > 0 ? div_nonneg(T + a.n_parts - 1, a.n_parts) : 0;
    if constexpr (PAGED) Q = (Q + a.page - 1) >> a.page_shift << a.page_shift;
    return Partition{T, Q};
}

// First key of sequence b in the end-to-end order.
template <bool PAGED>
__device__ __forceinline__ int64_t ctx_start(const DecodeArgs &a, int b) {
    int64_t S = 0;
    for (int i = 0; i < b; ++i) S += ctx_span<PAGED>(a, i);
    return S;
}

// Calls f(b, kbeg, kend, slot) for every sequence b that part `part`
// overlaps, with its keys [kbeg, kend) in that part.  The partial of
// (sequence b, part p) goes to workspace slot p + b: slots increase with
// (b, p) in order and a sequence's parts are consecutive, so no two pairs
// share a slot and P + B - 1 slots suffice.  The first segment is called
// outside the loop: as straight-line code its loads issue right after the
// partition arithmetic (inside a loop the compiler hoisted the invariant
// setup of every segment in front of them, which short layers paid for).
// Paged: a part that reaches only the page padding past a context's end has
// no keys of that sequence and writes no partial (the merge skips it too).
template <bool PAGED, typename F>
__device__ __forceinline__ void for_each_segment(const DecodeArgs &a, int part, F &&f) {
    const Partition pt = partition<PAGED>(a);
    if (pt.T == 0) return;
    const int64_t g0 = (int64_t)part * pt.Q;
    if (g0 >= pt.T) return;
    const int64_t g1 = g0 + pt.Q < pt.T ? g0 + pt.Q : pt.T;
    // The sequence holding key g0.
    int b = 0;
    int64_t S = 0, n = ctx_span<PAGED>(a, 0);
    while (b + 1 < a.B && S + n <= g0) {
        S += n;
        n = ctx_span<PAGED>(a, ++b);
    }
    if constexpr (PAGED) {
        const int64_t len = ctx_len(a, b);
        const int64_t kend = (g1 < S + n ? g1 : S + n) - S;
        if (g0 - S < len) f(b, g0 - S, kend < len ? kend : len, part + b);
    } else {
        f(b, g0 - S, (g1 < S + n ? g1 : S + n) - S, part + b);
    }
    // Sequences after it that the part still reaches.
    for (S += n, ++b; b < a.B && S < g1; ++b) {
        n = ctx_span<PAGED>(a, b);
        if constexpr (PAGED) {
            const int64_t len = ctx_len(a, b);
            const int64_t kend = (g1 < S + n ? g1 : S + n) - S;
            if (len > 0) f(b, (int64_t)0, kend < len ? kend : len, part + b);
        } else {
            if (n > 0) f(b, (int64_t)0, (g1 < S + n ? g1 : S + n) - S, part + b);
        }
        S += n;
    }
}

// Pool page of key `key` of sequence b in a paged cache (clamped to the pool,
// so a table entry out of range reads a wrong page instead of faulting).
// The table entry is uniform; it is read through the scalar cache and waited
// for in the same asm block: a vector load would make the wait for it also
// wait for the step's K and V loads issued before it.
__device__ __forceinline__ int64_t pool_page(const DecodeArgs &a, int b, int64_t key) {
    const int *p = a.block_table + ((int64_t)b * a.max_pages + (key >> a.page_shift));
    int pg;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(pg) : "s"(p));
    pg = pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);
    return pg;
}

// Partial state of (slot, query head h):
// ws[(slot * Hq + h) * (D + 2) + {0..D-1: o/l, D: m (log2), D+1: l}]
//
// Each wave streams its own 32-key steps of a segment (steps w, w+4, ...):
// K goes straight from global memory into the matrix-core A operand (lane
// (c, g) holds dims (D/4)g .. (D/4)(g+1)-1 of key c of a 16-key block,
// contiguous bytes), one step ahead in registers.  V rows are loaded one step
// ahead into registers too (coalesced 128-bit nontemporal loads), written at
// the start of their step into an LDS slot private to the wave and read back
// transposed.  All loads are register loads, so the compiler's
// load-counter waits stay exact (mixing in direct global->LDS loads made it
// wait for every outstanding load).  No workgroup barrier until the four
// waves merge their states at the end of the segment.
// UNIFORM (every context kv_len long): workgroup (split, b*Hkv + kv head)
// streams keys [split*kps, (split+1)*kps) of sequence b, kps = part_keys, and
// writes slot b*splits + split + b.  Otherwise (kv_lens): workgroup (part,
// kv head) streams its part of the end-to-end keys (for_each_segment).
// PAGED (per-sequence contexts in a page pool): each 16-key half of a step
// lies in one page, whose pool index is read once per step (twice with
// 16-row pages).
template <int D, bool UNIFORM, bool PAGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_bf16_kernel(DecodeArgs a) {
    static_assert(!(UNIFORM && PAGED), "paged caches take the per-sequence partition");
    constexpr int KS = D / 32;       // 32-dim steps (Q.K)
    constexpr int DB = D / 16;       // 16-dim blocks (O)
    constexpr int STEP = 32;         // keys per step
    constexpr int CPR = D / 8;       // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;    // V rows per wave-wide 128-bit load
    constexpr int NVL = STEP / RPI;  // V loads per lane and step
    constexpr int VTILE = STEP * D;  // elements per V step
    constexpr int KPL = D / 32;      // 16-byte K loads per lane and 16-key block (D/4 dims)
    // V slots (one step per wave) and, after the key loop, the merge buffer.
    constexpr int RING_BYTES = 4 * VTILE * (int)sizeof(bf16);
    constexpr int RED_BYTES = 4 * 16 * (D + 1) * (int)sizeof(float);
    __shared__ __attribute__((aligned(16))) char smem[RING_BYTES > RED_BYTES ? RING_BYTES : RED_BYTES];
    __shared__ float red_m[4][16], red_l[4][16];
    float (*const red_o)[16][D + 1] = (float (*)[16][D + 1])smem;

    // readfirstlane marks the wave index uniform, so the per-step tests are
    // scalar branches and the load counters are tracked exactly across them.
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c16 = lane & 15;
    const int hk = UNIFORM ? (int)(blockIdx.y % a.Hkv) : (int)blockIdx.y;
    // Query heads hk*G + hc .. + ncol - 1 of the group: the 16 columns of the
    // products hold at most 16 heads, so a group of more (G > 16) is served
    // in chunks of 16, one per grid z (each chunk streams the keys itself).
    const int hc = 16 * (int)blockIdx.z;
    const int ncol = a.G - hc < 16 ? a.G - hc : 16;
    poison_lds<256>(smem, (int)sizeof(smem), tid);
    poison_lds<256>(red_m, (int)sizeof(red_m), tid);
    poison_lds<256>(red_l, (int)sizeof(red_l), tid);
    read_now(a.q), read_now(a.k), read_now(a.v), read_now(a.ws);
    read_now(a.k_sb), read_now(a.k_sh), read_now(a.k_sn);
    read_now(a.v_sb), read_now(a.v_sh), read_now(a.v_sn);
    read_now(a.B), read_now(a.Hq), read_now(a.G), read_now(a.c);
    read_now(a.kv_len), read_now(a.kv_lens), read_now(a.part_keys), read_now(a.n_parts), read_now(a.splits);
    const int G = a.G;
    const float c = a.c;
    bf16 *const slot = (bf16 *)smem + wave * VTILE;

    // One segment: keys [kbeg, kend) of sequence b; the merged state of the
    // four waves goes to workspace slot ws_slot.
    auto segment = [&](int b, int64_t kbeg, int64_t kend, int ws_slot) {
        const int nsteps = (int)((kend - kbeg + STEP - 1) / STEP);
        const bf16 *kbase = (const bf16 *)a.k + b * a.k_sb + (int64_t)hk * a.k_sh;
        const bf16 *vbase = (const bf16 *)a.v + b * a.v_sb + (int64_t)hk * a.v_sh;

        // Q^T: lane holds column c16 (query head hk*G + c16, zero if c16 >= G),
        // dims (D/4)g + 8ks .. +7 of step ks -- the same dim order as the K operand.
        bf16x8 qreg[KS];
        {
            const bool col_ok = c16 < ncol;
            const bf16 *qp = (const bf16 *)a.q + ((int64_t)b * a.Hq + hk * G + hc + (col_ok ? c16 : 0)) * D + (D / 4) * g;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                bf16x8 v = *(const bf16x8 *)(qp + 8 * ks);
                qreg[ks] = col_ok ? v : bf16x8{};
            }
        }

        bf16x8 kreg[2][2][KPL];  // [buffer][16-key block][load]
        bf16x8 vreg[NVL];        // V rows of the next step: row RPI*u + lane/CPR, chunk lane%CPR
        auto issue = [&](int t, int buf) {
            const int64_t key0 = kbeg + (int64_t)t * STEP;
            if constexpr (PAGED) {
                // Rows r = key - key0 of the step, clamped to the segment's
                // last key (a uniform bound), are read from the page of key0
                // at its row of key0.  Pages of 32 rows or more hold the whole
                // step.  16-row pages hold one 16-key half each: the second
                // half (r >= 16, the K operand's second block and the second
                // half of the V loads) then comes from the page of key0 + 16,
                // looked up only when that half has keys.  The row strides
                // were checked on the host to keep 31 rows within 32-bit
                // offsets.
                const int64_t pg = pool_page(a, b, key0), r0 = key0 & (a.page - 1);
                const int64_t kA = pg * a.k_sb + (int64_t)hk * a.k_sh + r0 * a.k_sn;
                const int64_t vA = pg * a.v_sb + (int64_t)hk * a.v_sh + r0 * a.v_sn;
                int64_t kB = kA, vB = vA;  // element offsets of row 0 of the step, for rows r >= 16
                if (a.page_shift == 4 && key0 + 16 < kend) {
                    const int64_t pg2 = pool_page(a, b, key0 + 16);
                    kB = pg2 * a.k_sb + (int64_t)hk * a.k_sh - 16 * a.k_sn;
                    vB = pg2 * a.v_sb + (int64_t)hk * a.v_sh - 16 * a.v_sn;
                }
                const int64_t last = kend - 1 - key0;
                const int lim = last < STEP - 1 ? (int)last : STEP - 1;
                const int ksn = (int)a.k_sn, vsn = (int)a.v_sn;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int r = kb * 16 + c16 < lim ? kb * 16 + c16 : lim;
                    const bf16 *kp = (const bf16 *)a.k + (kb == 0 ? kA : kB) + (r * ksn + (D / 4) * g);
#pragma unroll
                    for (int u = 0; u < KPL; ++u) kreg[buf][kb][u] = *(const bf16x8 *)(kp + 8 * u);
                }
#pragma unroll
                for (int u = 0; u < NVL; ++u) {
                    const int r = RPI * u + lane / CPR < lim ? RPI * u + lane / CPR : lim;
                    vreg[u] = load_stream((const bf16 *)a.v + (RPI * u < 16 ? vA : vB) + (r * vsn + (lane % CPR) * 8));
                }
                return;
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                int64_t key = key0 + kb * 16 + c16;
                key = key < kend ? key : kend - 1;
                const bf16 *kp = kbase + key * a.k_sn + (D / 4) * g;
#pragma unroll
                for (int u = 0; u < KPL; ++u) kreg[buf][kb][u] = *(const bf16x8 *)(kp + 8 * u);
            }
#pragma unroll
            for (int u = 0; u < NVL; ++u) {
                int64_t key = key0 + RPI * u + lane / CPR;
                key = key < kend ? key : kend - 1;
                vreg[u] = load_stream(vbase + key * a.v_sn + (lane % CPR) * 8);
            }
    };
    // Write the staged V rows into the wave's slot, each 16-byte chunk at
    // its swizzled place.
    auto stage_v = [&]() {
#pragma unroll
        for (int u = 0; u < NVL; ++u) {
            const int row = RPI * u + lane / CPR, ph = lane % CPR;
            const int pc = D == 128 ? swz_v128(row, ph) : swz_v64(row, ph);
            *(bf16x8 *)(slot + row * D + pc * 8) = vreg[u];
        }
    };

    f32x4 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = kNegInf, l = 0.f;

    // One step of this wave: t is the step, BUF (compile time, so the K
    // registers stay registers) the buffer holding its K.  The step stages
    // its V rows, then (with PREFETCH) issues the loads of step t + 4, whose
    // latency the rest of the step covers.  The slot's previous contents
    // were consumed by the last step's transposing reads, which completed
    // before that step's products; LDS accesses of one wave run in order.
    auto step = [&](int t, auto buf_c, auto prefetch_c) {
        constexpr int BUF = decltype(buf_c)::value;
        stage_v();
        if constexpr (decltype(prefetch_c)::value) issue(t + 4, BUF ^ 1);
        // Lanes read rows other lanes wrote: keep the reads below the writes.
        asm volatile("" ::: "memory");
        const int64_t key0 = kbeg + (int64_t)t * STEP;

        f32x4 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kreg[BUF][kb][ks], qreg[ks], s[kb], 0, 0, 0);
        }
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                s[kb][r] = key0 + kb * 16 + 4 * g + r < kend ? s[kb][r] : kNegInf;
                mx = fmaxf(mx, s[kb][r]);
            }
        mx = group_max(mx);
        const float mnew = fmaxf(m, mx * c);
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);
        m = mnew;
        bf16x8 p8;
        float rs = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[0][e], c, -mnew));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[1][e], c, -mnew));
            rs += p0 + p1;
            p8[e] = (bf16)p0;
            p8[e + 4] = (bf16)p1;
        }
        l = l * alpha + rs;
        const bf16 *Vb = slot;
        const int row1 = 4 * g + (c16 >> 2), row2 = row1 + 16;
        const int half = (c16 & 1) * 4;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int lch = 2 * db + ((c16 & 3) >> 1);
            const int p1 = D == 128 ? swz_v128(row1, lch) : swz_v64(row1, lch);
            const int p2 = D == 128 ? swz_v128(row2, lch) : swz_v64(row2, lch);
            const bf16x8 A = __builtin_shufflevector(lds_read_tr(Vb + row1 * D + p1 * 8 + half),
                                                     lds_read_tr(Vb + row2 * D + p2 * 8 + half),
                                                     0, 1, 2, 3, 4, 5, 6, 7);
            o[db] *= alpha;
            o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, p8, o[db], 0, 0, 0);
        }
    };
    // The wave's steps are wave, wave + 4, ...; pairs whose successors all
    // exist run without a branch between issue and wait, so the compiler's
    // load-counter bookkeeping stays exact (a conditional prefetch made it
    // fall back to waiting for every load at each step).
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    using Pf = std::true_type;
    using Last = std::false_type;
    int t = wave;
    if (t < nsteps) issue(t, 0);
    for (; t + 8 < nsteps; t += 8) {
        step(t, B0{}, Pf{});
        step(t + 4, B1{}, Pf{});
    }
    if (t + 4 < nsteps) {
        step(t, B0{}, Pf{});
        step(t + 4, B1{}, Last{});
    } else if (t < nsteps) {
        step(t, B0{}, Last{});
    }

    // Merge the four waves' states for each column, then store the split's partial.
    __syncthreads();  // every wave is done with its V slot
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
    for (int e = tid; e < ncol * D; e += 256) {
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
        float *dst = a.ws + ((int64_t)ws_slot * a.Hq + hk * G + hc + col) * (D + 2);
        dst[d] = O / L;
        if (d == 0) {
            dst[D] = M;
            dst[D + 1] = L;
        }
    }
    __syncthreads();  // the merge buffers share LDS with the next segment's V slots
    };
    if constexpr (UNIFORM) {
        const int split = blockIdx.x, b = (int)(blockIdx.y / a.Hkv);
        const int64_t kbeg = (int64_t)split * a.part_keys;
        const int64_t kend = kbeg + a.part_keys < a.kv_len ? kbeg + a.part_keys : a.kv_len;
        if (kbeg < kend) segment(b, kbeg, kend, b * a.splits + split + b);
    } else {
        for_each_segment<PAGED>(a, (int)blockIdx.x, segment);
    }
}

// fp32: block of 64 lanes per (query head, part), looping over the part's
// segments; lane owns dims lane, lane+64.  Paged: the pool page is looked up
// at the segment's first key and at every page boundary.
template <int D, bool UNIFORM, bool PAGED>
__global__ __launch_bounds__(64) void decode_f32_kernel(DecodeArgs a) {
    constexpr int PER = D / 64;
    const int lane = threadIdx.x;
    const int h = UNIFORM ? (int)(blockIdx.y % a.Hq) : (int)blockIdx.y, hk = h / a.G;
    auto segment = [&](int b, int64_t kbeg, int64_t kend, int ws_slot) {
        const float *kbase = (const float *)a.k + b * a.k_sb + (int64_t)hk * a.k_sh;
        const float *vbase = (const float *)a.v + b * a.v_sb + (int64_t)hk * a.v_sh;
        float q[PER], o[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            q[u] = ((const float *)a.q)[((int64_t)b * a.Hq + h) * D + lane + 64 * u];
            o[u] = 0.f;
        }
        float m = kNegInf, l = 0.f;
        const float *kpg = nullptr, *vpg = nullptr;  // paged: the current page's rows of this KV head
        for (int64_t j = kbeg; j < kend; ++j) {
            const float *kr, *vr;
            if constexpr (PAGED) {
                const int64_t r = j & (a.page - 1);
                if (j == kbeg || r == 0) {
                    const int64_t pg = pool_page(a, b, j);
                    kpg = (const float *)a.k + pg * a.k_sb + (int64_t)hk * a.k_sh;
                    vpg = (const float *)a.v + pg * a.v_sb + (int64_t)hk * a.v_sh;
                }
                kr = kpg + r * a.k_sn;
                vr = vpg + r * a.v_sn;
            } else {
                kr = kbase + j * a.k_sn;
                vr = vbase + j * a.v_sn;
            }
            float dot = 0.f;
#pragma unroll
            for (int u = 0; u < PER; ++u) dot = __builtin_fmaf(q[u], kr[lane + 64 * u], dot);
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) dot += __shfl_xor(dot, off);
            const float s = dot * a.c;
            const float mnew = fmaxf(m, s);
            const float alpha = exp2f(m - mnew);
            const float p = exp2f(s - mnew);
            m = mnew;
            l = l * alpha + p;
#pragma unroll
            for (int u = 0; u < PER; ++u) o[u] = __builtin_fmaf(p, vr[lane + 64 * u], o[u] * alpha);
        }
        float *dst = a.ws + ((int64_t)ws_slot * a.Hq + h) * (D + 2);
#pragma unroll
        for (int u = 0; u < PER; ++u) dst[lane + 64 * u] = o[u] / l;
        if (lane == 0) {
            dst[D] = m;
            dst[D + 1] = l;
        }
    };
    if constexpr (UNIFORM) {
        const int split = blockIdx.x, b = (int)(blockIdx.y / a.Hq);
        const int64_t kbeg = (int64_t)split * a.part_keys;
        const int64_t kend = kbeg + a.part_keys < a.kv_len ? kbeg + a.part_keys : a.kv_len;
        if (kbeg < kend) segment(b, kbeg, kend, b * a.splits + split + b);
    } else {
        for_each_segment<PAGED>(a, (int)blockIdx.x, segment);
    }
}

// Merge split partials: out = sum_s w_s o_s / sum_s w_s, w_s = l_s 2^(m_s - M);
// lse = (M + log2 sum_s w_s) ln 2.  One block per (batch, query head), one
// thread per head dim.  The partials were written by workgroups on every XCD,
// so each load is a round trip to the shared memory level: all loads of up
// to CH splits are issued together, and chunks of CH splits are merged
// online (a running max M with L, O rescaled when it grows).
template <int D, typename T, bool PAGED>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
    constexpr int CH = 16;
    read_now(a.ws), read_now(a.o), read_now(a.lse), read_now(a.B), read_now(a.Hq);
    read_now(a.kv_len), read_now(a.kv_lens), read_now(a.part_keys), read_now(a.n_parts), read_now(a.splits);
    const int bh = blockIdx.x;
    const int b = bh / a.Hq, h = bh % a.Hq;
    const int d = threadIdx.x;
    // Sequence b's partial states in consecutive slots: its `splits` splits
    // from slot b*splits + b (uniform contexts), or the parts p0..p1 its
    // context overlaps, in slots p0 + b .. p1 + b (none for an empty one).
    int64_t p0 = (int64_t)b * a.splits;
    int n = a.splits;
    if (a.kv_lens != nullptr) {
        const Partition pt = partition<PAGED>(a);
        const int64_t S = ctx_start<PAGED>(a, b), len = ctx_len(a, b);
        p0 = len > 0 ? div_nonneg(S, pt.Q) : 0;
        n = len > 0 ? (int)(div_nonneg(S + len - 1, pt.Q) - p0) + 1 : 0;
    }
    const int64_t stride = (int64_t)a.Hq * (D + 2);
    const float *src = a.ws + (p0 + b) * stride + (int64_t)h * (D + 2);
    float M = kNegInf, L = 0.f, O = 0.f;
    for (int s0 = 0; s0 < n; s0 += CH) {
        float mv[CH], lv[CH], ov[CH];
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int sp = s0 + i < n ? s0 + i : n - 1;
            mv[i] = src[sp * stride + D];
            lv[i] = src[sp * stride + D + 1];
            ov[i] = src[sp * stride + d];
        }
        float Mc = M;
#pragma unroll
        for (int i = 0; i < CH; ++i)
            if (s0 + i < n) Mc = fmaxf(Mc, mv[i]);
        // Splits without keys carry m = -inf, l = 0: they get weight 0 (and
        // while every split so far is empty, M = Mc = -inf must not give NaN).
        const float f = M == kNegInf ? 0.f : __builtin_amdgcn_exp2f(M - Mc);
        L *= f;
        O *= f;
#pragma unroll
        for (int i = 0; i < CH; ++i)
            if (s0 + i < n) {
                const float w = mv[i] == kNegInf ? 0.f : lv[i] * __builtin_amdgcn_exp2f(mv[i] - Mc);
                L += w;
                O += w * ov[i];
            }
        M = Mc;
    }
    // An empty context (kv_lens[b] == 0): output 0, LSE -inf.
    ((T *)a.o)[(int64_t)bh * D + d] = (T)(L > 0.f ? O / L : 0.f);
    if (d == 0 && a.lse != nullptr) a.lse[bh] = (M + log2f(L)) * kLn2;
}

}  // namespace

int64_t decode_split_keys(int64_t kv_len, int splits) {
    const int64_t kps = (kv_len + splits - 1) / splits;
    return (kps + kTile - 1) / kTile * kTile;
}

int decode_num_splits(int B, int Hkv, int64_t kv_len) {
    // Every context kv_len long: about 512 workgroups (two per CU) over the
    // B*Hkv (sequence, KV head) pairs, splits of a multiple of kTile keys.
    const int64_t units = (int64_t)B * Hkv;
    int64_t want = (512 + units - 1) / units;
    const int64_t max_splits = (kv_len + kTile - 1) / kTile;
    if (want > max_splits) want = max_splits;
    if (want < 1) want = 1;
    const int64_t kps = decode_split_keys(kv_len, (int)want);
    return (int)((kv_len + kps - 1) / kps);
}

int decode_num_parts(int B, int Hkv, int64_t kv_len) {
    // Aim for about 512 workgroups (two per CU, eight waves streaming their
    // own steps) so enough loads are in flight to cover HBM latency; parts
    // of at least kTile keys when every context has its full length.
    int64_t want = (512 + Hkv - 1) / Hkv;
    const int64_t max_parts = ((int64_t)B * kv_len + kTile - 1) / kTile;
    if (want > max_parts) want = max_parts;
    if (want < 1) want = 1;
    return (int)want;
}

size_t decode_ws_bytes(int B, int Hq, int D, int n_parts) {
    return (size_t)(n_parts + B - 1) * Hq * (D + 2) * sizeof(float);
}

namespace {
// The split kernel, then the merge; each launch is checked, so a refused
// merge launch is reported even though the split kernel is already queued.
// PAGED: the per-sequence partition over pages of a pool.
template <int D, bool PAGED>
hipError_t launch_decode_dp(const DecodeArgs &a, int dtype, hipStream_t st) {
    const bool uni = a.kv_lens == nullptr;
    const char *kind = PAGED ? "paged" : uni ? "uniform" : "per-sequence";
    if (dtype == LT_BF16) {
        const unsigned chunks = (unsigned)((a.G + 15) / 16);  // query-head chunks of 16 per KV head
        const dim3 grid = uni ? dim3((unsigned)a.splits, (unsigned)(a.B * a.Hkv), chunks)
                              : dim3((unsigned)a.n_parts, (unsigned)a.Hkv, chunks);
        if (log_enabled())
            log_printf("  launch decode_bf16_kernel<D=%d, %s> grid %u x %u x %u x 256 threads (%s), then "
                       "decode_combine_kernel grid %d x %d threads", D, kind, grid.x, grid.y, grid.z,
                       uni ? "splits x (sequence, KV head) x head chunks" : "parts x KV head x head chunks",
                       a.B * a.Hq, D);
        if (PAGED)
            hipLaunchKernelGGL((decode_bf16_kernel<D, false, true>), grid, dim3(256), 0, st, a);
        else if (uni)
            hipLaunchKernelGGL((decode_bf16_kernel<D, true, false>), grid, dim3(256), 0, st, a);
        else
            hipLaunchKernelGGL((decode_bf16_kernel<D, false, false>), grid, dim3(256), 0, st, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((decode_combine_kernel<D, bf16, PAGED>), dim3(a.B * a.Hq), dim3(D), 0, st, a);
    } else {
        const dim3 grid = uni ? dim3((unsigned)a.splits, (unsigned)(a.B * a.Hq))
                              : dim3((unsigned)a.n_parts, (unsigned)a.Hq);
        if (log_enabled())
            log_printf("  launch decode_f32_kernel<D=%d, %s> grid %u x %u x 64 threads, then decode_combine_kernel",
                       D, kind, grid.x, grid.y);
        if (PAGED)
            hipLaunchKernelGGL((decode_f32_kernel<D, false, true>), grid, dim3(64), 0, st, a);
        else if (uni)
            hipLaunchKernelGGL((decode_f32_kernel<D, true, false>), grid, dim3(64), 0, st, a);
        else
            hipLaunchKernelGGL((decode_f32_kernel<D, false, false>), grid, dim3(64), 0, st, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((decode_combine_kernel<D, float, PAGED>), dim3(a.B * a.Hq), dim3(D), 0, st, a);
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs &a, int dtype, hipStream_t st) {
    return a.page > 0 ? launch_decode_dp<D, true>(a, dtype, st) : launch_decode_dp<D, false>(a, dtype, st);
}
}  // namespace

// Workspace of lt_hybrid_decode_attn_noalloc: the split partial states in a
// device array of fixed size, one copy per GPU, held until the process ends.
// Host code never passes `scratch` itself to a kernel (on the host the name
// stands for a host-side shadow, not a device address): the device address
// is looked up once per GPU and kept.
static __device__ __align__(256) char scratch[LT_DECODE_NOALLOC_SCRATCH_BYTES];

hipError_t decode_scratch(void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs &a, int dtype, hipStream_t st) {
    return a.D == 64 ? launch_decode_d<64>(a, dtype, st) : launch_decode_d<128>(a, dtype, st);
}

}  // namespace lt
