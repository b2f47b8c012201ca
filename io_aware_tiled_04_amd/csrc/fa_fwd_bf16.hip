// Attention forward pass, bf16 inputs, for gfx950 (MI355X).
//
// One workgroup owns one tile of kBr = 256 query rows of one query head and
// keeps it resident (in registers, 32 rows per wave) while it streams the
// K/V tiles of the matching K/V head through LDS: the tiling of the reading-notes page
// (Methods, step 1: Q stays on chip, K and V are read block by block) in the
// query-outer loop order the blog names at the end of its blocked derivation
// (section 带在线Softmax重缩放的分块模式, closing remark).  Per K/V tile j:
//
//   S^T = K_j Q_i^T                 bf16 MFMA 32x32x16, fp32 accumulate
//   mask (causal / past-the-end)    only on tiles that cross the diagonal or N
//   m' = max(m, rowmax S)           per lane + one permlane32 swap
//   P  = exp2(S*c - m'), l = l*2^(m-m') + rowsum P      (c = scale*log2 e)
//   O^T = 2^(m-m') O^T + V_j^T P^T  bf16 MFMA 32x32x16, fp32 accumulate
//
// which is the rescaled running sum and output of the reading-notes page
// (Methods, the two rescaling equations) in the unnormalised form of the
// Polish notes (section "Nie wystarczy uśrednić wyników bloków": keep m, l and
// u, divide u by l at the end).  The epilogue divides by l and writes the
// natural-log logsumexp m + ln l that the blog's backward section keeps.
// Two row sums are kept: l over the fp32 weights (for the logsumexp) and l~
// over the bf16-rounded weights that actually enter P V, formed on the
// matrix cores beside P V; O is divided by l~, so that it is exactly the
// weighted mean the matrix cores accumulated.  (Dividing by l instead adds
// the rounding error of the largest weight, up to 2^-9 |v|, to every row a
// single key dominates.)
//
// Scheduling choices (the arithmetic is that of the method):
//  * Ping-pong.  The 8 waves form two groups with one wave of each on every
//    SIMD.  Between workgroup barriers, one group runs a matrix phase
//    (S_t and P_{t-1} V_{t-1}) while the other runs a vector phase (the
//    softmax of its S), then they swap, so the matrix cores of each SIMD are
//    fed by one group while the other keeps the vector ALUs busy.  K tiles
//    run one tile ahead of V tiles through LDS to fit this order.  A wave
//    raises its issue priority for its matrix phase.
//  * Direct global-to-LDS copies.  K and V tiles go from HBM straight into
//    LDS (buffer loads with the LDS flag, no registers, no LDS store
//    instructions): the second group loads K tiles at the start of its
//    vector phase and the first group V tiles at the start of its matrix
//    phase, into two-deep rings whose target buffer the preceding barrier has
//    just freed.  Rows past the end of the sequence come back as zeros from
//    the buffer range check.
// and one change against a literal reading, exact in real arithmetic:
//  * Lazy rescaling.  The reference max m of a row is the exact row max of
//    the first tile; afterwards P is taken against it directly, and m only
//    moves (to the exact max, with a rescale of O and l and a redo of the
//    tile) when a row sum of the tile exceeds kSumLimit = 2^20, i.e. before
//    any p can leave [0, 2^20].  Any common reference value gives the same
//    O = sum p v / sum p and the same LSE = m + log2 l, and almost every
//    tile skips both the row max and the rescale.
//
// Layout choices (each checked against the MFMA lane layouts of gfx950):
//  * Computing S^T rather than S puts one query per lane (column of the
//    32x32 accumulator), so the row max and row sum are per-lane reductions
//    plus one exchange between lanes l and l+32.
//  * The S^T accumulator registers 8c..8c+7 of a 32-key block are exactly the
//    B operand (P^T, 16 keys x 32 queries) of the P V product for the 16-key
//    chunk c, once the keys of that chunk are taken in the order
//    {16c+4h+0..3, 16c+8+4h+0..3} for lane half h, so P never leaves
//    registers.  V stays row-major in LDS, and two transposing LDS reads
//    (ds_read_b64_tr_b16) per MFMA give the V^T operand in that key order.
//  * The O^T accumulator also has one query per lane, so the rescale and the
//    final 1/l are one multiplier per lane.
#include "fa_kernels.h"

#include <stdint.h>

#include "philox.h"

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LDS __attribute__((address_space(3)))

constexpr int kWaves = 8;
constexpr int kWaveRows = 32;                    // query rows per wave
constexpr int kThreads = kWaves * 64;
constexpr int kBr = kWaves * kWaveRows;          // query rows per workgroup
constexpr int kGroupThreads = kThreads / 2;      // threads of one wave group
static_assert(kBr == kBlockRowsBf16, "grid and kernel disagree on the query tile");
constexpr float kSumLimit = 1048576.0f;          // 2^20: largest row sum of a tile before a rescale
constexpr int kMatrixPrio = 3;                   // wave issue priority during a matrix phase
// s_getreg immediate for HW_REG_HW_ID (id 4), bits [5:4] = SIMD id
constexpr int kGetregSimdId = 4 | (4 << 6) | ((2 - 1) << 11);
// s_waitcnt immediates (vmcnt [3:0] and [15:14], expcnt [6:4], lgkmcnt
// [11:8]): wait for all vector memory operations, or for all LDS ones.
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitLgkm0 = 0xC07F;

// Workgroup barrier for the tile loop: this wave's LDS reads and writes are
// complete (lgkmcnt), then s_barrier; the empty asm statements keep the
// compiler from moving memory accesses across it.  Unlike __syncthreads it
// does not wait for outstanding vector memory operations: the direct K
// loads of one phase are meant to land during the next one, and their
// writer waits for them (vmcnt) before the barrier that publishes the tile.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// K/V tile geometry in LDS: two K buffers and two V buffers, all filled
// by direct global-to-LDS loads (one wave instruction writes 1 KiB: 16 bytes
// per lane, in lane order).
//  * K is stored chunk-major: the 16-byte chunk c (d = 8c .. 8c+7) of key r
//    sits in slot c * BC + r.  One direct load fills one chunk of all 64
//    keys, and the S operand read of 32 lanes (32 consecutive keys, one
//    chunk) is 512 contiguous bytes, free of bank conflicts.
//  * V is stored row-major ([key][d], 2D bytes per key), with the 16-byte
//    chunks of key r permuted: chunk c sits at position c ^ vswz(r).  The
//    P V operand is read with transposing 8-byte reads (ds_read_b64_tr_b16);
//    a half wave's read covers 4 consecutive keys x 64 bytes, and the
//    permutation puts those 4 rows on disjoint banks.
// Keys per tile: one K/V tile is the work of one tile step.  At d = 64 a
// step of 64 keys is only 16 MFMAs per wave and phase, so the fixed cost of
// a phase (barrier, first operand reads, the other group's vector work
// starting) weighs twice as much; 128-key tiles halve it and still fit the
// registers (at d = 128 they do not).
template <int D>
constexpr int kKeyTile = 64;
template <>
constexpr int kKeyTile<64> = 128;

template <int D>
struct Tile {
    static constexpr int BC = kKeyTile<D>;        // keys per tile
    static constexpr int KB = BC / 32;            // 32-key blocks per tile
    static constexpr int ROW_CHUNKS = D / 8;      // 16-byte chunks per row
    static constexpr int KBYTES = BC * D * 2;
    static constexpr int VBYTES = BC * D * 2;
    static constexpr int NBUF = 2;                // K and V rings: tile t in buffer t % 2
    static constexpr int VBASE = NBUF * KBYTES;
    static constexpr int ROLE = VBASE + NBUF * VBYTES;   // 16 ints for the wave roles
    static constexpr int LDS_BYTES = ROLE + 64;
    // Direct loads per tile: a K load fills 64 keys of one chunk column
    // (KH = BC / 64 loads per column), a V load 1 KiB of whole keys (V_ROWS
    // keys).  The K group's 4 waves share a K tile, the V group's 4 waves a V
    // tile.
    static constexpr int KH = BC / 64;
    static constexpr int KLOADS = ROW_CHUNKS * KH;
    static constexpr int K_DMA = KLOADS / 4;
    static constexpr int V_ROWS = 1024 / (2 * D);
    static constexpr int V_DMA = VBYTES / 1024 / 4;
    static_assert(BC % 64 == 0, "a direct K load covers 64 keys of one chunk column");
    static_assert(KLOADS % 4 == 0 && (VBYTES / 1024) % 4 == 0, "tiles must split evenly over a wave group");
    static_assert(KLOADS % kWaves == 0, "the first K tile splits evenly over all waves");
};

// Chunk permutation of V row r (in 16-byte chunks).  The transposing read of
// a half wave touches rows r0 .. r0+3 (r0 a multiple of 4) at the same 64
// bytes of the row; with 2D-byte rows these must land on 4 different 64-byte
// bank groups of the 256-byte bank space.
template <int D>
__device__ __forceinline__ int vswz(int r) {
    static_assert(D == 64 || D == 128, "head dimension");
    return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

// Buffer descriptor of a raw byte range: loads at or past `bytes` return
// zeros (the descriptor's range check), which is what the tile copies use
// for rows past the end of the sequence.  Words: base address (48 bits,
// stride 0), number of bytes, raw 32-bit data format.
constexpr uint32_t kBufferWord3 = 0x00020000u;
__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    u32x4 r;
    r[0] = (uint32_t)a;
    r[1] = (uint32_t)(a >> 32) & 0xFFFFu;
    r[2] = bytes;
    r[3] = kBufferWord3;
    return r;
}

// One direct global-to-LDS load: lane L's 16 bytes at (descriptor base +
// voff + soff) go to LDS address dst + 16 L.  Written as inline assembly
// on purpose: the compiler does not see it as a write to LDS, so it does not
// make the transposing LDS reads of other buffers wait for it (it cannot
// tell the ring buffers apart).  Completion is the caller's business: a
// vmcnt wait before the barrier that publishes the tile.  M0 holds the LDS
// address; nothing else in the kernel uses M0.
__device__ __forceinline__ void dma16(LDS char* dst, u32x4 rsrc, uint32_t voff, uint32_t soff) {
    const uint32_t m = (uint32_t)(uintptr_t)dst;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(m), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row sum of the rounded weights on the matrix cores.  The P operand pb[c]
// of a 16-key chunk (lane l: query l % 32, 8 of the chunk's keys) read as
// the B operand of a 16x16x32 product is B[k][n] with n = l % 16 and k in
// the 8-block l / 16.  The A operand `ones_pattern` has ones exactly where
// ((m >> 2) & 1) == (k-block & 1) (lane l holds row m = l % 16 of k-block
// l / 16), so output row m sums, for column n, the 16 keys of query n (m in
// 0..3, 8..11) or of query n + 16 (m in 4..7, 12..15).  The accumulator
// layout (lane l: rows 4 (l / 16) .. +3 of column l % 16) then gives every
// lane four copies of the chunk's sum for its own query l % 32.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 ones_pattern(int lane) {
    const bool one = (((lane & 15) >> 2) & 1) == ((lane >> 4) & 1);
    const uint32_t w = one ? 0x3F803F80u : 0u;    // two bf16 ones, or zeros
    return __builtin_bit_cast(bf16x8, (u32x4){w, w, w, w});
}

// Lane l and lane l^32 hold the same query: after the swap, out[0] and out[1]
// are x[l] and x[l^32] in some order, in every lane.
__device__ __forceinline__ float half_swap_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float half_swap_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// K/V copies.  Rows past the end of the sequence read as zeros (buffer
// range check): such keys are masked, and a zero V row is finite under a
// zero weight.  The loads complete asynchronously; the issuing wave waits
// for them (vmcnt) before the barrier that publishes the tile.  (idx, the
// wave's index in its group, is uniform over the wave; readfirstlane makes
// that visible, so the LDS address and the scalar offset need no per-lane
// handling.  The wave roles themselves stay per-lane values: as wave-uniform
// values they turn the role branches into scalar branches, and the register
// allocation of the two roles' code then spills.)

// Load n (0 <= n < KLOADS) of the K tile with first key key0 into `buf`:
// keys key0 + 64 j .. +63 (j = n % KH) of chunk column c = n / KH, lane L
// fetching key key0 + 64 j + L into slot c * BC + 64 j + L.
template <int D>
__device__ __forceinline__ void dma_k_load(u32x4 rk, LDS char* buf, int key0, int n, int lane) {
    using T = Tile<D>;
    const int c = n / T::KH, j = n % T::KH;
    dma16(buf + c * (T::BC * 16) + j * 1024, rk, lane * (2 * D), (key0 + 64 * j) * (2 * D) + 16 * c);
}
// K tile with first key key0 into `buf`: wave idx of the K group issues
// loads idx * K_DMA .. +K_DMA-1.
template <int D>
__device__ __forceinline__ void dma_k(u32x4 rk, LDS char* buf, int key0, int idx, int lane) {
    using T = Tile<D>;
    const int widx = __builtin_amdgcn_readfirstlane(idx);
#pragma unroll
    for (int i = 0; i < T::K_DMA; ++i) dma_k_load<D>(rk, buf, key0, widx * T::K_DMA + i, lane);
}

// V tile with first key key0 into `buf`: wave idx of the V group issues
// loads n = idx * V_DMA .. +V_DMA-1; load n fills bytes [1024 n, 1024 n +
// 1024) of the buffer, i.e. keys V_ROWS n + L / ROW_CHUNKS at chunk position
// L % ROW_CHUNKS for lane L, which fetches the chunk that the permutation
// puts there.  (V_ROWS n is a multiple of 4, so vswz sees only L's row.)
template <int D>
__device__ __forceinline__ void dma_v(u32x4 rv, LDS char* buf, int key0, int idx, int lane) {
    using T = Tile<D>;
    const int widx = __builtin_amdgcn_readfirstlane(idx);
    const int r = lane / T::ROW_CHUNKS;
    const int voff = r * (2 * D) + 16 * ((lane % T::ROW_CHUNKS) ^ vswz<D>(r));
#pragma unroll
    for (int i = 0; i < T::V_DMA; ++i) {
        const int n = widx * T::V_DMA + i;
        dma16(buf + 1024 * n, rv, voff, key0 * (2 * D) + 1024 * n);
    }
}

// The matrix phase of one tile step: S^T = K Q^T for the current tile
// (HAS_S) and O^T += V^T P^T for the previous one (HAS_PV), as one stream of LDS
// operand reads and MFMAs.  The reads run kAhead MFMAs ahead of their use
// (scheduling groups below), so the LDS latency stays hidden behind the
// matrix core instead of stalling every MFMA.
//
// The V^T operand of the P V product (32 d x 16 keys, keys in the order of
// P's registers: lane l holds d = 32 db + l % 32 and keys 16 cc + 4h + 0..3,
// then 16 cc + 8 + 4h + 0..3) comes from two transposing reads.  In a
// transposing read, lane i of each 16-lane group receives element i % 4 of
// the 4-element pieces addressed by lanes i / 4, i / 4 + 4, i / 4 + 8 and
// i / 4 + 12 of its group.  So lane j of group g addresses key
// 16 cc + 8q + 4h + j / 4 at d = 32 db + 16 (g % 2) + 4 (j % 4), and read q
// returns to each lane its 4 keys of run q for its d.
constexpr int kAhead = 4;

template <bool B>
struct MaskTag {
    static constexpr bool value = B;
};
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

template <int D, bool HAS_PV, bool HAS_S, bool LT>
__device__ __forceinline__ void gemm_phase(const LDS char* vl, const LDS char* kl,
                                           const bf16x8 (&pb)[Tile<D>::BC / 16],
                                           const bf16x8 (&qf)[D / 16], f32x16 (&oacc)[D / 32],
                                           f32x16 (&s)[Tile<D>::KB], f32x4& lt, bf16x8 ones, int lane) {
    using T = Tile<D>;
    constexpr int DB = D / 32;
    constexpr int NPV = HAS_PV ? (T::BC / 16) * DB : 0;
    constexpr int NS = HAS_S ? (D / 16) * T::KB : 0;
    constexpr int NF = NPV + NS;
    // LT: the row sum of the rounded weights of the previous tile, one small
    // product per 16-key chunk; they need no LDS operand, so they go first,
    // while the first operand reads are in flight.
    constexpr int NLT = (HAS_PV && LT) ? T::BC / 16 : 0;
    // Operands 0 .. NS-1 are those of S^T = K Q^T, then those of the P V
    // product: the S accumulators are complete first, so the wave's next
    // (vector) phase can start on them while the P V MFMAs drain.
    const int h = lane >> 5;
    const int l32 = lane & 31;
    const LDS char* krow = kl + (h * T::BC + l32) * 16;     // chunk h, key l32
    const int vr = 4 * h + ((lane & 15) >> 2);               // key of this lane's piece, within the run
    const int dlo = 16 * ((lane >> 4) & 1) + 4 * (lane & 3); // d of its piece, within the 32-d block
    bf16x8 fr[NF > 0 ? NF : 1];
#pragma unroll
    for (int i = 0; i < NF; ++i) {
        if (i >= NS) {
            const int j = i - NS;
            const int cc = j / DB, db = j % DB;
            const LDS char* vp = vl + (16 * cc + vr) * (2 * D) + 16 * ((4 * db + dlo / 8) ^ vswz<D>(vr)) +
                                 2 * (dlo % 8);
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)vp);
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)(vp + 8 * (2 * D)));
            fr[i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
            const int ks = i / T::KB, kb = i % T::KB;
            fr[i] = *(const LDS bf16x8*)(krow + (2 * ks * T::BC + 32 * kb) * 16);
        }
    }
    if constexpr (HAS_S) {
#pragma unroll
        for (int kb = 0; kb < T::KB; ++kb) s[kb] = (f32x16){};
    }
#pragma unroll
    for (int c = 0; c < NLT; ++c) lt = mfma16(ones, pb[c], lt);
#pragma unroll
    for (int i = 0; i < NF; ++i) {
        if (i >= NS) {
            const int j = i - NS;
            const int cc = j / DB, db = j % DB;
            oacc[db] = mfma32(fr[i], pb[cc], oacc[db]);
        } else {
            const int ks = i / T::KB, kb = i % T::KB;
            s[kb] = mfma32(fr[i], qf[ks], s[kb]);
        }
    }
    // A P V operand takes two reads, an S operand one.
    if constexpr (NF > kAhead) {
        constexpr int first_reads = NS >= kAhead ? kAhead : NS + 2 * (kAhead - NS);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, first_reads, 0);
        if constexpr (NLT > 0) __builtin_amdgcn_sched_group_barrier(kSchedMfma, NLT, 0);
#pragma unroll
        for (int i = 0; i < NF - kAhead; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            if (i + kAhead >= NS)
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
            else
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, kAhead, 0);
    }
}

// P = exp2(S*c - m) of one tile in bf16 for the P V product; returns this
// lane's share of the row sum (over the fp32 values).
template <int D>
__device__ __forceinline__ float exp_tile(const f32x16 (&s)[Tile<D>::KB], bf16x8 (&pb)[Tile<D>::BC / 16],
                                          float m_use, float c_log2) {
    // four partial sums, seeded with the first four weights (p >= 0, so this
    // equals summing from zero)
    float ps[4];
#pragma unroll
    for (int kb = 0; kb < Tile<D>::KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][i], c_log2, -m_use));
            if (kb == 0 && i < 4)
                ps[i] = p;
            else
                ps[i & 3] += p;
            pb[2 * kb + (i >> 3)][i & 7] = (__bf16)p;
        }
    return (ps[0] + ps[1]) + (ps[2] + ps[3]);
}

// Dropout on the bf16 weights of one tile (the row sum has already taken
// them whole): pb[s] holds this lane's keys key0 + 16s + 4h + {0..3, 8..11}
// of query row `row` in the order of the generator's 16-bit halves, so the
// call at counter (2 (key0/16 + s) + h, row, bh, offset) decides, word by
// word, the four packed pairs of pb[s].
template <int D>
__device__ __forceinline__ void apply_dropout(bf16x8 (&pb)[Tile<D>::BC / 16], int key0, int row, int bh,
                                              const Dropout& dr, int h) {
    // The first rounds depend only on the row, the head and the offset; the
    // empty asm hides that from the optimiser, which would otherwise keep
    // those partial states live across the whole key loop (and spill them).
    uint32_t row_u = (uint32_t)row;
    asm volatile("" : "+v"(row_u));
#pragma unroll
    for (int s = 0; s < Tile<D>::BC / 16; ++s) {
        const PhiloxOut r = philox4x32_10((uint32_t)(2 * ((key0 >> 4) + s) + h), row_u, (uint32_t)bh,
                                          dr.offset, dr.k0, dr.k1);
        u32x4 x = __builtin_bit_cast(u32x4, pb[s]);
#pragma unroll
        for (int m = 0; m < 4; ++m) x[m] = drop_pair(x[m], r.w[m], dr.t2);
        pb[s] = __builtin_bit_cast(bf16x8, x);
    }
}

// Online softmax of one tile of S^T: mask, P against the reference max m,
// row sum.  The reference max is lazy: after the first tile it only moves
// when some p of the wave would exceed kSumLimit (detected through the row
// sums, which also catch an overflow to inf); then the tile is redone
// against its exact row max, after rescaling O and l.  Any common
// reference gives the same O = sum p v / sum p and LSE = m + log2 l.
template <int D, bool CAUSAL, bool MASK>
__device__ __forceinline__ void softmax_tile(f32x16 (&s)[Tile<D>::KB], bf16x8 (&pb)[Tile<D>::BC / 16],
                                             f32x16 (&oacc)[D / 32], f32x4& lt, float& m_run, float& l_run,
                                             int key0, int N, int my_row, float c_log2, int lane,
                                             bool first) {
    using T = Tile<D>;
    constexpr int KB = T::KB;
    const int h = lane >> 5;

    if constexpr (MASK) {
        // Register i of block kb holds key key0 + 4h + off with
        // off = 32 kb + 8 (i / 4) + i % 4; the key is dead (past N, or after
        // the query when causal) iff off >= lim.  One limit per tile keeps
        // the offsets immediate.
        const int lim = (CAUSAL ? min(N, my_row + 1) : N) - key0 - 4 * h;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (32 * kb + 8 * (i >> 2) + (i & 3) >= lim) s[kb][i] = -__builtin_inff();
            }
        }
    }

    if (!first) {
        const float ps = exp_tile<D>(s, pb, m_run, c_log2);
        if (__builtin_amdgcn_ballot_w64(!(ps <= kSumLimit)) == 0) {
            l_run += ps;
            return;
        }
    }

    // exact row max: a tree over the lane's 32 values, then the other half's
    float mx[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) mx[t] = fmaxf(fmaxf(s[0][4 * t], s[0][4 * t + 1]), fmaxf(s[0][4 * t + 2], s[0][4 * t + 3]));
#pragma unroll
    for (int kb = 1; kb < KB; ++kb)
#pragma unroll
        for (int t = 0; t < 4; ++t)
            mx[t] = fmaxf(fmaxf(mx[t], s[kb][4 * t]), fmaxf(fmaxf(s[kb][4 * t + 1], s[kb][4 * t + 2]), s[kb][4 * t + 3]));
    const float tile_max = half_swap_max(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3])));

    const float m_new = fmaxf(m_run, tile_max * c_log2);
    const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);   // 1 where the max stayed
    l_run *= alpha;
    lt *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
    m_run = m_use;
    l_run += exp_tile<D>(s, pb, m_use, c_log2);
}

// c_log2 = |scale| * log2(e) (> 0); qsign flips the sign bit of every Q
// element when scale < 0 (exact), so that the kernel only sees c_log2 > 0.
//
// SPLIT: the launch covers n_splits disjoint ranges of the T key tiles:
// with kq = T / n_splits and kr = T % n_splits, split s = n_splits - 1 -
// blockIdx.y (the last range first, see the work decomposition) takes
// the tiles [s*kq + min(s, kr), (s+1)*kq + min(s+1, kr)) (kr ranges of kq+1
// tiles, then ranges of kq).  Without SPLIT, kq = T and kr = 0.  Each workgroup then writes the fp32 partial result
// of its range instead of O and LSE: the output normalised by its own row
// sum to OP[s][bh][row][d], and the logsumexp of its range to LP[s][bh][row]
// (O = 0 and LSE = -inf for a row of the tile that sees no key of the
// range).  A workgroup whose tile sees no key of its range writes nothing.
//
// DROP (never with SPLIT): dropout with the parameters `dr` on the weights
// that enter P V; the row sums, hence the logsumexp, take the weights whole,
// and the epilogue multiplies O by 1 / (1 - p).
template <int D, bool CAUSAL, bool SPLIT, bool DROP>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, float* __restrict__ LSE, int group, int N, int n_qtiles, int bh_total,
    float c_log2, uint32_t qsign, int kq, int kr, float* __restrict__ OP, float* __restrict__ LP,
    Dropout dr) {
    static_assert(!(SPLIT && DROP), "dropout runs on the direct path only");
    using T = Tile<D>;
    constexpr int BC = T::BC;
    constexpr int KB = T::KB;
    constexpr int DB = D / 32;
    constexpr int KSTEPS = D / 16;

    __shared__ __attribute__((aligned(16))) char smem_raw[T::LDS_BYTES];
    LDS char* smem = (LDS char*)smem_raw;
    LDS int* roles = (LDS int*)(smem + T::ROLE);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;
    const int l32 = lane & 31;

    // Work decomposition.  Workgroups are dealt round-robin to the 8 XCDs
    // (w % 8); give each XCD a contiguous range of heads so that the query
    // tiles sharing one K/V head (and a GQA group) share that XCD's L2 and
    // MALL slice.  Within an XCD the heads go four at a time, and the query
    // tiles of those four go out in rounds over them, latest (heaviest, when
    // causal) tiles first: four heads keep the K/V being read within the
    // XCD's L2 (half the L2 misses of rounds over all its heads, at the same
    // speed), and the short tiles of each group fill in behind the long ones.
    // Split ranges go out last range first: when causal, a late range holds
    // keys only for the late (long) query tiles, so the long pieces of work
    // start first and the short ones (early ranges of early tiles, and the
    // ranges a tile does not see at all, which return at once) fill in
    // behind them.  Consecutive workgroups read one key range.
    int bh, qt;
    const int split = SPLIT ? (int)(gridDim.y - 1 - blockIdx.y) : 0;
    {
        const int w = blockIdx.x;
        if ((bh_total & 31) == 0) {
            const int slot = w >> 3;
            const int r = slot % (4 * n_qtiles);
            bh = (w & 7) * (bh_total >> 3) + 4 * (slot / (4 * n_qtiles)) + (r & 3);
            qt = r >> 2;
        } else if ((bh_total & 7) == 0) {
            const int slot = w >> 3;
            bh = (w & 7) * (bh_total >> 3) + slot % (bh_total >> 3);
            qt = slot / (bh_total >> 3);
        } else {
            // (few heads) tile-major over all heads, so that when causal the
            // long tiles of every head go out before the short ones of any
            bh = w % bh_total;
            qt = w / bh_total;
        }
        if (CAUSAL) qt = n_qtiles - 1 - qt;
    }

    // The first K tile does not depend on the wave roles: all 8 waves start
    // loading it now, so that its latency overlaps the role set-up and the Q
    // loads.  (Not when the split range holds no visible tile: the
    // workgroup returns early and must leave no load in flight.)
    const size_t kv_head = (size_t)(bh / group) * N * D;
    const int kt_lo = split * kq + min(split, kr);
    const int kt_hi = kt_lo + kq + (split < kr ? 1 : 0);
    const int kv_end = CAUSAL ? min(N, qt * kBr + kBr) : N;  // keys this workgroup needs
    const int n_tiles = max(0, min(kt_hi, (kv_end + BC - 1) / BC) - kt_lo);
    const int Nl = N - kt_lo * BC;           // keys from the first tile of the range on
    const u32x4 rk = make_rsrc(K + kv_head + (size_t)kt_lo * BC * D, (uint32_t)Nl * (2 * D));
    const u32x4 rv = make_rsrc(V + kv_head + (size_t)kt_lo * BC * D, (uint32_t)Nl * (2 * D));
    if (n_tiles > 0) {
        const int w0 = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
        for (int i = 0; i < T::KLOADS / kWaves; ++i) dma_k_load<D>(rk, smem, 0, w0 * (T::KLOADS / kWaves) + i, lane);
    }

    // Wave roles.  Order the waves by (rank among the waves on the same SIMD,
    // SIMD id, wave id): the first four form the group that starts with a
    // matrix phase, the last four the group that starts one phase later, so
    // that each SIMD gets one wave of each group.  The order is a permutation
    // of the 8 waves whatever the placement, so the row blocks stay a
    // partition of the tile.
    int grp, idx;
    {
        const int simd = __builtin_amdgcn_s_getreg(kGetregSimdId) & 3;
        if (lane == 0) roles[wave] = simd;
        __syncthreads();
        int rank = 0;
        for (int v = 0; v < wave; ++v) rank += roles[v] == simd;
        const int key = (rank * 4 + simd) * kWaves + wave;
        __syncthreads();
        if (lane == 0) roles[8 + wave] = key;
        __syncthreads();
        int pos = 0;
        for (int v = 0; v < kWaves; ++v) pos += roles[8 + v] < key;
        grp = pos >> 2;
        idx = pos & 3;
    }
    // Row blocks: the first group takes blocks 0..3 and the second 7..4, so
    // SIMD k holds blocks k and 7 - k.  On the diagonal of a causal tile the
    // blocks need 1, 1, 2, 2, 3, 3, 4, 4 of its four key tiles; paired this
    // way, each SIMD has one working wave in the last two diagonal steps
    // (instead of one SIMD with two and two SIMDs with none), and a wave
    // alone on its SIMD runs its phase faster.
    const int rblock = grp == 0 ? idx : kWaves - 1 - idx;

    const size_t q_head = (size_t)bh * N * D;
    const int q0 = qt * kBr;
    const int wq0 = q0 + rblock * kWaveRows;  // first query row of this wave
    const int my_row = wq0 + l32;             // the query row this lane owns

    // Q fragments: B operand of S^T = K Q^T, lane holds d = 16*ks + 8*h .. +7.
    bf16x8 qf[KSTEPS];
    {
        const u32x4* qp = (const u32x4*)(Q + q_head + (size_t)min(my_row, N - 1) * D);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            u32x4 x = qp[2 * ks + h];
            if (my_row >= N) x = (u32x4){0u, 0u, 0u, 0u};
            x ^= qsign;
            qf[ks] = __builtin_bit_cast(bf16x8, x);
        }
    }

    // Key tiles: local tile t is global tile kt_lo + t (kt_lo = 0 unless SPLIT).
    const int w_kv_end = CAUSAL ? min(N, wq0 + kWaveRows) : N;
    const int w_tiles = (wq0 < N) ? max(0, min(kt_hi, (w_kv_end + BC - 1) / BC) - kt_lo) : 0;

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = (f32x16){};
    float m_run = -__builtin_inff();   // reference max of S*c (log2 domain)
    // Row sum of the bf16-rounded weights that enter P V (the same value in
    // all four registers): O is divided by it, so that O is exactly the
    // weighted mean the matrix cores formed, while l_run (fp32 weights)
    // gives the logsumexp.  With dropout the matrix phase sees the thinned
    // weights, so that path keeps l_run for both.
    f32x4 lt = (f32x4){};
    const bf16x8 ones = ones_pattern(lane);
    float l_run = 0.f;                 // this lane's share of the running sum
    f32x16 s[KB];
    bf16x8 pb[BC / 16];

    // K/V copies: direct loads, each wave of a group loading its share; tile
    // t of K and of V lives in ring buffer t & 1.  Each load is issued right
    // after a barrier that retired the previous readers of its buffer, and
    // has two phases to land before the barrier that publishes it.
    //   K (second group; K_0 by all waves before the loop).  At the start of its vector
    //   phase 2u the group issues K_{u+1}, over K_{u-1} (read in phases 2u-2
    //   and 2u-1), and waits for it at the end of its matrix phase 2u+1; it
    //   is first read in phase 2u+2.
    //   V (first group): at the start of its matrix phase 2u the group issues
    //   V_u, over V_{u-2} (read in phases 2u-2 and 2u-1), while that phase
    //   reads V_{u-1} from the other buffer, and waits for it at the end of
    //   its vector phase 2u+1; it is first read in phase 2u+2.
    // No key of the range is visible to the tile: nothing to write (the
    // merge takes split s for row r only when the range has keys and, when
    // causal, its first key is at most r, so it never reads this tile's
    // partials).
    if (SPLIT && n_tiles == 0) return;
    __builtin_amdgcn_s_waitcnt(kWaitVm0);      // this wave's share of K_0 (and its Q rows)
    __syncthreads();

    // Phases p = 0 .. 2*n_tiles+1, each closed by a workgroup barrier.  The
    // group's local phase lp = p - grp: even lp = 2t is the matrix phase t
    // (S_t, then P_{t-1} V_{t-1}; K_t and V_{t-1} are read), odd lp = 2t+1
    // the softmax of S_t.
    auto matrix_phase = [&](int t) __attribute__((always_inline)) {
        const bool has_pv = t >= 1 && t - 1 < w_tiles;
        const bool has_s = t < w_tiles;
        const LDS char* vl = smem + T::VBASE + ((t - 1) & 1) * T::VBYTES;
        const LDS char* kl = smem + (t & 1) * T::KBYTES;
        // The wave on the same SIMD runs vector work meanwhile; a higher
        // issue priority keeps the MFMAs from waiting behind it.
        __builtin_amdgcn_s_setprio(kMatrixPrio);
        if (has_pv && has_s)
            gemm_phase<D, true, true, !DROP>(vl, kl, pb, qf, oacc, s, lt, ones, lane);
        else if (has_pv)
            gemm_phase<D, true, false, !DROP>(vl, kl, pb, qf, oacc, s, lt, ones, lane);
        else if (has_s)
            gemm_phase<D, false, true, !DROP>(vl, kl, pb, qf, oacc, s, lt, ones, lane);
        __builtin_amdgcn_s_setprio(0);
    };
    // MASKED: the tile may hold dead keys (past N, or after some query of
    // the workgroup when causal); the masked softmax is exact on any tile.
    auto softmax_phase = [&](auto masked, int t) __attribute__((always_inline)) {
        if (t >= 0 && t < w_tiles) {
            const int key0 = (kt_lo + t) * BC;
            softmax_tile<D, CAUSAL, decltype(masked)::value>(s, pb, oacc, lt, m_run, l_run, key0, N, my_row,
                                                             c_log2, lane, t == 0);
            // Dropout thins the weights that enter P V; the row sum above
            // took them whole.
            if constexpr (DROP) apply_dropout<D>(pb, key0, my_row, bh, dr, h);
        }
    };
    // Phases 2u and 2u+1.
    auto tile_pair = [&](auto masked, int u) __attribute__((always_inline)) {
        if (grp == 0) {
            if (u < n_tiles) dma_v<D>(rv, smem + T::VBASE + (u & 1) * T::VBYTES, u * BC, idx, lane);
            matrix_phase(u);
        } else {            // vector phase of tile u-1 of the second group
            if (u + 1 < n_tiles) dma_k<D>(rk, smem + ((u + 1) & 1) * T::KBYTES, (u + 1) * BC, idx, lane);
            softmax_phase(masked, u - 1);
        }
        lds_barrier();
        if (grp == 0) {     // vector phase of tile u of the first group
            softmax_phase(masked, u);
            __builtin_amdgcn_s_waitcnt(kWaitVm0);    // V_u has landed
        } else {
            matrix_phase(u);
            __builtin_amdgcn_s_waitcnt(kWaitVm0);    // K_{u+1} has landed
        }
        lds_barrier();
    };
    // Local tile t holds keys from (kt_lo + t) BC on.  No key of a tile
    // before t_mask is dead for any row of the workgroup: the tail starts at
    // tile N / BC, and when causal the first row q0 sees every key of tiles
    // below q0 / BC (q0 is a multiple of BC).  The pair loop switches to the
    // masked softmax at the first pair that can run such a tile.
    int t_mask = N / BC - kt_lo;
    if (CAUSAL) t_mask = min(t_mask, q0 / BC - kt_lo);
    t_mask = max(0, min(t_mask, n_tiles + 1));
    int u = 0;
#pragma unroll 1
    for (; u < t_mask; ++u) tile_pair(MaskTag<false>{}, u);
#pragma unroll 1
    for (; u <= n_tiles; ++u) tile_pair(MaskTag<true>{}, u);

    if (wq0 >= N) return;
    const float l_tot = half_swap_sum(l_run);
    if constexpr (SPLIT) {
        if (my_row >= N) return;
        const bool seen = l_tot > 0.f;       // the row saw some key of the range
        // (a row that sees a key has its largest weight at 1 in the tile that
        // set its reference, so the rounded sum is at least 1)
        const float inv = seen ? 1.f / lt[0] : 0.f;
        const size_t prow = ((size_t)split * bh_total + bh) * N + my_row;
        float* opp = OP + prow * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *(float4*)(opp + 32 * db + 8 * g + 4 * h) =
                    make_float4(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv,
                                oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
        if (h == 0)
            LP[prow] = seen ? (m_run + __builtin_log2f(l_tot)) * 0.69314718055994531f : -__builtin_inff();
        return;
    }
    // O through LDS.  In registers a lane holds 4-element runs of its row,
    // so direct stores would write 16-byte pieces of 32 rows per instruction.
    // The wave writes its 32 x D tile (bf16) into its own slice of the idle
    // K/V rings, with the 16-byte chunk c of row r at position c ^ (r mod RC),
    // then reads back whole rows and stores 1 KiB of consecutive rows per
    // instruction.  (Every LDS read of the rings ended at the loop's last
    // barrier, and no copy is in flight.)
    constexpr int RC = D / 8;                        // 16-byte chunks per row
    constexpr int RPI = 1024 / (2 * D);              // rows per store instruction
    static_assert(kWaves * kWaveRows * 2 * D <= T::VBASE + T::NBUF * T::VBYTES, "O staging fits the rings");
    const float inv = DROP ? dr.factor / l_tot : 1.f / lt[0];
    LDS char* ot = smem + wave * (kWaveRows * 2 * D);
    // (the per-lane swizzle keys are hidden from the optimiser, which would
    // otherwise precompute all 24 addresses and keep them live from the start)
    int wsw = l32 % RC, rsw = (lane / RC) % RC;
    asm volatile("" : "+v"(wsw), "+v"(rsw));
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            bf16x4 out;
#pragma unroll
            for (int r = 0; r < 4; ++r) out[r] = (__bf16)(oacc[db][4 * g + r] * inv);
            *(LDS bf16x4*)(ot + l32 * (2 * D) + 16 * ((4 * db + g) ^ wsw) + 8 * h) = out;
        }
    }
    __bf16* otile = O + q_head + (size_t)wq0 * D;
#pragma unroll
    for (int i = 0; i < kWaveRows / RPI; ++i) {
        // row r = i RPI + lane / RC, and r mod RC = (i RPI + rsw) mod RC
        const int r = i * RPI + lane / RC, c = lane % RC;
        const u32x4 x = *(const LDS u32x4*)(ot + r * (2 * D) + 16 * (c ^ ((i * RPI + rsw) % RC)));
        if (wq0 + r < N) *(u32x4*)(otile + (size_t)r * D + 8 * c) = x;
    }
    if (h == 0 && my_row < N) LSE[(size_t)bh * N + my_row] = (m_run + __builtin_log2f(l_tot)) * 0.69314718055994531f;
}

template <int D, bool CAUSAL, bool SPLIT, bool DROP = false>
hipError_t launch(const FwdArgs& a, int n_splits, float* op, float* lp, hipStream_t stream,
                  Dropout dr = Dropout{}) {
    const int n_qtiles = (a.N + kBr - 1) / kBr;
    const int n_kt = (a.N + Tile<D>::BC - 1) / Tile<D>::BC;
    int kq = n_kt / n_splits, kr = n_kt % n_splits;
    const int bh_total = a.B * a.Hq;
    float c_log2 = fabsf(a.scale) * 1.4426950408889634f;
    // A zero scale makes every weight equal; a tiny positive factor gives the
    // same result to far below fp32 resolution and keeps the masked -inf
    // logits at -inf after scaling (0 * -inf would be NaN).
    if (!(c_log2 >= 1e-30f)) c_log2 = 1e-30f;
    uint32_t qsign = a.scale < 0.f ? 0x80008000u : 0u;
    int group = a.Hq / a.Hkv;
    int N = a.N;
    const __bf16* q = (const __bf16*)a.q;
    const __bf16* k = (const __bf16*)a.k;
    const __bf16* v = (const __bf16*)a.v;
    __bf16* o = (__bf16*)a.o;
    float* lse = a.lse;
    void* args[] = {&q, &k, &v, &o, &lse, &group, &N, (void*)&n_qtiles, (void*)&bh_total,
                    &c_log2, &qsign, &kq, &kr, &op, &lp, &dr};
    return hipLaunchKernel((const void*)fwd_bf16_kernel<D, CAUSAL, SPLIT, DROP>,
                           dim3(bh_total * n_qtiles, SPLIT ? n_splits : 1), dim3(kThreads), args, 0,
                           stream);
}

// Merge of the split partials: the reading-notes page's rescaling rule
// (Methods, the two rescaling equations) applied to whole ranges.  With
// LSE = ln sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.  One thread per
// (row, 4 consecutive d); kMergeRows rows per 256-thread block.
constexpr int kMergeThreads = 256;

// Number of key ranges that hold a key row r sees: the ranges with keys
// (kq + 1 tiles for s < kr, kq after), and, when causal, only those whose
// first key is at most r.  Range s starts at tile s (kq + 1) for s <= kr
// and at s kq + kr after, so with t = r / bc those are the s with start <= t.
// These are exactly the ranges whose partials the split kernel wrote for
// the row; the merge reads no other.
__device__ __forceinline__ int ranges_seen(int r, int n_splits, int kq, int kr, int bc, bool causal) {
    const int with_keys = kq > 0 ? n_splits : kr;
    if (!causal) return with_keys;
    const int t = r / bc;
    const int a = kr * (kq + 1);              // first tile of range kr
    const int c = t < a ? t / (kq + 1) + 1 : (kq > 0 ? (t - kr) / kq + 1 : kr);
    return min(c, with_keys);
}

template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_splits_kernel(
    const float* __restrict__ OP, const float* __restrict__ LP, __bf16* __restrict__ O,
    float* __restrict__ LSE, int n_splits, long long rows, int N, int kq, int kr, int causal) {
    constexpr int TPR = D / 4;                        // threads per row
    const long long row = (long long)blockIdx.x * (kMergeThreads / TPR) + threadIdx.x / TPR;
    if (row >= rows) return;
    const int c4 = threadIdx.x % TPR;
    const int ns = ranges_seen((int)(row % N), n_splits, kq, kr, Tile<D>::BC, causal != 0);
    float mx = -__builtin_inff();
    for (int sp = 0; sp < ns; ++sp) mx = fmaxf(mx, LP[sp * rows + row]);
    float wsum = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int sp = 0; sp < ns; ++sp) {
        const float l = LP[sp * rows + row];
        const float w = l == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f((l - mx) * 1.4426950408889634f);
        const float4 x = *(const float4*)(OP + (sp * rows + row) * D + 4 * c4);
        wsum += w;
        acc.x += w * x.x;
        acc.y += w * x.y;
        acc.z += w * x.z;
        acc.w += w * x.w;
    }
    const float inv = 1.f / wsum;
    bf16x4 out;
    out[0] = (__bf16)(acc.x * inv);
    out[1] = (__bf16)(acc.y * inv);
    out[2] = (__bf16)(acc.z * inv);
    out[3] = (__bf16)(acc.w * inv);
    *(bf16x4*)(O + row * D + 4 * c4) = out;
    if (c4 == 0) LSE[row] = mx + __builtin_logf(wsum);
}

template <int D>
hipError_t launch_merge(const FwdArgs& a, int n_splits, const float* op, const float* lp,
                        hipStream_t stream) {
    long long rows = (long long)a.B * a.Hq * a.N;
    const long long per_block = kMergeThreads / (D / 4);
    const int n_kt = (a.N + Tile<D>::BC - 1) / Tile<D>::BC;
    int kq = n_kt / n_splits, kr = n_kt % n_splits;
    int N = a.N, causal = a.causal;
    __bf16* o = (__bf16*)a.o;
    float* lse = a.lse;
    void* args[] = {(void*)&op, (void*)&lp, &o, &lse, &n_splits, &rows, &N, &kq, &kr, &causal};
    return hipLaunchKernel((const void*)merge_splits_kernel<D>, dim3((unsigned)((rows + per_block - 1) / per_block)),
                           dim3(kMergeThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
    if (a.d == 128)
        return a.causal ? launch<128, true, false>(a, 1, nullptr, nullptr, stream)
                        : launch<128, false, false>(a, 1, nullptr, nullptr, stream);
    return a.causal ? launch<64, true, false>(a, 1, nullptr, nullptr, stream)
                    : launch<64, false, false>(a, 1, nullptr, nullptr, stream);
}

hipError_t launch_fwd_bf16_dropout(const FwdArgs& a, const Dropout& dr, hipStream_t stream) {
    if (a.d == 128)
        return a.causal ? launch<128, true, false, true>(a, 1, nullptr, nullptr, stream, dr)
                        : launch<128, false, false, true>(a, 1, nullptr, nullptr, stream, dr);
    return a.causal ? launch<64, true, false, true>(a, 1, nullptr, nullptr, stream, dr)
                    : launch<64, false, false, true>(a, 1, nullptr, nullptr, stream, dr);
}

hipError_t launch_fwd_bf16_split(const FwdArgs& a, int n_splits, float* workspace, hipStream_t stream) {
    float* op = workspace;
    float* lp = workspace + (size_t)n_splits * a.B * a.Hq * a.N * a.d;
    hipError_t e;
    if (a.d == 128)
        e = a.causal ? launch<128, true, true>(a, n_splits, op, lp, stream)
                     : launch<128, false, true>(a, n_splits, op, lp, stream);
    else
        e = a.causal ? launch<64, true, true>(a, n_splits, op, lp, stream)
                     : launch<64, false, true>(a, n_splits, op, lp, stream);
    if (e != hipSuccess) return e;
    return a.d == 128 ? launch_merge<128>(a, n_splits, op, lp, stream)
                      : launch_merge<64>(a, n_splits, op, lp, stream);
}

}  // namespace fa
