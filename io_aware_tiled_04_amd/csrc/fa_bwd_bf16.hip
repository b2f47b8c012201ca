// Attention backward pass, bf16 inputs, for gfx950 (MI355X).
//
// The derivation blog (page "Flash Attention介绍", section Flash Attention
// 反向传播, 梯度推导) recomputes P block by block from the row statistics the
// forward stored, instead of keeping P: for a query block t and a key block
// tau,
//
//   P   = exp(scale * Q_t K_tau^T - LSE_t)            (LSE = m + ln l, stored)
//   dV_tau += P^T dO_t
//   dP  = dO_t V_tau^T,   dS = P (.) (dP - D_t),      D_i = sum_d dO_id O_id
//   dQ_t   += scale * dS K_tau
//   dK_tau += scale * dS^T Q_t
//
// (the section's dV, dP, dQ and dK equations, with the softmax scale of the
// forward; D is the diag(dO O^T) term of the blog's standard backward).
//
// Kernels.
//   dQ:  resident query rows, streamed key tiles: S^T = K Q^T and
//        dP^T = V dO^T put one query per lane (LSE and D per lane), and
//        dQ^T += K^T dS^T takes K^T from LDS in the key order of dS^T's
//        registers (the forward's V^T trick).  4 waves of 32 rows.  It
//        also forms D_i = sum_d dO_id O_id of its rows (it holds their dO)
//        and leaves D in the workspace for the dK/dV kernel, which runs
//        after it.
//   dK, dV: one launch (bwd_dkv_kernel below): resident key rows, streamed
//        query tiles, 8 waves in pairs: one wave of a pair forms S, P and
//        then dS and dK, the other dP and then dV, exchanging P and dP
//        through LDS.
// The accumulator of one 32-row block at d = 128 takes 64 VGPRs, so no wave
// holds two of them.  S and dP are computed twice in all (once for dQ, once
// for dK and dV): 7 products for the 5 of the definition.
// Streamed tiles are 32 rows, double-buffered in LDS and copied straight
// from global memory into LDS one step ahead (direct loads, no registers);
// a dQ step takes one tile, a dK/dV step kSub<D> of them (two at d = 128,
// three at d = 64).
//
// Dropout (DROP): the forward's output was O = (P (.) Z) V / (1 - p), so with
// f = 1 / (1 - p),  dV = (P (.) Z)^T dO f,  dP = (dO V^T) (.) Z f, and
// dS = P (.) (dP - D) as before (D = rowsum(dO (.) O) with the dropped O
// still equals sum_j P dP).  The keep bits Z are the forward's (philox.h).
// The dQ kernel holds one query per lane and keys in its registers, the
// forward's layout: two generator calls per step give its 16 decisions.  In
// the dK/dV kernel a lane holds one key: each lane makes the two calls of one
// streamed query and one half of the wave's keys, and sixteen wave ballots
// carry the bits to the lanes of their keys.
#include "fa_kernels.h"

#include <stdint.h>

#include "philox.h"

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LDS __attribute__((address_space(3)))

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRows = 32 * kWaves;      // resident rows per workgroup
static_assert(kRows == kBwdBlockRows, "grid and kernel disagree on the resident tile");
constexpr int kTile = 32;               // streamed rows per step
constexpr float kLog2e = 1.4426950408889634f;
// s_waitcnt immediate that waits for all vector memory operations only
// (vmcnt [3:0] and [15:14] zero, expcnt and lgkmcnt at their maximum)
constexpr int kWaitVm0 = 0x0F70;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Instruction order for a run of N MFMAs whose A operands are N * R LDS
// reads written before them: the reads go kAhead MFMAs ahead of their use, so that
// an MFMA does not wait for a read issued just before it.  (Groups for the
// scheduler: mask 0x100 = LDS reads, 0x008 = MFMAs.)
constexpr int kAhead = 4;
template <int N, int R = 1>
__device__ __forceinline__ void reads_ahead() {
    if constexpr (N > kAhead) {
        __builtin_amdgcn_sched_group_barrier(0x100, R * kAhead, 0);
#pragma unroll
        for (int i = 0; i < N - kAhead; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
    }
}

// Keep decision of the draw in 16-bit half `hi` of a generator word.
__device__ __forceinline__ bool keep_half(uint32_t word, int hi, uint32_t t) {
    return (hi ? word >> 16 : word & 0xFFFFu) >= t;
}

// LDS image of one streamed tile: kTile rows of D bf16, row-major and
// unpadded, with the 16-byte chunk c of row r at chunk position c ^ rswz(r).
// Both ways the kernels read a tile are then free of bank conflicts (64 banks
// of 4 bytes):
//   - 16-byte reads of one chunk on 16 consecutive rows (an MFMA operand with
//     one tile row per lane): rswz is one-to-one on r mod 16;
//   - transposing 8-byte reads, 16 lanes over 4 consecutive rows and 32
//     consecutive bytes of each (an MFMA operand with one column per lane):
//     rows r mod 4 = 0..3 land in four different 64-byte quarters.
// rswz depends on r mod 16 only.
template <int D>
__device__ __forceinline__ int rswz(int r) {
    static_assert(D == 64 || D == 128, "head dimensions 64 and 128");
    return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

// LDS layout of one buffer set (dQ kernel).
template <int D>
struct Lay {
    static constexpr int RBYTES = kTile * 2 * D;
    static constexpr int A = 0;                          // K rows
    static constexpr int B = RBYTES;                     // V rows
    static constexpr int SET = 2 * RBYTES;
    static constexpr int BYTES = 2 * SET;
};
// Per-lane offsets for the two operand forms of a tile.  Row operand (lane =
// tile row l32, d = 16 ks + 8 h .. + 7): offset rowop ^ (32 ks).  Transposed
// operand of chunk cc (lane = d 32 db + l32, tile rows {16 cc + 4 h + 0..3,
// 16 cc + 8 + 4 h + 0..3}, the key order of an accumulator's registers
// 8 cc .. 8 cc + 7): two transposing reads at 32 D cc + (trop[k] ^ (64 db)),
// k = 0, 1.  (The XORs act on the chunk bits alone: row offsets are multiples
// of 2D and element offsets stay below 16 bytes.)
template <int D>
__device__ __forceinline__ int rowop_off(int lane) {
    const int l32 = lane & 31, h = lane >> 5;
    return l32 * 2 * D + 16 * (h ^ rswz<D>(l32));
}
template <int D>
__device__ __forceinline__ int trop_off(int lane, int k) {
    const int vr = 4 * (lane >> 5) + ((lane & 15) >> 2) + 8 * k;     // tile row of this lane's piece
    const int dlo = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);          // its d within the 32-d block
    return vr * 2 * D + 16 * ((dlo >> 3) ^ rswz<D>(vr)) + 2 * (dlo & 7);
}
typedef short i16x4 __attribute__((ext_vector_type(4)));
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const LDS char* tile, int t0, int t1, int db, int cc) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)(tile + 32 * D * cc + (t0 ^ (64 * db))));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)(tile + 32 * D * cc + (t1 ^ (64 * db))));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Direct global-to-LDS copies of a streamed tile (buffer loads with the LDS
// flag): no registers and no LDS store instructions.  The descriptor covers
// one head's rows, so rows past N come back as zeros (its range check).
// Words: base address (48 bits, stride 0), number of bytes, raw 32-bit data
// format.  The arguments must be uniform over the wave; readfirstlane puts
// the words in scalar registers, where the copy instruction takes them,
// also where the compiler cannot prove the uniformity itself.
__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    u32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xFFFFu);
    r[2] = __builtin_amdgcn_readfirstlane(bytes);
    r[3] = 0x00020000u;
    return r;
}
// Lane L's 16 bytes at (descriptor base + voff + soff) go to LDS address dst
// + 16 L (M0 holds dst; nothing else in these kernels uses M0).  Inline
// assembly, so the compiler does not take it for an LDS write that other
// LDS reads must wait for; completion is the caller's vmcnt wait before the
// barrier that publishes the tile.
__device__ __forceinline__ void dma16(LDS char* dst, u32x4 rsrc, uint32_t voff, uint32_t soff) {
    const uint32_t m = (uint32_t)(uintptr_t)dst;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(m), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}
// One streamed tile (kTile rows from row0, uniform like dst and w) into
// `dst` in the layout above, copied by the wave of index w of NW: copy n fills bytes [1024 n, 1024 n +
// 1024), i.e. rows R n + L / (D/8) (R = 1024 / 2D rows per copy) at chunk
// position L % (D/8) for lane L, which fetches the chunk that rswz puts
// there.
template <int D>
constexpr int kTileCopies = kTile * 2 * D / 1024;
template <int D, int NW>
__device__ __forceinline__ void dma_tile(LDS char* dst, u32x4 rsrc, int row0, int w, int lane) {
    constexpr int RC = D / 8;                 // chunks per row
    constexpr int R = 1024 / (2 * D);         // rows per copy
    constexpr int PER = kTileCopies<D> / NW;
    static_assert(kTileCopies<D> % NW == 0, "copies split evenly over the waves");
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int n = w * PER + i;
        const int r = R * n + lane / RC;
        const uint32_t voff = (uint32_t)(r * 2 * D + 16 * ((lane % RC) ^ rswz<D>(r)));
        dma16(dst + 1024 * n, rsrc, voff, __builtin_amdgcn_readfirstlane((uint32_t)(row0 * 2 * D)));
    }
}

// Row statistics of the streamed query rows (dK/dV kernel): LSE * log2(e)
// and D.  Staged raw in registers, one step ahead like the tiles, and
// finished when stored: any arithmetic on the loaded values at load time
// would make the wave wait right there for every load it has in flight.
// Rows past N get +inf (so that p = 0) and D = 0.
__device__ __forceinline__ void stage_stats(const float* __restrict__ lse, const float* __restrict__ dd,
                                            int row0, int n, int tid, float& s0, float& s1, int& srow) {
    srow = row0 + (tid & 31);
    const int rc = min(srow, n - 1);
    s0 = lse[rc];
    s1 = dd[rc];
}
__device__ __forceinline__ void finish_stats(float s0, float s1, int srow, int n, float& lse2, float& dv) {
    const bool in = srow < n;
    lse2 = in ? s0 * kLog2e : __builtin_inff();
    dv = in ? s1 : 0.f;
}

// dQ: resident query rows of head hq, streamed key tiles of K/V head
// hq / group.  c = scale * log2(e) (signed).  LSE and D are [B, Hq, N] float32;
// the kernel writes D of its rows (from dO and the forward's output O).
// DROP: the forward ran with dropout `dr` (see the file header).
template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const __bf16* __restrict__ O, const float* __restrict__ LSE,
    float* __restrict__ Dd, __bf16* __restrict__ G, int Hq, int Hkv, int N, int n_rtiles, int bh_total,
    float c, float scale, Dropout dr) {
    using L = Lay<D>;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;

    __shared__ __attribute__((aligned(16))) char smem_raw[L::BYTES];
    LDS char* smem = (LDS char*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5;
    const int l32 = lane & 31;
    const int group = Hq / Hkv;

    // Work decomposition, XCD-aware as in the forward; for causal attention the
    // heaviest (last) query tiles go first.
    int bh, rt;
    {
        const int w = blockIdx.x;
        if ((bh_total & 7) == 0) {
            const int slot = w >> 3;
            bh = (w & 7) * (bh_total >> 3) + slot % (bh_total >> 3);
            rt = slot / (bh_total >> 3);
        } else {
            // (few heads) tile-major over all heads: the long causal tiles
            // of every head go out before the short ones of any
            bh = w % bh_total;
            rt = w / bh_total;
        }
        if (CAUSAL) rt = n_rtiles - 1 - rt;
    }
    const int b = bh / Hq;
    const int hr = bh % Hq;                              // query head
    const int r0 = rt * kRows;                           // first resident row of the workgroup
    const int wr0 = r0 + 32 * wave;                      // first resident row of this wave
    const int my_row = wr0 + l32;                        // the resident query of this lane

    // Resident Q and dO (B operands of S^T = K Q^T and dP^T = V dO^T): lane
    // holds d = 16*ks + 8*h .. +7 of its row.
    const size_t rhead = ((size_t)b * Hq + hr) * N * D;
    bf16x8 rf1[KS], rf2[KS];
    u32x4 orow[KS];                                      // the same d of the row of O
    {
        const int rr = min(my_row, N - 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 x = *(const u32x4*)(Q + rhead + (size_t)rr * D + 16 * ks + 8 * h);
            u32x4 y = *(const u32x4*)(dO + rhead + (size_t)rr * D + 16 * ks + 8 * h);
            orow[ks] = *(const u32x4*)(O + rhead + (size_t)rr * D + 16 * ks + 8 * h);
            if (my_row >= N) x = y = (u32x4){0u, 0u, 0u, 0u};
            rf1[ks] = __builtin_bit_cast(bf16x8, x);
            rf2[ks] = __builtin_bit_cast(bf16x8, y);
        }
    }
    const size_t srow = ((size_t)b * Hq + hr) * N + min(my_row, N - 1);
    float lse2_lane = LSE[srow] * kLog2e;
    float d_lane;

    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = (f32x16){};

    // Streamed key tiles 0 .. (last visible key)/32 of the K/V head.
    const int n_steps = ((CAUSAL ? min(N, r0 + kRows) : N) + kTile - 1) / kTile;
    const size_t kvhead = ((size_t)b * Hkv + hr / group) * N * D;

    // Each step's copy, straight into LDS: A = K rows, B = V rows (K^T is
    // read from A with transposing reads).
    const int rowop = rowop_off<D>(lane);
    const int trop0 = trop_off<D>(lane, 0), trop1 = trop_off<D>(lane, 1);
    const u32x4 rk = make_rsrc(K + kvhead, (uint32_t)N * (2 * D));
    const u32x4 rv = make_rsrc(V + kvhead, (uint32_t)N * (2 * D));
    auto copy_step = [&](int step, int set) __attribute__((always_inline)) {
        LDS char* base = smem + set * L::SET;
        dma_tile<D, kWaves>(base + L::A, rk, step * kTile, wave, lane);
        dma_tile<D, kWaves>(base + L::B, rv, step * kTile, wave, lane);
    };

    // n_steps >= 1: the workgroup's first row is below N, so key tile 0 is
    // always visible.
    copy_step(0, 0);
    // D of this lane's row: its 64 d (those of its dO fragments, zero past
    // N), then the other half from lane l ^ 32.  The loads of O arrived with
    // (before) the first tile's.
    {
        float part = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 ov = __builtin_bit_cast(bf16x8, orow[ks]);
#pragma unroll
            for (int e = 0; e < 8; ++e) part = fmaf((float)rf2[ks][e], (float)ov[e], part);
        }
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
        d_lane = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        if (h == 0 && my_row < N) Dd[srow] = d_lane;
    }
    // The row statistics arrived with (before) the first tile.  Redefining
    // them here tells the compiler so; otherwise it cannot prove it on every
    // path into the loop and waits for all loads in flight at their first
    // use in every step.
    asm volatile("" : "+v"(lse2_lane), "+v"(d_lane));
    __builtin_amdgcn_s_waitcnt(0);       // tile 0 (and every earlier load) has landed
    if (n_steps > 1) copy_step(1, 1);
    __syncthreads();

#pragma unroll 1
    for (int step = 0; step < n_steps; ++step) {
        const int set = step & 1;
        const LDS char* base = smem + set * L::SET;
        const int row0 = step * kTile;                          // first key of the tile
        // Does this wave see any pair of the tile?  (keys row0.. vs queries wr0..wr0+31)
        bool active = wr0 < N;
        bool masked = row0 + kTile > N;
        if (CAUSAL) {
            active = active && row0 <= wr0 + 31;
            masked = masked || row0 + kTile - 1 > wr0;
        }
        if (active) {
            // Dropout keep bits: lane = query my_row, register i = key row0 +
            // 16(i/8) + 8((i/4)%2) + 4h + i%4; call i/8 at counter
            // 2(row0/16 + i/8) + h holds register i's draw in half i%8.
            uint32_t kw[2][4];
            if constexpr (DROP) {
                // The empty asm hides which counter and key words stay fixed
                // over the steps; otherwise the optimiser keeps partial rounds
                // and the ten round keys live across the loop.
                uint32_t k0 = dr.k0, k1 = dr.k1;
                asm volatile("" : "+s"(k0), "+s"(k1));
                uint32_t row_u = (uint32_t)my_row;
                asm volatile("" : "+v"(row_u));
#pragma unroll
                for (int a2 = 0; a2 < 2; ++a2) {
                    const PhiloxOut r = philox4x32_10((uint32_t)(2 * ((row0 >> 4) + a2) + h), row_u, (uint32_t)bh,
                                                      dr.offset, k0, k1);
#pragma unroll
                    for (int m = 0; m < 4; ++m) kw[a2][m] = r.w[m];
                }
            }
            // score products: S^T and dP^T with one query per lane
            bf16x8 fa[2 * KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                fa[2 * ks] = *(const LDS bf16x8*)(base + L::A + (rowop ^ (32 * ks)));
                fa[2 * ks + 1] = *(const LDS bf16x8*)(base + L::B + (rowop ^ (32 * ks)));
            }
            f32x16 x = (f32x16){}, y = (f32x16){};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                x = mfma32(fa[2 * ks], rf1[ks], x);
                y = mfma32(fa[2 * ks + 1], rf2[ks], y);
            }
            reads_ahead<2 * KS>();
            // register i holds key row0 + (i/4)*8 + 4h + i%4
            float arg[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) arg[i] = fmaf(x[i], c, -lse2_lane);
            // Dead scores get exp2(-inf) = 0: selects under one uniform branch,
            // not a branch around each exponential.
            if (masked) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = row0 + (i >> 2) * 8 + 4 * h + (i & 3);
                    const bool dead = (key >= N) | (my_row >= N) | (CAUSAL & (key > my_row));
                    arg[i] = dead ? -__builtin_inff() : arg[i];
                }
            }
            bf16x8 w[2];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = __builtin_amdgcn_exp2f(arg[i]);
                float val;
                if constexpr (DROP) {
                    const bool kept = keep_half(kw[i >> 3][(i & 7) >> 1], i & 1, dr.t2 & 0xFFFFu);
                    val = p * ((kept ? y[i] * dr.factor : 0.f) - d_lane);
                } else {
                    val = p * (y[i] - d_lane);
                }
                w[i >> 3][i & 7] = (__bf16)val;
            }
            // dQ^T (d x queries) += (K^T) (d x keys) dS^T
            bf16x8 ft[2 * DB];
#pragma unroll
            for (int i = 0; i < 2 * DB; ++i) ft[i] = tr_operand<D>(base + L::A, trop0, trop1, i >> 1, i & 1);
#pragma unroll
            for (int i = 0; i < 2 * DB; ++i) acc[i >> 1] = mfma32(ft[i], w[i & 1], acc[i >> 1]);
            reads_ahead<2 * DB, 2>();
        }
        __builtin_amdgcn_s_waitcnt(kWaitVm0);    // this wave's copies of the next tile have landed
        __syncthreads();
        if (step + 2 < n_steps) copy_step(step + 2, set);
    }

    // Epilogue: this lane's query row, d = 32*db + 8*g + 4*h + r.
    if (my_row >= N) return;
    __bf16* gp = G + rhead + (size_t)my_row * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            bf16x4 out;
#pragma unroll
            for (int r = 0; r < 4; ++r) out[r] = (__bf16)(acc[db][4 * g + r] * scale);
            *(bf16x4*)(gp + 32 * db + 8 * g + 4 * h) = out;
        }
}

// dK and dV in one launch.  A workgroup of 8 waves holds 128 resident keys,
// 32 per wave pair (wave w and w + 4), and streams the query tiles of the
// GQA group once for both waves of every pair, kSub<D> 32-row tiles per step.
// Per step, for each of its tiles:
//   first half:  wave w     S = Q K^T (8 MFMAs), P (exp), P out to LDS;
//                wave w+4   dP = dO V^T (8 MFMAs), dP out to LDS;
//   barrier;
//   second half: wave w     dS = P (.) (dP - D), dK^T += Q^T dS (8 MFMAs);
//                wave w+4   dV^T += dO^T P (8 MFMAs);  next step's tiles to LDS;
//   barrier.
// So each SIMD (one wave of each kind) has 16 kSub<D> MFMAs in each half, and S
// and dP are computed once per pair (the separate DK and DV kernels computed
// S twice and streamed Q and dO twice).  P goes over in bf16 (it is rounded
// so for the products anyway, thinned by dropout); dP in fp32.  Several tiles
// per step cut the barriers, exchanges and pipeline fills per MFMA.
template <int D>
constexpr int kSub = D == 64 ? 3 : 2;     // as many as the LDS and registers hold
template <int D>
struct Lay2 {
    static constexpr int RBYTES = kTile * 2 * D;
    // one buffer set: for tile j of the step, Q rows at A(j), dO rows at
    // B(j), LSE*log2e and D of its 32 rows at S(j)
    static constexpr int A(int j) { return j * 2 * RBYTES; }
    static constexpr int B(int j) { return j * 2 * RBYTES + RBYTES; }
    static constexpr int S(int j) { return kSub<D> * 2 * RBYTES + j * 2 * kTile * 4; }
    static constexpr int SET = kSub<D> * (2 * RBYTES + 2 * kTile * 4);
    static constexpr int PXP = 2 * SET;                          // P:  [4 pairs][kSub<D>][2 chunks][64 lanes] x 16 B
    static constexpr int PXD = PXP + 4 * kSub<D> * 2 * 64 * 16;     // dP: [4 pairs][kSub<D>][4 quads][64 lanes] x 16 B
    static constexpr int BYTES = PXD + 4 * kSub<D> * 4 * 64 * 16;
};
constexpr int kDkvThreads = 512;

template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(kDkvThreads, 1) void bwd_dkv_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dd,
    __bf16* __restrict__ dK, __bf16* __restrict__ dV, int Hq, int Hkv, int N, int n_rtiles, int bh_total,
    float c, float scale, Dropout dr) {
    using L = Lay2<D>;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    static_assert(L::BYTES <= 160 * 1024, "fits the LDS of one compute unit");

    __shared__ __attribute__((aligned(16))) char smem_raw[L::BYTES];
    LDS char* smem = (LDS char*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // (readfirstlane: the wave index is uniform, so the role and block tests
    // below become scalar branches)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool dk_role = wave < 4;            // waves 0-3: S, P, dS, dK; waves 4-7: dP, dV
    const int wb = wave & 3;                  // resident block of the wave pair
    const int h = lane >> 5;
    const int l32 = lane & 31;
    const int group = Hq / Hkv;

    int bh, rt;
    {
        const int w = blockIdx.x;
        if ((bh_total & 7) == 0) {
            const int slot = w >> 3;
            bh = (w & 7) * (bh_total >> 3) + slot % (bh_total >> 3);
            rt = slot / (bh_total >> 3);
        } else {
            // (few heads) tile-major over all heads, the long key blocks
            // (first when causal) of every head before the short ones of any
            bh = w % bh_total;
            rt = w / bh_total;
        }
    }
    const int b = bh / Hkv;
    const int hr = bh % Hkv;                  // K/V head
    const int r0 = rt * kRows;
    const int wr0 = r0 + 32 * wb;
    const int my_row = wr0 + l32;             // this lane's key
    const size_t rhead = ((size_t)b * Hkv + hr) * N * D;

    // resident rows: K for the S waves, V for the dP waves (B operands)
    bf16x8 rf[KS];
    {
        const int rr = min(my_row, N - 1);
        const __bf16* src = (dk_role ? K : V) + rhead + (size_t)rr * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 x = *(const u32x4*)(src + 16 * ks + 8 * h);
            if (my_row >= N) x = (u32x4){0u, 0u, 0u, 0u};
            rf[ks] = __builtin_bit_cast(bf16x8, x);
        }
    }
    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = (f32x16){};

    // Streamed 32-row tiles t_begin .. t_end-1 of each query head of the
    // group, kSub<D> per step (the last step of a head may hold fewer: its
    // missing tiles lie past t_end and are skipped).
    const int t_begin = CAUSAL ? r0 / kTile : 0;
    const int t_end = (N + kTile - 1) / kTile;
    const int per_head = max(0, (t_end - t_begin + kSub<D> - 1) / kSub<D>);
    const int n_steps = group * per_head;
    auto q_head = [&](int hs) -> size_t { return ((size_t)b * Hq + hr * group + hs) * N; };
    // first tile of step st (in tiles), and its query head
    auto step_tile = [&](int st) { return t_begin + kSub<D> * (st % per_head); };

    // Copies of step `step` into its buffer set (step & 1): waves 0-3 copy
    // the Q rows and waves 4-7 the dO rows straight into LDS; threads
    // 0 .. 32 kSub - 1 stage the row statistics in registers (tile tid / 32
    // of the step), stored with store_stats.  The statistics are loaded
    // first, so the compiler's wait for them at the store also covers the
    // copies issued after them.
    const bool copy_do = wave >= 4;
    float s0 = 0.f, s1 = 0.f;
    int srow = 0;
    auto load_step = [&](int step) __attribute__((always_inline)) {
        const int st = min(step, n_steps - 1);
        const int hs = st / per_head;
        const int tile0 = step_tile(st);
        if (tid < kSub<D> * kTile)
            stage_stats(LSE + q_head(hs), Dd + q_head(hs), (tile0 + tid / kTile) * kTile, N, tid, s0, s1, srow);
        const u32x4 rs = make_rsrc((copy_do ? dO : Q) + q_head(hs) * D, (uint32_t)N * (2 * D));
        LDS char* base = smem + (step & 1) * L::SET;
#pragma unroll
        for (int j = 0; j < kSub<D>; ++j)
            dma_tile<D, 4>(base + (copy_do ? L::B(j) : L::A(j)), rs, (tile0 + j) * kTile, wave & 3, lane);
    };
    auto store_stats = [&](int set) __attribute__((always_inline)) {
        LDS char* base = smem + set * L::SET;
        if (tid < kSub<D> * kTile) {
            float lse2, dv;
            finish_stats(s0, s1, srow, N, lse2, dv);
            LDS float* st = (LDS float*)(base + L::S(tid / kTile));
            st[tid % kTile] = lse2;
            st[kTile + tid % kTile] = dv;
        }
    };

    if (n_steps > 0) {
        load_step(0);
        store_stats(0);
        __builtin_amdgcn_s_waitcnt(kWaitVm0);    // step 0's copies have landed
        if (n_steps > 1) load_step(1);
    }
    __syncthreads();

    const int rowop = rowop_off<D>(lane);
    const int trop0 = trop_off<D>(lane, 0), trop1 = trop_off<D>(lane, 1);

#pragma unroll 1
    for (int step = 0; step < n_steps; ++step) {
        const int set = step & 1;
        const LDS char* base = smem + set * L::SET;
        const int tile0 = step_tile(step);
        const int hs = step / per_head;
        bool active[kSub<D>], masked[kSub<D>];
#pragma unroll
        for (int j = 0; j < kSub<D>; ++j) {
            const int row0 = (tile0 + j) * kTile;
            active[j] = tile0 + j < t_end && wr0 < N;
            masked[j] = row0 + kTile > N || wr0 + 32 > N;
            if (CAUSAL) {
                active[j] = active[j] && row0 + kTile - 1 >= wr0;
                masked[j] = masked[j] || row0 < wr0 + 31;
            }
        }
        // register i of a 32x32 accumulator: streamed row (i/4)*8 + 4h + i%4 of the
        // tile (a query), resident key my_row (the lane)
        float p[kSub<D>][16];
        uint32_t zword[kSub<D>] = {};
#pragma unroll
        for (int j = 0; j < kSub<D>; ++j) {
            if (!active[j]) continue;
            const int row0 = (tile0 + j) * kTile;
            LDS bf16x8* pxp = (LDS bf16x8*)(smem + L::PXP) + (wb * kSub<D> + j) * 128;   // [cc][lane]
            LDS f32x4* pxd = (LDS f32x4*)(smem + L::PXD) + (wb * kSub<D> + j) * 256;     // [quad][lane]
            const int mine = dk_role ? L::A(j) : L::B(j);                            // the streamed tile this wave reads
            bf16x8 fa[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) fa[ks] = *(const LDS bf16x8*)(base + mine + (rowop ^ (32 * ks)));
            f32x16 x = (f32x16){};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) x = mfma32(fa[ks], rf[ks], x);
            reads_ahead<KS>();
            if (!dk_role) {            // dP out
#pragma unroll
                for (int qd = 0; qd < 4; ++qd)
                    pxd[qd * 64 + lane] = (f32x4){x[4 * qd], x[4 * qd + 1], x[4 * qd + 2], x[4 * qd + 3]};
            } else {                   // P (and the dropout bits), P out
                if constexpr (DROP) {
                    const uint32_t t = dr.t2 & 0xFFFFu;
                    // the key (and so its ten round keys) and the multipliers in
                    // vector registers: this kernel's scalar registers are nearly
                    // all taken
                    uint32_t k0 = dr.k0, k1 = dr.k1, m0 = kPhiloxM0, m1 = kPhiloxM1;
                    asm volatile("" : "+v"(k0), "+v"(k1), "+v"(m0), "+v"(m1));
                    const uint32_t bhq = (uint32_t)(b * Hq + hr * group + hs);
                    uint32_t mine_bits = 0;
                    uint32_t ctr0 = (uint32_t)(2 * (wr0 >> 4) + h);
                    asm volatile("" : "+v"(ctr0));
#pragma unroll
                    for (int al = 0; al < 2; ++al) {
                        const PhiloxOut r =
                            philox4x32_10(ctr0 + 2 * al, (uint32_t)(row0 + l32), bhq, dr.offset, k0, k1, m0, m1);
#pragma unroll
                        for (int k = 0; k < 8; ++k)
                            mine_bits |= (uint32_t)keep_half(r.w[k >> 1], k & 1, t) << (8 * al + k);
                    }
                    const int pos = ((l32 >> 4) << 3) | (((l32 >> 3) & 1) << 2) | (l32 & 3);
                    uint32_t sel = 1u << pos;
                    uint32_t sh = ((l32 >> 2) & 1) * 32u;
                    asm volatile("" : "+v"(sel), "+v"(sh));
                    uint32_t zw = 0;
#pragma unroll
                    for (int bit = 0; bit < 16; ++bit) {
                        const uint64_t bal = __builtin_amdgcn_ballot_w64((mine_bits >> bit) & 1u);
                        zw |= (uint32_t)(bal >> sh) & (0u - ((sel >> bit) & 1u));
                    }
                    zword[j] = zw >> (4 * h);
                }
                const LDS float* st = (const LDS float*)(base + L::S(j));
                float arg[16];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 lse4 = *(const LDS f32x4*)(st + 8 * g + 4 * h);
#pragma unroll
                    for (int e = 0; e < 4; ++e) arg[4 * g + e] = fmaf(x[4 * g + e], c, -lse4[e]);
                }
                // Dead scores get exp2(-inf) = 0: selects under one uniform
                // branch, not a branch around each exponential.
                if (masked[j]) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int qry = row0 + 8 * (i >> 2) + 4 * h + (i & 3);
                        const bool dead = (my_row >= N) | (qry >= N) | (CAUSAL & (my_row > qry));
                        arg[i] = dead ? -__builtin_inff() : arg[i];
                    }
                }
                bf16x8 pw[2];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    p[j][i] = __builtin_amdgcn_exp2f(arg[i]);
                    // keep bit as a 0/1 multiplier (no condition registers held)
                    const float keepf = DROP ? (float)((zword[j] >> (8 * (i >> 2) + (i & 3))) & 1u) : 1.f;
                    pw[i >> 3][i & 7] = (__bf16)(p[j][i] * keepf);
                }
                pxp[lane] = pw[0];
                pxp[64 + lane] = pw[1];
            }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kSub<D>; ++j) {
            if (!active[j]) continue;
            const LDS bf16x8* pxp = (const LDS bf16x8*)(smem + L::PXP) + (wb * kSub<D> + j) * 128;
            const LDS f32x4* pxd = (const LDS f32x4*)(smem + L::PXD) + (wb * kSub<D> + j) * 256;
            const int mine = dk_role ? L::A(j) : L::B(j);
            // operands of dK^T += (Q^T) dS  or  dV^T += (dO^T) P, read first so
            // that they arrive during the dS arithmetic
            bf16x8 ft[2 * DB];
#pragma unroll
            for (int i = 0; i < 2 * DB; ++i) ft[i] = tr_operand<D>(base + mine, trop0, trop1, i >> 1, i & 1);
            bf16x8 w[2];
            if (dk_role) {             // dS from the partner's dP
                const LDS float* st = (const LDS float*)(base + L::S(j));
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 dp = pxd[g * 64 + lane];
                    const f32x4 d4 = *(const LDS f32x4*)(st + kTile + 8 * g + 4 * h);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 4 * g + e;
                        float val;
                        if constexpr (DROP) {
                            const float keepf = (float)((zword[j] >> (8 * g + e)) & 1u) * dr.factor;
                            val = p[j][i] * fmaf(dp[e], keepf, -d4[e]);
                        } else {
                            val = p[j][i] * (dp[e] - d4[e]);
                        }
                        w[i >> 3][i & 7] = (__bf16)val;
                    }
                }
            } else {                   // P from the partner
                w[0] = pxp[lane];
                w[1] = pxp[64 + lane];
            }
            // dK^T += (Q^T) dS  or  dV^T += (dO^T) P
#pragma unroll
            for (int i = 0; i < 2 * DB; ++i) acc[i >> 1] = mfma32(ft[i], w[i & 1], acc[i >> 1]);
        }
        if (step + 1 < n_steps) store_stats(set ^ 1);
        __builtin_amdgcn_s_waitcnt(kWaitVm0);    // this wave's copies of the next step have landed
        __syncthreads();
        if (step + 2 < n_steps) load_step(step + 2);
    }

    if (my_row >= N) return;
    const float f = dk_role ? scale : (DROP ? dr.factor : 1.f);
    __bf16* gp = (dk_role ? dK : dV) + rhead + (size_t)my_row * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            bf16x4 out;
#pragma unroll
            for (int r = 0; r < 4; ++r) out[r] = (__bf16)(acc[db][4 * g + r] * f);
            *(bf16x4*)(gp + 32 * db + 8 * g + 4 * h) = out;
        }
}

template <int D, bool CAUSAL, bool DROP>
hipError_t launch_dkv(const BwdArgs& a, const float* dd, const Dropout& drop, hipStream_t stream) {
    int n_rtiles = (a.N + kRows - 1) / kRows;
    int bh_total = a.B * a.Hkv;
    float c = a.scale * kLog2e;
    float scale = a.scale;
    int Hq = a.Hq, Hkv = a.Hkv, N = a.N;
    const __bf16* q = (const __bf16*)a.q;
    const __bf16* k = (const __bf16*)a.k;
    const __bf16* v = (const __bf16*)a.v;
    const __bf16* dO = (const __bf16*)a.dO;
    const float* lse = a.lse;
    __bf16* gk = (__bf16*)a.dk;
    __bf16* gv = (__bf16*)a.dv;
    Dropout dr = drop;
    void* args[] = {(void*)&q, (void*)&k, (void*)&v, (void*)&dO, (void*)&lse, (void*)&dd, &gk, &gv,
                    &Hq, &Hkv, &N, &n_rtiles, &bh_total, &c, &scale, &dr};
    return hipLaunchKernel((const void*)bwd_dkv_kernel<D, CAUSAL, DROP>, dim3(bh_total * n_rtiles),
                           dim3(kDkvThreads), args, 0, stream);
}

template <int D, bool CAUSAL, bool DROP>
hipError_t launch_dq(const BwdArgs& a, float* dd, const Dropout& drop, hipStream_t stream) {
    int n_rtiles = (a.N + kRows - 1) / kRows;
    int bh_total = a.B * a.Hq;
    float c = a.scale * kLog2e;
    float scale = a.scale;
    int Hq = a.Hq, Hkv = a.Hkv, N = a.N;
    const __bf16* q = (const __bf16*)a.q;
    const __bf16* k = (const __bf16*)a.k;
    const __bf16* v = (const __bf16*)a.v;
    const __bf16* dO = (const __bf16*)a.dO;
    const float* lse = a.lse;
    __bf16* g = (__bf16*)a.dq;
    Dropout dr = drop;
    const __bf16* o = (const __bf16*)a.o;
    void* args[] = {(void*)&q, (void*)&k, (void*)&v, (void*)&dO, (void*)&o, (void*)&lse, (void*)&dd, &g,
                    &Hq, &Hkv, &N, &n_rtiles, &bh_total, &c, &scale, &dr};
    return hipLaunchKernel((const void*)bwd_dq_kernel<D, CAUSAL, DROP>, dim3(bh_total * n_rtiles),
                           dim3(kThreads), args, 0, stream);
}

// dQ first: it writes D, which the dK/dV kernel reads.
template <int D, bool CAUSAL, bool DROP>
hipError_t launch_all(const BwdArgs& a, float* workspace, const Dropout& dr, hipStream_t stream) {
    float* dd = workspace;
    hipError_t e = launch_dq<D, CAUSAL, DROP>(a, dd, dr, stream);
    if (e != hipSuccess) return e;
    return launch_dkv<D, CAUSAL, DROP>(a, dd, dr, stream);
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, float* workspace, hipStream_t stream) {
    const Dropout none{};
    if (a.d == 128)
        return a.causal ? launch_all<128, true, false>(a, workspace, none, stream)
                        : launch_all<128, false, false>(a, workspace, none, stream);
    return a.causal ? launch_all<64, true, false>(a, workspace, none, stream)
                    : launch_all<64, false, false>(a, workspace, none, stream);
}

hipError_t launch_bwd_bf16_dropout(const BwdArgs& a, const Dropout& dr, float* workspace, hipStream_t stream) {
    if (a.d == 128)
        return a.causal ? launch_all<128, true, true>(a, workspace, dr, stream)
                        : launch_all<128, false, true>(a, workspace, dr, stream);
    return a.causal ? launch_all<64, true, true>(a, workspace, dr, stream)
                    : launch_all<64, false, true>(a, workspace, dr, stream);
}

}  // namespace fa
