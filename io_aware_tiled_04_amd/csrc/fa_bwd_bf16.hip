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
// Kernels.  The accumulators of one 32-row block at d = 128 take 64 VGPRs
// each, so one wave cannot hold dK and dV (and K, V, S and dP) within the 256
// VGPRs of two waves per SIMD.  The work is split in three kernels of the
// forward's size, each with one accumulator:
//   DQ: resident query rows, streamed key tiles:  S^T = K Q^T and
//       dP^T = V dO^T put one query per lane (LSE and D per lane), and
//       dQ^T += K^T dS^T takes K^T from LDS in the key order of dS^T's
//       registers (the forward's V^T trick).
//   DK: resident key rows, streamed query tiles: S = Q K^T and dP = dO V^T
//       put one key per lane, and dK^T += Q^T dS takes Q^T from LDS.
//   DV: resident key rows: S = Q K^T, then dV^T += dO^T P.
// S and dP are recomputed by the kernels that need them (8 products instead
// of 5).  A first kernel forms D.
//
// Each workgroup: 4 waves of 32 resident rows (128 rows); streamed tiles of
// 32 rows, double-buffered in LDS, loaded into registers one tile ahead.
//
// Dropout (DROP): the forward's output was O = (P (.) Z) V / (1 - p), so with
// f = 1 / (1 - p),  dV = (P (.) Z)^T dO f,  dP = (dO V^T) (.) Z f, and
// dS = P (.) (dP - D) as before (D = rowsum(dO (.) O) with the dropped O
// still equals sum_j P dP).  The keep bits Z are the forward's (philox.h).
// DQ holds one query per lane and keys in its registers, the forward's
// layout: two generator calls per step give its 16 decisions.  DK and DV
// hold one key per lane: each lane makes the two calls of one streamed query
// and one half of the wave's keys, and sixteen wave ballots carry the bits
// to the lanes of their keys.
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

enum Mode { kDQ = 0, kDK = 1, kDV = 2 };

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Keep decision of the draw in 16-bit half `hi` of a generator word.
__device__ __forceinline__ bool keep_half(uint32_t word, int hi, uint32_t t) {
    return (hi ? word >> 16 : word & 0xFFFFu) >= t;
}

// Permuted position of row k (0..31) of a streamed tile inside a transposed
// LDS row: within each 16-row chunk, row 8*b3 + 4*b2 + b moves to
// 8*b2 + 4*b3 + b.  With it, accumulator registers 8c..8c+7 of a 32x32 MFMA
// (rows (r/4)*8 + h*4 + r%4) are the 16-element operand of chunk c.
__device__ __forceinline__ int tr_pos(int k) {
    return (k & ~15) | ((k & 4) << 1) | ((k & 8) >> 1) | (k & 3);
}

// LDS layout of one buffer set.
template <int D>
struct Lay {
    static constexpr int RPITCH = 2 * D + 16;            // row-major tile row
    static constexpr int TPITCH = 2 * kTile + 16;        // transposed row (one d)
    static constexpr int RBYTES = kTile * RPITCH;
    static constexpr int TBYTES = D * TPITCH;
    static constexpr int A = 0;                          // row-major tile 1
    static constexpr int B = RBYTES;                     // row-major tile 2
    static constexpr int T = 2 * RBYTES;                 // transposed tile
    static constexpr int S = 2 * RBYTES + TBYTES;        // two float[32] rows of statistics
    static constexpr int SET = S + 2 * kTile * 4;
    static constexpr int BYTES = 2 * SET;
    static constexpr int CHUNKS = D / 8;                 // 16-byte chunks per row
    static constexpr int ITEMS = (kTile / 2) * CHUNKS;   // (row pair, chunk) items per tile
};

// Per-thread staging of one streamed tile: the item (row pair j, chunk c8)
// of up to two tensors, and one statistic per row for up to two rows.
template <int D>
struct Stage {
    u32x4 x0, x1;     // tensor 1, rows 2j and 2j+1
    u32x4 y0, y1;     // tensor 2, rows 2j and 2j+1
    float s0, s1;     // statistics of row tid (tid < 32)
};

template <int D>
__device__ __forceinline__ void stage_rows(const __bf16* __restrict__ g, int row0, int n, int tid,
                                           u32x4& r0, u32x4& r1) {
    using L = Lay<D>;
    const int it = tid % L::ITEMS;
    const int j = it % (kTile / 2), c8 = it / (kTile / 2);
    const int a = min(row0 + 2 * j, n - 1), b = min(row0 + 2 * j + 1, n - 1);
    r0 = *(const u32x4*)(g + (size_t)a * D + 8 * c8);
    r1 = *(const u32x4*)(g + (size_t)b * D + 8 * c8);
}

template <int D>
__device__ __forceinline__ void put_rows(LDS char* dst, int tid, const u32x4& r0, const u32x4& r1) {
    using L = Lay<D>;
    if (tid >= L::ITEMS) return;
    const int j = tid % (kTile / 2), c8 = tid / (kTile / 2);
    *(LDS u32x4*)(dst + (2 * j) * L::RPITCH + 16 * c8) = r0;
    *(LDS u32x4*)(dst + (2 * j + 1) * L::RPITCH + 16 * c8) = r1;
}

template <int D>
__device__ __forceinline__ void put_transposed(LDS char* dst, int tid, const u32x4& r0, const u32x4& r1) {
    using L = Lay<D>;
    if (tid >= L::ITEMS) return;
    const int j = tid % (kTile / 2), c8 = tid / (kTile / 2);
    LDS char* p = dst + 8 * c8 * L::TPITCH + tr_pos(2 * j) * 2;   // rows 2j, 2j+1 stay adjacent
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t lo = __builtin_amdgcn_perm(r1[e], r0[e], 0x05040100u);
        const uint32_t hi = __builtin_amdgcn_perm(r1[e], r0[e], 0x07060302u);
        *(LDS uint32_t*)(p + (2 * e) * L::TPITCH) = lo;
        *(LDS uint32_t*)(p + (2 * e + 1) * L::TPITCH) = hi;
    }
}

// Row statistics of the streamed query rows (DK, DV): LSE * log2(e) and D.
// Rows past N get +inf (so that p = 0) and D = 0.
__device__ __forceinline__ void stage_stats(const float* __restrict__ lse, const float* __restrict__ dd,
                                            int row0, int n, int tid, float& s0, float& s1) {
    const int r = row0 + (tid & 31);
    const bool in = r < n;
    const int rc = min(r, n - 1);
    s0 = in ? lse[rc] * kLog2e : __builtin_inff();
    s1 = in && dd ? dd[rc] : 0.f;
}

// D_i = sum_d dO_id O_id for every row: D / 8 threads per row, one 16-byte
// chunk each, reduced across those threads.
template <int D>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const __bf16* __restrict__ dO,
                                                         const __bf16* __restrict__ O,
                                                         float* __restrict__ Dout, long long rows) {
    constexpr int TPR = D / 8;
    const long long row = (long long)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
    const int c = threadIdx.x % TPR;
    float acc = 0.f;
    if (row < rows) {
        const bf16x8 a = *(const bf16x8*)(dO + row * D + 8 * c);
        const bf16x8 b = *(const bf16x8*)(O + row * D + 8 * c);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += (float)a[e] * (float)b[e];
    }
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, TPR);
    if (row < rows && c == 0) Dout[row] = acc;
}

// One backward kernel per accumulator (MODE), see the file header.
//   resident rows: queries (DQ) or keys (DK, DV) of head rh;
//   streamed rows: keys of K/V head (DQ) or queries of the query heads of the
//   GQA group (DK, DV).
// c = scale * log2(e) (signed).  LSE and D are [B, Hq, N] float32.
// DROP: the forward ran with dropout `dr` (see the file header).
template <int D, bool CAUSAL, int MODE, bool DROP>
__global__ __launch_bounds__(kThreads, 2) void bwd_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dd,
    __bf16* __restrict__ G, int Hq, int Hkv, int N, int n_rtiles, int bh_total, float c, float scale,
    Dropout dr) {
    using L = Lay<D>;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    constexpr bool RES_Q = MODE == kDQ;

    __shared__ __attribute__((aligned(16))) char smem_raw[L::BYTES];
    LDS char* smem = (LDS char*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;
    const int l32 = lane & 31;
    const int group = Hq / Hkv;

    // Work decomposition, XCD-aware as in the forward; for causal attention the
    // heaviest resident tiles go first (last query tiles for DQ, first key
    // tiles for DK and DV).
    int bh, rt;
    {
        const int w = blockIdx.x;
        if ((bh_total & 7) == 0) {
            const int slot = w >> 3;
            bh = (w & 7) * (bh_total >> 3) + slot % (bh_total >> 3);
            rt = slot / (bh_total >> 3);
        } else {
            bh = w / n_rtiles;
            rt = w % n_rtiles;
        }
        if (CAUSAL && RES_Q) rt = n_rtiles - 1 - rt;
    }
    const int b = bh / (RES_Q ? Hq : Hkv);
    const int hr = bh % (RES_Q ? Hq : Hkv);             // resident head
    const int r0 = rt * kRows;                           // first resident row of the workgroup
    const int wr0 = r0 + 32 * wave;                      // first resident row of this wave
    const int my_row = wr0 + l32;                        // the resident row of this lane

    // Resident operands (B operand of the score products): lane holds
    // d = 16*ks + 8*h .. +7 of its row.
    const size_t rhead = ((size_t)b * (RES_Q ? Hq : Hkv) + hr) * N * D;
    bf16x8 rf1[KS], rf2[KS];
    {
        const __bf16* t1 = RES_Q ? Q : K;
        const __bf16* t2 = RES_Q ? dO : V;
        const int rr = min(my_row, N - 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 x = *(const u32x4*)(t1 + rhead + (size_t)rr * D + 16 * ks + 8 * h);
            if (my_row >= N) x = (u32x4){0u, 0u, 0u, 0u};
            rf1[ks] = __builtin_bit_cast(bf16x8, x);
            if constexpr (MODE != kDV) {
                u32x4 y = *(const u32x4*)(t2 + rhead + (size_t)rr * D + 16 * ks + 8 * h);
                if (my_row >= N) y = (u32x4){0u, 0u, 0u, 0u};
                rf2[ks] = __builtin_bit_cast(bf16x8, y);
            }
        }
    }
    // Per-lane statistics of a resident query row (DQ).
    float lse2_lane = 0.f, d_lane = 0.f;
    if constexpr (RES_Q) {
        const size_t srow = ((size_t)b * Hq + hr) * N + min(my_row, N - 1);
        lse2_lane = LSE[srow] * kLog2e;
        d_lane = Dd[srow];
    }

    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = (f32x16){};

    // Streamed range.  DQ: key tiles 0 .. (last visible key)/32 of K/V head
    // hq / group.  DK/DV: for each query head of the group, query tiles from
    // the first one that can see the workgroup's keys.
    const int heads = RES_Q ? 1 : group;
    int t_begin, t_end;
    if constexpr (RES_Q) {
        t_begin = 0;
        t_end = ((CAUSAL ? min(N, r0 + kRows) : N) + kTile - 1) / kTile;
    } else {
        t_begin = CAUSAL ? r0 / kTile : 0;
        t_end = (N + kTile - 1) / kTile;
    }
    const int per_head = max(0, t_end - t_begin);
    const int n_steps = heads * per_head;

    auto src_head = [&](int hs) -> size_t {
        // base element offset of the streamed head: K/V head for DQ, query head for DK/DV
        if constexpr (RES_Q) return ((size_t)b * Hkv + hr / group) * N * D;
        else return ((size_t)b * Hq + hr * group + hs) * N * D;
    };
    auto stat_base = [&](int hs) -> size_t { return ((size_t)b * Hq + hr * group + hs) * N; };

    Stage<D> stg;
    auto load_step = [&](int step) __attribute__((always_inline)) {
        const int s = min(step, n_steps - 1);
        const int hs = s / per_head;
        const int row0 = (t_begin + s % per_head) * kTile;
        const size_t base = src_head(hs);
        if constexpr (MODE == kDQ) {
            stage_rows<D>(K + base, row0, N, tid, stg.x0, stg.x1);
            stage_rows<D>(V + base, row0, N, tid, stg.y0, stg.y1);
        } else if constexpr (MODE == kDK) {
            stage_rows<D>(Q + base, row0, N, tid, stg.x0, stg.x1);
            stage_rows<D>(dO + base, row0, N, tid, stg.y0, stg.y1);
            stage_stats(LSE + stat_base(hs), Dd + stat_base(hs), row0, N, tid, stg.s0, stg.s1);
        } else {
            stage_rows<D>(Q + base, row0, N, tid, stg.x0, stg.x1);
            stage_rows<D>(dO + base, row0, N, tid, stg.y0, stg.y1);
            stage_stats(LSE + stat_base(hs), nullptr, row0, N, tid, stg.s0, stg.s1);
        }
    };
    // Writes the staged tile into buffer set `set`:
    //   DQ: A = K rows, B = V rows, T = K transposed;
    //   DK: A = Q rows, B = dO rows, T = Q transposed, stats = LSE*log2e, D;
    //   DV: A = Q rows, T = dO transposed, stats = LSE*log2e.
    auto store_step = [&](int set) __attribute__((always_inline)) {
        LDS char* base = smem + set * L::SET;
        put_rows<D>(base + L::A, tid, stg.x0, stg.x1);
        if constexpr (MODE != kDV) put_rows<D>(base + L::B, tid, stg.y0, stg.y1);
        if constexpr (MODE == kDV) put_transposed<D>(base + L::T, tid, stg.y0, stg.y1);
        else put_transposed<D>(base + L::T, tid, stg.x0, stg.x1);
        if constexpr (MODE != kDQ) {
            if (tid < kTile) {
                ((LDS float*)(base + L::S))[tid] = stg.s0;
                ((LDS float*)(base + L::S))[kTile + tid] = stg.s1;
            }
        }
    };

    if (n_steps > 0) {
        load_step(0);
        store_step(0);
        load_step(1);
    }
    __syncthreads();

#pragma unroll 1
    for (int step = 0; step < n_steps; ++step) {
        const int set = step & 1;
        const LDS char* base = smem + set * L::SET;
        const int row0 = (t_begin + step % per_head) * kTile;   // first streamed row of the tile

        // Does this wave see any pair of the tile?  (causal only)
        bool active = wr0 < N;
        bool masked = row0 + kTile > N;
        if (CAUSAL) {
            if (RES_Q) {   // keys row0.. vs queries wr0..wr0+31
                active = active && row0 <= wr0 + 31;
                masked = masked || row0 + kTile - 1 > wr0;
            } else {       // queries row0.. vs keys wr0..wr0+31
                active = active && row0 + kTile - 1 >= wr0;
                masked = masked || row0 < wr0 + 31;
            }
        }
        if (!RES_Q) masked = masked || wr0 + 32 > N;

        if (active) {
            // Dropout keep bits of this wave's pairs (the key j of a pair is
            // 16a + 8b + 4cc + w; its draw is half 4b + w of the call at
            // counter (2a + cc, query, query head unit, offset)).
            //   DQ: lane = query my_row, register i = key row0 + 16(i/8) +
            //       8((i/4)%2) + 4h + i%4: call i/8 at counter 2(row0/16 + i/8) + h
            //       holds register i's draw in half i%8.
            //   DK, DV: zword bit r = keep bit of (query row0 + 4h + r, my key).
            uint32_t kw[2][4];
            uint32_t zword = 0;
            if constexpr (DROP) {
                const uint32_t t = dr.t2 & 0xFFFFu;
                // The empty asm hides which counter and key words stay fixed
                // over the steps; otherwise the optimiser keeps partial rounds
                // and the ten round keys live across the loop (and spills them).
                uint32_t k0 = dr.k0, k1 = dr.k1;
                asm volatile("" : "+s"(k0), "+s"(k1));
                if constexpr (RES_Q) {
                    uint32_t row_u = (uint32_t)my_row;
                    asm volatile("" : "+v"(row_u));
#pragma unroll
                    for (int a2 = 0; a2 < 2; ++a2) {
                        const PhiloxOut r = philox4x32_10((uint32_t)(2 * ((row0 >> 4) + a2) + h), row_u,
                                                          (uint32_t)bh, dr.offset, k0, k1);
#pragma unroll
                        for (int m = 0; m < 4; ++m) kw[a2][m] = r.w[m];
                    }
                } else {
                    // Lane (l32, h) draws for query row0 + l32 and the keys
                    // wr0 + 16al + 4h + {0..3, 8..11}: bit 8al + k of `mine`
                    // is half k of call al.
                    const uint32_t bhq = (uint32_t)(b * Hq + hr * group + step / per_head);
                    uint32_t mine = 0;
                    uint32_t ctr0 = (uint32_t)(2 * (wr0 >> 4) + h);
                    asm volatile("" : "+v"(ctr0));
#pragma unroll
                    for (int al = 0; al < 2; ++al) {
                        const PhiloxOut r = philox4x32_10(ctr0 + 2 * al,
                                                          (uint32_t)(row0 + l32), bhq, dr.offset, k0, k1);
#pragma unroll
                        for (int k = 0; k < 8; ++k)
                            mine |= (uint32_t)keep_half(r.w[k >> 1], k & 1, t) << (8 * al + k);
                    }
                    // My key wr0 + l32 is bit pos of the lanes whose h equals
                    // its bit 2: lane l32' + 32 * that bit holds query l32'.
                    // The selection is arithmetic (one-hot `sel`, shift `sh`),
                    // and the asm keeps the optimiser from hoisting sixteen
                    // loop-invariant masks out of the step loop.
                    const int pos = ((l32 >> 4) << 3) | (((l32 >> 3) & 1) << 2) | (l32 & 3);
                    uint32_t sel = 1u << pos;
                    uint32_t sh = ((l32 >> 2) & 1) * 32u;
                    asm volatile("" : "+v"(sel), "+v"(sh));
#pragma unroll
                    for (int bit = 0; bit < 16; ++bit) {
                        const uint64_t bal = __builtin_amdgcn_ballot_w64((mine >> bit) & 1u);
                        zword |= (uint32_t)(bal >> sh) & (0u - ((sel >> bit) & 1u));
                    }
                    // Register i's query is (i/4)*8 + 4h + i%4: shift out 4h
                    // here so that the per-element shifts are immediates (a
                    // per-lane shift count per element would be 16 registers
                    // kept across the loop).
                    zword >>= 4 * h;
                }
            }
            // score products: X = A_tile (rows) x resident^T, one resident row per lane
            const LDS char* arow = base + L::A + l32 * L::RPITCH + 16 * h;
            f32x16 x = (f32x16){};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                x = mfma32(*(const LDS bf16x8*)(arow + 32 * ks), rf1[ks], x);
            f32x16 y = (f32x16){};
            if constexpr (MODE != kDV) {
                const LDS char* brow = base + L::B + l32 * L::RPITCH + 16 * h;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    y = mfma32(*(const LDS bf16x8*)(brow + 32 * ks), rf2[ks], y);
            }
            // register i holds streamed row sr(i) = (i/4)*8 + 4*h + i%4 of the tile;
            // the statistics of rows 8g + 4h .. +3 are one 16-byte LDS read
            const LDS float* st = (const LDS float*)(base + L::S);
            f32x4 lse4[4], d4[4];
            if constexpr (!RES_Q) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    lse4[g] = *(const LDS f32x4*)(st + 8 * g + 4 * h);
                    if constexpr (MODE == kDK) d4[g] = *(const LDS f32x4*)(st + kTile + 8 * g + 4 * h);
                }
            }
            bf16x8 w[2];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int sr = (i >> 2) * 8 + 4 * h + (i & 3);
                const int srow = row0 + sr;
                float lse2, dv;
                int key, qry;
                if constexpr (RES_Q) {
                    lse2 = lse2_lane;
                    dv = d_lane;
                    key = srow;
                    qry = my_row;
                } else {
                    lse2 = lse4[i >> 2][i & 3];
                    dv = MODE == kDK ? d4[i >> 2][i & 3] : 0.f;
                    key = my_row;
                    qry = srow;
                }
                bool dead = false;
                if (masked) dead = key >= N || qry >= N || (CAUSAL && key > qry);
                const float p = dead ? 0.f : __builtin_amdgcn_exp2f(fmaf(x[i], c, -lse2));
                bool kept = true;
                if constexpr (DROP) {
                    if constexpr (RES_Q) kept = keep_half(kw[i >> 3][(i & 7) >> 1], i & 1, dr.t2 & 0xFFFFu);
                    else kept = (zword >> ((i >> 2) * 8 + (i & 3))) & 1u;
                }
                float val;
                if constexpr (MODE == kDV) val = kept ? p : 0.f;              // times f in the epilogue
                else if constexpr (DROP) val = p * ((kept ? y[i] * dr.factor : 0.f) - dv);
                else val = p * (y[i] - dv);
                w[i >> 3][i & 7] = (__bf16)val;
            }
            // accumulator product: acc^T (d x resident) += T_tile^T (d x streamed) w
            const LDS char* trow = base + L::T + l32 * L::TPITCH + 16 * h;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int cc = 0; cc < 2; ++cc)
                    acc[db] = mfma32(*(const LDS bf16x8*)(trow + 32 * db * L::TPITCH + 32 * cc), w[cc],
                                     acc[db]);
        }
        if (step + 1 < n_steps) store_step(set ^ 1);
        __syncthreads();
        if (step + 2 < n_steps) load_step(step + 2);
    }

    // Epilogue: this lane's resident row, d = 32*db + 8*g + 4*h + r.
    if (my_row >= N) return;
    const float f = MODE == kDV ? (DROP ? dr.factor : 1.f) : scale;
    __bf16* gp = G + rhead + (size_t)my_row * D;
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

template <int D, bool CAUSAL, int MODE, bool DROP>
hipError_t launch_mode(const BwdArgs& a, const float* dd, const Dropout& drop, hipStream_t stream) {
    int n_rtiles = (a.N + kRows - 1) / kRows;
    int bh_total = a.B * (MODE == kDQ ? a.Hq : a.Hkv);
    float c = a.scale * kLog2e;
    float scale = a.scale;
    int Hq = a.Hq, Hkv = a.Hkv, N = a.N;
    const __bf16* q = (const __bf16*)a.q;
    const __bf16* k = (const __bf16*)a.k;
    const __bf16* v = (const __bf16*)a.v;
    const __bf16* dO = (const __bf16*)a.dO;
    const float* lse = a.lse;
    __bf16* g = (__bf16*)(MODE == kDQ ? a.dq : MODE == kDK ? a.dk : a.dv);
    Dropout dr = drop;
    void* args[] = {(void*)&q, (void*)&k, (void*)&v, (void*)&dO, (void*)&lse, (void*)&dd, &g,
                    &Hq, &Hkv, &N, &n_rtiles, &bh_total, &c, &scale, &dr};
    return hipLaunchKernel((const void*)bwd_kernel<D, CAUSAL, MODE, DROP>, dim3(bh_total * n_rtiles),
                           dim3(kThreads), args, 0, stream);
}

template <int D, bool CAUSAL, bool DROP>
hipError_t launch_all(const BwdArgs& a, float* workspace, const Dropout& dr, hipStream_t stream) {
    long long rows = (long long)a.B * a.Hq * a.N;
    const __bf16* dO = (const __bf16*)a.dO;
    const __bf16* o = (const __bf16*)a.o;
    float* dd = workspace;
    void* args[] = {(void*)&dO, (void*)&o, &dd, &rows};
    const long long per_block = 256 / (D / 8);
    hipError_t e = hipLaunchKernel((const void*)bwd_rowdot_kernel<D>,
                                   dim3((unsigned)((rows + per_block - 1) / per_block)), dim3(256), args,
                                   0, stream);
    if (e != hipSuccess) return e;
    if ((e = launch_mode<D, CAUSAL, kDQ, DROP>(a, dd, dr, stream)) != hipSuccess) return e;
    if ((e = launch_mode<D, CAUSAL, kDK, DROP>(a, dd, dr, stream)) != hipSuccess) return e;
    return launch_mode<D, CAUSAL, kDV, DROP>(a, dd, dr, stream);
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
