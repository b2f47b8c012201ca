// Attention forward pass, bf16 inputs, for gfx950 (MI355X).
//
// One workgroup owns one tile of kBr = 128 query rows of one query head and
// keeps it resident (in registers) while it streams the K/V tiles of the
// matching K/V head through LDS: the tiling of the reading-notes page
// (Methods, step 1: Q stays on chip, K and V are read block by block) in the
// query-outer loop order the blog names at the end of its blocked derivation
// (section 带在线Softmax重缩放的分块模式, closing remark).  Per K/V tile:
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
//
// Layout choices (each checked against the MFMA lane layouts of gfx950):
//  * Computing S^T rather than S puts one query per lane (column of the
//    32x32 accumulator), so the row max and row sum are per-lane reductions
//    plus one exchange between lanes l and l+32.
//  * The S^T accumulator registers 8c..8c+7 of a 32-key block are exactly the
//    B operand (P^T, 16 keys x 32 queries) of the P V product for the 16-key
//    chunk c, once the keys of that chunk are taken in the order
//    {16c+4h+0..3, 16c+8+4h+0..3} for lane half h.  V is read in the same
//    key order with the LDS transpose read (ds_read_b64_tr_b16), so P never
//    leaves registers and V keeps its natural [key][d] layout in LDS.
//  * The O^T accumulator also has one query per lane, so the rescale by
//    2^(m-m') and the final 1/l are one multiplier per lane.
#include "fa_kernels.h"

#include <stdint.h>

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS __attribute__((address_space(3)))

constexpr int kWaves = 4;
constexpr int kWaveRows = 32;                    // query rows per wave
constexpr int kThreads = kWaves * 64;
constexpr int kBr = kWaves * kWaveRows;          // query rows per workgroup
static_assert(kBr == kBlockRowsBf16, "grid and kernel disagree on the query tile");

// K/V tile geometry in LDS.  Row pitches are padded so that the MFMA operand
// reads are free of bank conflicts: K rows are read 16 bytes per lane with
// consecutive lanes on consecutive keys (pitch = 16 mod 128 bytes); V rows
// are read 4 rows x 32 bytes per 16 lanes by the transpose read (pitch = 32
// mod 128 bytes).
template <int D>
struct Tile {
    static constexpr int BC = 8192 / D;           // keys per tile: 64 (d=128), 128 (d=64)
    static constexpr int KPITCH = 2 * D + 16;
    static constexpr int VPITCH = 2 * D + 32;
    static constexpr int KBYTES = BC * KPITCH;
    static constexpr int VBYTES = BC * VPITCH;
    static constexpr int STAGE = KBYTES + VBYTES;
    static constexpr int ROW_CHUNKS = D / 8;       // 16-byte chunks per row
    static constexpr int CHUNKS_PER_THREAD = BC * ROW_CHUNKS / kThreads;
    static_assert(BC * ROW_CHUNKS % kThreads == 0, "tile must split evenly over the threads");
    static_assert(BC % 32 == 0, "");
};

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Sum or max across the two lane halves (lane l and lane l^32 hold the same
// query): after the swap, out[0] + out[1] is x[l] + x[l^32] in every lane.
__device__ __forceinline__ float half_swap_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float half_swap_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Global -> registers for one K/V tile; rows at or past N read as zero so
// that masked keys meet finite values.
template <int D>
__device__ __forceinline__ void load_kv(const u32x4* __restrict__ kg, const u32x4* __restrict__ vg,
                                        int key0, int N, int tid,
                                        u32x4 (&kr)[Tile<D>::CHUNKS_PER_THREAD],
                                        u32x4 (&vr)[Tile<D>::CHUNKS_PER_THREAD]) {
    using T = Tile<D>;
#pragma unroll
    for (int c = 0; c < T::CHUNKS_PER_THREAD; ++c) {
        const int u = c * kThreads + tid;
        const int row = u / T::ROW_CHUNKS;
        const int col = u % T::ROW_CHUNKS;
        const int key = key0 + row;
        if (key < N) {
            const size_t off = (size_t)key * T::ROW_CHUNKS + col;
            kr[c] = kg[off];
            vr[c] = vg[off];
        } else {
            kr[c] = (u32x4){0u, 0u, 0u, 0u};
            vr[c] = (u32x4){0u, 0u, 0u, 0u};
        }
    }
}

template <int D>
__device__ __forceinline__ void store_kv(LDS char* stage, int tid,
                                         const u32x4 (&kr)[Tile<D>::CHUNKS_PER_THREAD],
                                         const u32x4 (&vr)[Tile<D>::CHUNKS_PER_THREAD]) {
    using T = Tile<D>;
    LDS char* kl = stage;
    LDS char* vl = stage + T::KBYTES;
#pragma unroll
    for (int c = 0; c < T::CHUNKS_PER_THREAD; ++c) {
        const int u = c * kThreads + tid;
        const int row = u / T::ROW_CHUNKS;
        const int col = u % T::ROW_CHUNKS;
        *(LDS u32x4*)(kl + row * T::KPITCH + col * 16) = kr[c];
        *(LDS u32x4*)(vl + row * T::VPITCH + col * 16) = vr[c];
    }
}

// c_log2 = |scale| * log2(e) (> 0); qsign flips the sign bit of every Q
// element when scale < 0 (exact), so that the kernel only sees c_log2 > 0.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, float* __restrict__ LSE, int group, int N, int n_qtiles, int bh_total,
    float c_log2, uint32_t qsign) {
    using T = Tile<D>;
    constexpr int BC = T::BC;
    constexpr int KB = BC / 32;        // 32-key blocks per tile
    constexpr int DB = D / 32;         // 32-wide d blocks of the output
    constexpr int KSTEPS = D / 16;     // contraction steps of S

    __shared__ __attribute__((aligned(16))) char smem_raw[2 * T::STAGE];
    LDS char* smem = (LDS char*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;           // lane half
    const int l32 = lane & 31;

    // Work decomposition.  Workgroups are dealt round-robin to the 8 XCDs
    // (w % 8); give each XCD a contiguous range of heads so that the query
    // tiles sharing one K/V head (and a GQA group) share that XCD's L2.
    // Causal tiles run heaviest (latest) first.
    int bh, qt;
    {
        const int w = blockIdx.x;
        if ((bh_total & 7) == 0) {
            const int slot = w >> 3;
            bh = (w & 7) * (bh_total >> 3) + slot / n_qtiles;
            qt = slot % n_qtiles;
        } else {
            bh = w / n_qtiles;
            qt = w % n_qtiles;
        }
        if (CAUSAL) qt = n_qtiles - 1 - qt;
    }
    const size_t q_head = (size_t)bh * N * D;
    const size_t kv_head = (size_t)(bh / group) * N * D;
    const int q0 = qt * kBr;
    const int wq0 = q0 + wave * kWaveRows;    // first query row of this wave
    const int my_row = wq0 + l32;             // the query row this lane owns

    // Q fragments: B operand of S^T = K Q^T, lane holds d = 16*ks + 8*h .. +7.
    bf16x8 qf[KSTEPS];
    {
        const u32x4* qp = (const u32x4*)(Q + q_head + (size_t)(my_row < N ? my_row : N - 1) * D);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            u32x4 x = qp[2 * ks + h];
            if (my_row >= N) x = (u32x4){0u, 0u, 0u, 0u};
            x ^= qsign;
            qf[ks] = __builtin_bit_cast(bf16x8, x);
        }
    }

    const int kv_end = CAUSAL ? min(N, q0 + kBr) : N;       // keys this workgroup needs
    const int n_tiles = (kv_end + BC - 1) / BC;
    const int w_kv_end = CAUSAL ? min(N, wq0 + kWaveRows) : N;
    const int w_tiles = (wq0 < N) ? (w_kv_end + BC - 1) / BC : 0;   // tiles this wave computes

    const u32x4* kg = (const u32x4*)(K + kv_head);
    const u32x4* vg = (const u32x4*)(V + kv_head);

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = (f32x16){};
    float m_run = -__builtin_inff();   // running max of S*c (log2 domain)
    float l_run = 0.f;                 // this lane's share of the running sum

    u32x4 kr[T::CHUNKS_PER_THREAD], vr[T::CHUNKS_PER_THREAD];
    load_kv<D>(kg, vg, 0, N, tid, kr, vr);
    store_kv<D>(smem, tid, kr, vr);
    __syncthreads();

    // lane-constant parts of the V transpose-read address
    const int v_row_lane = 4 * h + ((lane & 15) >> 2);
    const int v_col_lane = 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));

    for (int j = 0; j < n_tiles; ++j) {
        const bool more = j + 1 < n_tiles;
        if (more) load_kv<D>(kg, vg, (j + 1) * BC, N, tid, kr, vr);

        if (j < w_tiles) {
            LDS char* kl = smem + (j & 1) * T::STAGE;
            LDS char* vl = kl + T::KBYTES;

            f32x16 s[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) s[kb] = (f32x16){};
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const bf16x8 a = *(LDS bf16x8*)(kl + (32 * kb + l32) * T::KPITCH + (16 * ks + 8 * h) * 2);
                    s[kb] = mfma32(a, qf[ks], s[kb]);
                }
            }

            // Accumulator register 4g+r of block kb holds key 32kb + 8g + 4h + r.
            const int key0 = j * BC;
            const bool need_mask = (key0 + BC > N) || (CAUSAL && key0 + BC - 1 > wq0);
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = key0 + 32 * kb + 8 * (i >> 2) + 4 * h + (i & 3);
                        const bool dead = key >= N || (CAUSAL && key > my_row);
                        if (dead) s[kb][i] = -__builtin_inff();
                    }
                }
            }

            float mx = s[0][0];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
            mx = half_swap_max(mx);
            const float m_new = fmaxf(m_run, mx * c_log2);
            const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);

            float psum = 0.f;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][i], c_log2, -m_use));
                    s[kb][i] = p;
                    psum += p;
                }
            l_run = fmaf(l_run, alpha, psum);
            m_run = m_new;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;

#pragma unroll
            for (int cc = 0; cc < BC / 16; ++cc) {
                bf16x8 pb;
#pragma unroll
                for (int t = 0; t < 8; ++t) pb[t] = (__bf16)s[cc >> 1][8 * (cc & 1) + t];
                LDS char* vrow = vl + (16 * cc + v_row_lane) * T::VPITCH + v_col_lane;
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)(vrow + 64 * db));
                    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)(vrow + 8 * T::VPITCH + 64 * db));
                    const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    oacc[db] = mfma32(a, pb, oacc[db]);
                }
            }
        }

        if (more) store_kv<D>(smem + ((j + 1) & 1) * T::STAGE, tid, kr, vr);
        __syncthreads();
    }

    if (wq0 >= N) return;
    const float l_tot = half_swap_sum(l_run);
    if (my_row >= N) return;
    const float inv = 1.f / l_tot;
    __bf16* op = O + q_head + (size_t)my_row * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            bf16x4 out;
#pragma unroll
            for (int r = 0; r < 4; ++r) out[r] = (__bf16)(oacc[db][4 * g + r] * inv);
            *(bf16x4*)(op + 32 * db + 8 * g + 4 * h) = out;
        }
    }
    if (h == 0) LSE[(size_t)bh * N + my_row] = (m_run + __builtin_log2f(l_tot)) * 0.69314718055994531f;
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
    const int n_qtiles = (a.N + kBr - 1) / kBr;
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
    void* args[] = {&q, &k, &v, &o, &lse, &group, &N, (void*)&n_qtiles, (void*)&bh_total, &c_log2, &qsign};
    return hipLaunchKernel((const void*)fwd_bf16_kernel<D, CAUSAL>, dim3(bh_total * n_qtiles),
                           dim3(kThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
    if (a.d == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
    return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

}  // namespace fa
