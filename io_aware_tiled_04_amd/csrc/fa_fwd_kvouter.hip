// Attention forward in the K/V-outer loop order, bf16, for gfx950: the loop
// order the reading-notes page describes (Methods: K and V read from HBM once,
// Q, O, l and m read and written block by block), kept as a measured
// alternative to the query-outer hot path.
//
// One workgroup per (batch, head).  For each 64-key tile j (outer loop) the
// workgroup loads K_j and V_j into LDS once; its 8 waves then sweep the
// 32-row query blocks (inner loop, block rb on wave rb mod 8).  Per (block,
// tile) pair a wave reads Q_rb, the running output accumulator O_rb and the
// row statistics m, l from HBM, applies the reading-notes page's two
// rescaling equations (Methods) with the tile's exact row max, and writes
// O_rb, m and l back; at the last tile a block sees it writes O / l (bf16)
// and LSE = m + ln l instead.  K and V are read once per head; Q, O, m and l
// once per visible (block, tile) pair, which is the traffic this order costs.
//
// Arithmetic and operand layouts are those of the query-outer kernel: S^T =
// K Q^T with one query per lane (MFMA 32x32x16 bf16), P rounded to bf16 after
// the fp32 row sum, O^T += V^T P^T with V^T key-permuted in LDS.  The
// accumulator state lives in the caller's workspace in the MFMA register
// layout (per block: lane-major float4 chunks), so every wave load and store
// of it is a contiguous 1 KiB.
#include "fa_kernels.h"

#include <stdint.h>

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LDS __attribute__((address_space(3)))

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBlk = 32;      // query rows per block (one wave)
constexpr int kBc = 64;       // keys per tile
static_assert(kBc == kKeyTileBf16, "key tile of the K/V-outer kernel");

template <int D>
struct KvLay {
    static constexpr int KPITCH = 2 * D + 16;
    static constexpr int VPITCH = 2 * kBc + 16;
    static constexpr int K0 = 0;
    static constexpr int V0 = kBc * KPITCH;
    static constexpr int BYTES = V0 + D * VPITCH;
    static constexpr int CHUNKS = D / 8;
};

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float swap_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Key k of a tile at its permuted place in a V^T row (the query-outer
// kernel's order: P^T's accumulator registers are then the MFMA operand).
__device__ __forceinline__ int vt_pos(int k) {
    return (k & ~15) | ((k & 4) << 1) | ((k & 8) >> 1) | (k & 3);
}

// Workspace per (head, block): the O^T accumulator as 64 lanes x D/2 floats
// (float4 chunk (db, g) of lane l at ((db*4 + g)*64 + l)), then m and l, one
// float per lane each.
template <int D>
struct KvWs {
    static constexpr int O_FLOATS = 64 * (D / 2);
    static constexpr int PER_BLOCK = O_FLOATS + 128;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd_kvouter_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, float* __restrict__ LSE, float* __restrict__ WS, int group, int N,
    float c_log2, uint32_t qsign) {
    using L = KvLay<D>;
    constexpr int DB = D / 32;
    constexpr int KS = D / 16;

    __shared__ __attribute__((aligned(16))) char smem_raw[L::BYTES];
    LDS char* smem = (LDS char*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;
    const int l32 = lane & 31;
    const int bh = blockIdx.x;
    const int nblk = (N + kBlk - 1) / kBlk;
    const int ntile = (N + kBc - 1) / kBc;

    const __bf16* qh = Q + (size_t)bh * N * D;
    const __bf16* kh = K + (size_t)(bh / group) * N * D;
    const __bf16* vh = V + (size_t)(bh / group) * N * D;
    float* wsh = WS + (size_t)bh * nblk * KvWs<D>::PER_BLOCK;

#pragma unroll 1
    for (int j = 0; j < ntile; ++j) {
        const int key0 = j * kBc;
        // K_j row-major and V_j transposed into LDS, once per head (rows past
        // N repeat row N-1: their keys are masked, and V must stay finite).
        for (int u = tid; u < kBc * L::CHUNKS; u += kThreads) {
            const int r = u / L::CHUNKS, c8 = u % L::CHUNKS;
            const int row = min(key0 + r, N - 1);
            const u32x4 kx = *(const u32x4*)(kh + (size_t)row * D + 8 * c8);
            *(LDS u32x4*)(smem + L::K0 + r * L::KPITCH + 16 * c8) = kx;
            const bf16x8 vx = *(const bf16x8*)(vh + (size_t)row * D + 8 * c8);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                *(LDS __bf16*)(smem + L::V0 + (8 * c8 + e) * L::VPITCH + 2 * vt_pos(r)) = vx[e];
        }
        __syncthreads();

        // the query blocks that see some key of tile j
        const int rb_first = CAUSAL ? key0 / kBlk : 0;
#pragma unroll 1
        for (int rb = wave; rb < nblk; rb += kWaves) {
            if (rb < rb_first) continue;
            const int q0 = rb * kBlk;
            const int my_row = q0 + l32;
            // last tile this block sees: it finalises there
            const int j_last = CAUSAL ? min(ntile - 1, (min(N, q0 + kBlk) - 1) / kBc) : ntile - 1;

            bf16x8 qf[KS];
            {
                const u32x4* qp = (const u32x4*)(qh + (size_t)min(my_row, N - 1) * D);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    u32x4 x = qp[2 * ks + h];
                    if (my_row >= N) x = (u32x4){0u, 0u, 0u, 0u};
                    x ^= qsign;
                    qf[ks] = __builtin_bit_cast(bf16x8, x);
                }
            }
            f32x16 s[2];
            s[0] = (f32x16){};
            s[1] = (f32x16){};
            const LDS char* krow = smem + L::K0 + l32 * L::KPITCH + 16 * h;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    s[kb] = mfma32(*(const LDS bf16x8*)(krow + 32 * kb * L::KPITCH + 32 * ks), qf[ks], s[kb]);

            // mask: register i of block kb is key key0 + 32kb + 8(i/4) + 4h + i%4
            if (key0 + kBc > N || (CAUSAL && key0 + kBc - 1 > q0)) {
                int lim = (CAUSAL ? min(N, my_row + 1) : N) - key0 - 4 * h;
                // (opaque, so that 32 per-lane limits are not hoisted out of
                // the loops when the limit does not depend on the row)
                asm volatile("" : "+v"(lim));
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (32 * kb + 8 * (i >> 2) + (i & 3) >= lim) s[kb][i] = -__builtin_inff();
            }

            // running state of the block
            float* ob = wsh + (size_t)rb * KvWs<D>::PER_BLOCK;
            f32x16 oacc[DB];
            float m_run = -__builtin_inff(), l_run = 0.f;
            if (j == 0) {
#pragma unroll
                for (int db = 0; db < DB; ++db) oacc[db] = (f32x16){};
            } else {
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const float4 x = *(const float4*)(ob + ((db * 4 + g) * 64 + lane) * 4);
                        oacc[db][4 * g] = x.x;
                        oacc[db][4 * g + 1] = x.y;
                        oacc[db][4 * g + 2] = x.z;
                        oacc[db][4 * g + 3] = x.w;
                    }
                m_run = ob[KvWs<D>::O_FLOATS + lane];
                l_run = ob[KvWs<D>::O_FLOATS + 64 + lane];
            }

            // the reading-notes page's rescaling with the tile's exact row max
            float mx = -__builtin_inff();
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
            const float m_new = fmaxf(m_run, swap_max(mx) * c_log2);
            const float m_use = m_new == -__builtin_inff() ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
            bf16x8 pb[4];
            float ps = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][i], c_log2, -m_use));
                    ps += p;
                    pb[2 * kb + (i >> 3)][i & 7] = (__bf16)p;
                }
            l_run = l_run * alpha + ps;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
            const LDS char* vrow = smem + L::V0 + l32 * L::VPITCH + 16 * h;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc)
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    oacc[db] = mfma32(*(const LDS bf16x8*)(vrow + 32 * db * L::VPITCH + 32 * cc), pb[cc], oacc[db]);

            if (j == j_last) {
                const float l_tot = swap_sum(l_run);
                if (my_row < N) {
                    const float inv = 1.f / l_tot;
                    __bf16* op = O + (size_t)bh * N * D + (size_t)my_row * D;
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            bf16x4 out;
#pragma unroll
                            for (int r = 0; r < 4; ++r) out[r] = (__bf16)(oacc[db][4 * g + r] * inv);
                            *(bf16x4*)(op + 32 * db + 8 * g + 4 * h) = out;
                        }
                    if (h == 0) LSE[(size_t)bh * N + my_row] = (m_use + __builtin_log2f(l_tot)) * 0.69314718055994531f;
                }
            } else {
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        *(float4*)(ob + ((db * 4 + g) * 64 + lane) * 4) =
                            make_float4(oacc[db][4 * g], oacc[db][4 * g + 1], oacc[db][4 * g + 2],
                                        oacc[db][4 * g + 3]);
                ob[KvWs<D>::O_FLOATS + lane] = m_use;
                ob[KvWs<D>::O_FLOATS + 64 + lane] = l_run;
            }
        }
        __syncthreads();   // K_j and V_j stay until every wave is done with them
    }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, float* ws, hipStream_t stream) {
    float c_log2 = fabsf(a.scale) * 1.4426950408889634f;
    if (!(c_log2 >= 1e-30f)) c_log2 = 1e-30f;
    uint32_t qsign = a.scale < 0.f ? 0x80008000u : 0u;
    int group = a.Hq / a.Hkv;
    int N = a.N;
    const __bf16* q = (const __bf16*)a.q;
    const __bf16* k = (const __bf16*)a.k;
    const __bf16* v = (const __bf16*)a.v;
    __bf16* o = (__bf16*)a.o;
    float* lse = a.lse;
    void* args[] = {&q, &k, &v, &o, &lse, &ws, &group, &N, &c_log2, &qsign};
    return hipLaunchKernel((const void*)fwd_kvouter_kernel<D, CAUSAL>, dim3(a.B * a.Hq), dim3(kThreads), args, 0,
                           stream);
}

}  // namespace

long long kvouter_workspace_floats(long long B, long long Hq, long long N, long long d) {
    return B * Hq * ((N + kBlk - 1) / kBlk) * (64 * (d / 2) + 128);
}

hipError_t launch_fwd_bf16_kvouter(const FwdArgs& a, float* workspace, hipStream_t stream) {
    if (a.d == 128)
        return a.causal ? launch<128, true>(a, workspace, stream) : launch<128, false>(a, workspace, stream);
    return a.causal ? launch<64, true>(a, workspace, stream) : launch<64, false>(a, workspace, stream);
}

}  // namespace fa
