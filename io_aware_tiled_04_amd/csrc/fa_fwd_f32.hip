// Attention forward pass, fp32 inputs and arithmetic, for gfx950.
//
// Same method as the bf16 kernel (query tile resident, K/V tiles streamed
// through LDS, online rescale of the running sum and of the unnormalised
// output; reading-notes page, Methods, and the Polish notes' m / l / u state),
// with every product and sum in fp32 and no reduced-precision rounding.
// gfx950 has no reduced-precision fp32 matrix instruction, and this path
// serves small fp32 problems, so it uses plain vector FMA: one lane owns one
// query row (its q and unnormalised output stay in registers) and all lanes
// read the same K/V row from LDS (a broadcast, free of bank conflicts).
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kRows = kBlockRowsF32;   // query rows (lanes) per workgroup
constexpr int kTileKeys = 32;          // keys staged in LDS per step
constexpr int kSub = 16;               // keys per online update

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kRows) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int group, int N, int n_qtiles, float c_log2,
    float qsign) {
    __shared__ float ks[kTileKeys][D];
    __shared__ float vs[kTileKeys][D];

    const int bh = blockIdx.x / n_qtiles;
    const int qt = blockIdx.x % n_qtiles;
    const int t = threadIdx.x;
    const int row = qt * kRows + t;
    const size_t q_head = (size_t)bh * N * D;
    const size_t kv_head = (size_t)(bh / group) * N * D;

    float q[D], o[D];
    {
        const float* qp = Q + q_head + (size_t)(row < N ? row : N - 1) * D;
#pragma unroll
        for (int i = 0; i < D; ++i) {
            q[i] = row < N ? qp[i] * qsign : 0.f;
            o[i] = 0.f;
        }
    }
    float m_run = -__builtin_inff();
    float l_run = 0.f;

    const int kv_end = CAUSAL ? min(N, qt * kRows + kRows) : N;
    for (int key0 = 0; key0 < kv_end; key0 += kTileKeys) {
        __syncthreads();
        for (int e = t; e < kTileKeys * D; e += kRows) {
            const int r = e / D, col = e % D;
            const int key = key0 + r;
            ks[r][col] = key < N ? K[kv_head + (size_t)key * D + col] : 0.f;
            vs[r][col] = key < N ? V[kv_head + (size_t)key * D + col] : 0.f;
        }
        __syncthreads();
        for (int sb = 0; sb < kTileKeys; sb += kSub) {
            float s[kSub];
            float mx = -__builtin_inff();
#pragma unroll
            for (int jj = 0; jj < kSub; ++jj) {
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < D; ++i) acc = fmaf(q[i], ks[sb + jj][i], acc);
                const int key = key0 + sb + jj;
                const bool dead = key >= N || (CAUSAL && key > row);
                s[jj] = dead ? -__builtin_inff() : acc;
                mx = fmaxf(mx, s[jj]);
            }
            const float m_new = fmaxf(m_run, mx * c_log2);
            const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
            const float alpha = exp2f(m_run - m_use);
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < D; ++i) o[i] *= alpha;
#pragma unroll
            for (int jj = 0; jj < kSub; ++jj) {
                const float p = exp2f(fmaf(s[jj], c_log2, -m_use));
                l_run += p;
#pragma unroll
                for (int i = 0; i < D; ++i) o[i] = fmaf(p, vs[sb + jj][i], o[i]);
            }
            m_run = m_new;
        }
    }
    if (row >= N) return;
    const float inv = 1.f / l_run;
    float* op = O + q_head + (size_t)row * D;
#pragma unroll
    for (int i = 0; i < D; ++i) op[i] = o[i] * inv;
    LSE[(size_t)bh * N + row] = (m_run + log2f(l_run)) * 0.69314718055994531f;
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
    int n_qtiles = (a.N + kRows - 1) / kRows;
    float c_log2 = fabsf(a.scale) * 1.4426950408889634f;
    // zero scale: see the bf16 launcher (keeps masked -inf logits at -inf)
    if (!(c_log2 >= 1e-30f)) c_log2 = 1e-30f;
    float qsign = a.scale < 0.f ? -1.f : 1.f;
    int group = a.Hq / a.Hkv;
    int N = a.N;
    const float* q = (const float*)a.q;
    const float* k = (const float*)a.k;
    const float* v = (const float*)a.v;
    float* o = (float*)a.o;
    float* lse = a.lse;
    void* args[] = {&q, &k, &v, &o, &lse, &group, &N, &n_qtiles, &c_log2, &qsign};
    return hipLaunchKernel((const void*)fwd_f32_kernel<D, CAUSAL>, dim3(a.B * a.Hq * n_qtiles),
                           dim3(kRows), args, 0, stream);
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream) {
    if (a.d == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
    return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

}  // namespace fa
