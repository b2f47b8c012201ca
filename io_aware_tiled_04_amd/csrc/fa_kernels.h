// Internal launchers of the attention forward kernels (not part of the C ABI).
// Arguments are validated by the caller (fa_api.cpp) before these run.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, Hq, Hkv, N, d;
    int causal;
    float scale;
};

// Arguments of the backward pass (validated by fa_api.cpp).
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dO;
    const float* lse;
    void* dq;
    void* dk;
    void* dv;
    int B, Hq, Hkv, N, d;
    int causal;
    float scale;
};

// Dropout on the attention weights: the Philox4x32-10 key (the seed), the
// call offset, the keep threshold t = floor(p * 2^16) in both 16-bit halves
// of t2, and the survivors' factor 1 / (1 - p).  The draws are defined in
// philox.h.
struct Dropout {
    uint32_t k0, k1;   // seed mod 2^32, seed >> 32
    uint32_t offset;
    uint32_t t2;       // t | t << 16
    float factor;      // 1 / (1 - p)
};

// Each returns hipSuccess or the launch error.
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
// Split-KV form of launch_fwd_bf16: partials of n_splits key ranges into
// `workspace` (float32, split_workspace_floats(...) elements), then a merge
// into a.o and a.lse.  Both kernels are enqueued on `stream`.
hipError_t launch_fwd_bf16_split(const FwdArgs& a, int n_splits, float* workspace, hipStream_t stream);
// launch_fwd_bf16 with dropout on the weights (the logsumexp is that of the
// weights before dropout).
hipError_t launch_fwd_bf16_dropout(const FwdArgs& a, const Dropout& dr, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);
// The forward in the K/V-outer loop order: one workgroup per (batch, head),
// the running O, m and l of each 32-row query block in `workspace` (float32,
// kvouter_workspace_floats(...) elements).
hipError_t launch_fwd_bf16_kvouter(const FwdArgs& a, float* workspace, hipStream_t stream);
long long kvouter_workspace_floats(long long B, long long Hq, long long N, long long d);
// Device address of the current device's fixed scratch array of the
// allocation-free split-KV entry point (FA_NOALLOC_SCRATCH_BYTES bytes),
// looked up on the first call on each device.
hipError_t noalloc_scratch(float** out);
// Backward pass: D = rowsum(dO * O) into `workspace` (B*Hq*N floats), then
// the dQ, dK and dV kernels, all enqueued on `stream`.
hipError_t launch_bwd_bf16(const BwdArgs& a, float* workspace, hipStream_t stream);
// launch_bwd_bf16 for a forward that ran with dropout `dr`.
hipError_t launch_bwd_bf16_dropout(const BwdArgs& a, const Dropout& dr, float* workspace, hipStream_t stream);

// Query rows per workgroup of the bf16 kernel (the grid is B*Hq*ceil(N/kBlockRowsBf16)).
constexpr int kBlockRowsBf16 = 256;
// Query rows per workgroup of the fp32 kernel.
constexpr int kBlockRowsF32 = 64;
// Longest sequence: the bf16 forward addresses one head's K or V (N * d * 2
// bytes) through buffer descriptors with 32-bit byte offsets.
constexpr int kMaxSeqLen = 1 << 23;
// Resident rows per workgroup of the backward kernels.
constexpr int kBwdBlockRows = 128;
// Keys per tile of the K/V-outer kernel (the bf16 forward's key tile at
// d = 128; at d = 64 the forward takes 128 keys per tile).
constexpr int kKeyTileBf16 = 64;
// Largest split count of the split-KV entry point.
constexpr int kMaxSplits = 256;

// float32 elements of the split-KV workspace: partial O then partial LSE.
inline long long split_workspace_floats(long long B, long long Hq, long long N, long long d,
                                        long long n_splits) {
    return n_splits * B * Hq * N * (d + 1);
}

}  // namespace fa
