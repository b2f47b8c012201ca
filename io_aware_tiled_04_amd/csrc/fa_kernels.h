// Internal launchers of the attention forward kernels (not part of the C ABI).
// Arguments are validated by the caller (fa_api.cpp) before these run.
#pragma once
#include <hip/hip_runtime.h>

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

// Each returns hipSuccess or the launch error.
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);

// Query rows per workgroup of the bf16 kernel (the grid is B*Hq*ceil(N/kBlockRowsBf16)).
constexpr int kBlockRowsBf16 = 256;
// Query rows per workgroup of the fp32 kernel.
constexpr int kBlockRowsF32 = 64;

}  // namespace fa
