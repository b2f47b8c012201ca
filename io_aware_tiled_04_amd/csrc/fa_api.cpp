// C ABI entry points: argument validation, instance dispatch and launch.
// Validation runs before any HIP call, so a rejected call touches neither the
// device nor the outputs.
#include "fa.h"

#include <climits>
#include <cstdint>
#include <cmath>

#include "fa_kernels.h"

namespace {

int validate(const void* q, const void* k, const void* v, const void* o, const void* lse, int B,
             int Hq, int Hkv, int N, int d, float scale) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || N > fa::kMaxSeqLen) return FA_ERR_SHAPE;
    // Every grid must fit one launch dimension (the fp32 kernel has the
    // smallest query tile), and every tensor must be indexable in 64 bits
    // with room to spare (elements < 2^50).
    const long long bh = (long long)B * Hq;
    const long long tiles = ((long long)N + fa::kBlockRowsF32 - 1) / fa::kBlockRowsF32;
    if (bh > INT_MAX || bh * tiles > INT_MAX) return FA_ERR_SHAPE;
    if ((double)bh * (double)N * 128.0 >= 1125899906842624.0) return FA_ERR_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_HEADS;
    if (d != 64 && d != 128) return FA_ERR_HEADDIM;
    if (!std::isfinite(scale)) return FA_ERR_ARG;
    // the kernels move whole 16-byte pieces of rows
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) return FA_ERR_ALIGN;
    if ((uintptr_t)lse & 3) return FA_ERR_ALIGN;
    return FA_OK;
}

fa::FwdArgs pack(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                 int Hkv, int N, int d, int causal, float scale) {
    fa::FwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.N = N;
    a.d = d;
    a.causal = causal != 0;
    a.scale = scale;
    return a;
}

}  // namespace

extern "C" int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int Hq, int Hkv, int N, int d, int causal, float scale, hipStream_t stream) {
    const int rc = validate(q, k, v, o, lse, B, Hq, Hkv, N, d, scale);
    if (rc != FA_OK) return rc;
    const hipError_t e =
        fa::launch_fwd_bf16(pack(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale), stream);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                          hipStream_t stream) {
    const int rc = validate(q, k, v, o, lse, B, Hq, Hkv, N, d, scale);
    if (rc != FA_OK) return rc;
    const hipError_t e =
        fa::launch_fwd_f32(pack(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale), stream);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

namespace {

// Dropout parameters: 0 <= p < 1; t = floor(p * 2^16) (exact in double).
int make_dropout(float p, unsigned long long seed, unsigned int offset, fa::Dropout* dr) {
    if (!(p >= 0.f && p < 1.f)) return FA_ERR_ARG;
    const uint32_t t = (uint32_t)std::floor((double)p * 65536.0);
    dr->k0 = (uint32_t)(seed & 0xFFFFFFFFull);
    dr->k1 = (uint32_t)(seed >> 32);
    dr->offset = offset;
    dr->t2 = t | (t << 16);
    dr->factor = 1.f / (1.f - p);
    return FA_OK;
}

}  // namespace

extern "C" int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                              int Hq, int Hkv, int N, int d, int causal, float scale, float p_drop,
                              unsigned long long seed, unsigned int offset, hipStream_t stream) {
    int rc = validate(q, k, v, o, lse, B, Hq, Hkv, N, d, scale);
    if (rc != FA_OK) return rc;
    fa::Dropout dr;
    rc = make_dropout(p_drop, seed, offset, &dr);
    if (rc != FA_OK) return rc;
    const fa::FwdArgs a = pack(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale);
    // p = 0 keeps every weight with factor 1: the plain kernel computes exactly that.
    const hipError_t e = p_drop == 0.f ? fa::launch_fwd_bf16(a, stream) : fa::launch_fwd_bf16_dropout(a, dr, stream);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

namespace {

// Split count and workspace checks of the split-KV entry point (after the
// common validation).
int validate_split(int B, int Hq, int N, int d, int num_splits, const void* workspace,
                   size_t workspace_bytes) {
    if (num_splits < 1 || num_splits > fa::kMaxSplits) return FA_ERR_ARG;
    const long long bh = (long long)B * Hq;
    const long long qtiles = ((long long)N + fa::kBlockRowsBf16 - 1) / fa::kBlockRowsBf16;
    if (bh * qtiles * num_splits > INT_MAX) return FA_ERR_SHAPE;
    // the split kernels store float4 values into the workspace
    if (!workspace || ((uintptr_t)workspace & 15) != 0) return FA_ERR_WORKSPACE;
    const long long need = fa::split_workspace_floats(B, Hq, N, d, num_splits) * 4;
    if ((unsigned long long)need > (unsigned long long)workspace_bytes) return FA_ERR_WORKSPACE;
    return FA_OK;
}

}  // namespace

extern "C" size_t fa_fwd_splitkv_workspace_size(int B, int Hq, int N, int d, int num_splits) {
    if (B <= 0 || Hq <= 0 || N <= 0 || (d != 64 && d != 128)) return 0;
    if (num_splits < 1 || num_splits > fa::kMaxSplits) return 0;
    if ((double)B * Hq * (double)N * 128.0 >= 1125899906842624.0) return 0;
    return (size_t)fa::split_workspace_floats(B, Hq, N, d, num_splits) * 4;
}

extern "C" int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                              int num_splits, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
    int rc = validate(q, k, v, o, lse, B, Hq, Hkv, N, d, scale);
    if (rc != FA_OK) return rc;
    rc = validate_split(B, Hq, N, d, num_splits, workspace, workspace_bytes);
    if (rc != FA_OK) return rc;
    const hipError_t e = fa::launch_fwd_bf16_split(pack(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale),
                                                   num_splits, (float*)workspace, stream);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                      int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                                      int num_splits, hipStream_t stream) {
    int rc = validate(q, k, v, o, lse, B, Hq, Hkv, N, d, scale);
    if (rc != FA_OK) return rc;
    if (num_splits < 1 || num_splits > fa::kMaxSplits) return FA_ERR_ARG;
    const long long need = fa::split_workspace_floats(B, Hq, N, d, num_splits) * 4;
    if (need > (long long)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
    // the split checks proper, with the scratch standing in for a workspace
    // (its address is 256-byte aligned, so a stand-in with that alignment
    // is checked here, before any HIP call)
    rc = validate_split(B, Hq, N, d, num_splits, (const void*)(uintptr_t)256, FA_NOALLOC_SCRATCH_BYTES);
    if (rc != FA_OK) return rc;
    float* ws = nullptr;
    if (fa::noalloc_scratch(&ws) != hipSuccess) return FA_ERR_HIP;
    const hipError_t e = fa::launch_fwd_bf16_split(pack(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale),
                                                   num_splits, ws, stream);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" size_t fa_fwd_kvouter_workspace_size(int B, int Hq, int N, int d) {
    if (B <= 0 || Hq <= 0 || N <= 0 || (d != 64 && d != 128)) return 0;
    if ((double)B * Hq * (double)N * 128.0 >= 1125899906842624.0) return 0;
    return (size_t)fa::kvouter_workspace_floats(B, Hq, N, d) * 4;
}

extern "C" int fa_fwd_kvouter(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                              int Hkv, int N, int d, int causal, float scale, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    const int rc = validate(q, k, v, o, lse, B, Hq, Hkv, N, d, scale);
    if (rc != FA_OK) return rc;
    if (!workspace || ((uintptr_t)workspace & 15) != 0) return FA_ERR_WORKSPACE;
    if ((unsigned long long)fa::kvouter_workspace_floats(B, Hq, N, d) * 4 > (unsigned long long)workspace_bytes)
        return FA_ERR_WORKSPACE;
    const hipError_t e = fa::launch_fwd_bf16_kvouter(pack(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale),
                                                     (float*)workspace, stream);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" size_t fa_bwd_workspace_size(int B, int Hq, int N) {
    if (B <= 0 || Hq <= 0 || N <= 0) return 0;
    if ((double)B * Hq * (double)N * 128.0 >= 1125899906842624.0) return 0;
    return (size_t)B * Hq * N * 4;
}

namespace {

// Validation and packing shared by the backward entry points.
int check_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
              void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N, int d, float scale,
              const void* workspace, size_t workspace_bytes) {
    if (!dout || !dq || !dk || !dv) return FA_ERR_NULL;
    const int rc = validate(q, k, v, o, lse, B, Hq, Hkv, N, d, scale);
    if (rc != FA_OK) return rc;
    if (((uintptr_t)dout | (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv) & 15) return FA_ERR_ALIGN;
    const long long bh = (long long)B * Hq;
    const long long rtiles = ((long long)N + fa::kBwdBlockRows - 1) / fa::kBwdBlockRows;
    if (bh * rtiles > INT_MAX) return FA_ERR_SHAPE;
    if (!workspace) return FA_ERR_WORKSPACE;
    if ((unsigned long long)B * Hq * N * 4 > (unsigned long long)workspace_bytes) return FA_ERR_WORKSPACE;
    return FA_OK;
}

fa::BwdArgs pack_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N, int d,
                     int causal, float scale) {
    fa::BwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.dO = dout;
    a.lse = lse;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.N = N;
    a.d = d;
    a.causal = causal != 0;
    a.scale = scale;
    return a;
}

}  // namespace

extern "C" int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N,
                      int d, int causal, float scale, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
    const int rc = check_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, scale, workspace,
                             workspace_bytes);
    if (rc != FA_OK) return rc;
    const hipError_t e = fa::launch_bwd_bf16(pack_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d,
                                                      causal, scale),
                                             (float*)workspace, stream);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N,
                              int d, int causal, float scale, float p_drop, unsigned long long seed,
                              unsigned int offset, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
    int rc = check_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, scale, workspace, workspace_bytes);
    if (rc != FA_OK) return rc;
    fa::Dropout dr;
    rc = make_dropout(p_drop, seed, offset, &dr);
    if (rc != FA_OK) return rc;
    const fa::BwdArgs a = pack_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, causal, scale);
    // p = 0: every weight kept with factor 1, the plain backward.
    const hipError_t e = p_drop == 0.f ? fa::launch_bwd_bf16(a, (float*)workspace, stream)
                                       : fa::launch_bwd_bf16_dropout(a, dr, (float*)workspace, stream);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" const char* fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "ok";
        case FA_ERR_NULL: return "null pointer argument";
        case FA_ERR_SHAPE: return "invalid shape (B, Hq, Hkv and N must be positive and the problem indexable)";
        case FA_ERR_HEADS: return "Hq must be a multiple of Hkv";
        case FA_ERR_HEADDIM: return "unsupported head size d (supported: 64, 128)";
        case FA_ERR_ARG: return "invalid scalar argument (scale must be finite, num_splits in 1..256, p_drop in [0, 1))";
        case FA_ERR_WORKSPACE: return "workspace is null, not 16-byte aligned or smaller than the size the entry point needs";
        case FA_ERR_SCRATCH: return "problem needs more than the 64 MiB fixed scratch of fa_fwd_splitkv_noalloc (use fewer splits or a workspace)";
        case FA_ERR_ALIGN: return "a tensor pointer is misaligned (16 bytes for q, k, v, o, dout, dq, dk, dv; 4 bytes for lse)";
        case FA_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}
