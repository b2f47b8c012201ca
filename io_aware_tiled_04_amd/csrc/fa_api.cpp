// C ABI entry points: argument validation, instance dispatch and launch.
// Validation runs before any HIP call, so a rejected call touches neither the
// device nor the outputs.
#include "fa.h"

#include <climits>
#include <cmath>

#include "fa_kernels.h"

namespace {

int validate(const void* q, const void* k, const void* v, const void* o, const void* lse, int B,
             int Hq, int Hkv, int N, int d, float scale) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0) return FA_ERR_SHAPE;
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

extern "C" const char* fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "ok";
        case FA_ERR_NULL: return "null pointer argument";
        case FA_ERR_SHAPE: return "invalid shape (B, Hq, Hkv and N must be positive and the problem indexable)";
        case FA_ERR_HEADS: return "Hq must be a multiple of Hkv";
        case FA_ERR_HEADDIM: return "unsupported head size d (supported: 64, 128)";
        case FA_ERR_ARG: return "scale must be finite";
        case FA_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}
