/*
 * fa.h - C ABI of the FlashAttention forward pass for AMD Instinct MI355X
 * (gfx950).
 *
 * The operation is exact softmax attention, computed tile by tile so that the
 * N x N score and probability matrices never reach device memory:
 *
 *   O   = softmax(scale * Q K^T, masked) V
 *   LSE = ln sum_{j allowed} exp(scale * q_i . k_j)       (natural log, fp32)
 *
 * Sources for the definition (the three pages on FlashAttention):
 *  - the derivation blog ("Flash Attention介绍"), section 标准注意力 / 前向传播:
 *    O = Diag((exp(QK^T) (.) M) 1)^-1 (exp(QK^T) (.) M) V with M causal or
 *    absent (section 分块递推模式);
 *  - the reading-notes page, Background (S = QK^T, P = softmax(S), O = PV, per
 *    head, Q, K, V in R^{N x d}) and Methods (Q resident on chip, K/V read in
 *    blocks, running sum and output rescaled at each block);
 *  - the blog's backward section (comment under 梯度推导): the forward keeps
 *    the row max and row sum for the backward pass, delivered here as LSE;
 *  - the Polish notes, closing paragraph: grouped-query attention combines
 *    with the method (fewer K/V heads than query heads).
 *
 * Conventions shared by every entry point
 *  - Layout: q and o are [B, Hq, N, d], k and v are [B, Hkv, N, d], all
 *    contiguous row-major; lse is [B, Hq, N] float32.  Queries and keys have
 *    the same length N.  There are no stride arguments.
 *  - Grouped-query attention: query head hq reads K/V head hq / (Hq / Hkv)
 *    (contiguous groups); Hq must be a multiple of Hkv.  Hkv == Hq is plain
 *    multi-head attention.
 *  - causal != 0: key j is visible to query i iff j <= i.  Masked pairs get
 *    weight exactly zero.  Every query sees at least key 0, so no row is empty.
 *  - scale multiplies Q K^T before the mask and the softmax; any finite value
 *    (negative and zero included).  Results are finite as long as
 *    |scale * q_i . k_j| stays below about 1e38.
 *  - All pointers are device pointers (hipMalloc'd or equivalent), owned by the
 *    caller; the library allocates nothing, frees nothing and keeps no state
 *    between calls, so it is reentrant and thread-safe.  Outputs must not
 *    alias inputs.
 *  - Asynchronous: the work is enqueued on `stream` (NULL = the default
 *    stream) and the call returns without synchronising.  The caller orders
 *    and synchronises as for any kernel launch.
 *  - Errors: arguments are validated before any HIP call; on a validation
 *    error nothing is launched and the outputs are untouched.  FA_ERR_HIP
 *    reports a launch failure (for example no gfx950 device).  Faults inside
 *    the kernel surface on the caller's next synchronising HIP call.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fa_status {
    FA_OK = 0,
    FA_ERR_NULL = -1,      /* a null pointer argument (lse included) */
    FA_ERR_SHAPE = -2,     /* B, Hq, Hkv or N <= 0, N > 2^23, or the problem is too large to index */
    FA_ERR_HEADS = -3,     /* Hq is not a multiple of Hkv */
    FA_ERR_HEADDIM = -4,   /* d is not one of the supported head sizes (64, 128) */
    FA_ERR_ARG = -5,       /* scale is not finite, num_splits or p_drop is out of range */
    FA_ERR_HIP = -6,       /* the HIP runtime rejected the launch */
    FA_ERR_WORKSPACE = -7, /* a workspace argument is null, misaligned or too small */
    FA_ERR_SCRATCH = -8,   /* the problem needs more than the fixed scratch of fa_fwd_splitkv_noalloc */
    FA_ERR_ALIGN = -9      /* a tensor pointer is misaligned: 16 bytes for q, k, v, o, dout, dq, dk, dv; 4 for lse */
};

/* Bytes of the fixed device scratch array of fa_fwd_splitkv_noalloc (64 MiB). */
#define FA_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * fa_fwd - attention forward pass on bfloat16 inputs (the hot path).
 *
 * q [B,Hq,N,d], k [B,Hkv,N,d], v [B,Hkv,N,d]: bfloat16 device pointers.
 * o [B,Hq,N,d]: bfloat16 device pointer, written with O rounded to nearest
 *   even from its fp32 value.
 * lse [B,Hq,N]: float32 device pointer, written with the natural-log
 *   logsumexp of the scaled, masked scores of each query row.
 * q, k, v and o must be 16-byte aligned (the kernels move whole 16-byte
 * pieces of rows) and lse 4-byte aligned, or the call returns FA_ERR_ALIGN;
 * the same holds for every entry point below (fp32 tensors included).
 * d in {64, 128}; N >= 1 (any length; partial tiles are masked).
 * Products Q K^T and P V run on bf16 matrix cores with fp32 accumulation; the
 * softmax state (row max, row sums, output accumulator) is fp32.  The
 * logsumexp takes the row sum of the fp32 weights; O is divided by the row
 * sum of the same weights rounded to bf16, the values that enter P V.
 * Returns FA_OK or a negative fa_status.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Hq, int Hkv, int N, int d, int causal, float scale,
           hipStream_t stream);

/*
 * fa_fwd_f32 - the same operation on float32 inputs and output, with fp32
 * arithmetic throughout (no reduced-precision rounding of P or O).
 * Arguments, layouts, errors and stream behaviour as for fa_fwd.
 */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
               int B, int Hq, int Hkv, int N, int d, int causal, float scale,
               hipStream_t stream);

/*
 * fa_fwd_splitkv_workspace_size - bytes of device workspace that
 * fa_fwd_splitkv needs for these sizes: num_splits * B * Hq * N * (d + 1) * 4
 * (a float32 partial output and a float32 partial logsumexp per split and
 * query row).  Returns 0 for arguments that fa_fwd_splitkv would reject
 * (non-positive sizes, d not in {64, 128}, num_splits outside 1..256).
 */
size_t fa_fwd_splitkv_workspace_size(int B, int Hq, int N, int d, int num_splits);

/*
 * fa_fwd_splitkv - the result of fa_fwd (same o and lse, up to float
 * rounding order), computed as num_splits independent passes over disjoint
 * ranges of the keys followed by a merge.  This is the per-block rescaling
 * of the reading-notes page (Methods, the two rescaling equations) applied
 * to whole key ranges: each pass produces a partial output O_s (normalised by
 * its own row sum) and a partial logsumexp LSE_s, and the merge forms
 * LSE = ln sum_s exp(LSE_s) and O = sum_s exp(LSE_s - LSE) O_s.  More passes
 * give more independent workgroups, which fills the GPU when B * Hq * N is
 * small.
 *
 * Arguments q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, stream: as for
 *   fa_fwd (bf16 inputs and output, float32 lse).
 * num_splits: 1..256.  The keys are cut into T = ceil(N/BC) tiles of BC
 *   keys, the kernel's key tile: BC = 64 at d = 128 and BC = 128 at d = 64.
 *   The splits take consecutive ranges of them: with q = T / num_splits and
 *   r = T % num_splits, the first r splits take q + 1 tiles and the others
 *   q.  More splits than tiles leave some ranges empty, which is allowed.
 * workspace: device memory of at least workspace_bytes bytes, owned by the
 *   caller, 16-byte aligned; workspace_bytes must be at least
 *   fa_fwd_splitkv_workspace_size(B, Hq, N, d, num_splits).  Its contents on
 *   entry do not matter and are overwritten; it must not be used by another
 *   call that runs at the same time.
 * Both kernels are enqueued on `stream`; the library allocates nothing.
 * Returns FA_OK or a negative fa_status (FA_ERR_ARG for num_splits,
 * FA_ERR_WORKSPACE for a null, misaligned or small workspace).
 */
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                   int num_splits, void* workspace, size_t workspace_bytes,
                   hipStream_t stream);

/*
 * fa_fwd_splitkv_noalloc - fa_fwd_splitkv without a workspace argument and
 * without any allocation, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).
 *
 * The split partials go to a fixed device array inside the library of
 * FA_NOALLOC_SCRATCH_BYTES bytes (64 MiB).  Each GPU the entry point runs on
 * gets its own copy on the first call there (the library looks up its
 * address once per device; that first call loads the array) and keeps it
 * until the process ends.  The call itself allocates and frees nothing.
 *
 * Arguments: as for fa_fwd_splitkv without workspace and workspace_bytes;
 * the result is fa_fwd_splitkv's, bit for bit, for the same num_splits.
 * Limit: fa_fwd_splitkv_workspace_size(B, Hq, N, d, num_splits) must not
 * exceed FA_NOALLOC_SCRATCH_BYTES; larger problems return FA_ERR_SCRATCH
 * before any HIP call (use fewer splits, or fa_fwd_splitkv with a caller
 * workspace).
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap in time on one GPU (two streams, two host
 * threads) race on it and may give wrong results.  Calls on one stream, or
 * otherwise ordered, are safe.  Nothing in the array needs to be cleared
 * between calls: the first kernel writes every partial the merge reads.
 * Returns FA_OK or a negative fa_status (FA_ERR_ARG for num_splits,
 * FA_ERR_SCRATCH for a problem too large for the array, FA_ERR_HIP if the
 * array's address cannot be obtained or a launch fails, otherwise as
 * fa_fwd).
 */
int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                           int num_splits, hipStream_t stream);

/*
 * fa_fwd_dropout - fa_fwd with dropout on the attention weights.
 *
 * The reading-notes page (section 其他算子) has dropout set attention weights
 * to zero at random with probability p and keep the random generator's
 * state for the backward pass.  Here:
 *   O   = (P (.) Z) V / (1 - p_drop),   LSE as for fa_fwd (before dropout),
 * with P the softmax weights of fa_fwd and Z_ij in {0, 1} drawn by
 * Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011), a counter-based
 * generator, so the whole state is (seed, offset):
 *   for head unit bh = b * Hq + hq, query row i and key
 *   j = 16a + 8b + 4c + w (b, c in {0, 1}, w in 0..3), the draw u_ij is the
 *   16-bit half number 4b + w (low half of output word 0 first) of the call
 *   at counter (2a + c, i, bh, offset) with key (seed mod 2^32, seed >> 32);
 *   Z_ij = 1 iff u_ij >= floor(p_drop * 2^16).
 * The keep probability is thus within 2^-16 of 1 - p_drop.  Passing the
 * same (seed, offset) to another call draws the same Z.
 *
 * Arguments q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, stream: as for
 *   fa_fwd.
 * p_drop: the drop probability, 0 <= p_drop < 1 (FA_ERR_ARG otherwise).
 *   p_drop = 0 gives exactly fa_fwd's result.
 * seed: 64-bit generator key.  offset: 32-bit stream number; calls with one
 *   seed that must draw independent masks use different offsets.
 * Returns FA_OK or a negative fa_status.
 */
int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                   float p_drop, unsigned long long seed, unsigned int offset,
                   hipStream_t stream);

/*
 * fa_fwd_kvouter_workspace_size - bytes of device workspace fa_fwd_kvouter
 * needs: B * Hq * ceil(N/32) * (32 * d + 128) * 4 (the running output, row
 * max and row sum of every 32-row query block, float32).  Returns 0 for
 * arguments fa_fwd_kvouter would reject.
 */
size_t fa_fwd_kvouter_workspace_size(int B, int Hq, int N, int d);

/*
 * fa_fwd_kvouter - the result of fa_fwd (same o and lse up to float rounding
 * order), computed in the loop order of the reading-notes page (Methods):
 * the K/V blocks are the outer loop, each read from HBM once per head, and
 * for every K/V block the query blocks read their Q, running output O and
 * row statistics m, l from device memory, apply the page's two rescaling
 * equations and write them back.  fa_fwd keeps the query block on chip
 * instead (the interchanged order).  This entry point exists to measure that
 * trade: one workgroup per (batch, head), and HBM traffic that grows with
 * N^2 / 64 instead of N.
 *
 * Arguments q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, stream: as for
 *   fa_fwd.
 * workspace: device memory of at least fa_fwd_kvouter_workspace_size(B, Hq,
 *   N, d) bytes, 16-byte aligned, owned by the caller; its contents on entry
 *   do not matter; it must not be shared with a call that runs at the same
 *   time.
 * Returns FA_OK or a negative fa_status (FA_ERR_WORKSPACE for a null,
 * misaligned or small workspace, otherwise as fa_fwd).
 */
int fa_fwd_kvouter(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fa_bwd_workspace_size - bytes of device workspace that fa_bwd needs:
 * B * Hq * N * 4 (one float32 per query row).  Returns 0 for non-positive
 * sizes.
 */
size_t fa_bwd_workspace_size(int B, int Hq, int N);

/*
 * fa_bwd - gradients of the attention forward pass (bfloat16), from its
 * saved output and logsumexp.
 *
 * The derivation blog's backward sections define the operation: the
 * standard attention backward (section 反向传播) gives
 *   dV = P^T dO,  dS = P (.) (dO V^T - D 1^T) with D_i = sum_d dO_id O_id,
 *   dQ = scale * dS K,  dK = scale * dS^T Q,
 * and its FlashAttention backward (section Flash Attention 反向传播, 梯度推导)
 * computes them without storing P: only the row statistics of the forward
 * are kept, here the logsumexp, and P = exp(scale * q_i . k_j - LSE_i) is
 * recomputed block by block.
 *
 * q, k, v, o, lse: exactly the inputs and outputs of a previous fa_fwd call
 *   with the same B, Hq, Hkv, N, d, causal and scale (o bf16 [B,Hq,N,d],
 *   lse float32 [B,Hq,N]).
 * dout [B,Hq,N,d]: bfloat16 upstream gradient dL/dO.
 * dq [B,Hq,N,d], dk [B,Hkv,N,d], dv [B,Hkv,N,d]: bfloat16 outputs, written
 *   (not accumulated into) with the gradients rounded to nearest even from
 *   fp32.  With GQA, dk and dv of a K/V head are the sums over the query
 *   heads of its group.
 * workspace: device memory of at least fa_bwd_workspace_size(B, Hq, N)
 *   bytes, owned by the caller, 4-byte aligned; its contents on entry do not
 *   matter; it must not be shared with a call that runs at the same time.
 * d in {64, 128}.  Products run on bf16 matrix cores with fp32 accumulation;
 * P and dS are rounded to bf16 for their products.
 * All work is enqueued on `stream`.  Returns FA_OK or a negative fa_status
 * (FA_ERR_NULL for any null pointer, FA_ERR_WORKSPACE for a null or small
 * workspace, otherwise as fa_fwd).
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv,
           int B, int Hq, int Hkv, int N, int d, int causal, float scale,
           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fa_bwd_dropout - gradients of an fa_fwd_dropout call.
 *
 * With W = P (.) Z / (1 - p_drop) the forward's output was O = W V, so
 *   dV = W^T dO,  dP = (dO V^T) (.) Z / (1 - p_drop),
 *   dS = P (.) (dP - D 1^T) with D_i = sum_d dO_id O_id,
 *   dQ = scale * dS K,  dK = scale * dS^T Q,
 * the backward of fa_bwd with the dropout factor in the chain rule; Z is
 * regenerated from (seed, offset), the generator state the reading-notes
 * page (section 其他算子) has the forward keep for the backward pass.
 *
 * Arguments: as for fa_bwd, with o and lse the outputs of the fa_fwd_dropout
 * call and p_drop, seed, offset exactly the values passed to it.
 * p_drop = 0 gives fa_bwd's result.  Returns FA_OK or a negative fa_status
 * (FA_ERR_ARG for p_drop outside [0, 1), otherwise as fa_bwd).
 */
int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv,
                   int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                   float p_drop, unsigned long long seed, unsigned int offset,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fa_status_string - a static, human-readable description of a status code
 * returned by the entry points above ("unknown status" for anything else).
 * The string is owned by the library and must not be freed.
 */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
