/*
 * sana_linattn.h - C ABI of the ReLU linear self-attention forward pass
 * (Sana's Linear DiT block) for AMD Instinct MI355X (gfx950).
 *
 * The operation, per batch item b and head h, with x_n = x[b, n, h, :]:
 *
 *     phi(x)  = max(x, 0)
 *     KV      = sum_n phi(k_n) v_n^T            (d x d)
 *     ksum    = sum_n phi(k_n)                  (d)
 *     out_i   = phi(q_i) KV / (phi(q_i) . ksum + eps)
 *
 * Sources: Sana course notes (papers-3lj.pages.dev, "08 Sana 高效高分辨率
 * 生成"), section "Linear Attention 的原理" (phi = ReLU; KV = phi(K)^T V is a
 * d x d matrix whatever n is; A = phi(Q) KV); Linear-DiT 4K blog
 * (blog.hotdry.top), section "核心架构" (the normalised form
 * phi(Q)(phi(K)^T V) / (phi(Q) phi(K)^T 1)); Sana paper review
 * (phd-frog.tistory.com/40), section 2.2, "선형 어텐션 블럭" (ReLU linear
 * attention; the shared terms computed once and reused by every query).
 * eps is on no page: it is added to the denominator, outside the dot product.
 * Attention is non-causal except in the block-causal and token-causal entry
 * points below; no positional term touches q or k.
 *
 * Layout. q, k, v and out are dense, row-major [B][N][H][d] tensors of one
 * dtype: element (b, n, h, c) sits at index ((b*N + n)*H + h)*d + c. This is
 * the natural output layout of a (B, N, D = H*d) projection, so no transpose
 * is needed. bf16 in gives bf16 out (fp32 accumulation, round-to-nearest-even
 * on the final store); fp32 in gives fp32 out.
 *
 * The augmented state of one (b, h) is a d x (d+1) fp32 matrix, row-major:
 * state[c][j] = KV[c][j] for j < d and state[c][d] = ksum[c]. It is the
 * contraction phi(K)^T [V | 1]; its size does not depend on N.
 *
 * Ownership. Every pointer is a device pointer owned by the caller (q, k, v,
 * out, state, workspace). The library allocates no device memory and keeps no
 * per-call state. q, k and v are only read. out must not overlap q, k, v, the
 * state or the workspace, and a workspace must not overlap any tensor of the
 * call, inputs included (its partial results are written while other blocks
 * still read the inputs); a detected overlap returns SANA_ERR_INVALID_ARG.
 *
 * Streams. Every call enqueues its kernels on `stream` (NULL = the default
 * stream) and returns without synchronising. Results are defined once the
 * stream reaches that point. Calls that share a workspace must be ordered on
 * one stream.
 *
 * Graph capture. A call makes no allocation, copy, memset or synchronising
 * HIP call on its way to the launches, so it can be captured into a HIP
 * graph (make one ordinary call on the device first: the device's properties
 * are looked up once, on first use). A replay reads the captured pointers'
 * current contents and recomputes the result in full; replays that share a
 * workspace must not overlap in time. (On ROCm 7 a graph launch costs a few
 * microseconds more than the call's own launches, so capture pays only where
 * it removes host work.)
 *
 * Errors. Calls return a status code and never throw. All argument checks run
 * on the host before any HIP call, so an invalid call enqueues nothing. A
 * failed kernel launch returns SANA_ERR_HIP.
 *
 * Domain. B, N, H >= 1; d == 32 (other head widths return
 * SANA_ERR_UNSUPPORTED); B*N*H*d must fit in int64, every tensor must be
 * addressable (total bytes < 2^62) and B*ceil(H/2), the number of head pairs,
 * must be at most 2^22 (kernel grids over head pairs must stay within 2^32
 * work-items). eps must be finite and
 * >= 0; with
 * eps = 0 a query row with phi(q_i) = 0 gives 0/0 = NaN, otherwise such a row
 * gives exactly 0. Tensor pointers must be 16-byte aligned
 * (SANA_ERR_ALIGNMENT otherwise). Inputs must be finite.
 *
 * Language. The header is C99 as well as C++; from a C or C++ compiler other
 * than hipcc, define __HIP_PLATFORM_AMD__ (as hipcc does) so that
 * <hip/hip_runtime_api.h> declares hipStream_t and hipEvent_t, and link the
 * library (it brings its HIP runtime dependency with it).
 */
#ifndef SANA_LINATTN_H
#define SANA_LINATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SANA_LINATTN_VERSION 1

typedef enum {
  SANA_DTYPE_F32 = 0,  /* IEEE binary32 in and out */
  SANA_DTYPE_BF16 = 1  /* bfloat16 in and out, fp32 accumulation */
} sana_dtype_t;

typedef enum {
  SANA_OK = 0,
  SANA_ERR_INVALID_ARG = 1,  /* null pointer, size < 1, overflow, bad eps, overlap */
  SANA_ERR_UNSUPPORTED = 2,  /* d != 32, unknown dtype or variant */
  SANA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than the query says */
  SANA_ERR_ALIGNMENT = 4,    /* a tensor pointer is not 16-byte aligned */
  SANA_ERR_HIP = 5           /* a HIP launch failed */
} sana_status_t;

typedef enum {
  SANA_VARIANT_AUTO = 0,   /* by shape and device: SPLIT for N > 1024; for N <= 1024,
                              FUSED when N <= 512, or the call is tiny (P * N <= 4096 for
                              P = B * ceil(H/2) head pairs), or P * N >= CUs * 512 (P >= 128
                              at N = 1024 on MI355X's 256 CUs), SPLIT otherwise */
  SANA_VARIANT_SPLIT = 1,  /* two launches: split-N state reduction into per-block partials,
                              then the apply, which sums a head pair's partials in fixed
                              order (bf16); fp32 folds them at the end of the reduction */
  SANA_VARIANT_FUSED = 2   /* one launch, one block per (b, head pair): reduce into LDS,
                              then apply; for short sequences */
} sana_variant_t;

/* Feature maps phi for sana_linattn_fwd_fmap, sana_linattn_fwd_strided,
 * sana_linattn_bwd_fmap, sana_linattn_bwd_state and sana_linattn_kv_state_fmap
 * (Sana course notes, "Linear
 * Attention 的原理": ReLU, or another non-linear kernel such as ELU + 1 or
 * cos, chosen by a kernel-function parameter). Applied element by element. */
typedef enum {
  SANA_FMAP_RELU = 0,  /* max(x, 0): the forward of sana_linattn_fwd */
  SANA_FMAP_ELU1 = 1,  /* ELU(x) + 1, alpha = 1: x + 1 for x > 0, exp(x) otherwise */
  SANA_FMAP_COS = 2    /* cos(x); can be negative, so den + eps can vanish or turn
                          negative: the formula is evaluated as it stands */
} sana_fmap_t;

/*
 * Bytes of device workspace that sana_linattn_fwd, sana_linattn_fwd_variant
 * and sana_linattn_kv_state need for this shape. The size depends on
 * (B, N, H, d) only through the number of token chunks of the split
 * reduction, which stops growing once N is large: it is constant for N at
 * or above a fixed threshold (the state is independent of n). Every variant
 * uses at most this many bytes. Writes *bytes; returns SANA_OK or an
 * argument error (same checks as the forward call).
 */
sana_status_t sana_linattn_workspace_size(int64_t B, int64_t N, int64_t H, int64_t d,
                                          sana_dtype_t dtype, size_t* bytes);

/*
 * The forward pass: out = phi(Q)(phi(K)^T [V|1]) split into numerator and
 * normaliser, per (b, h). Equivalent to sana_linattn_fwd_variant with
 * SANA_VARIANT_AUTO. workspace must hold at least
 * sana_linattn_workspace_size(...) bytes (it may be NULL only when that size
 * is 0), be 256-byte aligned, and must not be used by another call in flight.
 * Its contents on entry do not matter (it needs no clearing, ever) and are
 * undefined on return.
 */
sana_status_t sana_linattn_fwd(const void* q, const void* k, const void* v, void* out,
                               int64_t B, int64_t N, int64_t H, int64_t d, float eps,
                               sana_dtype_t dtype, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the forward
 * pass of sana_linattn_fwd - same arguments, checks and result bits - with
 * its workspace in a static device array of SANA_LINATTN_SCRATCH_BYTES that
 * the library holds on each GPU it runs on until the process ends. The call
 * allocates nothing. A shape whose workspace (sana_linattn_workspace_size)
 * exceeds SANA_LINATTN_SCRATCH_BYTES returns SANA_ERR_WORKSPACE before any
 * HIP call. Every call on one GPU shares that GPU's array, and the array
 * keeps the last call's contents (the kernels need none of it cleared):
 * calls on one GPU that may run at the same time (different streams not
 * ordered against each other, or different host threads) race, so the
 * caller must order them. The first call on a device looks up the array's
 * device address there (SANA_ERR_HIP if that fails).
 */
#define SANA_LINATTN_SCRATCH_BYTES ((size_t)64 << 20)
sana_status_t sana_linattn_fwd_noalloc(const void* q, const void* k, const void* v, void* out,
                                       int64_t B, int64_t N, int64_t H, int64_t d, float eps,
                                       sana_dtype_t dtype, hipStream_t stream);

/*
 * Same as sana_linattn_fwd with an explicit kernel variant (sana_variant_t).
 * Every variant computes the same function; results of one variant are
 * bitwise repeatable for the same inputs and shape on the same device.
 */
sana_status_t sana_linattn_fwd_variant(const void* q, const void* k, const void* v, void* out,
                                       int64_t B, int64_t N, int64_t H, int64_t d, float eps,
                                       sana_dtype_t dtype, sana_variant_t variant, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream);

/*
 * sana_linattn_fwd_variant that also times its kernels: it records events[0]
 * on `stream` before the first kernel and events[i] right after kernel i, so
 * hipEventElapsedTime(events[i-1], events[i]) is the duration of kernel i.
 * The kernels, in order: SPLIT - the state reduction over token ranges,
 * then the apply (which, in bf16, also sums the reduction's partials); FUSED -
 * its single kernel; AUTO - those of the variant it picks. *n_kernels (if not
 * NULL) receives that count (2 or 1) whenever the shape, dtype and variant
 * are valid, even when the call fails otherwise. The events are created by the caller (hipEventCreate);
 * n_events must be at least *n_kernels + 1, else SANA_ERR_INVALID_ARG.
 * Computes exactly what sana_linattn_fwd_variant computes.
 */
sana_status_t sana_linattn_fwd_profiled(const void* q, const void* k, const void* v, void* out,
                                        int64_t B, int64_t N, int64_t H, int64_t d, float eps,
                                        sana_dtype_t dtype, sana_variant_t variant, void* workspace,
                                        size_t workspace_bytes, hipEvent_t* events,
                                        int n_events, int* n_kernels, hipStream_t stream);

/*
 * The forward pass with feature map `fmap` (sana_fmap_t) in place of ReLU:
 * out_i = phi(q_i) KV / (phi(q_i) . ksum + eps) with KV = phi(K)^T V and
 * ksum = phi(K)^T 1 (course notes, "Linear Attention 的原理", with the blog's
 * normalised form, "核心架构"). Same tensors, layout, dtypes, workspace
 * (sana_linattn_workspace_size), checks and errors as sana_linattn_fwd;
 * always the SPLIT kernels. SANA_FMAP_RELU computes exactly what
 * sana_linattn_fwd_variant(SPLIT) computes. In bf16, phi of ELU + 1 and cos
 * is evaluated in fp32 and split into bf16 hi + lo parts for the MFMAs. An
 * fmap outside sana_fmap_t returns SANA_ERR_UNSUPPORTED. events may be NULL;
 * otherwise n_events >= 3 and events[0..2] are recorded before the state
 * reduction, after it and after the apply (else SANA_ERR_INVALID_ARG).
 */
sana_status_t sana_linattn_fwd_fmap(const void* q, const void* k, const void* v, void* out,
                                    int64_t B, int64_t N, int64_t H, int64_t d, float eps,
                                    sana_dtype_t dtype, sana_fmap_t fmap, void* workspace, size_t workspace_bytes,
                                    hipEvent_t* events, int n_events, hipStream_t stream);

/*
 * The forward pass of sana_linattn_fwd_fmap on q, k and v read with a token
 * stride: element (b, n, h, c) of each is at index (b N + n) ld + h d + c
 * from its pointer. This reads the output of one fused QKV linear layer in
 * place (Sana review, section 4, projection and attention as one unit):
 * for a [B][N][3][H][d] tensor qkv, pass q = qkv, k = qkv + H d,
 * v = qkv + 2 H d and ld = 3 H d; ld = H d is the contiguous layout of
 * sana_linattn_fwd. out stays contiguous [B][N][H][d].
 *
 * ld: elements, >= H d (else SANA_ERR_INVALID_ARG); ld * element size must
 * be a multiple of 16 bytes (else SANA_ERR_ALIGNMENT), so every token row
 * stays 16-byte aligned. q, k and v may overlap each other (they are only
 * read); out must not overlap the (B N - 1) ld + H d elements any of them
 * spans, nor the workspace. Workspace (sana_linattn_workspace_size with the
 * same B, N, H, d, dtype), dtypes, fmap, events and the other checks and
 * errors as sana_linattn_fwd_fmap; always the SPLIT kernels. The result is
 * bitwise that of sana_linattn_fwd_fmap on contiguous copies of q, k, v.
 */
sana_status_t sana_linattn_fwd_strided(const void* q, const void* k, const void* v, int64_t ld,
                                       void* out, int64_t B, int64_t N, int64_t H, int64_t d,
                                       float eps, sana_dtype_t dtype, sana_fmap_t fmap, void* workspace,
                                       size_t workspace_bytes, hipEvent_t* events, int n_events,
                                       hipStream_t stream);

/*
 * QKV projection with the attention state in its epilogue, then the forward
 * pass (Sana review, section 4: the deployment kernels fold linear
 * attention's ReLU(K)^T V into the QKV projection layer). bf16 only.
 *
 *   [q | k | v] = x W^T, each rounded to bf16 (round to nearest even), then
 *   out = the forward of sana_linattn_fwd on (q, k, v).
 *
 * x:     [B][N][C] bf16 token features (device, read-only).
 * w_qkv: [3 D][C] bf16 weight, D = H d, the [out][in] layout of a linear
 *        layer without bias: rows 0..D-1 give q, D..2D-1 k, 2D..3D-1 v, head
 *        h at rows h d .. h d + d - 1 of each (device, read-only).
 * q:     [B][N][H][d] bf16, written: the projected, rounded q.
 * out:   [B][N][H][d] bf16, written.
 * k and v are never written to memory: the projection's blocks that compute
 * a head pair's k and v columns reduce them to that pair's state over their
 * 256 tokens (one fp32 partial state each, in the workspace), and the apply
 * sums a pair's partials in fixed order. The result equals, up to fp32
 * summation order, sana_linattn_fwd on the q, k, v an unfused bf16
 * projection would store.
 *
 * Domain: d == 32; 1 <= C < 2^22 and C % 8 == 0 (C % 8 != 0 returns
 * SANA_ERR_UNSUPPORTED);
 * B, N, H as for sana_linattn_fwd; x, w_qkv, q, out 16-byte aligned;
 * q and out must not overlap x, w_qkv, each other or the workspace. The
 * workspace (256-byte aligned, >= sana_linattn_qkv_workspace_size) needs no
 * clearing. events may be NULL; otherwise n_events >= 3 and events[0..2]
 * are recorded before the projection, after it and after the apply.
 * Checks run before any HIP call; a failed launch returns SANA_ERR_HIP.
 */
sana_status_t sana_linattn_qkv_workspace_size(int64_t B, int64_t N, int64_t C, int64_t H,
                                              int64_t d, size_t* bytes);
sana_status_t sana_linattn_qkv_fwd(const void* x, const void* w_qkv, void* q, void* out, int64_t B,
                                   int64_t N, int64_t C, int64_t H, int64_t d, float eps,
                                   void* workspace, size_t workspace_bytes, hipEvent_t* events,
                                   int n_events, hipStream_t stream);

/*
 * First half of the forward pass: the augmented state of every (b, h),
 * written to `state` as fp32 [B][H][d][d+1] (see the layout note above), by
 * a split-N reduction over token chunks and a fixed-order sum of the chunk
 * partials (deterministic, no float atomics). workspace as for
 * sana_linattn_fwd. The state is additive over tokens: states of disjoint
 * token ranges sum to the state of their union.
 */
sana_status_t sana_linattn_kv_state(const void* k, const void* v, float* state,
                                    int64_t B, int64_t N, int64_t H, int64_t d, sana_dtype_t dtype,
                                    void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/*
 * sana_linattn_kv_state with feature map `fmap` (sana_fmap_t) in place of
 * ReLU: KV = phi(K)^T V and ksum = phi(K)^T 1 of that map (in bf16, phi of
 * ELU + 1 and cos is evaluated in fp32 and split into bf16 hi + lo parts for
 * the MFMAs, as in sana_linattn_fwd_fmap). The state a training step keeps
 * for sana_linattn_bwd_state with the same map. Tensors, workspace, checks
 * and errors as sana_linattn_kv_state; an fmap outside sana_fmap_t returns
 * SANA_ERR_UNSUPPORTED. SANA_FMAP_RELU is sana_linattn_kv_state.
 */
sana_status_t sana_linattn_kv_state_fmap(const void* k, const void* v, float* state,
                                         int64_t B, int64_t N, int64_t H, int64_t d,
                                         sana_dtype_t dtype, sana_fmap_t fmap, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream);

/*
 * Second half of the forward pass: out_i = phi(q_i) KV / (phi(q_i) . ksum + eps)
 * for every token of every (b, h), reading `state` (fp32 [B][H][d][d+1], as
 * written by sana_linattn_kv_state or computed elsewhere, e.g. summed over
 * token shards). q and out as for sana_linattn_fwd. Needs no workspace.
 */
sana_status_t sana_linattn_apply(const void* q, const float* state, void* out,
                                 int64_t B, int64_t N, int64_t H, int64_t d, float eps,
                                 sana_dtype_t dtype, hipStream_t stream);

/* Bytes of one [B][H][d][d+1] fp32 state (0 and SANA_ERR_* on bad arguments). */
sana_status_t sana_linattn_state_size(int64_t B, int64_t H, int64_t d, size_t* bytes);

/*
 * Backward pass (bf16 only). Given g = dL/dout for the forward pass with the
 * same q, k, v and eps, writes dq = dL/dq, dk = dL/dk, dv = dL/dv, per (b, h):
 *
 *     dnum_i = g_i / den_i,   dden_i = -(g_i . out_i) / den_i
 *     dq_i   = (KV dnum_i + ksum dden_i) * [q_i > 0]
 *     dKV    = sum_i phi(q_i)^T dnum_i,    dksum = sum_i phi(q_i) dden_i
 *     dk_n   = (dKV v_n + dksum) * [k_n > 0],   dv_n = phi(k_n) dKV
 *
 * (with den_i = phi(q_i) . ksum + eps). These are the chain rule through the
 * forward definition; the Sana paper review, section 2.2 "Triton을 통한
 * 학습/추론 가속화", fuses this attention for training, which needs them, but
 * no page writes them out. The derivative of phi at exactly 0 is taken as 0.
 * The forward state is recomputed from k and v (one extra read of both).
 *
 * q, k, v, dout (read) and dq, dk, dv (written): dense [B][N][H][d] bf16,
 * 16-byte aligned; fp32 accumulation, round-to-nearest-even on the stores.
 * An output may not overlap another output, an input or the workspace
 * (SANA_ERR_INVALID_ARG); inputs may alias each other. workspace: at least
 * sana_linattn_bwd_workspace_size(...) bytes, 256-byte aligned, contents
 * irrelevant on entry and undefined on return. SANA_DTYPE_F32 returns
 * SANA_ERR_UNSUPPORTED. With eps = 0, rows whose phi(q_i) is 0 give NaN
 * gradients, as the forward gives NaN outputs there. All checks run before
 * any HIP call; three kernels are enqueued on `stream`.
 */
sana_status_t sana_linattn_bwd_workspace_size(int64_t B, int64_t N, int64_t H, int64_t d,
                                              sana_dtype_t dtype, size_t* bytes);
sana_status_t sana_linattn_bwd(const void* q, const void* k, const void* v, const void* dout,
                               void* dq, void* dk, void* dv, int64_t B, int64_t N, int64_t H,
                               int64_t d, float eps, sana_dtype_t dtype, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * sana_linattn_bwd that records events[0] before its first kernel and
 * events[i] after kernel i (i = 1..3: the state reduction, the q pass that
 * also reduces dKV and dksum, the k/v pass); n_events must be >= 4 and the
 * events created by the caller. Computes exactly what sana_linattn_bwd does.
 */
sana_status_t sana_linattn_bwd_profiled(const void* q, const void* k, const void* v,
                                        const void* dout, void* dq, void* dk, void* dv,
                                        int64_t B, int64_t N, int64_t H, int64_t d, float eps,
                                        sana_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                        hipEvent_t* events, int n_events, hipStream_t stream);

/*
 * sana_linattn_bwd (fmap = SANA_FMAP_RELU) or sana_linattn_bwd_fmap from a
 * saved forward state: `state` is the fp32 [B][H][d][d+1] state of the same
 * k, v and map, as sana_linattn_kv_state / sana_linattn_kv_state_fmap write
 * it (KV in the first d columns, ksum in the last; 16-byte aligned,
 * sana_linattn_state_size bytes, read only). The state is the only part of
 * the forward a training step needs to keep (d (d + 1) floats per head,
 * independent of N); with it the backward skips the state reduction and
 * reads k and v once (two kernels: the q pass and the k/v pass). With the
 * state of sana_linattn_kv_state_fmap(k, v, fmap) the gradients are bitwise
 * those of the recomputing backward. Tensors, workspace
 * (sana_linattn_bwd_workspace_size), checks and errors as sana_linattn_bwd;
 * an fmap outside sana_fmap_t is SANA_ERR_UNSUPPORTED; a NULL state is
 * SANA_ERR_INVALID_ARG, an output or the workspace overlapping it too.
 * events may be NULL; otherwise n_events >= 3 and events[0..2] are recorded
 * before the q pass, after it and after the k/v pass.
 */
sana_status_t sana_linattn_bwd_state(const void* q, const void* k, const void* v,
                                     const void* dout, const float* state, void* dq, void* dk,
                                     void* dv, int64_t B, int64_t N, int64_t H, int64_t d,
                                     float eps, sana_dtype_t dtype, sana_fmap_t fmap,
                                     void* workspace, size_t workspace_bytes, hipEvent_t* events,
                                     int n_events, hipStream_t stream);

/*
 * The backward pass of sana_linattn_fwd_fmap (bf16 only): the gradients of
 * sana_linattn_bwd with feature map `fmap` (sana_fmap_t) in place of ReLU,
 * the map's derivative in place of the mask [x > 0]:
 *
 *     dq_i = (KV dnum_i + ksum dden_i) * phi'(q_i)
 *     dk_n = (dKV v_n + dksum) * phi'(k_n),   dv_n = phi(k_n) dKV
 *
 * with KV, ksum, dnum, dden, dKV and dksum as there, from phi of this map.
 * phi'(x): ELU + 1, 1 for x > 0 and exp(x) otherwise; cos, -sin(x); ReLU, as
 * sana_linattn_bwd (SANA_FMAP_RELU computes exactly what sana_linattn_bwd
 * computes). No page writes these gradients out: the chain rule through the
 * course notes' kernel-function form ("Linear Attention 的原理") with the
 * blog's normaliser ("核心架构"). In bf16, phi and phi' of ELU + 1 and cos
 * are evaluated in fp32 and phi is split into bf16 hi + lo parts for the
 * MFMAs. Tensors, workspace (sana_linattn_bwd_workspace_size), checks and
 * errors as sana_linattn_bwd; an fmap outside sana_fmap_t returns
 * SANA_ERR_UNSUPPORTED. events may be NULL; otherwise as for
 * sana_linattn_bwd_profiled (n_events >= 4).
 */
sana_status_t sana_linattn_bwd_fmap(const void* q, const void* k, const void* v,
                                    const void* dout, void* dq, void* dk, void* dv, int64_t B,
                                    int64_t N, int64_t H, int64_t d, float eps,
                                    sana_dtype_t dtype, sana_fmap_t fmap, void* workspace,
                                    size_t workspace_bytes, hipEvent_t* events, int n_events,
                                    hipStream_t stream);

/*
 * Block-causal forward pass. The N tokens of each batch item form N / block
 * consecutive blocks of `block` tokens (a video frame is such a block); a
 * query in block c attends to every key in blocks 0..c - its own block
 * included, earlier blocks in full:
 *
 *     S_c   = sum over tokens n in blocks 0..c of phi(k_n)^T [v_n | 1]
 *     out_i = phi(q_i) S_c(i)[:, :d] / (phi(q_i) . S_c(i)[:, d] + eps)
 *
 * The Linear-DiT 4K blog, section "技术演进", names Block Causal Linear
 * Attention (SANA-Video) without a formula; this is its plainest reading.
 * block = N is sana_linattn_fwd's non-causal attention; block = 1 is
 * token-causal attention. N must be a multiple of block
 * (SANA_ERR_INVALID_ARG otherwise). Tensors, dtypes, eps, alignment and
 * overlap rules as for sana_linattn_fwd; workspace: at least
 * sana_linattn_block_causal_workspace_size(...) bytes, 256-byte aligned,
 * contents irrelevant on entry. Three kernels, in fixed order (results are
 * bitwise repeatable): in general the state reduction per block, an
 * inclusive prefix sum over each batch item's blocks, the apply. In bf16,
 * short blocks run chunk-wise instead (one state per chunk of consecutive
 * tokens, not per block): blocks of 1, 2, 4, 8 or 16 tokens (which never
 * straddle a 16-token tile) on the kernels of sana_linattn_fwd_causal with
 * their in-tile mask widened to whole blocks (block = 1 gives bitwise the
 * result of sana_linattn_fwd_causal), and blocks of 32 to 256 tokens that
 * are whole 16-token tiles on a block-wise apply over chunks of whole
 * blocks (each block's states first, then its queries).
 */
sana_status_t sana_linattn_block_causal_workspace_size(int64_t B, int64_t N, int64_t H,
                                                      int64_t d, int64_t block, sana_dtype_t dtype,
                                                      size_t* bytes);
sana_status_t sana_linattn_fwd_block_causal(const void* q, const void* k, const void* v,
                                            void* out, int64_t B, int64_t N, int64_t H,
                                            int64_t d, int64_t block, float eps, sana_dtype_t dtype,
                                            void* workspace, size_t workspace_bytes,
                                            hipStream_t stream);
/* The same, recording events[0] before and events[1..3] after its three
 * kernels (n_events >= 4, caller-created events). */
sana_status_t sana_linattn_fwd_block_causal_profiled(const void* q, const void* k, const void* v,
                                                     void* out, int64_t B, int64_t N, int64_t H,
                                                     int64_t d, int64_t block, float eps,
                                                     sana_dtype_t dtype, void* workspace,
                                                     size_t workspace_bytes, hipEvent_t* events,
                                                     int n_events, hipStream_t stream);

/*
 * Token-causal attention: query i of a batch item attends to keys 0..i of
 * the same item. This is the block-causal attention above (the blog's
 * "技术演进" section) with blocks of one token, computed with chunked
 * prefix states instead of one state per token:
 *
 *     out_i = phi(q_i) S_i[:, :d] / (phi(q_i) . S_i[:, d] + eps),
 *     S_i   = sum_{n <= i} phi(k_n)^T [v_n | 1].
 *
 * bf16 only (SANA_DTYPE_F32 returns SANA_ERR_UNSUPPORTED); same tensors,
 * layout, alignment, overlap and eps rules as sana_linattn_fwd. The result
 * equals sana_linattn_fwd_block_causal's with block = 1, bit for bit.
 * Three kernels: the states of chunks of consecutive
 * tokens, their exclusive prefix over each head's chunks (fixed order:
 * results are bitwise repeatable), and the apply, which walks each chunk
 * tile by tile from its prefix. workspace: at least
 * sana_linattn_causal_workspace_size(...) bytes, 256-byte aligned, contents
 * irrelevant on entry and undefined on return, overlapping no tensor of the
 * call. events (may be NULL): events[0] is recorded before the first kernel
 * and events[i] after kernel i (n_events >= 4).
 */
sana_status_t sana_linattn_causal_workspace_size(int64_t B, int64_t N, int64_t H, int64_t d,
                                                sana_dtype_t dtype, size_t* bytes);
sana_status_t sana_linattn_fwd_causal(const void* q, const void* k, const void* v, void* out,
                                      int64_t B, int64_t N, int64_t H, int64_t d, float eps,
                                      sana_dtype_t dtype, void* workspace,
                                      size_t workspace_bytes, hipEvent_t* events, int n_events,
                                      hipStream_t stream);

/* Static, human-readable name of a status code ("unknown status" for a value
 * outside sana_status_t). Never NULL; the string is owned by the library. */
const char* sana_linattn_strerror(sana_status_t status);

/* SANA_LINATTN_VERSION of the built library. */
int sana_linattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SANA_LINATTN_H */
