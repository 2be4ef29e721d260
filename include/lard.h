/*
 * lard.h -- C ABI of the linear-memory attention-relation KL library (LinearARD) for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (pith.science verdict page on LinearARD, pith_extraction.key_machinery
 * and core_discovery; arXiv abstract on mlsanity.com):
 *   for each batch b and relation head h, with X_m = x_m[b, head_map[h]] (N x d) for the
 *   teacher m = t and the student m = s,
 *     Z_m   = scale * X_m X_m^T + M        (M: 0 where kept, -inf where masked)
 *     R_m   = row-softmax(Z_m)
 *     KL_i  = sum_j R_t(i,j) * (log R_t(i,j) - log R_s(i,j))        (forward KL, nats)
 *     loss  = sum over b, h, i of KL_i
 *   and, for an upstream gradient g of the loss,
 *     dZ    = g * (R_s - R_t)  (0 where masked)
 *     dX_s  = scale * (dZ + dZ^T) X_s       (the teacher is frozen: no teacher gradient)
 * "Phase 1" keeps only per-row statistics; the backward recomputes the logits tile by tile
 * from them, so no N x N matrix is ever stored.  The forward returns, per row i, the
 * log-sum-exp LSE_m(i) of both sides and diag_delta(i) = R_s(i,i) - R_t(i,i); the backward
 * takes exactly these three fp32 vectors (12 bytes per row and head) plus the inputs.  The
 * diagonal entry Z_m(i,i) = scale |X_m(i)|^2 carries most of a row's mass, so the fp32 LSE
 * alone cannot resolve R_m(i,i) to the precision a nearly-equal teacher and student need;
 * the forward computes that entry from |X_m(i)|^2 in fp64 and hands over the difference.
 *
 * Mask: causal = 1 keeps j <= i (the diagonal included); causal = 0 keeps every entry.
 * The returned loss is the plain sum; the pages' mean over rows is loss / N and its
 * gradient is obtained by passing g = 1 / N.
 *
 * Conventions shared by every entry point:
 *  - Pointers named x_*, lse_*, diag_delta, row_kl, loss, reserve, grad_loss, dx_student
 *    and workspace are DEVICE pointers; head_map and the descriptors are HOST pointers.
 *  - All validation happens on the host before any HIP call; a failed validation
 *    returns LARD_ERR_INVALID_ARGUMENT / LARD_ERR_UNSUPPORTED /
 *    LARD_ERR_WORKSPACE_TOO_SMALL and touches no device memory.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the null
 *    stream).  The library never allocates, frees or synchronises, keeps no global
 *    state and is safe to call from several threads.  A failed launch returns
 *    LARD_ERR_HIP.  No exception or abort crosses the ABI.
 *  - The caller owns every buffer, including the workspace, and must keep them alive
 *    until the enqueued work has completed.
 *  - Results are bitwise reproducible for a fixed shape and split count.
 *  - NaN / Inf inputs are not checked and propagate.
 *  - For bf16 inputs the backward recomputes the scores on the bf16 rows as given and
 *    contracts the gradient in IEEE fp16: each staged student tile is converted on chip
 *    (bf16 -> fp16 is exact for 2^-17 <= |x| < 65504; smaller magnitudes are rounded toward
 *    zero onto the fp16 subnormal grid, an absolute error below 2^-24), and dZ is carried as
 *    fp16 scaled by 2^14.  Inputs with
 *    |x| >= 65504 are not supported by the bf16 backward.
 */
#ifndef LARD_H
#define LARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lard_status {
  LARD_OK = 0,
  LARD_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, stride, alignment or map */
  LARD_ERR_UNSUPPORTED = 2,      /* valid request the library does not implement     */
  LARD_ERR_WORKSPACE_TOO_SMALL = 3,
  LARD_ERR_HIP = 4               /* a HIP launch or runtime call failed              */
} lard_status;

typedef enum lard_dtype { LARD_FP32 = 0, LARD_BF16 = 1 } lard_dtype;

/* Largest sequence length N (rows per head); longer descriptors return LARD_ERR_UNSUPPORTED. */
#define LARD_MAX_N (1 << 30)

/* Largest number of relation heads one call may compute (length of head_map). */
#define LARD_MAX_HEADS 256

/* Largest number of relation problems one grouped call computes together. */
#define LARD_MAX_GROUP 4

/*
 * Problem descriptor.  Teacher and student are [B, H_in, N, d] tensors of the same dtype
 * with element strides (stride over d must be 1, i.e. each row of d elements is
 * contiguous).  Requirements checked by every entry point:
 *   B >= 1, H_in >= 1, 1 <= N <= LARD_MAX_N, d in {64, 128};
 *   all strides >= 0 and multiples of 8 (bf16) or 4 (fp32) elements, so that every row
 *   starts on a 16-byte boundary; x pointers 16-byte aligned;
 *   for N > 1: t_stride_n, s_stride_n >= d, and their byte sizes below 2^24 (16 MiB;
 *   else LARD_ERR_UNSUPPORTED: the backward addresses the rows of a key tile as 24-bit
 *   offsets from the tile's first row);
 *   1 <= H <= LARD_MAX_HEADS;
 *   head_map == NULL  -> H == H_in and relation head h reads input head h;
 *   head_map != NULL  -> H entries, each in [0, H_in), pairwise distinct (injective:
 *                        e.g. the distinct KV heads of a repeated GQA tensor);
 *   causal in {0, 1}; scale finite and > 0 (normally float32(1/sqrt(d)), used for
 *   teacher and student alike).
 */
typedef struct lard_relkl_desc {
  int32_t dtype;          /* lard_dtype of x_teacher and x_student                    */
  int32_t B, H_in, N, d;
  int64_t t_stride_b, t_stride_h, t_stride_n;   /* teacher strides, in elements       */
  int64_t s_stride_b, s_stride_h, s_stride_n;   /* student strides, in elements       */
  int32_t H;              /* relation heads computed                                   */
  int32_t causal;         /* 1: keep j <= i;  0: keep all                              */
  const int32_t* head_map;/* HOST int32[H] or NULL                                     */
  float scale;            /* logit scale                                               */
} lard_relkl_desc;

/*
 * Output layout of the student gradient: [B, H_in, N, d] in `dtype` (LARD_FP32 or the
 * input dtype), element strides with unit stride over d; same alignment rules as the
 * inputs.  Heads listed in head_map (all heads when NULL) are overwritten; the other
 * heads are left untouched.
 */
typedef struct lard_grad_desc {
  int32_t dtype;
  int32_t reserved;
  int64_t stride_b, stride_h, stride_n;
} lard_grad_desc;

/*
 * Bytes of device workspace that lard_relkl_fwd (pass = 0) or lard_relkl_bwd (pass = 1)
 * needs for this descriptor (the RoPE-fused and cross entry points use the same sizes).
 * Returns 0 and sets *status (if non-NULL) on an invalid descriptor.  The forward's
 * workspace holds one fp64 loss partial per workgroup (8 * B * H * ceil(N / 128) bytes,
 * rounded up to 256); the backward's holds fp32 split-K partials and is 0 bytes unless the
 * library splits the key range, which it does only when the (batch, head, row tile) work
 * alone cannot fill the chip (environment variable LARD_SPLITK overrides the split count).
 */
size_t lard_relkl_workspace_size(const lard_relkl_desc* desc, int pass, lard_status* status);

/*
 * Forward ("phase 1" plus the KL accumulation; key_machinery of the verdict page).
 *   x_teacher, x_student : device, desc layout and dtype, read only.
 *   lse_teacher, lse_student : device fp32 [B, H, N] (dense), written: LSE_m(i) in nats.
 *   diag_delta : device fp32 [B, H, N] or NULL; written: R_s(i,i) - R_t(i,i).  Required by
 *            lard_relkl_bwd (a caller that only wants the loss may pass NULL).
 *   row_kl : device fp32 [B, H, N] or NULL; written: KL_i.
 *   loss   : device fp32 scalar, written (not accumulated): sum of KL_i over b, h, i,
 *            reduced in a fixed order in fp64.
 *   workspace : device, >= lard_relkl_workspace_size(desc, 0) bytes, 8-byte aligned.
 */
lard_status lard_relkl_fwd(const lard_relkl_desc* desc, const void* x_teacher,
                           const void* x_student, float* lse_teacher, float* lse_student,
                           float* diag_delta, float* row_kl, float* loss, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Backward (logit recomputation fused with the gradient; key_machinery and the gradient
 * identity of core_discovery on the verdict page).
 *   x_teacher, x_student : the inputs given to lard_relkl_fwd.
 *   lse_teacher, lse_student, diag_delta : device fp32 [B, H, N], as written by
 *            lard_relkl_fwd for the same inputs and descriptor (the only state kept
 *            between the two passes).
 *   grad_loss : device fp32 scalar g (the upstream gradient of `loss`).
 *   dx_student : device, layout and dtype given by `grad`; see lard_grad_desc.
 *   workspace : device, >= lard_relkl_workspace_size(desc, 1) bytes, 16-byte aligned
 *            (may be NULL when that size is 0).
 */
lard_status lard_relkl_bwd(const lard_relkl_desc* desc, const void* x_teacher,
                           const void* x_student, const float* lse_teacher,
                           const float* lse_student, const float* diag_delta,
                           const float* grad_loss, const lard_grad_desc* grad,
                           void* dx_student, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * RoPE-fused entry points.  The pages distil the relations of queries and keys after the
 * rotary embedding -- the teacher with its native RoPE, the student with a rescaled one --
 * and send the gradient to the student's Q/K/V projections (verdict page,
 * pith_extraction.key_machinery; arXiv abstract).  These entry points take the
 * activations BEFORE the rotation, rotate them inside the operation, and return the
 * gradient with respect to the student's pre-rotation input.
 *
 * The rotation (rotate-half pairing of dimension k with k + d/2, the reading taken where
 * the pages leave it open): for token p and k < d/2,
 *     X[p, k]       = Xpre[p, k] cos[p][k] - Xpre[p, k + d/2] sin[p][k]
 *     X[p, k + d/2] = Xpre[p, k + d/2] cos[p][k] + Xpre[p, k] sin[p][k]
 * and the loss is the one of lard_relkl_fwd on (X_teacher, X_student).  The returned
 * gradient is dXpre = R^T dX_s, i.e. (g_k c + g_{k+d/2} s, g_{k+d/2} c - g_k s).
 *
 * Tables: device fp32, dense [N][d/2] (row p holds the cos / sin of token p's angles;
 * the caller's recipe -- base, position interpolation, NTK base -- lives entirely in
 * them), 16-byte aligned.  Each side's pair is either both non-NULL or both NULL (that
 * side is not rotated, e.g. the V relation).  Every relation head uses the same tables.
 *
 * The rotated rows are rounded to the input dtype (bf16: nearest even), as the model would
 * hand them to the plain operation, and the plain kernels run on them.  The reserve holds
 * them for the backward (a caller-owned buffer of 2 * e * B * H * N * d bytes, e the
 * element size, from lard_relkl_rope_reserve_size); the row statistics are the outputs, as
 * for the plain entry points.  Workspaces are those of lard_relkl_workspace_size.
 * Validation, ownership, stream and error conventions are those of the plain entry points.
 */
typedef struct lard_rope_desc {
  const float* cos_teacher;  /* device fp32 [N][d/2] or NULL */
  const float* sin_teacher;  /* device fp32 [N][d/2] or NULL (NULL iff cos_teacher is) */
  const float* cos_student;
  const float* sin_student;
} lard_rope_desc;

/* Bytes of the reserve the RoPE-fused forward writes: 2 * c * B * H * N * d (c = 2 for
 * bf16, 4 for fp32 inputs), each copy rounded up to 256 bytes.  Returns 0 and sets *status
 * on an invalid descriptor. */
size_t lard_relkl_rope_reserve_size(const lard_relkl_desc* desc, lard_status* status);

/*
 * RoPE-fused forward.  x_teacher, x_student: pre-rotation inputs (desc layout and dtype).
 * Outputs and workspace as for lard_relkl_fwd; reserve: device, 256-byte aligned, at least
 * lard_relkl_rope_reserve_size bytes, written (the rotated rows).
 */
lard_status lard_relkl_rope_fwd(const lard_relkl_desc* desc, const lard_rope_desc* rope,
                                const void* x_teacher, const void* x_student,
                                float* lse_teacher, float* lse_student, float* diag_delta,
                                float* row_kl, float* loss, void* reserve, size_t reserve_bytes,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * RoPE-fused backward: the gradient of g * loss with respect to the student's
 * PRE-rotation input, written like lard_relkl_bwd's (heads outside head_map untouched).
 * Needs the reserve the fused forward wrote (it holds the rotated operands), the forward's
 * lse_teacher, lse_student and diag_delta, and the same `rope` tables (the student's
 * rotate the gradient back).
 */
lard_status lard_relkl_rope_bwd(const lard_relkl_desc* desc, const lard_rope_desc* rope,
                                const void* reserve, size_t reserve_bytes,
                                const float* lse_teacher, const float* lse_student,
                                const float* diag_delta, const float* grad_loss,
                                const lard_grad_desc* grad, void* dx_student, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * Cross-relation entry points: the same row-wise KL for the relation between two different
 * matrices per side, softmax(scale * A B^T + M) -- e.g. the attention map of queries A and
 * keys B -- the general form the verdict page's own inference on the method's scope
 * points to (the relation case is A = B).  Per side m = t, s:
 *     Z_m = scale * A_m B_m^T + M,  R_m = row-softmax(Z_m),  loss = sum_i KL(R_t(i,:) || R_s(i,:))
 * and, for an upstream gradient g, with dZ = g (R_s - R_t) (0 where masked):
 *     dA_s = scale * dZ B_s,   dB_s = scale * dZ^T A_s      (teacher frozen).
 * A and B have the same shape [B, H_in, N, d] and dtype; `desc` describes A (its t_ / s_
 * strides) together with the mask, scale and head map, which apply to B too; `keys` gives
 * B's strides (same rules as the descriptor's).  With `rope` non-NULL each side's tables
 * rotate both its A and its B (as RoPE rotates queries and keys alike; see the RoPE-fused
 * entry points for the rotation, rounding and table layout) and the gradients are returned
 * with respect to the pre-rotation inputs.  The reserve holds copies of all four matrices
 * (fp16 images of bf16 values, or fp32); size from lard_relkl_cross_reserve_size.  The row
 * statistics are the LSE outputs (no matrix entry is special here, so there is no
 * diag_delta).  Workspaces are those of lard_relkl_workspace_size.
 * Validation, ownership, stream and error conventions are those of the plain entry points.
 */
typedef struct lard_cross_desc {
  int64_t bt_stride_b, bt_stride_h, bt_stride_n;  /* teacher B strides, in elements */
  int64_t bs_stride_b, bs_stride_h, bs_stride_n;  /* student B strides, in elements */
} lard_cross_desc;

/* Bytes of the reserve the cross forward writes: 4 * c * B * H * N * d (c = 2 for bf16, 4
 * for fp32 inputs), each copy rounded up to 256 bytes.  Returns 0 and sets *status on an
 * invalid descriptor. */
size_t lard_relkl_cross_reserve_size(const lard_relkl_desc* desc, lard_status* status);

/*
 * Cross forward.  a_*, b_*: device, A in desc's layout, B in `keys`' layout, desc's dtype.
 * rope: NULL (no rotation) or tables as for lard_relkl_rope_fwd.  Outputs (LSE and row KL
 * per row of A), reserve and workspace as for lard_relkl_fwd.
 */
lard_status lard_relkl_cross_fwd(const lard_relkl_desc* desc, const lard_cross_desc* keys,
                                 const lard_rope_desc* rope, const void* a_teacher,
                                 const void* b_teacher, const void* a_student,
                                 const void* b_student, float* lse_teacher, float* lse_student,
                                 float* row_kl, float* loss, void* reserve, size_t reserve_bytes,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Cross backward: dA_s and dB_s of g * loss, each written like lard_relkl_bwd's gradient
 * (layout and dtype from grad_a / grad_b; heads outside head_map untouched).  Needs the
 * reserve the cross forward wrote, its lse_teacher and lse_student, and the same `rope`
 * (NULL if the forward had none).
 */
lard_status lard_relkl_cross_bwd(const lard_relkl_desc* desc, const lard_rope_desc* rope,
                                 const void* reserve, size_t reserve_bytes,
                                 const float* lse_teacher, const float* lse_student,
                                 const float* grad_loss, const lard_grad_desc* grad_a,
                                 void* da_student, const lard_grad_desc* grad_b,
                                 void* db_student, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * Grouped entry points: up to LARD_MAX_GROUP relation problems ("members") in one launch of
 * each kernel.  The method's loss has three relation terms per layer, Q/Q, K/K and V/V
 * (verdict page: pith_extraction.core_discovery; the referee report places the V/V term in
 * Eq. (4c) of section 3.2), and with grouped-query attention the query relation runs on
 * more heads than the key and value relations (e.g. 32 query heads, 8 KV heads).  One grouped call computes
 * all of them with one forward and one backward launch, so small problems (short
 * sequences, few heads) fill the chip together instead of one after another.
 *
 * Each member carries its own descriptor, inputs and outputs.  Members must share dtype,
 * d and causal; B, H_in, N, H, strides, head maps and scale may differ.  The head maps of
 * one group hold at most 512 entries in total (a member without a head map takes none);
 * beyond that the call returns LARD_ERR_UNSUPPORTED.  Per member, the results are those of
 * the single-problem entry points on the same inputs: the forward outputs bitwise, the
 * gradient bitwise for the same backward split count (a group picks one split count from
 * its total work; LARD_SPLITK overrides it as for the single calls).
 *
 * with_rope = 0: members are post-rotation inputs (as lard_relkl_fwd / _bwd).
 * with_rope = 1: members are pre-rotation inputs rotated inside the call with their own
 *   `rope` tables (a pair of NULL tables: that side is not rotated, e.g. the V relation),
 *   as lard_relkl_rope_fwd / _bwd; the gradients are with respect to the pre-rotation
 *   inputs.
 * With with_rope = 1 the reserve holds every member's rotated rows (as sized by
 * lard_relkl_rope_reserve_size) back to back; with with_rope = 0 no reserve is needed (it
 * may be NULL with reserve_bytes 0).  Sizes from lard_relkl_group_reserve_size and
 * lard_relkl_group_workspace_size.  Validation, ownership, stream and error conventions
 * are those of the single-problem entry points.
 */
typedef struct lard_relkl_member {
  lard_relkl_desc desc;
  const void* x_teacher;    /* device, desc layout and dtype                          */
  const void* x_student;    /* (with_rope = 1: before the rotation)                   */
  float* lse_teacher;       /* device fp32 [B, H, N], written by the forward, read by  */
  float* lse_student;       /*   the backward                                          */
  float* diag_delta;        /* device fp32 [B, H, N] (as lard_relkl_fwd's); the forward */
                            /*   may take NULL, the backward needs it                   */
  float* row_kl;            /* device fp32 [B, H, N] or NULL                          */
  float* loss;              /* device fp32 scalar or NULL: this member's own sum      */
  lard_rope_desc rope;      /* tables of this member (read when with_rope = 1)        */
} lard_relkl_member;

/* Bytes of the reserve a grouped forward writes: 0 for with_rope = 0, else the sum of the
 * members' lard_relkl_rope_reserve_size.  Returns 0 and sets *status on an invalid
 * group. */
size_t lard_relkl_group_reserve_size(int n, const lard_relkl_member* members, int with_rope,
                                     lard_status* status);

/* Bytes of device workspace of the grouped forward (pass = 0) or backward (pass = 1). */
size_t lard_relkl_group_workspace_size(int n, const lard_relkl_member* members, int pass,
                                       lard_status* status);

/*
 * Grouped forward.  Writes every member's LSE vectors, diag_delta and row KL (if
 * requested) and own loss (if requested), and `loss`: device fp32 scalar = the sum over all
 * members, reduced in a fixed order in fp64.  reserve (with_rope = 1) and workspace sized
 * by the group functions above.
 */
lard_status lard_relkl_group_fwd(int n, const lard_relkl_member* members, int with_rope,
                                 float* loss, void* reserve, size_t reserve_bytes,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Grouped backward: the gradient of g * loss (g = *grad_loss, loss = the group's sum) with
 * respect to every member's student input, written to dx_student[k] with layout grads[k]
 * (all members' gradients of one dtype; heads outside a member's head map untouched).
 * members, with_rope and reserve: as given to lard_relkl_group_fwd; the backward reads the
 * members' lse_teacher, lse_student and diag_delta as the forward wrote them (row_kl and
 * loss are not read; with with_rope = 1 neither are the inputs).
 */
lard_status lard_relkl_group_bwd(int n, const lard_relkl_member* members, int with_rope,
                                 const void* reserve, size_t reserve_bytes,
                                 const float* grad_loss, const lard_grad_desc* grads,
                                 void* const* dx_student, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * Allocation-free forward, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): lard_relkl_fwd
 * without the workspace argument.  The forward's per-workgroup loss partials go to a
 * device array the library holds per GPU (LARD_NOALLOC_MAX_PARTIALS fp64 values, 512 KiB,
 * kept until the process ends); the address is looked up on the first call on each device.
 * The caller still passes inputs and outputs, as for lard_relkl_fwd.  The call allocates
 * nothing.  A descriptor needing more than LARD_NOALLOC_MAX_PARTIALS partials
 * (B * H * ceil(N / 128) of them) returns LARD_ERR_WORKSPACE_TOO_SMALL.  Every call on one
 * GPU shares the array: calls that overlap on a GPU (e.g. on two streams at once) race.
 * Results are bitwise those of lard_relkl_fwd.
 */
#define LARD_NOALLOC_MAX_PARTIALS 65536
lard_status lard_relkl_fwd_noalloc(const lard_relkl_desc* desc, const void* x_teacher,
                                   const void* x_student, float* lse_teacher,
                                   float* lse_student, float* diag_delta, float* row_kl,
                                   float* loss, void* stream);

/*
 * Matrix-core throughput probe (measurement, not part of the relation KL): enqueues one
 * kernel of `workgroups` workgroups of LARD_PROBE_THREADS threads (two waves per SIMD when
 * one workgroup runs per CU, the relation backward's occupancy), in which every wave issues
 * iters * LARD_PROBE_MFMA_PER_ITER independent v_mfma_f32_32x32x16_bf16 (32768 flops each)
 * with register operands that change from one MFMA to the next (pseudo-random bf16 values).  vector_work = 1 adds, per four MFMAs, the vector work of four
 * backward probability differences (two FMAs, two exp2 and a subtraction each).  Timing the
 * launch gives the dense bf16 rate the part sustains under that load, beside the published
 * peak the roofline is quoted against.  sink: device buffer of workgroups *
 * LARD_PROBE_THREADS floats, written with values that depend on every result.  Returns
 * LARD_ERR_INVALID_ARGUMENT for a null sink, iters outside [1, 2^20], workgroups outside
 * [1, 2^16] or vector_work other than 0 or 1; LARD_ERR_HIP if the launch fails.
 */
#define LARD_PROBE_THREADS 512
#define LARD_PROBE_MFMA_PER_ITER 24
lard_status lard_probe_mfma(int vector_work, int iters, int workgroups, float* sink,
                            void* stream);

/* Static, NUL-terminated description of a status code. */
const char* lard_status_string(lard_status status);

/* Library version as major * 10000 + minor * 100 + patch. */
int lard_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LARD_H */
