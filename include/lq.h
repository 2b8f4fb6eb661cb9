/*
 * lq.h -- C ABI of the LiftQuant lift-then-project linear layer on MI355X.
 *
 * The layer (LiftQuant notes, "LiftQuant: Continuous Bit-Width LLM via
 * Dimensional Lifting and Projection", section 关键设计 4 and the 推理 node of
 * the 整体框架 flowchart) is
 *
 *     o = diag(s) . W_q . lift(T^-1 a)
 *
 *   * W_q in {+-1}^(m x K) holds one sign per bit (关键设计 1: a d-wide weight
 *     group is w = M y with y in {+-1}^D, so K = n*D/d and the bit-width is D/d);
 *   * T^-1 is a per-layer transform, here block-diagonal with square blocks;
 *   * lift applies M^T (M is d x D) to every d-wide group of u = T^-1 a:
 *     a_hat[g*D + j] = sum_r M[r][j] u[g*d + r].  Since y.(M^T u_g) = (M y).u_g
 *     this equals the product with the reconstructed weights;
 *   * s is a per-output-row scale (the notes write diag(s) and nothing more).
 * The notes split the run-time work into one small transform of the
 * activations and then the product of the 1-bit weights with the result
 * (关键设计 4); the calls below are those two steps.
 *
 * Conventions (all calls):
 *   - Every pointer except host-side size outputs is a DEVICE pointer owned by
 *     the caller.  The library keeps no buffers of its own.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  A
 *     call validates its arguments on the host, enqueues its kernels on
 *     `stream` and returns without synchronising.
 *   - On any validation failure the call returns a nonzero lq_status, sets a
 *     thread-local message (lq_last_error) and launches nothing.  A failed
 *     launch returns LQ_ERR_HIP.
 *   - Outputs must not alias inputs.  All arrays are row-major and dense in
 *     their last dimension; leading dimensions are given where they may differ.
 *   - Calls are thread-safe; calls that share a workspace must not overlap.
 */
#ifndef LQ_H_
#define LQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t lq_status;
#define LQ_OK              0
#define LQ_ERR_NULL        1  /* a required pointer is NULL                        */
#define LQ_ERR_SHAPE       2  /* sizes inconsistent or out of range                */
#define LQ_ERR_DTYPE       3  /* unsupported element type for this argument        */
#define LQ_ERR_ALIGN       4  /* a pointer or leading dimension is misaligned      */
#define LQ_ERR_UNSUPPORTED 5  /* valid request this build does not implement        */
#define LQ_ERR_HIP         6  /* the HIP runtime reported an error                  */
#define LQ_ERR_WORKSPACE   7  /* workspace missing or too small                     */

typedef int32_t lq_dtype;
#define LQ_F32  0
#define LQ_F16  1
#define LQ_BF16 2

/* Human-readable name of a status code (static string). */
const char* lq_status_string(lq_status st);
/* Message of the last failed call on this thread ("" if none). */
const char* lq_last_error(void);
/* Library version string. */
const char* lq_version(void);

/*
 * lq_pack_signs -- pack signs into W_q words.
 * Storage of W_q (关键设计 1: one bit per lifted sign, D signs per d weights):
 *   packed: uint32 [rows][ldw]; lifted position k of a row is bit (k & 31) of
 *   word (k >> 5); the bit is 1 iff signs[row][k] > 0 (0 and negatives pack as
 *   0, i.e. -1).  Bits at positions >= K and words >= ceil(K/32) are written 0.
 * signs:  int8 [rows][lds], lds >= K.
 * Requires rows >= 0, K >= 0, ldw >= ceil(K/32), lds >= K; rows == 0 or
 * K == 0 with ldw == 0 is a no-op.
 */
lq_status lq_pack_signs(const int8_t* signs, int64_t rows, int64_t K, int64_t lds,
                        uint32_t* packed, int64_t ldw, void* stream);

/*
 * lq_unpack_signs -- inverse of lq_pack_signs: signs[row][k] = +1 if the bit
 * is 1 else -1, for k < K (columns K..lds-1 are not written).
 */
lq_status lq_unpack_signs(const uint32_t* packed, int64_t rows, int64_t K, int64_t ldw,
                          int8_t* signs, int64_t lds, void* stream);

/*
 * lq_lift_activations -- the small transform of the activations
 * (关键设计 4, T* a, with T* read as T^-1 followed by M^T per group).
 *   u[b][tb*q + r] = sum_c T_q[r][c] * a[b][tb*q + c]      (block q of T^-1)
 *   a_lift[b][g*D + j] = sum_{r<d} M[r][j] * u[b][g*d + r]
 * a:      [B][n] of a_dtype (LQ_F16 | LQ_BF16 | LQ_F32)
 * t_inv:  [n/t_block][t_block][t_block] of t_dtype (LQ_F16 | LQ_BF16 | LQ_F32)
 * M:      float [d][D]
 * a_lift: [B][K] of lift_dtype, K = n*D/d.  LQ_F32 feeds lq_gemv; LQ_F16 or
 *         LQ_BF16 (round to nearest even) feed lq_gemm.
 * Accumulation is float32.  Requires t_block == 128, n % 128 == 0,
 * n % d == 0, 1 <= d <= 64, 1 <= D <= 256, d*D <= 8192, B >= 1; a and t_inv
 * 16-byte aligned (16-byte loads), M and a_lift aligned to their element.
 */
lq_status lq_lift_activations(const void* a, lq_dtype a_dtype, int64_t B, int64_t n,
                              const void* t_inv, lq_dtype t_dtype, int32_t t_block,
                              const float* M, int32_t d, int32_t D,
                              void* a_lift, lq_dtype lift_dtype, void* stream);

/*
 * lq_lift_kron -- the lift with the Kronecker-factored whitening of
 * 关键设计 3, T = diag(s1) (P1 (x) P2) diag(s2) with P1 n1 x n1, P2 n2 x n2,
 * n = n1 n2 and s2 constant over each d-wide lift group (so that it folds
 * into M):
 *   u      = diag(1/s2) (P1^-1 (x) P2^-1) diag(1/s1) a
 *   a_lift = (I (x) M^T) u,  a_lift[b][g*D + j] = sum_{r<d} M[r][j] u[b][g*d + r]
 * Channel c = i*n2 + j of a token is entry (i, j) of its n1 x n2 reshape.
 * a:        [B][n] of a_dtype (LQ_F16 | LQ_BF16 | LQ_F32).
 * s1:       float [n];  s2: float [n/d] (one scale per group).
 * p1_inv:   float [n1][n1] (P1^-1);  p2_inv: float [n2][n2] (P2^-1).
 * M:        float [d][D].
 * a_lift:   [B][K] of lift_dtype, K = n*D/d.
 * workspace: device buffer of >= lq_lift_kron_workspace_size bytes (the
 *           intermediate n1 x n2 products, float32), 256-byte aligned,
 *           caller-owned, no initialisation needed.
 * Requires 1 <= B <= 65535, n % n1 == 0, n2 = n/n1 <= 128, n1 <= 256,
 * n2 % d == 0, 1 <= d <= 64, 1 <= D <= 256, d*D <= 8192 (else LQ_ERR_SHAPE or
 * LQ_ERR_UNSUPPORTED, nothing launched).  float32 arithmetic throughout.
 */
lq_status lq_lift_kron_workspace_size(int64_t B, int64_t n, size_t* bytes);
lq_status lq_lift_kron(const void* a, lq_dtype a_dtype, int64_t B, int64_t n, int32_t n1,
                       const float* s1, const float* p1_inv, const float* p2_inv,
                       const float* s2, const float* M, int32_t d, int32_t D, void* a_lift,
                       lq_dtype lift_dtype, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * lq_encode -- quantise weight groups to lattice codes: for each d-wide group
 * w, the code y in {+-1}^D whose projection M y is nearest to w (w ~ M y with
 * M of shape d x D, 关键设计 1; the nearest-point search of 关键设计 2).
 *   A == NULL: exhaustive, every y (2^D candidates; candidate t has y_j = +1
 *              iff bit j of t is set).
 *   A != NULL: the pseudo-inverse start plus auxiliary vector of 关键设计 2,
 *              read as y(v) = sign([M; A]^-1 [w; v]) for every auxiliary sign
 *              vector v in {+-1}^(D-d) (v_k = +1 iff bit k of t is set),
 *              2^(D-d) candidates.  A ((D-d) x D) completes M to an
 *              invertible matrix; with [M; A] orthogonal the candidate is
 *              sign(M^+ w + A^T v).
 * The candidate with the smallest ||w - M y||^2 is chosen, ties to the
 * smallest t, sign(0) = +1.  Arithmetic is float32 (the inverse is formed in
 * float64 and rounded), so groups whose best candidates are within float32
 * rounding of each other may resolve to either.
 * w:     float [groups][d] (group g is weights g*d .. g*d + d - 1; a weight
 *        matrix [m][n] in row-major order is groups = m*n/d).
 * M:     float [d][D];  A: float [D-d][D] or NULL (with D == d, A has no
 *        rows: pass any non-null pointer to select the search).
 * codes: int8 [groups][D], +1 / -1 (the lq_pack_signs input for a matrix of
 *        m rows and K = n*D/d).
 * err:   float [groups], the squared error of the chosen code, or NULL.
 * workspace: with A, >= lq_encode_workspace_size bytes, 256-byte aligned,
 *        caller-owned, no initialisation needed (it receives [M; A]^-1); may
 *        be NULL without A.
 * Requires 1 <= d <= D <= 32 and at most 2^24 candidates (D - d <= 24 with
 * A, D <= 24 without); else LQ_ERR_SHAPE or LQ_ERR_UNSUPPORTED, nothing
 * launched.  groups == 0 is a no-op.  A singular [M; A] gives unspecified
 * codes.  Work grows as groups * 2^(D-d) (or 2^D) * d * D.
 */
lq_status lq_encode_workspace_size(int32_t d, int32_t D, size_t* bytes);
lq_status lq_encode(const float* w, int64_t groups, const float* M, const float* A, int32_t d,
                    int32_t D, int8_t* codes, float* err, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * lq_gemm_decoded -- the layer's product for large batches with the weights
 * decoded instead of the activations lifted: W_hat[i][g*d + r] =
 * sum_j M[r][j] sigma_{i, g*D + j} (w = M y, 关键设计 1), then
 *   out[b][i] = s[i] * sum_{k<n} W_hat[i][k] * u[b][k],
 * the same linear map as lq_gemm on the lifted activations (y . (M^T x) =
 * (M y) . x), at 2 m n B flops for the product plus the reconstruction,
 * instead of 2 m K B (fewer once B > D d / (D - d)).
 * w_packed: uint32 [m][ldw] (layout of lq_pack_signs), ldw >= ceil(K/32),
 *           K = n*D/d.
 * M:        float [d][D];  s: float [m].
 * u:        float16 [B][n], the whitened activations T^-1 a (for example
 *           lq_lift_activations with M = I_4, d = D = 4).
 * out:      float [B][m].
 * workspace: none is needed (lq_gemm_decoded_workspace_size gives 0); the
 *           pointer may be null.
 * Arithmetic: one kernel reconstructs the weights on the matrix cores from
 * M rounded to float16 (exact +-1 signs, float32 sums), rounds them to
 * float16 (relative 2^-11) and contracts them with u on the matrix cores in
 * float32; s[i] scales the float32 result.  The weights never leave the
 * chip.
 * Requires n % d == 0, 1 <= d <= 64, 1 <= D <= 256, n <= 2^22, ldw <= 2^22,
 * m, B <= 2^31 - 1; u must be LQ_F16 (else LQ_ERR_DTYPE).
 */
lq_status lq_gemm_decoded_workspace_size(int64_t m, int64_t n, size_t* bytes);
lq_status lq_gemm_decoded(const uint32_t* w_packed, int64_t m, int64_t n, int64_t ldw,
                          const float* M, int32_t d, int32_t D, const float* s, const void* u,
                          lq_dtype u_dtype, int64_t B, float* out, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * lq_softmin_grad -- the objective that learns M (关键设计 2: M* minimises
 * E_w[min_y ||w - M y||] over Gaussian w, M initialised orthogonal, the inner
 * argmin replaced by a soft-argmin at temperature T, 10 in the notes) on one
 * batch, and its gradient.  Over all 2^D codes y_t (y_tj = +1 iff bit j of t):
 *   p_nt  = softmax_t(-T ||w_n - M y_t||^2),  y_hat_n = sum_t p_nt y_t,
 *   *loss = (1/N) sum_n ||w_n - M y_hat_n||^2,   grad = d loss / d M.
 * w:     float [N][d] samples (drawn by the caller).
 * M:     float [d][D].
 * loss:  device float (one value);  grad: float [d][D].
 * workspace: >= lq_softmin_workspace_size bytes, 256-byte aligned,
 *        caller-owned, no initialisation needed.
 * Requires 1 <= N <= 2^31 - 1, 1 <= d <= D <= 24 (D <= 32 is a valid shape the
 * build does not implement: LQ_ERR_UNSUPPORTED), T finite and >= 0.  float32
 * arithmetic; the result does not depend on timing (fixed partition and
 * summation order).  Work grows as N * 2^D * (d + D).
 */
lq_status lq_softmin_workspace_size(int64_t N, int32_t d, int32_t D, size_t* bytes);
lq_status lq_softmin_grad(const float* w, int64_t N, const float* M, int32_t d, int32_t D,
                          float T, float* loss, float* grad, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * lq_adam_update -- one Adam step on `count` floats in place (the optimiser
 * that learns M; the notes name none, this is the textbook bias-corrected
 * form): m1 = beta1 m1 + (1 - beta1) g, m2 = beta2 m2 + (1 - beta2) g^2,
 * M -= lr (m1 / (1 - beta1^step)) / (sqrt(m2 / (1 - beta2^step)) + eps).
 * m1, m2: caller-owned moment buffers, zero before step 1.  step >= 1,
 * 0 <= beta1, beta2 < 1, eps >= 0; count == 0 is a no-op.
 */
lq_status lq_adam_update(float* M, const float* grad, float* m1, float* m2, int64_t count,
                         int32_t step, float lr, float beta1, float beta2, float eps,
                         void* stream);

/*
 * lq_gemv_workspace_size -- bytes of workspace lq_gemv needs for this shape
 * (0 when none).  Written to *bytes.
 */
lq_status lq_gemv_workspace_size(int64_t m, int64_t K, int64_t B, size_t* bytes);

/*
 * lq_workspace_clear -- zero `bytes` bytes of a workspace on `stream` with a
 * fill kernel.  lq_gemv needs no cleared workspace (every call writes what it
 * reads back); this is a convenience for callers that want a known state.
 */
lq_status lq_workspace_clear(void* workspace, size_t bytes, void* stream);

/*
 * lq_gemv -- the product of the 1-bit weights with the float lifted
 * activations for small batches (关键设计 4 calls this the main body: an
 * ordinary GEMM between 1-bit weights and floats, with no weight codebook to
 * look up):
 *   out[b][i] = s[i] * sum_{k<K} sigma_ik * a_lift[b][k],
 *   sigma_ik = +1 if bit k of row i is 1, else -1.
 * w_packed: uint32 [m][ldw] (layout of lq_pack_signs), ldw >= ceil(K/32),
 *           ldw a multiple of 4 and w_packed 16-byte aligned (16-byte loads).
 * s:        float [m].
 * a_lift:   float [B][K] (lq_lift_activations with LQ_F32), 16-byte aligned,
 *           K % 4 == 0.
 * out:      float [B][m].
 * workspace: device buffer of >= lq_gemv_workspace_size bytes, 256-byte
 *           aligned, owned by the caller; may be NULL when that size is 0.
 *           Its contents need no initialisation.  Calls that share a
 *           workspace must not overlap.
 * Requires 1 <= B <= 16, m >= 1, K >= 1, m*ldw*4 <= 2^30 bytes (split
 * larger matrices by rows over several calls) and K <= 2^24.  Accumulation
 * is float32 and the result does not depend on timing (partial sums over the
 * lifted dimension are added in a fixed order, no float atomics).
 * Arithmetic: the product runs on the matrix cores with the signs as
 * float4 values (exact) and each activation carried by three float8 (E4M3)
 * parts of 4 significant bits each, kept in range by a power-of-two scale
 * per block of positions (1024 positions for B <= 5, 128 for B >= 6): 12
 * significant bits per value (relative error at most 2^-12 of the value,
 * less than 2^-17 of the block's largest one for small values), exact
 * products, float32 sums; about 2e-5 relative output error on the workload
 * shapes.  For B <= 5 the signs enter as 0 / c nibbles and each block adds
 * 2 R - sum(a) (R: the sum over set bits, the block's sum taken in float32).
 */
lq_status lq_gemv(const uint32_t* w_packed, int64_t m, int64_t K, int64_t ldw,
                  const float* s, const float* a_lift, int64_t B, float* out,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * lq_lift_parts_size -- bytes of the operand image lq_lift_parts writes for
 * K lifted positions (written to *bytes).
 */
lq_status lq_lift_parts_size(int64_t K, size_t* bytes);

/*
 * lq_lift_parts -- the lift of lq_lift_activations (关键设计 4: the small
 * transform of the activations, done once per input; 关键设计 1 for M),
 * written not as a_lift but as the operand image that lq_gemv_parts reads,
 * so that the product needs no conversion launch of its own.
 * a, t_inv: [B][n] and [n/t_block][t_block][t_block] of one 16-bit type
 *           (LQ_F16 or LQ_BF16: their products are exact), 16-byte aligned.
 * M:        float [d][D], 4-byte aligned.
 * parts:    device buffer of >= lq_lift_parts_size(n*D/d) bytes, 16-byte
 *           aligned, owned by the caller.  Layout (opaque to callers, fixed
 *           by this library): per 512-position span of the lifted dimension
 *           (whole groups of eight spans, padding spans zero), each token's
 *           lifted values as three float8 (E4M3) parts in the order the
 *           product's matrix operands hold them, then an int power-of-two
 *           exponent per 128 positions and token; a value is p0 + p1/16 +
 *           p2/256 times 2^-e, 12 significant bits.
 * Requires 1 <= B <= 16, t_block == 128, n % 128 == 0, d in {4, 8, 16, 32},
 * n % d == 0, d <= D <= 256.  Accumulation float32.  Errors as
 * lq_lift_activations; LQ_ERR_WORKSPACE if parts_bytes is too small.
 */
lq_status lq_lift_parts(const void* a, lq_dtype a_dtype, int64_t B, int64_t n,
                        const void* t_inv, lq_dtype t_dtype, int32_t t_block,
                        const float* M, int32_t d, int32_t D, void* parts,
                        size_t parts_bytes, void* stream);

/*
 * lq_gemv_parts_workspace_size -- bytes of workspace lq_gemv_parts needs
 * (the partial sums over splits of K), written to *bytes.
 */
lq_status lq_gemv_parts_workspace_size(int64_t m, int64_t K, int64_t B, size_t* bytes);

/*
 * lq_gemv_parts -- lq_gemv on the image of lq_lift_parts instead of float
 * lifted activations (关键设计 4, the 1-bit x float product), for 1 <= B <=
 * 16 tokens on the matrix-core kernel of lq_gemv's 6 - 16 token range:
 *   out[b][i] = s[i] * sum_{k<K} sigma_ik * a_hat[b][k].
 * w_packed, ldw, s, out, K: as lq_gemv.  parts: the image of lq_lift_parts
 * for the same K and B (parts_bytes >= lq_lift_parts_size(K)).  workspace:
 * >= lq_gemv_parts_workspace_size bytes, 256-byte aligned, caller-owned, no
 * initialisation needed; calls sharing it must not overlap.  Deterministic
 * (fixed-order sums).  Errors as lq_gemv.
 */
lq_status lq_gemv_parts(const uint32_t* w_packed, int64_t m, int64_t K, int64_t ldw,
                        const float* s, const void* parts, size_t parts_bytes, int64_t B,
                        float* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * lq_stream_read -- a plain read of `bytes` bytes of device memory at
 * `buffer` (16-byte aligned, bytes % 16 == 0), each byte once: the HBM read
 * rate the one-token lq_gemv (which reads each weight byte once) is
 * measured against.  sink: device uint32 [4 * compute units], caller-owned;
 * written only in the unlikely case that the buffer's words fold to one
 * fixed value (which keeps the loads from being removed).  Errors as the
 * other calls; bytes == 0 is a no-op.
 */
lq_status lq_stream_read(const void* buffer, size_t bytes, uint32_t* sink, void* stream);

/*
 * lq_gemv_noalloc -- lq_gemv for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, kernels and result, without a workspace
 * argument.  The partial sums go to a scratch array the library holds in its
 * code object, one per GPU, LQ_GEMV_NOALLOC_MAX_BYTES bytes, kept until the
 * process ends; its device address is looked up once per device on the
 * first call there.  The call allocates nothing.
 * Every lq_gemv_noalloc call on one GPU uses that GPU's one array: calls
 * that may overlap on one GPU (other streams, other host threads) race and
 * must be ordered by the caller.  Each call writes all of the scratch it
 * reads, so no clearing is needed.
 * Errors as lq_gemv; a shape whose lq_gemv_workspace_size exceeds
 * LQ_GEMV_NOALLOC_MAX_BYTES returns LQ_ERR_WORKSPACE and launches nothing
 * (every workload shape of 1 to 16 tokens up to 28672 x 68096 fits).
 */
#define LQ_GEMV_NOALLOC_MAX_BYTES (16u << 20)
lq_status lq_gemv_noalloc(const uint32_t* w_packed, int64_t m, int64_t K, int64_t ldw,
                          const float* s, const float* a_lift, int64_t B, float* out,
                          void* stream);

/*
 * lq_layer_b1 -- the whole layer for one token, o = diag(s) W_q lift(T^-1 a)
 * (关键设计 4), with the lift computed inside the one-token product: each
 * workgroup of the weight stream computes the lifted activations of the
 * 1024-position slices its tables serve (u = T^-1 a for the slices'
 * channels, then a_hat_g = M^T u_g, float32) before building the tables,
 * while its first weights stream in.  No a_hat buffer, no lift launch; the
 * result is lq_lift_activations followed by lq_gemv with B == 1 (same table
 * arithmetic, a_hat summed in another order).
 * a:      [n] of a_dtype;  t_inv: [n/128][128][128] of t_dtype == a_dtype
 *         (LQ_F16, LQ_BF16 or LQ_F32), both 16-byte aligned;  t_block: 128.
 * M:      float [d][D];  w_packed: uint32 [m][ldw] (lq_pack_signs layout),
 *         ldw >= ceil(K/32), a multiple of 4, 16-byte aligned, K = n*D/d.
 * s:      float [m];  out: float [m].
 * workspace: >= lq_layer_b1_workspace_size bytes (0 when K <= 1024),
 *         256-byte aligned, caller-owned, no initialisation needed.
 * Requires n % 128 == 0, n % d == 0, 1 <= d <= D <= 256, d <= 64,
 * d*D <= 8192, K % 4 == 0, K <= 2^24, m*ldw*4 <= 2^30 (else LQ_ERR_SHAPE,
 * LQ_ERR_UNSUPPORTED or LQ_ERR_ALIGN; nothing launched).  Arithmetic as
 * lq_gemv with B == 1 (float16 activation-sum tables, exact power-of-two
 * scaling, float32 sums).
 */
lq_status lq_layer_b1_workspace_size(int64_t m, int64_t n, int32_t d, int32_t D,
                                     size_t* bytes);
lq_status lq_layer_b1(const void* a, lq_dtype a_dtype, int64_t n, const void* t_inv,
                      lq_dtype t_dtype, int32_t t_block, const float* M, int32_t d, int32_t D,
                      const uint32_t* w_packed, int64_t m, int64_t ldw, const float* s,
                      float* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * lq_gemm -- the same product for large batches, contracted on the matrix
 * cores: out[b][i] = s[i] * sum_k sigma_ik * a_lift[b][k] with a_lift in
 * 16-bit (LQ_F16 or LQ_BF16) [B][K]; signs are expanded to exact +-1 16-bit
 * tiles and multiplied with float32 accumulation.
 * w_packed: uint32 [m][ldw] (layout of lq_pack_signs), ldw >= ceil(K/32),
 *           4-byte aligned.
 * a_lift:   16-byte aligned, K % 8 == 0.
 * out:      float [B][m].
 * Requires 1 <= B < 2^31, 1 <= m < 2^31, 1 <= K <= 2^22 and ldw <= 2^22;
 * otherwise LQ_ERR_SHAPE, LQ_ERR_ALIGN or LQ_ERR_DTYPE and nothing is
 * launched.  Each output is one float32 sum in a fixed order (deterministic).
 */
lq_status lq_gemm(const uint32_t* w_packed, int64_t m, int64_t K, int64_t ldw,
                  const float* s, const void* a_lift, lq_dtype lift_dtype, int64_t B,
                  float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LQ_H_ */
