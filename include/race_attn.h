/*
 * race_attn.h -- C ABI of the RACE attention library for AMD Instinct MI355X
 * (gfx950).  Build: librace_attn.so (hand-written HIP kernels).
 *
 * RACE attention replaces softmax attention by a strictly linear sketch
 * (page "RACE Attention: A Strictly Linear-Time Attention for Long-Sequence
 * Training", gist.science/zh/paper/2510.04008, technical summary §2.2 and
 * §2.3; the es/pt/fr/de pages of the same paper, technical summaries §2):
 *
 *   1. each row x of Q and K is L2-normalised, projected on Gaussian
 *      hyperplanes W[L][P][d] and squashed, z = tanh(W x_hat);
 *   2. per table l, the row is soft-assigned over the R = 2^P hypercube
 *      corners c_r in {-1,+1}^P: phi_l = softmax_r(<z_l, c_r> / tau), with
 *      c_rp = +1 when bit p of r is set;
 *   3. the keys are summed into per-table bucket statistics
 *      A_l = sum_j phi_l(k_j) and B_l = sum_j phi_l(k_j) v_j^T;
 *   4. query i reads out o_i = sum_l phi_l(q_i)^T B_l / sum_l phi_l(q_i)^T A_l;
 *   5. in causal mode the sums run over keys j <= i only (streaming
 *      cumulative statistics, zh §2.3).
 *   tau is the soft-hash temperature (tau = 1/beta of zh §3).
 *
 * Conventions shared by every entry point
 *   - Q, K, V, O, dO, dQ, dK, dV: device pointers to contiguous [B][H][N][d]
 *     tensors of type `dt` (RACE_F32: float, RACE_BF16: bfloat16 bits,
 *     RACE_F16: IEEE half bits).  RACE_F16 rows are read exactly, staged
 *     and multiplied as bf16 like RACE_BF16 rows (the matrix-core operands
 *     of both are bf16, with fp32 sums) and the outputs are rounded to fp16.
 *   - W: device pointer, contiguous fp32 [L][P][d], shared by every (b, h).
 *   - den: device pointer, fp32 [B][H][N]: the readout denominator
 *     m_i = sum_l phi_l(q_i)^T A_l of every row, written by the forward and
 *     read by the backward (the analogue of a softmax log-sum-exp).
 *   - workspace: device pointer of at least race_attn_workspace_bytes() bytes,
 *     256-byte aligned, owned by the caller; its contents are scratch and
 *     need not be preserved between calls.
 *   - stream: a hipStream_t.  Every kernel is enqueued on it; calls return
 *     after enqueueing, without synchronising.  The library never allocates,
 *     frees or synchronises, keeps no global mutable state and is safe to
 *     call from several threads.
 *   - Supported: d = 64, P = 4, 1 <= L <= 128 (L <= 32 for RACE_F32; for
 *     16-bit rows L > 32 runs as passes over tables 0..31, 32..63, ..., each
 *     adding its fp32 partial sums to the previous passes' before the last
 *     pass finishes the outputs); for RACE_BF16 and
 *     RACE_F16 with L <= 32 also d = 32 (the
 *     rows are zero-padded to 64 columns on chip: the same work per token as
 *     d = 64, half the memory traffic) and P = 1, 2, 3 (the kernels keep 4
 *     hyperplanes per table with t = 0 on the padding ones, an exact
 *     reduction to the P-plane corner product at the work of P = 4);
 *     for RACE_BF16 and RACE_F16 also P = 5 and 6 at any L <= 128 (a table of
 *     2^P buckets runs as 2^(P-4) virtual tables of 16: the Walsh features
 *     of hyperplanes 0..3 times those of hyperplanes 4, 5, whose kernels add
 *     up to the table's; the work of L 2^(P-4) tables of P = 4, in passes of
 *     32) and d = 128 with L <= 32, P <= 4 (the rows are hashed once over all
 *     128 elements, then the chunk kernels run on value columns 0..63 and
 *     64..127; the saved buffer keeps the hash features of Q and K, without
 *     it the backward rehashes),
 *     any B, H, N >= 1 (int64 offsets), tau finite and > 0.
 *   - chunk: tokens per scan segment, 0 = the library chooses; otherwise a
 *     multiple of 16.  It changes only the order of the floating-point sums.
 *
 * Errors are returned synchronously, before anything is enqueued, and leave
 * every output untouched:
 *   RACE_ERR_NULL        a required pointer is NULL
 *   RACE_ERR_SHAPE       B, H, N, d, L or P not positive, or N too large
 *   RACE_ERR_UNSUPPORTED valid but not implemented (d, P, L, dtype)
 *   RACE_ERR_TAU         tau not finite or tau <= 0
 *   RACE_ERR_CHUNK       chunk not 0 and not a positive multiple of 16
 *   RACE_ERR_WORKSPACE   ws_bytes smaller than required, or misaligned
 *   RACE_ERR_HIP         a kernel launch failed (hipGetLastError)
 * Non-finite input values propagate to the outputs; they are not checked.
 */
#ifndef RACE_ATTN_H
#define RACE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Both enums are int-sized.  Seen from C++ they have int as fixed underlying
 * type, so any int a C caller passes (an unknown dtype, say) is a value the
 * library can test and refuse rather than an out-of-range enum. */
#ifdef __cplusplus
#define RACE_ENUM_INT : int
#else
#define RACE_ENUM_INT
#endif

typedef enum RACE_ENUM_INT {
    RACE_OK = 0,
    RACE_ERR_NULL = 1,
    RACE_ERR_SHAPE = 2,
    RACE_ERR_UNSUPPORTED = 3,
    RACE_ERR_TAU = 4,
    RACE_ERR_CHUNK = 5,
    RACE_ERR_WORKSPACE = 6,
    RACE_ERR_HIP = 7
} race_status_t;

typedef enum RACE_ENUM_INT { RACE_F32 = 0, RACE_BF16 = 1, RACE_F16 = 2 } race_dtype_t;

/* Workspace size, in bytes, that race_attn_forward (for_backward = 0),
 * race_attn_backward (for_backward = 1), race_attn_backward_dw
 * (for_backward = 2; RACE_ERR_UNSUPPORTED where that entry point is),
 * race_attn_state_add_fast (for_backward = 3, with causal = 1, chunk = 0;
 * RACE_ERR_UNSUPPORTED where that entry point is) or race_attn_forward_hard
 * and race_attn_forward_hard_counts (for_backward = 4) needs
 * for this problem.  Pure host function; `bytes` (host pointer) receives the
 * size. */
race_status_t race_attn_workspace_bytes(int B, int H, int64_t N, int d, int L, int P,
                                        int causal, int chunk, race_dtype_t dt,
                                        int for_backward, size_t *bytes);

/* Forward pass, steps 1-5 above (zh §2.2 bucket aggregation and output
 * reconstruction; zh §2.3 causal streaming).  Writes O [B][H][N][d] (type dt)
 * and den [B][H][N] (fp32). */
race_status_t race_attn_forward(const void *Q, const void *K, const void *V, const float *W,
                                int L, int P, float tau, int causal, int B, int H, int64_t N,
                                int d, race_dtype_t dt, int chunk, void *O, float *den,
                                void *workspace, size_t ws_bytes, void *stream);

/* Forward pass with hard hashing: each row falls in exactly one corner per
 * table, r_l(x) = sum_p [u_lp >= 0] 2^p with u = W x (the signs of W x_hat),
 * and the bucket sums of steps 3-5 are true counts and value sums (the
 * tau -> 0 limit of step 2: the original RACE sketch and YOSO-style
 * attention the pages contrast soft hashing with, zh §2.2 and §3).
 * o_i = sum_l B_l[r_l(q_i)] / sum_l A_l[r_l(q_i)] over keys j <= i (causal)
 * or all keys; den_i = that count.  No tau.  Inference only: the hash has no
 * gradient.  A query that collides with no visible key in any table (the
 * sums are empty) gets den = 0 and o = 0.
 * RACE_BF16 / RACE_F16 rows with d = 32 or 64 and L <= 32, P <= 4 (or, for
 * P = 5 and 6, L 2^(P-4) <= 32: each table of 2^P buckets as 2^(P-4) tables
 * of 16), with N L < 2^31, run on the bucket ids of race_attn_hash_ids (every
 * sign decided on exact products):
 * int32 counts, kept and gathered exactly, and fp32 value sums (read as
 * bf16 matrix-core operands, the precision of the outputs); den is the count
 * (exact below 2^24).  Other shapes with P <= 4 (fp32 rows, L > 32) run the
 * chunked soft kernels with t = +-1 (counts through the sums' fp32 and bf16
 * arithmetic); P = 5, 6 elsewhere, and P > 6, return RACE_ERR_UNSUPPORTED.
 * workspace: race_attn_workspace_bytes(..., for_backward = 4). */
race_status_t race_attn_forward_hard(const void *Q, const void *K, const void *V,
                                     const float *W, int L, int P, int causal, int B, int H,
                                     int64_t N, int d, race_dtype_t dt, int chunk, void *O,
                                     float *den, void *workspace, size_t ws_bytes, void *stream);

/* race_attn_forward_hard that also writes every row's count
 * sum_l A_l[r_l(q_i)] as int32 [B][H][N] (device pointer `count`, exact at any
 * length).  Only where the bucket-id kernels run (see above);
 * RACE_ERR_UNSUPPORTED otherwise. */
race_status_t race_attn_forward_hard_counts(const void *Q, const void *K, const void *V,
                                            const float *W, int L, int P, int causal, int B, int H,
                                            int64_t N, int d, race_dtype_t dt, int chunk, void *O,
                                            float *den, int32_t *count, void *workspace,
                                            size_t ws_bytes, void *stream);

/* Backward pass: the exact gradient of the forward (the pages state the
 * method is differentiable end to end, es §2 item 3, fr §3 item 3).  Given
 * Q, K, V, W, the forward's O and den, and dO = dLoss/dO, writes dQ, dK, dV
 * (type dt, [B][H][N][d]).  W is a fixed random projection: no dW. */
race_status_t race_attn_backward(const void *Q, const void *K, const void *V, const float *W,
                                 const void *O, const float *den, const void *dO, int L,
                                 int P, float tau, int causal, int B, int H, int64_t N, int d,
                                 race_dtype_t dt, int chunk, void *dQ, void *dK, void *dV,
                                 void *workspace, size_t ws_bytes, void *stream);

/* Right-padded batches: batch b holds seqlens[b] rows (0 <= seqlens[b] <= N
 * after clamping) followed by padding.  Each sequence is attended on its own
 * rows only (causal or not), as if it had been passed alone with N =
 * seqlens[b]; padding rows are never read and their outputs (O, den; dQ, dK,
 * dV) are left as they are, so padding costs no work.  seqlens: device
 * pointer, int32 [B], read by the kernels.  Otherwise as race_attn_forward /
 * race_attn_backward; the backward also writes dW when dW is not NULL (as
 * race_attn_backward_dw: RACE_BF16 / RACE_F16, workspace with
 * for_backward = 2).  No saved state.  chunk = 0 picks the dense default
 * (about one segment per compute unit over all B H N rows); with unequal
 * lengths the segments past a sequence's end have no work, and a smaller
 * chunk (about B H N / 2048) keeps more workgroups busy.  d = 128 rows:
 * RACE_ERR_UNSUPPORTED. */
race_status_t race_attn_forward_padded(const void *Q, const void *K, const void *V,
                                       const float *W, int L, int P, float tau, int causal, int B,
                                       int H, int64_t N, int d, race_dtype_t dt, int chunk,
                                       const int *seqlens, void *O, float *den, void *workspace,
                                       size_t ws_bytes, void *stream);
race_status_t race_attn_backward_padded(const void *Q, const void *K, const void *V,
                                        const float *W, const void *O, const float *den,
                                        const void *dO, int L, int P, float tau, int causal, int B,
                                        int H, int64_t N, int d, race_dtype_t dt, int chunk,
                                        const int *seqlens, void *dQ, void *dK, void *dV,
                                        float *dW, void *workspace, size_t ws_bytes, void *stream);

/* Packed batches (variable-length sequences without padding): every head's
 * rows are the B sequences back to back, Q, K, V, O, dO, dQ, dK, dV being
 * [H][T][d] and den [H][T]; sequence b holds rows cu_seqlens[b] ..
 * cu_seqlens[b + 1] - 1 of each head (cu_seqlens: device pointer, int32
 * [B + 1], non-decreasing from 0 to T, read by the kernels; values are
 * clamped to [0, T]).  Each sequence is attended on its own rows only, as if
 * it had been passed alone (causal or not); every row of T belongs to one
 * sequence.  max_seqlen bounds every sequence's length (longer ones are cut
 * to it) and sizes the workspace: race_attn_workspace_bytes(B, H,
 * max_seqlen, ...), as for race_attn_forward_padded.  T <= B max_seqlen.
 * RACE_BF16 and RACE_F16 rows only (the fused kernels: d = 32 or 64; any L up
 * to 128, P up to 6); RACE_ERR_UNSUPPORTED otherwise.  The backward writes dW when dW
 * is not NULL (workspace with for_backward = 2).  chunk = 0 as for the padded
 * entry points. */
race_status_t race_attn_forward_varlen(const void *Q, const void *K, const void *V,
                                       const float *W, int L, int P, float tau, int causal, int B,
                                       int H, int64_t T, int64_t max_seqlen, int d,
                                       race_dtype_t dt, int chunk, const int *cu_seqlens, void *O,
                                       float *den, void *workspace, size_t ws_bytes, void *stream);
race_status_t race_attn_backward_varlen(const void *Q, const void *K, const void *V,
                                        const float *W, const void *O, const float *den,
                                        const void *dO, int L, int P, float tau, int causal, int B,
                                        int H, int64_t T, int64_t max_seqlen, int d,
                                        race_dtype_t dt, int chunk, const int *cu_seqlens,
                                        void *dQ, void *dK, void *dV, float *dW, void *workspace,
                                        size_t ws_bytes, void *stream);

/* Per-kernel timing for the *_ex entry points.  The caller creates the HIP
 * events (hipEventCreate, timing enabled) and owns them; the library records
 * start[i] / stop[i] on the call's stream around the i-th kernel it enqueues
 * (at most `capacity` kernels, capacity <= RACE_TRACE_MAX) and sets count
 * and name[i] (static strings).  Elapsed times are read by the caller after
 * the stream has completed. */
#define RACE_TRACE_MAX 24
typedef struct {
    int capacity;
    int count;
    void *start[RACE_TRACE_MAX];
    void *stop[RACE_TRACE_MAX];
    const char *name[RACE_TRACE_MAX];
} race_trace_t;

/* Size, in bytes, of the state that race_attn_forward_ex can save for
 * race_attn_backward_ex.  16-bit rows: the per-segment prefix sums of the
 * keys' bucket statistics with the per-head totals (step 3 / zh §2.3, fp32),
 * and the squashed projections t of Q and K with their derivatives (steps
 * 1-2, fp16, 512 bytes per row of Q and of K at L = 32).  RACE_F32 rows: t
 * and its derivative of Q and of K in fp32 (1024 bytes per row of each at
 * L = 32); the fp32 backward keeps the key statistics in another layout and
 * sums them again.  Pure host function. */
race_status_t race_attn_saved_bytes(int B, int H, int64_t N, int d, int L, int P, int causal,
                                    int chunk, race_dtype_t dt, size_t *bytes);

/* race_attn_forward / race_attn_backward with optional tracing and an
 * optional saved state.
 *   trace: may be NULL.
 *   saved: device pointer (256-byte aligned, race_attn_saved_bytes bytes,
 *     owned by the caller) or NULL.  The forward writes the state there
 *     (its outputs are the same either way); a backward given the same
 *     buffer, for the same Q, K, V, W, tau, causal and chunk, reads it
 *     instead of recomputing it (the gradients agree to rounding; bitwise
 *     for RACE_F32 rows).  Ignored when race_attn_saved_bytes is 0.  A misaligned saved buffer is
 *     RACE_ERR_WORKSPACE.
 * With trace = NULL and saved = NULL these are exactly the plain entry
 * points. */
race_status_t race_attn_forward_ex(const void *Q, const void *K, const void *V, const float *W,
                                   int L, int P, float tau, int causal, int B, int H, int64_t N,
                                   int d, race_dtype_t dt, int chunk, void *O, float *den,
                                   void *workspace, size_t ws_bytes, void *stream, void *saved,
                                   race_trace_t *trace);
race_status_t race_attn_backward_ex(const void *Q, const void *K, const void *V,
                                    const float *W, const void *O, const float *den,
                                    const void *dO, int L, int P, float tau, int causal, int B,
                                    int H, int64_t N, int d, race_dtype_t dt, int chunk, void *dQ,
                                    void *dK, void *dV, void *workspace, size_t ws_bytes,
                                    void *stream, const void *saved, race_trace_t *trace);

/* Diagnostic: the polynomials the bf16 kernels (RACE_BF16 and RACE_F16 rows)
 * use for the squash
 * t = tanh(tanh(v) / tau) and its derivative dt/dv (steps 1-2; zh §2.2).
 * With e = exp(-2|v|) and y = 2e - 1, the kernels evaluate
 *   t = sign(v) |sum_k coef[k] y^k|      (race_attn_squash_coeffs)
 *   dt/dv = sum_k coef[k] y^k            (race_attn_squash_deriv_coeffs)
 * for k = 0 .. *deg, in fp16 arithmetic (y rounded from fp32, fused
 * multiply-adds), with fp16 coefficients (returned exactly as floats): a
 * Chebyshev interpolation on e in [0, 1] fitted in fp64 on the host and kept
 * when its fp16 evaluation stays within 1.5e-3 of t and 1.5e-3 max(1, 1/tau)
 * of dt/dv.  coef receives RACE_SQUASH_MAXDEG + 1 floats (zeros past *deg).
 * *deg = -1 means the kernels evaluate the functions directly in fp32 (always
 * so for RACE_F32).  Pure host functions. */
#define RACE_SQUASH_MAXDEG 16
race_status_t race_attn_squash_coeffs(float tau, race_dtype_t dt, float *coef, int *deg);
race_status_t race_attn_squash_deriv_coeffs(float tau, race_dtype_t dt, float *coef, int *deg);

/* race_attn_backward_ex that also returns the gradient of the projection,
 * for learned hyperplanes: dW = sum over the rows x of Q and K (every batch
 * and head) of dLoss/du (x / max(|x|, 1e-12))^T, u = W x_hat (step 1), into
 * dW (device, fp32 [L][P][d], overwritten).  dQ, dK and dV are the same as
 * race_attn_backward_ex's.  The per-workgroup sums are added in a fixed order,
 * so the result does not depend on the launch.  Supported for RACE_BF16 and
 * RACE_F16 with d = 32 or 64 (RACE_ERR_UNSUPPORTED for RACE_F32 and d = 128);
 * workspace: race_attn_workspace_bytes with for_backward = 2. */
race_status_t race_attn_backward_dw(const void *Q, const void *K, const void *V,
                                    const float *W, const void *O, const float *den,
                                    const void *dO, int L, int P, float tau, int causal, int B,
                                    int H, int64_t N, int d, race_dtype_t dt, int chunk, void *dQ,
                                    void *dK, void *dV, float *dW, void *workspace,
                                    size_t ws_bytes, void *stream, const void *saved,
                                    race_trace_t *trace);

/* Streaming state (inference).  The causal recurrence of step 5 keeps running
 * bucket sums and reads them at every step (zh §2.3: each step costs the same
 * however long the prefix), so a head can be carried as a fixed-size state
 * that tokens are appended to and read from, one step at a time.
 *
 * State of one head: fp32 S[F][d + 1], F = 16 L, row f = 16 l + s:
 *   S[f][c] = sum_j psi_f(k_j) v_j[c] for c < d,  S[f][d] = sum_j psi_f(k_j),
 *   psi_{16 l + s}(x) = 2^(-P/2) prod_{p in s} t_lp(x),  t_lp = tanh(z_lp / tau),
 * over the keys j appended so far, where s is a subset of the table's
 * hyperplanes (bit p of s set when p is in it; 2^(-P/2) = 1/4 for P = 4).  For
 * P < 4 the rows are still 16 per table; those whose s contains a p >= P are
 * zero.  The corner weights of step 2
 * are phi_lr = prod_p (1 + c_rp t_lp) / 2, so psi_l is their Walsh-Hadamard
 * transform, psi(q).psi(k) = phi(q).phi(k), and S holds the bucket sums A_l,
 * B_l of step 3 in that basis.  A readout is [n | m] = sum_f psi_f(q) S[f][:],
 * o = n / m, den = m (step 4).  The states of all heads are one contiguous
 * device array [B][H][F][d + 1], owned by the caller; all zeros is the empty
 * prefix.  These entry points compute in fp32 (t with tanhf) whatever dt is.
 * Supported for 1 <= d <= 64, 1 <= P <= 4, L <= 64 and B * H <= 65535; N or T = 0
 * is a no-op (the row pointers may then be NULL; W and state may not).  Calls
 * that write one state must not overlap. */

/* Bytes of the states of B * H heads (F * (d + 1) floats each).  Pure host
 * function. */
race_status_t race_attn_state_bytes(int B, int H, int d, int L, int P, size_t *bytes);

/* Workspace bytes that race_attn_state_add needs for N tokens per head (0 for
 * N = 0).  Pure host function. */
race_status_t race_attn_state_add_workspace_bytes(int B, int H, int64_t N, int d, int L, int P,
                                                  size_t *bytes);

/* Appends N tokens per head to the states: state += sum_j psi(k_j)^T [v_j | 1]
 * for the rows of K, V ([B][H][N][d], type dt).  The tokens are summed in
 * blocks in parallel and the block sums added to the state in block order
 * (the result does not depend on the launch).  workspace: 256-byte aligned,
 * race_attn_state_add_workspace_bytes bytes, scratch. */
race_status_t race_attn_state_add(const void *K, const void *V, const float *W, int L, int P,
                                  float tau, int B, int H, int64_t N, int d, race_dtype_t dt,
                                  float *state, void *workspace, size_t ws_bytes, void *stream);

/* race_attn_state_add through the fused matrix-core kernels (RACE_BF16 /
 * RACE_F16 rows, L <= 32, d = 32 or 64): the keys' segment sums of the
 * forward (bf16 features and values, fp32 sums) and their scan give the
 * total, which is added into the state.  Much faster for long prompts; the
 * state then carries the bf16 rounding of the features and values (about
 * 1e-3 relative, the forward's own precision) instead of race_attn_state_add's
 * fp32 arithmetic.  workspace: race_attn_workspace_bytes(B, H, N, d, L, P, 1,
 * 0, dt, 3, ...) bytes (the segment states and the scan's group totals),
 * 256-byte aligned.  RACE_ERR_UNSUPPORTED for other configurations. */
race_status_t race_attn_state_add_fast(const void *K, const void *V, const float *W, int L, int P,
                                       float tau, int B, int H, int64_t N, int d,
                                       race_dtype_t dt, float *state, void *workspace,
                                       size_t ws_bytes, void *stream);

/* Decode step: appends T tokens per head in order and returns their causal
 * outputs; token i reads the state after its own key is added (step 5: keys
 * j <= i).  Q, K, V: [B][H][T][d] (type dt); O: [B][H][T][d] (type dt); den:
 * fp32 [B][H][T].  Started from the empty state, a call over a sequence gives
 * the rows of race_attn_forward with causal = 1; started from
 * race_attn_state_add of a prefix, the rows that follow it. */
race_status_t race_attn_decode(const void *Q, const void *K, const void *V, const float *W,
                               int L, int P, float tau, int B, int H, int64_t T, int d,
                               race_dtype_t dt, float *state, void *O, float *den, void *stream);

/* Readout without appending: o_i = n_i / m_i with [n_i | m_i] = psi(q_i) S
 * for the T rows of Q ([B][H][T][d]); the state is only read.  Over the
 * state of a key set this is race_attn_forward with causal = 0 on those keys.
 * A state with no keys gives m = 0 and non-finite o. */
race_status_t race_attn_state_readout(const void *Q, const float *W, int L, int P, float tau,
                                      int B, int H, int64_t T, int d, race_dtype_t dt,
                                      const float *state, void *O, float *den, void *stream);

/* Static, NUL-terminated description of a status code. */
const char *race_attn_status_string(race_status_t status);

/* Hard-hash bucket ids (the tau -> 0 limit of step 2, zh §2.2 and §3: the
 * original RACE count arrays): ids[row][l] = sum_p [u_lp >= 0] 2^p with
 * u = W x over the `rows` rows of X ([rows][d], type dt; d a multiple of 8,
 * at most 128; 1 <= L <= 128, 1 <= P <= 6), as uint8 [rows][L] (device
 * pointer).  The sign of x / |x| is that of x, so rows are not normalised; a
 * zero row falls in the last corner (every u = 0 counts as >= 0).  W and the
 * row are split into bf16 terms that add up to their values exactly, so
 * every product is exact and only the fp32 additions round: a decision can
 * differ from the exact sign only where |sum_t W_t x_t| <= n 2^-24 sum_t
 * |W_t x_t|, n = 3 t (d rounded up to 32) + 16, t = 1, 2, 3 row terms for
 * bf16, fp16, fp32.  workspace: race_attn_hash_ids_workspace_bytes (the W
 * terms), 256-byte aligned.  rows = 0 returns RACE_OK without enqueueing. */
race_status_t race_attn_hash_ids_workspace_bytes(int L, int P, int d, size_t *bytes);
race_status_t race_attn_hash_ids(const void *X, int64_t rows, int d, race_dtype_t dt,
                                 const float *W, int L, int P, uint8_t *ids, void *workspace,
                                 size_t ws_bytes, void *stream);

/* Bytes of the device scratch array that race_attn_forward_noalloc uses as
 * its workspace (one array per GPU, held until the process ends). */
#define RACE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/* race_attn_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The workspace race_attn_forward would
 * take is a file-scope device array of RACE_NOALLOC_SCRATCH_BYTES bytes in
 * the library instead (one per GPU; its address is looked up once per
 * device, on the first call with that device current).  This entry point
 * calls no hipMalloc, hipFree or allocating routine, and no saved state or
 * trace is taken.  Problems whose race_attn_workspace_bytes(..., 0) exceeds
 * RACE_NOALLOC_SCRATCH_BYTES return RACE_ERR_WORKSPACE before anything is
 * enqueued (with chunk = 0 and 16-bit rows that is about 300,000 tokens at
 * L = 32, the segment states taking about 42 MB of it).  `stream` must
 * belong to the current device.  Every call on a GPU shares that GPU's
 * array: calls that overlap on one GPU (two streams, or two threads) race
 * and must be ordered by the caller.  Every scratch element the kernels read
 * is written earlier in the same call, so nothing needs clearing and the
 * contents left by a previous call do not matter.  Results equal
 * race_attn_forward's for the same arguments. */
race_status_t race_attn_forward_noalloc(const void *Q, const void *K, const void *V,
                                        const float *W, int L, int P, float tau, int causal,
                                        int B, int H, int64_t N, int d, race_dtype_t dt, int chunk,
                                        void *O, float *den, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RACE_ATTN_H */
