/*
 * ttt.h -- C ABI of libttt.so: the forward scan of a Test-Time-Training (TTT)
 * layer on one AMD Instinct MI355X (gfx950).
 *
 * The layer's hidden state is a per-head fast weight W.  Each mini-batch of
 * b tokens takes one gradient step of the reconstruction loss
 *     l(W; k, v) = 1/2 || f(k; W) - v ||^2
 * and every token reads out y = f(q; W) with the weights after its own
 * update.  Definitions: "Test-Time Training Layers: How Inner-Loop Gradient
 * Descent Replaces the Transformer KV Cache with Expressive Hidden Models"
 * (news.premlal.in), section "The Core Mechanism", steps 1-3, and section
 * "Hardware Parallelization: The Dual Form and Mini-Batch GPU Acceleration";
 * "Test-Time Training (TTT) Layers for Sequence Modeling"
 * (dileepadev.github.io), sections "Mathematical Formulation" and
 * "Variants: TTT-Linear vs. TTT-MLP".
 *
 * Conventions shared by every entry point:
 *   - Row-vector form f(z; W) = z W; W[i][j] has i = input, j = output.
 *   - Within a mini-batch every gradient is taken at the chunk-start W and
 *     summed (no 1/b) in token order; a final partial mini-batch
 *     (T mod b != 0) follows the same rules.
 *   - eta is one fp32 learning rate per head.
 *   - All arrays are dense, row-major, and live in DEVICE memory owned by the
 *     caller.  The library allocates no memory and keeps no state between
 *     calls.  The TTT-Linear scan and its backward take a caller-owned device
 *     workspace (sized by ttt_linear_workspace_bytes /
 *     ttt_linear_backward_workspace_bytes for the same sizes); its contents
 *     need no initialisation and are scratch after the call.  Calls that use
 *     one workspace must be ordered (e.g. on one stream).
 *   - qkv_dtype selects the element type of Q/K/V/Y (and q/k/v/y): TTT_F32
 *     (float) or TTT_BF16 (bfloat16 bits, round-to-nearest-even on output).
 *     Fast-weight state is always fp32.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and the call returns without synchronising; no call makes a
 *     synchronising HIP call, so every call can be captured into a HIP graph.
 *     Segment plans and workspace sizes use the current device's
 *     compute-unit count, as the size queries do: pass a stream of the
 *     current device (or of a device with as many compute units).
 *   - Arguments are validated before any HIP call; on an error nothing is
 *     launched and nothing is written.  No C++ exception crosses the ABI.
 *   - Results are deterministic run to run (no atomics, fixed reduction
 *     order).
 */
#ifndef TTT_H
#define TTT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TTT_F32 = 0,
    TTT_BF16 = 1
} ttt_dtype;

typedef enum {
    TTT_OK = 0,
    TTT_ERR_INVALID_ARG = -1,   /* null pointer, negative size, b < 1, aliasing */
    TTT_ERR_UNSUPPORTED = -2,   /* shape or dtype outside what the kernels cover */
    TTT_ERR_HIP = -3            /* a HIP call or kernel launch failed */
} ttt_status;

/*
 * TTT-Linear, chunked dual form.  Inner model f(z; W) = z W with W [d][d].
 * Per mini-batch (rows = tokens of the chunk, W = chunk-start weights):
 *     E      = K W - V
 *     Y      = Q W - eta_h * tril(Q K^T) E        (diagonal kept)
 *     W_next = W - eta_h * K^T E
 * which is exactly mini-batch gradient descent on the loss above with the
 * readout after each token's update (the dual form named in the section
 * "Hardware Parallelization" of the news.premlal.in page; the dual-form
 * paragraph of the ren-xubin.github.io essay).
 *
 *   Q, K, V      [B][H][T][d], qkv_dtype, read only.
 *   W0           fp32, [H][d][d] shared over the batch (w0_per_batch = 0) or
 *                [B][H][d][d] (w0_per_batch = 1).
 *   eta          fp32 [H].
 *   Y            [B][H][T][d], qkv_dtype, written.
 *   W_out        fp32 [B][H][d][d], the weights after the last token.  It may
 *                be the same pointer as W0 when w0_per_batch = 1 (in-place
 *                state update); no other overlap between an output and any
 *                argument is allowed.
 *   B, H, T      >= 0.  B*H = 0 is a no-op.  T = 0 writes W_out = W0.
 *                B*H above 2^20 returns TTT_ERR_UNSUPPORTED (for every entry
 *                point).
 *   d            16, 32, 64 or 128.
 *   b            mini-batch size, 1 <= b <= 64.  (d = 64, b = 16 runs the
 *                MFMA kernels; other shapes run a plainer kernel.)
 *
 * Segmented scan (d = 64, b = 16, when the chains are too few to fill the
 * GPU).  A mini-batch maps the weights affinely,
 *     W_next = (I - eta_h K^T K) W + eta_h K^T V,
 * so a run of mini-batches does too: W_end = M W_start + N.  The T tokens of
 * each chain are then cut into segments (a whole number of mini-batches
 * each); one launch computes (M, N) of every segment but the last, one
 * composes them into every segment's start state, and one runs all segments'
 * scans at once.  The result is the same mini-batch descent; only the fp32
 * rounding order of the state differs from a single-segment scan.  The
 * maps and start states (B*H*(3 nseg - 2)*d*d*4 bytes) live in the caller's
 * workspace.  The call uses the segment count ttt_linear_segments reports
 * when workspace_bytes >= ttt_linear_workspace_bytes(B, H, T, d, b,
 * qkv_dtype); with less it uses the fastest count whose maps and states fit
 * (NULL / 0 bytes: one segment, which needs none).  The environment variable
 * TTT_LINEAR_SEGMENTS=S (1..30) forces S segments (fewer if they do not fit).
 * bf16 at d = 64, b = 16 may use the fused layout (ttt_linear_fused
 * reports it; ttt_linear_forward_ex with the prologue weighs it the same
 * way): the first launch also scans segment 0,
 * which then needs no map and is shorter than the others, and the
 * composition starts from its end state; with S - 1 workgroups per chain in
 * each launch, one more segment fits the GPU.  TTT_LINEAR_FUSED=0 turns it
 * off.  Same workspace size.
 *
 * fp32 Q/K/V at d = 64, b = 16 with B*H*4 <= the GPU's compute units: each
 * chain's W is split by columns over 4 workgroups (the dual form keeps W's
 * output columns apart), and the segments compose their own start states
 * (no composition launch).  Same arithmetic, another order of the sums over
 * the 64 input rows.  TTT_LINEAR_F32_COLS=0 keeps one workgroup per chain.
 *
 *   workspace    device memory of workspace_bytes bytes (may be NULL when
 *                workspace_bytes is 0), owned by the caller; must not overlap
 *                any other argument.
 *
 * Errors: TTT_ERR_INVALID_ARG (also workspace_bytes < 0, or a NULL workspace
 * with workspace_bytes > 0), TTT_ERR_UNSUPPORTED (d, b, dtype, T above
 * 2^31 - 1 or the kernels' own length bound, or on-chip memory the shape
 * needs), TTT_ERR_HIP (a kernel launch failed).
 */
int ttt_linear_forward(const void* Q, const void* K, const void* V, int qkv_dtype,
                       const float* W0, int w0_per_batch, const float* eta,
                       int64_t B, int64_t H, int64_t T, int d, int b,
                       void* Y, float* W_out, void* workspace, int64_t workspace_bytes,
                       void* stream);

/*
 * ttt_linear_forward for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments without the workspace, same plan
 * and kernels as ttt_linear_forward given at least
 * ttt_linear_workspace_bytes of workspace, so the results are identical bit
 * for bit.  The segment maps and start states go to a static device array of
 * ttt_linear_noalloc_max_workspace_bytes() (16 MiB) that every device the
 * library runs on holds until the process ends (the copy of the device that
 * `stream` belongs to is used); sizes whose plan needs more
 * return TTT_ERR_UNSUPPORTED (every planned call on a 256-CU MI355X fits:
 * at most B*H*(3 S - 2) matrices of 16 KB with B*H*S <= 256).  The call
 * allocates nothing.  Its contents need no clearing (every byte read is
 * written first in the same call).  All calls on one device share that
 * array: calls that overlap in time on one device (different streams, or
 * host threads without ordering) race on it and must be serialised by the
 * caller.  Errors as for ttt_linear_forward; TTT_ERR_HIP also if the array's
 * device address cannot be obtained.
 */
int ttt_linear_forward_noalloc(const void* Q, const void* K, const void* V, int qkv_dtype,
                               const float* W0, int w0_per_batch, const float* eta,
                               int64_t B, int64_t H, int64_t T, int d, int b,
                               void* Y, float* W_out, void* stream);

/* Bytes of the static array ttt_linear_forward_noalloc uses. */
int64_t ttt_linear_noalloc_max_workspace_bytes(void);

/*
 * Workspace bytes ttt_linear_forward (and ttt_linear_forward_ex) uses for
 * these sizes on the current device: B*H*(3 S - 2)*d*d*4 for the S segments
 * ttt_linear_segments reports, 0 when unsegmented.  Negative ttt_status for
 * sizes the forward would reject.  Needs no device memory; queries the
 * device's compute-unit count.
 */
int64_t ttt_linear_workspace_bytes(int64_t B, int64_t H, int64_t T, int d, int b, int qkv_dtype);

/*
 * ttt_linear_forward with the layer's input prologue fused into the scan:
 *   - LayerNorm of every q and k row over the head dim before the inner loop
 *     (the TTT-Linear listing in the "Hardware Parallelization" section of the
 *     news.premlal.in page normalises the projected keys and queries):
 *         x <- (x - mean) / sqrt(var + ln_eps) * gamma_h + beta_h,
 *     biased variance, one (gamma, beta) pair per head; V is not normalised;
 *   - a step size per token instead of the head's (the uTTT write-up on
 *     thelatestinai.com, Table D3: learning rates per token, head and
 *     matrix): token t's gradient term is scaled by eta_tok[b][h][t], i.e.
 *         Y = Q W - tril(Q K^T) diag(eta) E,   W_next = W - K^T diag(eta) E.
 *
 *   eta_tok      fp32 [B][H][T], or NULL for the head's eta (then eta [H]).
 *   ln_q, ln_k   fp32 [H][2][d] (gamma row, then beta row), or NULL for none.
 *   ln_eps       > 0 when either LayerNorm is given.
 *   read_mode    0: token t reads out with the weights after its own update
 *                (the pages' rule, as ttt_linear_forward); 1: every token of
 *                a mini-batch reads out with the mini-batch's start weights,
 *                Y = Q W (the uTTT write-up, Figure 2(a): forward reads use
 *                the chunk-start state).  The state recurrence is the same.
 * Everything else as for ttt_linear_forward (eta [H] must be valid even when
 * eta_tok is given).  With all three NULL and read_mode 0 this is
 * ttt_linear_forward.  The
 * prologue runs in the d = 64, b = 16 MFMA kernels (and their segment maps)
 * only: other shapes return TTT_ERR_UNSUPPORTED.  With bf16 inputs the
 * normalised rows are rounded to bf16 before the products, as the inputs
 * would be.  eta_tok, ln_q and ln_k must not overlap Y or W_out.
 */
int ttt_linear_forward_ex(const void* Q, const void* K, const void* V, int qkv_dtype,
                          const float* W0, int w0_per_batch, const float* eta,
                          const float* eta_tok, const float* ln_q, const float* ln_k, float ln_eps,
                          int read_mode, int64_t B, int64_t H, int64_t T, int d, int b,
                          void* Y, float* W_out, void* workspace, int64_t workspace_bytes,
                          void* stream);
/*
 * TTT-MLP, chunked dual form.  Inner model f(z) = SiLU(z W1) W2, W1 [d][m],
 * W2 [m][d], no biases ("Test-Time Training (TTT) Layers for Sequence
 * Modeling", section "Variants": a two-layer MLP with a SiLU non-linearity).
 * Per mini-batch, all gradients at the chunk-start (W1, W2), the inner
 * backward pass fused into the scan:
 *     Hk = K W1, Ak = SiLU(Hk), E = Ak W2 - V
 *     D  = (E W2^T) * SiLU'(Hk)
 *     Hq = Q W1 - eta_h tril(Q K^T) D,   Aq = SiLU(Hq)
 *     Y  = Aq W2 - eta_h tril(Aq Ak^T) E
 *     W1 <- W1 - eta_h K^T D,  W2 <- W2 - eta_h Ak^T E
 *
 *   Q, K, V, Y   as for ttt_linear_forward.
 *   W1_0, W2_0   fp32 [H][d][m], [H][m][d] (w0_per_batch = 0) or with a
 *                leading [B] (w0_per_batch = 1).
 *   W1_out, W2_out  fp32 [B][H][d][m], [B][H][m][d].  They may equal
 *                W1_0 / W2_0 when w0_per_batch = 1.
 *   d            16, 32 or 64;  m a multiple of 16 in [16, 512];  1 <= b <= 64.
 *                (d = 64, m = 256, b = 16 runs the MFMA kernel.)
 * Errors as for ttt_linear_forward.
 */
int ttt_mlp_forward(const void* Q, const void* K, const void* V, int qkv_dtype,
                    const float* W1_0, const float* W2_0, int w0_per_batch,
                    const float* eta, int64_t B, int64_t H, int64_t T, int d, int m, int b,
                    void* Y, float* W1_out, float* W2_out, void* stream);

/*
 * TTT-Linear single-token step (online gradient descent, the b = 1 case; the
 * "Hardware Parallelization" section of the news.premlal.in page names this
 * sequential form as the one for token-by-token decoding):
 *     r = k W - v;   W <- W - eta_h k^T r;   y = q W   (updated W)
 *
 *   q, k, v      [B][H][d], qkv_dtype, read only; q and k 16-byte aligned.
 *   W            fp32 [B][H][d][d], updated IN PLACE; 16-byte aligned.
 *   eta          fp32 [H].
 *   y            [B][H][d], qkv_dtype, written; must not overlap any input.
 *   d            16, 32, 64 or 128.
 * Errors as for ttt_linear_forward.
 */
int ttt_linear_decode_step(const void* q, const void* k, const void* v, int qkv_dtype,
                           float* W, const float* eta, int64_t B, int64_t H, int d,
                           void* y, void* stream);

/*
 * Backward of the TTT-Linear scan, for outer-loop training: the gradients of
 *     L = <dY, Y> + <dW_out, W_out>
 * with respect to Q, K, V, W0 and eta, where (Y, W_out) is what
 * ttt_linear_forward computes from the same arguments.  Training the outer
 * model differentiates the layer output through the inner gradient steps
 * (the dual form of the "Hardware Parallelization" section of the
 * news.premlal.in page exists for training; the uTTT write-up on
 * thelatestinai.com, Figure 2(b): the read-output Jacobian runs backward
 * through the earlier inner updates).  Per mini-batch, in reverse order,
 * with W the chunk-start weights, E = K W - V, A = tril(Q K^T) and G the
 * gradient with respect to the weights after the chunk (G = dW_out after the
 * last one):
 *     P  = A^T dY + K G,   dV = eta_h P,   deta_h += -<P, E>
 *     dA = -eta_h tril(dY E^T)
 *     dQ = dY W^T + dA K
 *     dK = -eta_h (P W^T + E G^T) + dA^T Q
 *     G <- G + Q^T dY - eta_h K^T P
 * and dW0 = G after the first mini-batch.  The chunk-start weights are
 * recomputed from Q, K, V, W0 (nothing from the forward call is needed).
 *
 *   Q, K, V, W0, eta, B, H, T, b, w0_per_batch: as for ttt_linear_forward.
 *   dY           [B][H][T][d], qkv_dtype, read only.
 *   dW_out       fp32 [B][H][d][d], read only (pass zeros if W_out is unused).
 *   dQ, dK, dV   [B][H][T][d], qkv_dtype, written.
 *   dW0          fp32, W0's shape: [H][d][d] summed over the batch
 *                (w0_per_batch = 0) or [B][H][d][d] (w0_per_batch = 1).
 *   deta         fp32 [H], summed over the batch.
 *   d = 64 and b = 16 only (other shapes: TTT_ERR_UNSUPPORTED).
 *   B*H = 0 writes dW0 = 0 and deta = 0 (sums over an empty batch); T = 0
 *   gives dW0 = dW_out (summed over the batch when W0 is shared), deta = 0.
 * No output may overlap any other argument.
 *
 * Segments.  When the chains are too few for the GPU, the backward is cut
 * into sequence segments like the forward scan.  The cotangent G is affine
 * too: per mini-batch G_start = (I - eta_h K^T K) G_end + (Q - eta_h A K)^T dY,
 * which needs no W.  So the forward's maps and composition give every
 * segment's start W, cotangent maps composed from dW_out backwards give every
 * segment's end G, and then all segments run at once (deta and dW0 are
 * summed in a fixed order).  ttt_linear_backward_segments reports the count;
 * TTT_LINEAR_BWD_SEGMENTS=S (1..30) forces it.  Workspace, caller-owned, in
 * d*d*4-byte matrices per chain: S*ceil(ceil(T/16)/S) recomputed chunk-start
 * states (fp32 inputs; bf16 inputs keep instead each chunk's 2 KB update
 * operand, from which the kernel walks the states back: an eighth of
 * that), with S > 1 another 6 S - 4 (maps, start and end states), and one
 * more when W0 is shared (per-chain dW0).  With workspace_bytes >=
 * ttt_linear_backward_workspace_bytes(...) the call uses the count
 * ttt_linear_backward_segments reports (the prologue call of
 * ttt_linear_backward_ex may plan more segments; the query covers both);
 * with less, the fastest count that fits; if not even one segment's
 * states fit, TTT_ERR_INVALID_ARG.
 * Errors as for ttt_linear_forward.
 */
int ttt_linear_backward(const void* Q, const void* K, const void* V, int qkv_dtype,
                        const float* W0, int w0_per_batch, const float* eta,
                        int64_t B, int64_t H, int64_t T, int d, int b,
                        const void* dY, const float* dW_out,
                        void* dQ, void* dK, void* dV, float* dW0, float* deta,
                        void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Workspace bytes that serve every ttt_linear_backward and
 * ttt_linear_backward_ex call of these sizes on the current device (shared or
 * per-batch W0, with or without the prologue).  Negative ttt_status for sizes
 * the backward would reject.
 */
int64_t ttt_linear_backward_workspace_bytes(int64_t B, int64_t H, int64_t T, int d, int b,
                                            int qkv_dtype);
/*
 * ttt_linear_backward with the input prologue of ttt_linear_forward_ex: the
 * gradients of L = <dY, Y> + <dW_out, W_out> for (Y, W_out) =
 * ttt_linear_forward_ex of the same arguments, so a model whose layer
 * LayerNorms q and k (the TTT-Linear listing of the "Hardware
 * Parallelization" section of the news.premlal.in page), learns a step size
 * per token (the uTTT write-up on thelatestinai.com, Table D3) or reads out
 * with the chunk-start weights (its Figure 2(a)) trains through this call.
 * With Qn, Kn the LayerNorm'd rows, eta_t the step sizes and Et = diag(eta_t) E,
 * per mini-batch in reverse order:
 *     P  = A^T dY + Kn G,  dV = diag(eta_t) P,  deta_t = -<P_t, E_t>
 *     dA = -tril(dY Et^T)          (A = 0 and dA = 0 with read_mode 1)
 *     dQn = dY W^T + dA Kn,  dKn = -diag(eta_t) (P W^T + E G^T) + dA^T Qn
 *     G <- G + Qn^T dY - Kn^T diag(eta_t) P
 * and the LayerNorm backward takes dQn, dKn to the raw rows:
 *     dx = rstd (g gamma - mean(g gamma) - xh mean(g gamma xh)),
 *     dgamma += g xh, dbeta += g  (xh the normalised row, g its gradient).
 *
 *   Q, K            the raw rows (before the LayerNorm), as for
 *                   ttt_linear_forward_ex; eta, eta_tok, ln_q, ln_k, ln_eps,
 *                   read_mode: its prologue arguments (eta is read always).
 *   deta_tok        fp32 [B][H][T], written: d L / d eta_tok.  Must be given
 *                   exactly when eta_tok is; deta is then all zero.
 *   dln_q, dln_k    fp32 [H][2][d] (gamma row, beta row), written: summed over
 *                   the batch.  Must be given exactly when ln_q / ln_k are.
 *   the rest        as for ttt_linear_backward (dQ, dK are the gradients of
 *                   the raw rows; deta is the head step's gradient).
 * d = 64 and b = 16 only.  Computed like ttt_linear_backward (bf16 Q/K/V:
 * normalised rows rounded to bf16 for the MFMA operands; the LayerNorm and its
 * backward in fp32).  The per-token eta gradients need no reduction; gamma,
 * beta sums run over (batch, segment) in a fixed order: deterministic.
 * TTT_ERR_INVALID_ARG also for a prologue input without its gradient output
 * (or the reverse), ln_eps <= 0 with a LayerNorm, read_mode not 0 or 1, or
 * any overlap of an output with another argument.
 */
int ttt_linear_backward_ex(const void* Q, const void* K, const void* V, int qkv_dtype,
                           const float* W0, int w0_per_batch, const float* eta,
                           const float* eta_tok, const float* ln_q, const float* ln_k,
                           float ln_eps, int read_mode, int64_t B, int64_t H, int64_t T, int d,
                           int b, const void* dY, const float* dW_out, void* dQ, void* dK,
                           void* dV, float* dW0, float* deta, float* deta_tok, float* dln_q,
                           float* dln_k, void* workspace, int64_t workspace_bytes, void* stream);
/*
 * Number of sequence segments ttt_linear_backward would cut each chain into
 * for these sizes on the current device (1 = unsegmented).  Negative
 * ttt_status for arguments ttt_linear_backward would reject.
 */
int ttt_linear_backward_segments(int64_t B, int64_t H, int64_t T, int d, int b, int qkv_dtype);
/*
 * ttt_linear_decode_step with the input prologue of ttt_linear_forward_ex,
 * for one token: q and k LayerNorm'd over the head dim (ln_q, ln_k [H][2][d],
 * NULL for none; ln_eps > 0 when used), the token's own step size eta_tok
 * [B][H] (NULL: the head's eta), and read_mode 1 reading out before the
 * update (y = q W, the one-token case of the chunk-start read).  So a
 * sequence prefilled with ttt_linear_forward_ex continues token by token with
 * the same rules.  Any d of ttt_linear_decode_step; computed in fp32 (the
 * normalised rows are not rounded to bf16).  Errors as for
 * ttt_linear_decode_step; eta_tok, ln_q, ln_k must not overlap y or W.
 */
int ttt_linear_decode_step_ex(const void* q, const void* k, const void* v, int qkv_dtype,
                              float* W, const float* eta, const float* eta_tok,
                              const float* ln_q, const float* ln_k, float ln_eps, int read_mode,
                              int64_t B, int64_t H, int d, void* y, void* stream);
/*
 * Number of sequence segments ttt_linear_forward would cut each chain into
 * for these sizes on the current device, given at least
 * ttt_linear_workspace_bytes of workspace (1 = one workgroup scans the whole
 * chain).  Returns a negative ttt_status for arguments ttt_linear_forward
 * would reject.  Needs no device memory; queries the device's compute-unit
 * count.
 */
int ttt_linear_segments(int64_t B, int64_t H, int64_t T, int d, int b, int qkv_dtype);

/*
 * 1 if ttt_linear_forward uses the fused segment layout for these sizes on
 * the current device (segment 0 scanned in the maps launch), 0 if not;
 * a negative ttt_status for arguments ttt_linear_forward would reject.
 * Needs no device memory.
 */
int ttt_linear_fused(int64_t B, int64_t H, int64_t T, int d, int b, int qkv_dtype);

/*
 * TTT-Linear with momentum gradient descent.  The E2-TTT write-up
 * (zhichai.net), sections "E2-TTT's Breakthrough: A Closed-Form Solution"
 * and "Core Math (Simplified)": fast weights W and a momentum M of the same
 * shape, one step per token t on the loss above,
 *     r_t = k_t W_g - v_t,  M_t = beta_h M_{t-1} + k_t^T r_t,
 *     W_t = W_{t-1} - eta_h M_t,  y_t = q_t W_t,
 * with the gradient point W_g chosen by grad_mode:
 *   0  W_g = W_{t-1}: exact token-level steps (with beta = 0, exact online
 *      gradient descent, the same result as ttt_linear_forward with b = 1);
 *   1  W_g = the weights at the start of the token's mini-batch of b tokens
 *      (the chunk-start gradients of the section "The Curse of Efficiency";
 *      with beta = 0 the result of ttt_linear_forward with the same b).
 * The kernels run each mini-batch in a closed form: for exact steps the
 * residuals R of the chunk solve a unit lower triangular system built from
 * K K^T (one forward substitution per chunk), and the chunk-end W and M
 * follow from R with geometric sums of beta.  So b sets only the work split
 * when grad_mode = 0 (the result is the same up to rounding for every b).
 * On the MFMA path a few long chains are split into sequence segments as in
 * ttt_linear_forward: a chunk maps each column [W; M] of the state affinely,
 * so each segment's map (A of 2d x 2d, N of 2d x d) is computed from the
 * segment's inputs alone, the maps are composed into every segment's start
 * state, and the segments then run at once
 * (ttt_linear_momentum_segments gives the count).
 *
 *   Q, K, V, Y   as for ttt_linear_forward.
 *   W0           fp32, [H][d][d] (w0_per_batch = 0) or [B][H][d][d] (= 1).
 *   M0           fp32 [B][H][d][d] start momentum, or NULL for zero.
 *   eta, beta    fp32 [H]: learning rate and momentum coefficient per head.
 *   grad_mode    0 or 1 (above).
 *   W_out, M_out fp32 [B][H][d][d]: the weights and momentum after the last
 *                token.  W_out may be W0 when w0_per_batch = 1, and M_out may
 *                be M0 (in-place state update); no other overlap between an
 *                output and any argument is allowed.
 *   B, H, T, d   as for ttt_linear_forward; T = 0 writes W_out = W0 and
 *                M_out = M0 (or zero).
 *   b            1 <= b <= 64.  bf16 Q/K/V with d = 64 and b = 16 run the
 *                MFMA kernels; other shapes run a plain fp32 kernel whose
 *                on-chip memory bounds b for d = 128 (b <= 19, else
 *                TTT_ERR_UNSUPPORTED).
 *   workspace    caller-owned device memory (must not overlap any other
 *                argument): the per-chunk triangular inverses of exact steps
 *                on the MFMA path, and with sequence segments their maps and
 *                start states.  ttt_linear_momentum_workspace_bytes gives the
 *                size of the planned split; less (down to what one segment
 *                needs, 0 bytes off the MFMA path or for grad_mode 1) runs
 *                with fewer segments.
 *
 * Errors: TTT_ERR_INVALID_ARG (null or overlapping buffers, grad_mode not 0
 * or 1, a workspace smaller than required), TTT_ERR_UNSUPPORTED (sizes as for
 * ttt_linear_forward, or on-chip memory), TTT_ERR_HIP.
 */
int ttt_linear_momentum_forward(const void* Q, const void* K, const void* V, int qkv_dtype,
                                const float* W0, int w0_per_batch, const float* M0,
                                const float* eta, const float* beta, int grad_mode,
                                int64_t B, int64_t H, int64_t T, int d, int b,
                                void* Y, float* W_out, float* M_out,
                                void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Workspace bytes ttt_linear_momentum_forward uses for these sizes with its
 * planned number S of sequence segments: for exact steps on the MFMA path
 * B*H*ceil(T/32)*1024 (one 16x16 bf16 inverse per chunk of 16 tokens, stored
 * in pairs), rounded up to 256; with S > 1 also B*H*(S-1)*6*d*d*4 (the
 * segments' maps, rounded up to 256) plus B*H*S*2*d*d*4 (their start
 * states); 0 when none of these apply.  Negative ttt_status for sizes the
 * call would reject.
 */
int64_t ttt_linear_momentum_workspace_bytes(int64_t B, int64_t H, int64_t T, int d, int b,
                                            int qkv_dtype, int grad_mode);

/*
 * Sequence segments per (batch, head) chain that ttt_linear_momentum_forward
 * plans for these sizes with the workspace of
 * ttt_linear_momentum_workspace_bytes (1: no split; only the bf16 MFMA path
 * splits), or a negative ttt_status.  The environment variable
 * TTT_MOMENTUM_SEGMENTS=S (1 <= S <= 12) forces S segments (each a multiple
 * of 32 tokens, so fewer for short sequences).
 */
int ttt_linear_momentum_segments(int64_t B, int64_t H, int64_t T, int d, int b, int qkv_dtype,
                                 int grad_mode);

/* Static, human-readable text for a status code (never NULL). */
const char* ttt_status_string(int status);

/* ABI version of this header: (major << 16) | minor. */
int ttt_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TTT_H */
