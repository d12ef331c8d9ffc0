/*
 * prn.h -- C ABI of libprn: parallel Newton forward of diagonal GRU / LSTM
 * recurrences on AMD Instinct MI355X (gfx950).
 *
 * The sequential recurrence s_t = f(s_{t-1}, x_t) is replaced by K Newton
 * iterations over the whole trajectory.  Each iteration evaluates the cell
 * and its per-channel Jacobian J_t at the previous guess, forms the affine
 * maps s_t = J_t s_{t-1} + b_t with b_t = f(s^old_{t-1}, x_t) - J_t s^old_{t-1},
 * solves them with a chunked parallel scan over time, and reduces the
 * residual max|F(H)|, F_t = h_t - f(h_{t-1}, x_t).
 *
 * Sources (pararnn-torch pages):
 *   FAQs, "Does parallel Newton match sequential unroll?"    agreement tau
 *   FAQs, "How many Newton iterations should I use?"         K pinned or per T
 *   FAQs, "Does torch.compile / autocast work?"              fixed K, no host sync
 *   FAQs, "train() vs eval()"                                Newton vs sequential
 *   Numerics contract, "Two thresholds", "1. Runtime"       residual max|F(H)|
 *   shapes/layout page, contiguity and ragged packs           (1, N, d) + cu_seqlens,
 *                                                             J = 0 at segment heads,
 *                                                             unsupported pins raise
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers (hipMalloc'd or equivalent)
 *     unless a comment says "host".  Every tensor is dense, row-major and
 *     contiguous in the layout given; callers copy strided views first.
 *   - The caller owns every buffer.  The library allocates no device memory,
 *     keeps no pointer after a call returns, and is re-entrant: concurrent
 *     calls are fine as long as they use distinct workspaces and outputs.
 *   - All work is enqueued on params->stream (a hipStream_t; NULL = the null
 *     stream).  No entry point synchronises the host with the device.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     non-OK status means nothing was launched (except PRN_ERR_DEVICE, which
 *     reports a launch failure).  prn_last_error() gives the reason.
 *   - Storage dtype (params->dtype) applies to x, W, xproj, h0, H_out,
 *     state_last_out and the iterates kept in the workspace.  Arithmetic is
 *     fp32 whatever the storage dtype; stores round to nearest even.
 */
#ifndef PRN_H_
#define PRN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PRN_OK = 0,
  PRN_ERR_INVALID_ARG = 1,  /* null pointer, bad size, K < 1, bad cu_seqlens  */
  PRN_ERR_UNSUPPORTED = 2,  /* valid request this library does not implement */
  PRN_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required    */
  PRN_ERR_DEVICE = 4        /* a HIP call or kernel launch failed            */
} prn_status;

/* Cells.  Gate order inside a token's projected row:
 *   PRN_CELL_DIAG_GRU   G = 3 gates [z | r | c], state S = 1 (h)
 *       z = sig(x_z + a_z h), r = sig(x_r + a_r h), c = tanh(x_c + a_c r h),
 *       h' = (1 - z) h + z c
 *   PRN_CELL_DIAG_LSTM  G = 4 gates [i | f | o | g], state S = 2 (c, h)
 *       i,f,o = sig(x_* + a_* h), g = tanh(x_g + a_g h),
 *       c' = f c + i g, h' = o tanh(c')
 * (diagonal "mix='diag'" cells of the shapes/layout page's support table) */
enum { PRN_CELL_DIAG_GRU = 0, PRN_CELL_DIAG_LSTM = 1 };

/* Storage dtypes. */
enum { PRN_F32 = 0, PRN_BF16 = 1 };

typedef struct {
  int32_t cell;            /* PRN_CELL_DIAG_GRU | PRN_CELL_DIAG_LSTM                     */
  int32_t dtype;           /* PRN_F32 | PRN_BF16                                          */
  int64_t B;               /* batch rows; must be 1 for a ragged pack                     */
  int64_t T;               /* steps per row; for a ragged pack the total token count N    */
  int64_t d_in;            /* input width (the entry points that take x)                  */
  int64_t d_h;             /* hidden width = channels per gate                            */
  int64_t n_seqs;          /* 0: rectangular batch; > 0: segments in the ragged pack      */
  const float* a;          /* (G, d_h) fp32 diagonal recurrent weights, gate order above  */
  void* state_last_out;    /* optional (rows, S, d_h) storage dtype: final state of every
                              sequence (rows = B, or n_seqs for a pack); LSTM order (c, h) */
  void* workspace;         /* device scratch owned by the caller, 256-byte aligned         */
  size_t workspace_bytes;  /* its size; must be >= prn_workspace_bytes(params, K) (forward)
                              or prn_backward_workspace_bytes(params) (backward)          */
  void* stream;            /* hipStream_t                                                 */
  void* states_out;        /* optional (B, T, S, d_h) storage dtype, forward entry points:
                              every state s_t of the returned trajectory (LSTM (c, h);
                              for the GRU it equals H_out).  The backward pass takes it as
                              its trajectory                                                */
  int32_t picard_iters;    /* prn_newton_forward: P >= 0 Picard (Jacobi) sweeps
                              H <- f(shift(H), x) from 0 before the K Newton iterations
                              (FAQs "How many Newton iterations should I use?":
                              picard_iters), each sweep rounded to the storage dtype;
                              r_0 is then the residual of the guess H^(P).  Every sub-chunk
                              builds its own guess (H^(P)_t depends on the P steps up to t
                              only): about P * (L + P / 2) cell evaluations per sub-chunk
                              of L = 8 to 16 steps, so it is meant for a few sweeps.
                              P >= T gives the unroll itself and runs as P = T.
                              Single-pass schedule only (PRN_ALGO=tp: PRN_ERR_UNSUPPORTED) */
  void* error_out;         /* optional device uint32 word (4-byte aligned), forward and
                              backward entry points: bit 0 (PRN_FAULT_LOOKBACK) is ORed in
                              when a wait for a preceding chunk's record gave up (after about
                              65 ms of polling: another process starving this kernel); the
                              results of that call are then NaN from the chunk on (the
                              forward's residual reads +Inf).  Never cleared by the library:
                              the caller zeroes it and reads it after the stream work is
                              done.  NULL: the bit goes to a word in the workspace only     */
} prn_params;

/* Bits of prn_params.error_out. */
enum { PRN_FAULT_LOOKBACK = 1 };

/* Input projection, once per forward:
 *   xproj[b,t,g,i] = sum_j x[b,t,j] * W[g*d_h + i, j] + bias[g*d_h + i]
 * (the input weight W_x of the FAQs "decode_wx" / shapes page "W_x").
 *   x      (B, T, d_in)  storage dtype
 *   W      (G*d_h, d_in) storage dtype, rows gate-major
 *   bias   (G*d_h) fp32, or NULL for none (LSTM callers fold the +1 forget
 *          bias in here)
 *   xproj_out (B, T, G, d_h) storage dtype
 * fp32 storage: fp32-accurate products on the bf16 matrix cores (each
 * operand split exactly into three bf16 terms; the six term products of
 * weight 2^-16 or more, so the dropped part is below 3 * 2^-24 |a b|),
 * accumulated in fp32; non-finite inputs give non-finite outputs.  bf16
 * multiplies bf16 with fp32 accumulation and rounds the result to bf16.
 * Uses no workspace. */
prn_status prn_input_proj(const void* x, const void* W, const float* bias,
                          const prn_params* params, void* xproj_out);

/* Gradients of the input projection (its train-mode backward: FAQs "train()
 * vs eval()"; shapes/layout page, the train forward+backward surface and
 * W_x), given dL/dxproj:
 *   dx[b,t,j]  = sum_n dxproj[b,t,n] W[n,j]        (n = g*d_h + i)
 *   dW[n,j]    = sum_{b,t} dxproj[b,t,n] x[b,t,j]
 *   dbias[n]   = sum_{b,t} dxproj[b,t,n]
 *   dxproj     (B, T, G, d_h) storage dtype (prn_newton_backward's dxproj_out)
 *   x, W       the forward's operands: (B, T, d_in), (G*d_h, d_in) storage dtype
 *   dx_out     (B, T, d_in) storage dtype, or NULL (not computed)
 *   dW_out     (G*d_h, d_in) storage dtype, or NULL
 *   dbias_out  (G*d_h) fp32, or NULL
 * params: cell, dtype, B, T, d_in, d_h, workspace (at least
 * prn_input_proj_backward_workspace_bytes(params); it covers all three
 * outputs), stream; n_seqs must be 0 (a ragged pack is B = 1, T = N).
 * dxproj must be 16-byte aligned (it is read by the matrix-core tiles);
 * so must x when dW_out is asked for and G*d_h and d_in are multiples of
 * 256 (dW then reads both operands along their rows); the other pointers
 * need only their element alignment.
 * Products on the matrix cores as in prn_input_proj (fp32, or bf16 with fp32
 * accumulation); every sum is taken in a fixed order (the result is bitwise
 * reproducible) and rounded once to the storage dtype; dbias sums in fp32.
 * The weight gradient is split over token slices whose fp32 partial sums are
 * added in slice order.  When G*d_h and d_in are multiples of 256 its tiles
 * read both operands along their rows, and also take dbias's column sums
 * per token slice (so dbias asked for with dW_out may differ in the last
 * bits from dbias asked for without it, which sums 64-token tiles; each is
 * bitwise reproducible); otherwise both are first transposed into the
 * workspace (which then holds dxproj and x once more). */
prn_status prn_input_proj_backward(const void* dxproj, const void* x, const void* W,
                                   const prn_params* params, void* dx_out, void* dW_out,
                                   float* dbias_out);
size_t prn_input_proj_backward_workspace_bytes(const prn_params* params);

/* Parallel Newton forward (the train-mode path of the FAQs' "train() vs
 * eval()"): K iterations from the guess H = 0, then the final trajectory.
 *   xproj      (B, T, G, d_h) storage dtype, biases included
 *   h0         initial state (rows, S, d_h) storage dtype, or NULL for zeros;
 *              rows = B, or n_seqs for a ragged pack (one per segment)
 *   K          >= 1 Newton iterations (fixed; no early exit, no host sync)
 *   cu_seqlens NULL for a rectangular batch, else (n_seqs + 1) int32
 *              offsets with cu[0] = 0, non-decreasing, cu[n_seqs] = T, B = 1
 *              (shapes/layout page, ragged packs).  Each segment start is a
 *              head: J = 0 and the previous state is that segment's h0.
 *              Empty segments are allowed; their final state is their h0.
 *              Its contents are not read on the host; prn_validate_cu_seqlens
 *              checks a host copy.  Malformed contents give wrong results
 *              but never out-of-bounds accesses.
 *   H_out      (B, T, d_h) storage dtype: h of the K-th iterate (and, when
 *              params->states_out is set, every state component there)
 *   residual_out  NULL, or (K + 1) fp32: residual_out[k] = max|F(H^(k))| over
 *              batch, time, state component and channel, of the iterate as
 *              stored (H^(0) = 0).  A non-finite value reads as +Inf.  The
 *              caller applies the gate (Numerics contract: fail above 1.0).
 * Divergence is reported through the residual, never as a status.
 * Reproducibility: every output is a fixed function of the inputs and the
 * launch geometry (which depends on cell, dtype, T and the number of
 * (row, 64-channel) chains): two calls with the same arguments give
 * bitwise-equal results.  The carry into a chunk is defined as the serial
 * application of the preceding chunks' composed maps to the initial state,
 * and the look-back, whichever published prefix it starts from, performs
 * exactly those operations.
 * Environment (read at every call): PRN_ALGO=tp selects the multi-kernel
 * three-phase schedule; PRN_SPIN_LIMIT overrides the number of polls before a
 * wait for a preceding chunk gives up (0: every wait gives up at once, the
 * way to exercise the error_out path). */
prn_status prn_newton_forward(const void* xproj, const prn_params* params, const void* h0,
                              int32_t K, const int32_t* cu_seqlens, void* H_out,
                              float* residual_out);

/* prn_input_proj followed by prn_newton_forward, in one kernel: each Newton
 * workgroup computes its chunk's projected inputs on the matrix cores from x
 * and W (FAQs "How do I pass recurrent state between decode steps?":
 * decode_wx is this projection; shapes page: W_x), so the projected inputs
 * never pass through device memory unless xproj_out asks for them.
 *   x, W, bias as for prn_input_proj (d_in % 4 == 0 for fp32 storage,
 *              % 8 for bf16; x and W 16-byte aligned)
 *   h0, K, cu_seqlens, H_out, residual_out as for prn_newton_forward
 *   xproj_out  NULL, or (B, T, G, d_h) storage dtype, 16-byte aligned: also
 *              store the projected inputs (the backward pass needs them)
 * The projected inputs are bitwise those prn_input_proj computes (same
 * matrix-core instruction and summation order), so H_out and residual_out
 * equal those of prn_input_proj + prn_newton_forward bitwise whenever both
 * take the same chunk length (every LSTM, and the GRU below 64 chains), and
 * up to the rounding of another chunking otherwise.  params->d_in must be set and
 * params->picard_iters must be 0 (else PRN_ERR_UNSUPPORTED); the single-pass
 * schedule always runs (PRN_ALGO is not read).  Workspace:
 * prn_workspace_bytes(params, K), which covers both forwards.  Errors as
 * for prn_newton_forward and prn_input_proj. */
prn_status prn_newton_forward_fused(const void* x, const void* W, const float* bias,
                                    const prn_params* params, const void* h0, int32_t K,
                                    const int32_t* cu_seqlens, void* H_out, float* residual_out,
                                    void* xproj_out);

/* prn_newton_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, kernels and results as prn_newton_forward (the
 * single-pass schedule; PRN_ALGO is not read), but params->workspace and
 * workspace_bytes are ignored: the scratch (chunk records, status words,
 * residual partials) is a file-scope device array of
 * PRN_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends.  The call
 * allocates nothing (no hipMalloc, no hipFree, no allocating library call);
 * the first call on a device looks up that device's copy of the array.
 * A call needing more scratch than the array holds (prn_workspace_bytes
 * tells how much) returns PRN_ERR_WORKSPACE before anything is launched.
 * Every call on a GPU shares its array: calls that overlap on one GPU (two
 * streams, two host threads) race and must be serialised by the caller.
 * The current device must be the stream's device. */
#define PRN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
prn_status prn_newton_forward_noalloc(const void* xproj, const prn_params* params, const void* h0,
                                      int32_t K, const int32_t* cu_seqlens, void* H_out,
                                      float* residual_out);

/* Sequential unroll s_t = f(s_{t-1}, x_t) (the eval-mode path and the truth
 * the Newton result must match within tau).  Arguments as for
 * prn_newton_forward.  Uses no workspace. */
prn_status prn_sequential_forward(const void* xproj, const prn_params* params, const void* h0,
                                  const int32_t* cu_seqlens, void* H_out);

/* Bytes of workspace prn_newton_forward (and prn_newton_forward_fused)
 * needs for these params and K.  0 on invalid params, with the reason in
 * prn_last_error; the workspace-size queries clear that message first, so 0
 * with an empty message means no workspace is needed (e.g. T = 0). */
size_t prn_workspace_bytes(const prn_params* params, int32_t K);

/* Backward pass: gradients of a loss L through the recurrence, the step a
 * training iteration needs after the Newton forward (FAQs "train() vs
 * eval()"; shapes/layout page, the train forward+backward surface of the
 * diagonal cells and ragged packs).  The pages do not print the backward
 * equations; this takes the gradient of the sequential recurrence
 * s_t = f(s_{t-1}, x_t) at the given trajectory, which is the solution of
 * the adjoint (transposed, reverse-time) linear recurrence
 *     lam_t = dL/ds_t + J_{t+1}^T lam_{t+1}
 * with J_{t+1} = df/ds at step t+1, cut to 0 where step t+1 is a segment
 * head (its previous state is the segment's h0) and past the end of a row;
 * dL/ds_t is dH_t in the h component plus, at the last step of a sequence,
 * dstate_last.  It runs as a chunked parallel scan backwards in time (the
 * forward's scan machinery with the chunk order reversed), then per step
 *     dxproj_t = (ds_t/dxproj_t)^T lam_t
 *     da      += (ds_t/da)^T lam_t          (summed over rows and steps)
 *     dh0_j    = J_t^T lam_t                at the head t of sequence j
 * and an empty segment passes its dstate_last to its dh0 unchanged.
 *   xproj       (B, T, G, d_h) storage dtype, as given to the forward
 *   h0          (rows, S, d_h) storage dtype or NULL (zeros), as given to the forward
 *   cu_seqlens  NULL or the forward's ragged offsets (same contract)
 *   states      (B, T, S, d_h) storage dtype: the trajectory s_1..s_T at which
 *               the gradient is taken (states_out of the forward)
 *   dH          (B, T, d_h) storage dtype: dL/dH_out
 *   dstate_last (rows, S, d_h) storage dtype, or NULL for zero: dL/d state_last_out
 *   dxproj_out  (B, T, G, d_h) storage dtype: dL/dxproj.  The projection's own
 *               gradients are plain products of it: dW = dxproj^T x,
 *               dx = dxproj W, dbias = sum of dxproj over tokens
 *   da_out      (G, d_h) fp32: dL/da (overwritten, not accumulated)
 *   dh0_out     (rows, S, d_h) storage dtype, or NULL
 * params->a is the forward's a; params->workspace must hold at least
 * prn_backward_workspace_bytes(params); state_last_out and states_out are
 * not used.  The result is deterministic (fixed reduction orders). */
prn_status prn_newton_backward(const void* xproj, const prn_params* params, const void* h0,
                               const int32_t* cu_seqlens, const void* states, const void* dH,
                               const void* dstate_last, void* dxproj_out, float* da_out,
                               void* dh0_out);

/* Bytes of workspace prn_newton_backward needs for these params (0 on
 * invalid params; see prn_last_error). */
size_t prn_backward_workspace_bytes(const prn_params* params);

/* One T = 1 step for B independent slots: the serving decode step (FAQs,
 * "How do I pass recurrent state between decode steps?": a fixed-size carry
 * (slots, d_h) per layer; prefill with the sequential or Newton forward, then
 * decode_wx + decode_step for each T = 1 token; "train() vs eval()": T = 1
 * decode).  The token's projection and the cell step are fused:
 *   xproj_g = x W_g^T + bias_g (fp32 sums, rounded to the storage dtype as
 *             prn_input_proj's output is), s' = f(state_in, xproj).
 *   x          (B, d_in) storage dtype
 *   W, bias    (G*d_h, d_in) storage dtype and (G*d_h) fp32 or NULL, as for
 *              prn_input_proj
 *   state_in   (B, S, d_h) storage dtype, the carry, or NULL for zeros
 *   state_out  (B, S, d_h) storage dtype: the new carry; must not alias state_in
 *              (callers ping-pong two buffers)
 *   h_out      (B, d_h) storage dtype, or NULL
 * params: cell, dtype, B = slots, T = 1, d_in, d_h, a, stream.  One kernel
 * launch, no workspace, no memory set: it can be captured in a HIP graph with
 * its buffers pinned.  The result equals prn_input_proj + prn_sequential_forward
 * on the same token up to the summation order of the projection.
 * Errors (nothing is launched): PRN_ERR_INVALID_ARG for T != 1, a ragged pack
 * (n_seqs > 0), d_in < 1, NULL x / W / a / state_out, a pointer not aligned
 * to its element size, or state_in == state_out. */
prn_status prn_decode_step(const void* x, const void* W, const float* bias, const prn_params* params,
                           const void* state_in, void* state_out, void* h_out);

/* ---- Head-mix GRU (shapes/layout page, support table: the GRU with
 * mix='head'; FAQs, memory notes: heads of d_head channels).  Reading: the
 * hidden width splits into n_heads = d_h / d_head heads, and each gate's
 * recurrent term becomes a dense d_head x d_head block per head:
 *   z = sig(x_z + A_z h)  r = sig(x_r + A_r h)  c = tanh(x_c + A_c (r * h))
 *   h' = (1 - z) * h + z * c         (A_g h: each head's block times its slice)
 * Newton as for the diagonal cells, with dense Jacobian blocks per head.
 *   A          (3, n_heads, d_head, d_head) fp32, gate order z, r, c; A[g][k][i][j]
 *              multiplies channel j of head k into channel i (row-major blocks)
 *   xproj      (B, T, 3, d_h) storage dtype, as for the diagonal GRU; aligned
 *              to 4 elements (16 bytes fp32, 8 bytes bf16)
 *   h0         (B, d_h) storage dtype or NULL (zeros); aligned to 4 elements
 *   H_out      (B, T, d_h) storage dtype; aligned to 4 elements (the Newton
 *              forward reads the iterates in 4-channel vectors)
 * params: cell = PRN_CELL_DIAG_GRU, dtype (PRN_F32 or PRN_BF16: the storage
 * of xproj, h0, the iterates, H_out and state_last_out; A and every
 * operation are fp32, each stored iterate is rounded once to nearest even),
 * B, T, d_h, n_seqs = 0, state_last_out ((B, d_h) or NULL), workspace,
 * stream; a, states_out and picard_iters are not used (states_out /
 * picard_iters must be 0).
 * Supported: d_head = 16, rectangular batches (the pages' head-mix fused
 * path takes no ragged pack); anything else is PRN_ERR_UNSUPPORTED.
 * Errors as for prn_newton_forward; residual_out as there (K + 1 values). */
size_t prn_head_workspace_bytes(const prn_params* params, int32_t d_head, int32_t K);
prn_status prn_head_newton_forward(const void* xproj, const prn_params* params, const float* A, int32_t d_head,
                                   const void* h0, int32_t K, void* H_out, float* residual_out);
/* The unroll h_t = f(h_{t-1}, x_t) of the head-mix GRU, the state chain in
 * fp32 and every output rounded once to the storage dtype; no workspace;
 * pointers aligned to their element size. */
prn_status prn_head_sequential_forward(const void* xproj, const prn_params* params, const float* A,
                                       int32_t d_head, const void* h0, void* H_out);

/* Host-side check of ragged offsets (the validate_cu_seqlens contract of
 * the shapes/layout page): cu_host has n_seqs + 1 entries, cu[0] = 0,
 * non-decreasing, cu[n_seqs] = N.  cu_host is a HOST pointer. */
prn_status prn_validate_cu_seqlens(const int32_t* cu_host, int64_t n_seqs, int64_t N);

/* Message for the last non-OK status returned on the calling thread. */
const char* prn_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t prn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PRN_H_ */
