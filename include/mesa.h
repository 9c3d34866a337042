/*
 * libmesa -- forward pass of the Mesa layer on one AMD MI355X (gfx950).
 *
 * Method: MesaNet, "Sequence Modeling by Locally Optimal Test-Time Training"
 * (technical summary, "Mesa layer" section).  For every token t the layer
 * keeps two decayed states,
 *
 *     H_t = gamma_t H_{t-1} + beta_t k_t k_t^T        (dk x dk, symmetric)
 *     G_t = gamma_t G_{t-1} + beta_t v_t k_t^T        (dv x dk)
 *
 * solves (H_t + Lambda) x_t = q_t by conjugate gradient and emits
 * o_t = G_t x_t.  This is the closed-form optimum of the section's
 * forget-weighted, Lambda-regularised least-squares objective with cumulative
 * forget factor zeta_{tt'} = beta_t' prod_{i=t'+1..t} gamma_i, reached
 * approximately by CG as the section prescribes; the number of CG steps is
 * either fixed or set per token by a residual test (the section's "dynamic
 * compute" paragraph).  Chunkwise-parallel evaluation over the sequence
 * (same section, "parallelisation") gives mesa_fwd_chunked; the O(1)
 * recurrent form gives mesa_decode_step.
 *
 * CG: Hestenes-Stiefel from x_0 = 0 with the recursive residual r.  Before
 * each iteration a token stops if max_steps iterations are done, if
 * tol > 0 and ||r||_2 <= tol, or if r.r is zero; it also stops (without
 * updating) if p.(A p) is zero or negative.  "Zero" means below 2^-126, the
 * smallest normal float: in the fixed-step mode a system solved to rounding
 * keeps shrinking its recursive residual until r.r underflows, and the
 * iteration ends there.  A stopped token never restarts.  steps[t] is the
 * number of executed updates.  tol <= 0 selects the fixed-step mode.
 *
 * Conventions common to every call
 *   - All tensor pointers are device pointers owned by the caller.  The
 *     library never allocates or frees device memory; scratch memory comes in
 *     through `workspace`.
 *   - Every call is asynchronous on `stream` (0 = the null stream) and holds
 *     no global mutable state, so calls on different streams may overlap as
 *     long as they do not write the same buffers.
 *   - All arguments are validated before anything is launched.  On any error
 *     the call returns a non-zero status, launches nothing and writes nothing.
 *     Launch failures reported by the runtime return MESA_ERR_HIP.
 *   - Numeric preconditions are documented, not checked: 0 < gamma <= 1,
 *     beta >= 0, lambda > 0, finite inputs, symmetric h0 / h_state.
 *   - An output buffer may not overlap another output or an input, except
 *     where a call updates a state in place (the decode steps) or says
 *     otherwise.  Only the preprocessing calls check this.
 *   - Tensors are dense and row-major with the last index fastest.  States are
 *     [.., dk, dk] for H and [.., dv, dk] for G (row = value dimension).
 *   - Supported sizes: dk == dv; dk in {16, 32, 64, 128} for MESA_F32 inputs
 *     and dk in {32, 64, 128} for MESA_BF16 inputs; chunk in {16, 32, 64};
 *     any T >= 0 (a last, shorter chunk is handled); B, H >= 1.
 *   - Pointers must be 16-byte aligned.
 */
#ifndef MESA_H_
#define MESA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MESA_ABI_VERSION 1

typedef enum {
  MESA_OK = 0,
  MESA_ERR_INVALID_ARG = 1,  /* null required pointer, negative size, ...        */
  MESA_ERR_UNSUPPORTED = 2,  /* valid but not implemented (d, chunk, dk != dv)  */
  MESA_ERR_ALIGNMENT = 3,    /* a pointer is not 16-byte aligned                 */
  MESA_ERR_WORKSPACE = 4,    /* workspace missing or smaller than required       */
  MESA_ERR_HIP = 5           /* the HIP runtime reported an error                */
} mesa_status;

typedef enum {
  MESA_F32 = 0,   /* q, k, v are float32; states and arithmetic are fp32          */
  MESA_BF16 = 1   /* q, k, v are bfloat16; MFMA in bf16 with fp32 accumulation,
                     CG vectors, scalars and carried states in fp32             */
} mesa_dtype;

typedef struct {
  int32_t B, H, T;      /* batch, heads, tokens per sequence                       */
  int32_t dk, dv;       /* key / value head dims (dk == dv)                        */
  int32_t chunk;        /* tokens per chunk of the parallel form                   */
  int32_t max_steps;    /* CG iteration cap, >= 0                                  */
  float tol;            /* residual tolerance; <= 0 runs exactly max_steps         */
  mesa_dtype in_dtype;  /* dtype of q, k, v                                        */
} mesa_fwd_desc;

/* Bytes of scratch memory mesa_fwd_chunked needs for `d`: the decayed
 * chunk-boundary states and, for MESA_BF16 inputs, one int32 per chunk
 * (rounded up to 256 bytes) recording which chunks the strong-decay kernel
 * solves.  Returns 0 for an invalid or unsupported descriptor, and for
 * T == 0. */
size_t mesa_fwd_workspace_bytes(const mesa_fwd_desc* d);

/* Chunkwise-parallel Mesa forward over whole sequences
 * (MesaNet page, technical summary, "Mesa layer": objective, CG query
 * response, chunk-parallel states, dynamic CG step count).
 *
 *   q, k   [B, H, T, dk]  in_dtype        queries / keys
 *   v      [B, H, T, dv]  in_dtype        values
 *   gamma  [B, H, T]      fp32            forget factor of each token
 *   beta   [B, H, T]      fp32            write strength of each token
 *   lambda [H, dk]        fp32            diagonal of Lambda per head (> 0)
 *   h0     [B, H, dk, dk] fp32 or NULL    state before token 0 (NULL = 0)
 *   g0     [B, H, dv, dk] fp32 or NULL
 *   o      [B, H, T, dv]  fp32            out: o_t = G_t x_t
 *   h_final, g_final      fp32 or NULL    out: states after token T-1
 *   steps  [B, H, T]      int32 or NULL   out: CG iterations per token
 *   x_out  [B, H, T, dk]  fp32 or NULL    out: the CG solution x_t
 *   workspace             device memory of at least
 *                         mesa_fwd_workspace_bytes(d) bytes (may be NULL
 *                         when that is 0)
 *
 * h_final / g_final of one call are valid h0 / g0 of the next call on the
 * continuation of the sequence, and valid decode states. */
mesa_status mesa_fwd_chunked(const mesa_fwd_desc* d,
                             const void* q, const void* k, const void* v,
                             const float* gamma, const float* beta, const float* lambda,
                             const float* h0, const float* g0,
                             float* o, float* h_final, float* g_final,
                             int32_t* steps, float* x_out,
                             void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* mesa_fwd_chunked with warm-started CG (MesaNet page, technical summary,
 * "significance": warm-started optimisation as a way to cut the solver's
 * cost).  The chunks of a sequence are solved in parallel and the tokens of a
 * chunk in tiles of 16, so a token can start from a solution that an earlier
 * tile of its own chunk produced: token t starts its CG from x_{t-16}, the
 * solution of token t-16, when both lie in one chunk, and from 0 otherwise
 * (the first 16 tokens of every chunk).  The residual starts at
 * q_t - (H_t + Lambda) x_{t-16}; that product is not counted in steps.  With
 * a tolerance a good start saves steps; with a fixed step count the result is
 * the n-step CG iterate from that start.
 *
 * Supported for in_dtype MESA_BF16 and every chunk and dk of mesa_fwd_chunked
 * (at chunk 16 no token has a start in its chunk); fp32 inputs return
 * MESA_ERR_UNSUPPORTED and launch nothing.  Every argument, the workspace and
 * the error behaviour are those of mesa_fwd_chunked. */
mesa_status mesa_fwd_chunked_warm(const mesa_fwd_desc* d,
                                  const void* q, const void* k, const void* v,
                                  const float* gamma, const float* beta, const float* lambda,
                                  const float* h0, const float* g0,
                                  float* o, float* h_final, float* g_final,
                                  int32_t* steps, float* x_out,
                                  void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/* mesa_fwd_chunked on raw queries and keys, with the preprocessing of
 * mesa_qk_preprocess fused into the forward's loads (MesaNet page,
 * "architecture" section: queries and keys are convolved with a small causal
 * window and normalised before the Mesa layer).  The result equals
 * mesa_qk_preprocess (bf16 outputs) followed by mesa_fwd_chunked on its
 * outputs, bit for bit, without the processed q and k ever reaching memory:
 * the scan and solve kernels convolve and normalise the raw rows they load.
 *
 *   q_raw, k_raw   [B, H, T, dk] bf16      raw projections (the q, k of
 *                                          mesa_fwd_chunked before processing)
 *   w_q, w_k       [H, dk, window] fp32    taps; tap i weighs token t-i
 *   window         1..4
 *   eps            > 0, finite             out_t = y_t / max(||y_t||, eps)
 *   q_hist, k_hist [B, H, window-1, dk] bf16 or NULL: raw vectors before
 *                                          t = 0, oldest first (NULL: zeros)
 *   q_hist_out, k_hist_out [B, H, window-1, dk] bf16 or NULL: the last
 *                  window-1 raw vectors of history + sequence (the next
 *                  call's histories); they may not overlap q_raw, k_raw,
 *                  q_hist, k_hist or each other (MESA_ERR_INVALID_ARG)
 *
 * Every other argument, the workspace (mesa_fwd_workspace_bytes(d)) and the
 * error behaviour are those of mesa_fwd_chunked.  Supported for in_dtype
 * MESA_BF16, chunk 64 and dk = dv in {64, 128}; other descriptors, and
 * window > 4, return MESA_ERR_UNSUPPORTED.  window < 1, eps <= 0 or not
 * finite, or a NULL w_q / w_k return MESA_ERR_INVALID_ARG.  Nothing is
 * launched on an error. */
mesa_status mesa_fwd_chunked_prep(const mesa_fwd_desc* d,
                                  const void* q_raw, const void* k_raw, const void* v,
                                  const float* w_q, const float* w_k, int32_t window, float eps,
                                  const void* q_hist, const void* k_hist,
                                  const float* gamma, const float* beta, const float* lambda,
                                  const float* h0, const float* g0,
                                  float* o, float* h_final, float* g_final,
                                  int32_t* steps, float* x_out,
                                  void* q_hist_out, void* k_hist_out,
                                  void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/* Size of the static scratch array behind mesa_fwd_chunked_noalloc: 64 MiB
 * per GPU the library runs on (for example B*H*T = 65536 token-heads at
 * dk = 128, chunk 64, or the B=4, H=8, T=2048, dk=64 workload's 16 MiB). */
#define MESA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* mesa_fwd_chunked for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and error behaviour as mesa_fwd_chunked, without the
 * workspace: the scratch is a file-scope device array of
 * MESA_NOALLOC_SCRATCH_BYTES, one per GPU, held until the process ends.  The
 * call itself allocates nothing (no hipMalloc, no hipFree); its first call on
 * a device looks the array's address up once with hipGetSymbolAddress.
 *
 *   - A descriptor whose mesa_fwd_workspace_bytes exceeds
 *     MESA_NOALLOC_SCRATCH_BYTES returns MESA_ERR_UNSUPPORTED and launches
 *     nothing; every argument check runs before any HIP call.
 *   - `stream` must belong to the current device (else MESA_ERR_INVALID_ARG);
 *     the current device's array is used.
 *   - Every call on a GPU shares that GPU's array, and the array keeps the
 *     last call's contents.  Calls that overlap in time on one GPU (different
 *     streams, or host threads racing) race on it: serialise them.
 *   - Nothing in the array needs clearing between calls: every byte a call
 *     reads, the same call wrote first. */
mesa_status mesa_fwd_chunked_noalloc(const mesa_fwd_desc* d,
                                     const void* q, const void* k, const void* v,
                                     const float* gamma, const float* beta, const float* lambda,
                                     const float* h0, const float* g0,
                                     float* o, float* h_final, float* g_final,
                                     int32_t* steps, float* x_out,
                                     hipStream_t stream);

/* mesa_fwd_chunked with the regulariser given either as before or as a full
 * matrix per head (MesaNet page, technical summary, "Mesa layer": Lambda is a
 * symmetric positive definite regulariser of the objective).
 *
 *   lambda_full = 0: lambda [H, dk] fp32, the diagonal, exactly as
 *                    mesa_fwd_chunked (the same kernels run).
 *   lambda_full = 1: lambda [H, dk, dk] fp32, row-major, symmetric positive
 *                    definite.  This is not checked: with an indefinite
 *                    matrix a token can meet p.Ap <= 0, and CG's breakdown
 *                    rule stops it there, as for any token.  The matrix is
 *                    rounded to bf16 for its MFMA products; lambda is only
 *                    read.
 *                    Supported for in_dtype MESA_BF16, chunk 64 and
 *                    dk = dv in {64, 128}; other descriptors return
 *                    MESA_ERR_UNSUPPORTED and launch nothing.
 *
 * Any other value of lambda_full returns MESA_ERR_INVALID_ARG and launches
 * nothing, as in mesa_bwd_chunked_ex and mesa_decode_step_ex.  Every other
 * argument, the workspace and the error behaviour are those of
 * mesa_fwd_chunked. */
mesa_status mesa_fwd_chunked_ex(const mesa_fwd_desc* d,
                                const void* q, const void* k, const void* v,
                                const float* gamma, const float* beta, const float* lambda,
                                int32_t lambda_full, const float* h0, const float* g0,
                                float* o, float* h_final, float* g_final,
                                int32_t* steps, float* x_out,
                                void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* The two phases of mesa_fwd_chunked, for callers that want them apart
 * (e.g. building decode states from a prompt without solving, or timing).
 *
 * mesa_fwd_scan: the inter-chunk state scan only.  Reads k, v, gamma, beta,
 * h0, g0; writes the chunk-boundary states into `workspace` and, when given,
 * h_final / g_final.  q, lambda and o are not needed.
 *
 * mesa_fwd_solve: the chunked CG solve and read-out only.  Reads q, k, v,
 * gamma, beta, lambda and the boundary states a preceding mesa_fwd_scan
 * with the same descriptor and inputs left in `workspace` (stream order);
 * writes o, steps, x_out.  Same arguments and rules as mesa_fwd_chunked. */
mesa_status mesa_fwd_scan(const mesa_fwd_desc* d, const void* k, const void* v,
                          const float* gamma, const float* beta,
                          const float* h0, const float* g0,
                          float* h_final, float* g_final,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

mesa_status mesa_fwd_solve(const mesa_fwd_desc* d,
                           const void* q, const void* k, const void* v,
                           const float* gamma, const float* beta, const float* lambda,
                           float* o, int32_t* steps, float* x_out,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* One recurrent step for N sequences x H heads, states updated in place
 * (MesaNet page, technical summary, "Mesa layer": O(1) inference form).
 *
 *   q, k    [N, H, dk]  in_dtype; v [N, H, dv] in_dtype
 *   gamma, beta [N, H]  fp32
 *   lambda  [H, dk]     fp32
 *   h_state [N, H, dk, dk] fp32, in/out: H_{t-1} -> H_t
 *   g_state [N, H, dv, dk] fp32, in/out: G_{t-1} -> G_t
 *   o       [N, H, dv]  fp32 out
 *   steps   [N, H]      int32 out or NULL
 *   x_out   [N, H, dk]  fp32 out or NULL
 * Supported: dk == dv == 128 or 64, either in_dtype. */
mesa_status mesa_decode_step(int32_t N, int32_t H, int32_t dk, int32_t dv,
                             const void* q, const void* k, const void* v, mesa_dtype in_dtype,
                             const float* gamma, const float* beta, const float* lambda,
                             float* h_state, float* g_state,
                             float* o, int32_t* steps, float* x_out,
                             int32_t max_steps, float tol, hipStream_t stream);

/* ---- packed-symmetric key-covariance state for the decode step -------------
 *
 * H is symmetric (each update adds beta k k^T), so its upper triangle holds all
 * of it.  The "blocked upper-triangular" layout stores, for d in {64, 128},
 * the (d/16)(d/16+1)/2 blocks of 16x16 on or above the block diagonal, in
 * row-major block order (0,0), (0,1), ..., (0,d/16-1), (1,1), ...; each block
 * is 16x16 fp32 row-major (1 KB) and block (bi, bj) holds
 * H[16 bi + r][16 bj + c].  Diagonal blocks are stored whole.  At d = 128 a
 * state takes 36 KB instead of 64 KB, so the HBM-bound decode step moves about
 * 22 % fewer bytes. */

/* Floats of one state in the blocked layout (0 for an unsupported d). */
size_t mesa_sym_state_floats(int32_t d);

/* full [count, d, d] fp32 -> packed [count, mesa_sym_state_floats(d)] fp32
 * (the blocks on and above the block diagonal are copied; the rest of `full`
 * is not read).  Device pointers, 16-byte aligned; asynchronous on `stream`. */
mesa_status mesa_sym_pack(int32_t count, int32_t d, const float* full, float* packed,
                          hipStream_t stream);

/* packed -> full [count, d, d]: the blocks below the block diagonal are the
 * transposes of the stored ones, so the result is exactly symmetric when the
 * stored diagonal blocks are. */
mesa_status mesa_sym_unpack(int32_t count, int32_t d, const float* packed, float* full,
                            hipStream_t stream);

/* mesa_decode_step with h_sym [N, H, mesa_sym_state_floats(dk)] in the
 * blocked layout (in/out); every other argument, the arithmetic and the
 * results are those of mesa_decode_step.  Supported: dk == dv == 64 or 128. */
mesa_status mesa_decode_step_symh(int32_t N, int32_t H, int32_t dk, int32_t dv,
                                  const void* q, const void* k, const void* v, mesa_dtype in_dtype,
                                  const float* gamma, const float* beta, const float* lambda,
                                  float* h_sym, float* g_state,
                                  float* o, int32_t* steps, float* x_out,
                                  int32_t max_steps, float tol, hipStream_t stream);

/* ---- warm-started decode step -----------------------------------------------
 *
 * The "significance" section of the MesaNet page names warm-starting the
 * optimisation as a way to cut the solver's cost.  This step starts CG from a
 * per-pair guess instead of 0 -- in decoding, the previous token's solution,
 * which the step itself leaves behind:
 *
 *   x_state [N, H, dk] fp32, in/out (required): on entry the CG start x_0
 *           (zeros give the cold start of mesa_decode_step), on return this
 *           token's solution x_t, the next call's start.
 *   h_packed 0: h_state is [N, H, dk, dk]; 1: h_state is [N, H,
 *           mesa_sym_state_floats(dk)] in the blocked layout above.
 *
 * CG then begins from r_0 = q - (H_t + Lambda) x_0, tests the tolerance
 * before every iteration as usual, and `steps` counts its iterations (the
 * product A x_0 is one more, uncounted).  Everything else is as in
 * mesa_decode_step.  Calls that share x_state must not overlap.
 * Errors: MESA_ERR_INVALID_ARG for a NULL x_state or h_packed not 0/1. */
mesa_status mesa_decode_step_warm(int32_t N, int32_t H, int32_t dk, int32_t dv,
                                  const void* q, const void* k, const void* v, mesa_dtype in_dtype,
                                  const float* gamma, const float* beta, const float* lambda,
                                  float* h_state, int32_t h_packed, float* g_state, float* x_state,
                                  float* o, int32_t* steps,
                                  int32_t max_steps, float tol, hipStream_t stream);

/* ---- backward pass (training) -------------------------------------------------
 *
 * Gradients of a mesa_fwd_chunked call by implicit differentiation of its
 * solves (MesaNet page, technical summary, "Mesa layer"; the layer is trained
 * end to end).  The scalar differentiated is
 *   L = sum_t <d_o_t, o_t> + <d_hfinal, H_T> + <d_gfinal, G_T>.
 * Each x_t is treated as the solution of (H_t + Lambda) x_t = q_t; the adjoint
 * systems (H_t + Lambda) y_t = G_t^T d_o_t are solved by the same CG (the
 * descriptor's max_steps; its tol taken relative to ||G_t^T d_o_t||), and
 *   dq_t = y_t,  dk_t = beta_t ((Hh_t + Hh_t^T) k_t + Gh_t^T v_t),  dv_t = beta_t Gh_t k_t,
 *   dbeta_t = k_t^T Hh_t k_t + v_t^T Gh_t k_t,  dgamma_t = <Hh_t, H_{t-1}> + <Gh_t, G_{t-1}>,
 *   dlambda = -sum_{b,t} y_t * x_t,  dh0 = sym(gamma_0 Hh_0),  dg0 = gamma_0 Gh_0,
 * with Hh_t = -y_t x_t^T + gamma_{t+1} Hh_{t+1} (Hh_T = d_hfinal) and
 * Gh_t = d_o_t x_t^T + gamma_{t+1} Gh_{t+1} (Gh_T = d_gfinal).
 *
 *   desc          the forward's descriptor; supported: bf16 inputs, dk == dv in
 *                 {64, 128}, chunk 64 (else MESA_ERR_UNSUPPORTED)
 *   q ... g0      the forward's inputs (h0, g0 may be NULL)
 *   x             the forward's x_out, fp32 [B, H, T, d]
 *   d_o           dL/do, fp32 [B, H, T, dv]
 *   d_hfinal, d_gfinal  fp32 [B, H, d, d] or NULL (zero)
 *   dq, dk, dv    fp32 [B, H, T, d] out;  dgamma, dbeta fp32 [B, H, T] out
 *   dlambda       fp32 [H, dk] out (summed over batch and time)
 *   dh0, dg0      fp32 [B, H, d, d] out or NULL; dh0 is symmetric (h0 is a
 *                 symmetric state)
 *   adj_steps     int32 [B, H, T] out or NULL: CG steps of the adjoint solves
 *   states_in_workspace  0: the call recomputes the forward's boundary
 *                 states; 1: the forward call ran with this same workspace
 *                 (its first mesa_fwd_workspace_bytes(desc) bytes are the
 *                 forward's workspace layout) and the states it left there
 *                 are used (same descriptor, same k, v, gamma, beta, h0, g0)
 *   workspace     mesa_bwd_workspace_bytes(desc) bytes, which is at least
 *                 mesa_fwd_workspace_bytes(desc)
 * The products inside use bf16 operands with fp32 accumulation, like the
 * forward's bf16 path.  Asynchronous on `stream`; device pointers, 16-byte
 * aligned; validation failures write nothing. */
size_t mesa_bwd_workspace_bytes(const mesa_fwd_desc* d);

mesa_status mesa_bwd_chunked(const mesa_fwd_desc* d,
                             const void* q, const void* k, const void* v,
                             const float* gamma, const float* beta, const float* lambda,
                             const float* h0, const float* g0,
                             const float* x, const float* d_o,
                             const float* d_hfinal, const float* d_gfinal,
                             float* dq, float* dk, float* dv, float* dgamma, float* dbeta,
                             float* dlambda, float* dh0, float* dg0, int32_t* adj_steps,
                             int32_t states_in_workspace,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* mesa_bwd_chunked with Lambda either diagonal (lambda_full = 0: exactly
 * mesa_bwd_chunked) or a full symmetric positive definite matrix per head
 * (lambda_full = 1; MesaNet page, technical summary, "Mesa layer": Lambda is
 * a symmetric positive definite regulariser):
 *   lambda   fp32 [H, dk, dk] in, the matrix of the forward call
 *            (mesa_fwd_chunked_ex with lambda_full = 1)
 *   dlambda  fp32 [H, dk, dk] out: -sum_{b,t} y_t x_t^T, the partial
 *            derivative of each entry of the solves' matrix (not
 *            symmetrised; a caller that ties Lambda_ij to Lambda_ji adds the
 *            transpose).  Its diagonal is the diagonal case's dlambda.
 * The adjoint solves take the full matrix like the forward's.  Descriptors,
 * workspace (mesa_bwd_workspace_bytes) and errors are those of
 * mesa_bwd_chunked; lambda_full other than 0 or 1 is MESA_ERR_INVALID_ARG. */
mesa_status mesa_bwd_chunked_ex(const mesa_fwd_desc* d,
                                const void* q, const void* k, const void* v,
                                const float* gamma, const float* beta, const float* lambda,
                                int32_t lambda_full, const float* h0, const float* g0,
                                const float* x, const float* d_o,
                                const float* d_hfinal, const float* d_gfinal,
                                float* dq, float* dk, float* dv, float* dgamma, float* dbeta,
                                float* dlambda, float* dh0, float* dg0, int32_t* adj_steps,
                                int32_t states_in_workspace,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- general decode step --------------------------------------------------------
 *
 * Every decode variant in one call, with the Lambda of the pages' objective
 * either diagonal or a full symmetric positive definite matrix per head
 * ("technical summary / Mesa layer": Lambda is a symmetric positive definite
 * regulariser):
 *
 *   lambda       [H, dk] fp32 (lambda_full = 0: the diagonal) or
 *                [H, dk, dk] fp32 (lambda_full = 1: symmetric positive definite,
 *                row-major; the kernel relies on its symmetry)
 *   h_packed     0: h_state [N, H, dk, dk]; 1: [N, H, mesa_sym_state_floats(dk)]
 *   x_state      [N, H, dk] fp32 in/out, or NULL: as in mesa_decode_step_warm
 *                (CG starts at x_state and leaves the solution there), or a
 *                cold start from 0
 *   x_out        [N, H, dk] fp32 out or NULL (cold start only)
 * Everything else as in mesa_decode_step.  Errors: MESA_ERR_INVALID_ARG for
 * flags other than 0/1, or x_out given together with x_state. */
mesa_status mesa_decode_step_ex(int32_t N, int32_t H, int32_t dk, int32_t dv,
                                const void* q, const void* k, const void* v, mesa_dtype in_dtype,
                                const float* gamma, const float* beta,
                                const float* lambda, int32_t lambda_full,
                                float* h_state, int32_t h_packed, float* g_state, float* x_state,
                                float* o, int32_t* steps, float* x_out,
                                int32_t max_steps, float tol, hipStream_t stream);

/* ---- query/key preprocessing -------------------------------------------------
 *
 * MesaNet page, "architecture" section: queries and keys are normalised and
 * convolved with a small window before the Mesa layer.  Computed here as a
 * causal depthwise convolution along time followed by L2 normalisation of
 * every token vector (so the layer receives unit-norm queries and keys), for
 * queries and keys in one call, each with its own taps:
 *
 *   y_t[j] = sum_{i < window} w[h][j][i] * x_{t-i}[j]
 *   out_t  = y_t / max(||y_t||_2, eps)
 *
 *   q_raw, k_raw [B, H, T, d] dtype (raw projections)
 *   w_q, w_k     [H, d, window] fp32; tap i weighs token t-i
 *   q_hist, k_hist [B, H, window-1, d] dtype, or NULL: the raw vectors before
 *                t = 0, oldest first (NULL: zeros -- a sequence start)
 *   q_out, k_out [B, H, T, d] dtype (bf16 outputs are rounded to nearest even)
 *   q_hist_out, k_hist_out [B, H, window-1, d] dtype, or NULL: the last
 *                window-1 raw vectors of history + sequence, the next call's
 *                history (also for T < window-1, and for a decode step, T = 1)
 *
 * The scale 1 / max(||y||, eps) is formed as min(1/sqrt(||y||^2), 1/eps)
 * with the hardware reciprocal square root (1 ulp).
 *
 * Supported: d in {16, 64, 128}, 1 <= window <= 4, B*H <= 65535, and
 * 2^-63 <= eps < inf (else MESA_ERR_INVALID_ARG).
 * Outputs may not overlap the raw inputs or histories (MESA_ERR_INVALID_ARG):
 * every raw vector is read by up to `window` outputs.  Device pointers,
 * 16-byte aligned; asynchronous on `stream`. */
mesa_status mesa_qk_preprocess(int32_t B, int32_t H, int32_t T, int32_t d, int32_t window,
                               mesa_dtype dtype, const void* q_raw, const void* k_raw,
                               const float* w_q, const float* w_k,
                               const void* q_hist, const void* k_hist, float eps,
                               void* q_out, void* k_out, void* q_hist_out, void* k_hist_out,
                               hipStream_t stream);

/* Static text for a status code. */
const char* mesa_status_string(mesa_status s);

/* MESA_ABI_VERSION of the built library. */
int32_t mesa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MESA_H_ */
