/*
 * tango.h - C ABI of the MI355X (gfx950) TANGO / WANGO block forward library.
 *
 * The operation is the gated-aggregation block of "TANGO: Token-Aggregated
 * Nonlinear Gating Operators for Natural and Formal Language Modeling"
 * (arXiv 2608.22117 v1):
 *
 *   x_i    = RMSNorm(h_i)                                       (§2.1)
 *   g_i    = SiLU(W_g x_i),  v_i = W_v x_i                      (§2.1, eq. 2)
 *   q_ia, k_ia = per-head W_q x_i, W_k x_i; RoPE, unit length   (§2.1)
 *   l_ija  = tau_a q_ia . k_ja,  tau_a = exp(min(theta_a, log 20))   (§2.1, eq. 4)
 *   gbar_ia = sum_j m_ija g_ja / (sum_j m_ija + n_i exp(b_a))   (§2.1, eq. 5)
 *   h+_i   = h_i + W_o (gbar_i * v_i)                           (§2.1, eq. 3)
 *
 * with m_ija = exp(l_ija) over the whole causal prefix for TANGO (§2.2, eq. 6),
 * and for WANGO exp(l_ija) inside the trailing window of W positions and
 * phi(sqrt(tau) q)^T phi(sqrt(tau) k) for older sources, phi(u) =
 * max(ELU(u)+1+1e-4, 1e-4)/sqrt(d_h), carried as running sums (§2.2, eqs. 7-10).
 *
 * Readings where the text is open: RMSNorm eps = shape.rms_eps with an optional
 * gain; heads own contiguous column blocks of the gate and of q/k; RoPE rotates
 * interleaved pairs (2c, 2c+1) by angle i * rope_base^(-2c/d_h) at the 0-based
 * position i of each batch row (rope_base = 0 turns it off); a zero-length q or
 * k is divided by 1e-12; ELU alpha = 1; n_i = i + 1; the WANGO feature map
 * keeps the head width (phi_dim must equal head_dim).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller, row-major and
 *    contiguous, 16-byte aligned.  x and out have shape->io_dtype; the five
 *    weight matrices, the gain and the intermediate activations have
 *    shape->dtype; theta, null_bias and every float32 buffer below are float32.
 *    Accumulation is float32 for both dtypes.
 *  - Calls are asynchronous on `hip_stream` (a hipStream_t; NULL = the default
 *    stream) and never synchronise the host.  The library allocates no memory
 *    on any call and keeps no per-call state; scratch space is the caller's
 *    `workspace`, whose minimum size the *_workspace_size functions return.
 *    A call only launches kernels on `hip_stream` (no memset, copy or host
 *    wait; the first call on a device also sets kernel attributes), so after
 *    one call on the device it can be captured into a HIP graph and replayed.
 *  - A workspace must not be shared by calls that can run concurrently.
 *  - Inputs are never modified.  `out` may equal `x` (in place); any other
 *    overlap between `out`, `workspace` and the inputs is TANGO_ERR_ALIAS.
 *  - Every argument is validated before anything is launched: on a non-zero
 *    status nothing was written.  A launch failure returns TANGO_ERR_HIP.
 *    tango_last_error() then holds a message for the calling thread.
 *  - No C++ exception and no abort crosses this interface.
 *
 * Supported shapes (otherwise TANGO_ERR_UNSUPPORTED; F % H != 0,
 * phi_dim != head_dim and window < 1 are TANGO_ERR_SHAPE):
 *    batch >= 1, seq_len >= 1, batch * seq_len <= 2^26,
 *    d_model % 128 == 0 and d_model <= 4096,
 *    d_gate % 64 == 0, (d_gate / n_heads) % 4 == 0,
 *    head_dim in {32, 64, 128}, n_heads * head_dim <= 1024,
 *    WANGO: chunk in {64, 128}, window % chunk == 0.
 */
#ifndef TANGO_H_
#define TANGO_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TANGO_ABI_VERSION 10

typedef enum { TANGO_F32 = 0, TANGO_BF16 = 1 } tango_dtype_t;

typedef enum {
  TANGO_OK = 0,
  TANGO_ERR_NULL = -1,        /* a required pointer is NULL                        */
  TANGO_ERR_SHAPE = -2,       /* inconsistent sizes (F % H, phi_dim, window < 1 ...) */
  TANGO_ERR_DTYPE = -3,       /* dtype or io_dtype is not TANGO_F32 or TANGO_BF16  */
  TANGO_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned                  */
  TANGO_ERR_UNSUPPORTED = -5, /* a consistent shape the kernels do not cover        */
  TANGO_ERR_WORKSPACE = -6,   /* workspace smaller than *_workspace_size()          */
  TANGO_ERR_ALIAS = -7,       /* outputs overlap inputs or the workspace            */
  TANGO_ERR_HIP = -8          /* the HIP runtime reported an error                  */
} tango_status_t;

/* Sizes of one block call.  B sequences of T positions, residual width d,
 * gate width F split over H heads of F/H gate columns and d_h query/key
 * columns each. */
typedef struct {
  int32_t batch;      /* B                                                */
  int32_t seq_len;    /* T                                                */
  int32_t d_model;    /* d                                                */
  int32_t d_gate;     /* F                                                */
  int32_t n_heads;    /* H                                                */
  int32_t head_dim;   /* d_h                                              */
  int32_t dtype;      /* tango_dtype_t: dtype of the weights and of every
                         intermediate activation (accumulation is float32) */
  int32_t io_dtype;   /* tango_dtype_t: dtype of x and out, the residual
                         stream (float32 keeps it exact between stacked
                         applications)                                     */
  float rope_base;    /* RoPE base (10000 in the shipped workloads); 0 = off */
  float rms_eps;      /* RMSNorm epsilon (1e-6 in the shipped workloads)  */
  int32_t operand_parts; /* How the float32 activation operand of the
                         projection and output GEMMs (h*gain, gbar*v;
                         [TANGO] §2.1 eqs. 2-3) enters the bf16 MFMA:
                         0 or 1 = rounded once to bf16 (the pages' bf16
                         compute); 2 = as two bf16 parts hi = bf16(e),
                         lo = bf16(e - hi) summed into one float32
                         accumulator (about 2^-16 relative, twice the MFMA
                         work; for long shared-weight stacks).  2 requires
                         dtype TANGO_BF16, else TANGO_ERR_SHAPE.  The
                         decode step always takes two parts in bf16.      */
} tango_shape_t;

/* Block parameters ([TANGO] §2.1; the count in Table 1 fixes this list):
 * bias-free projections, one RMSNorm gain, a temperature logit and a null-gate
 * bias per head. */
typedef struct {
  const void* w_g;        /* [F, d]                                          */
  const void* w_v;        /* [F, d]                                          */
  const void* w_q;        /* [H*d_h, d]                                      */
  const void* w_k;        /* [H*d_h, d]                                      */
  const void* w_o;        /* [d, F]                                          */
  const void* rms_gain;   /* [d] in dtype, or NULL for a gain of 1           */
  const float* theta;     /* [H]; tau_a = exp(min(theta_a, log 20))  (eq. 4) */
  const float* null_bias; /* [H] b_a, or NULL: null gate off          (eq. 5) */
} tango_weights_t;

/* ---- Whole block --------------------------------------------------------- */

/* Bytes of workspace tango_block_fwd needs for `shape`; 0 if the shape is
 * invalid (the call itself then reports why). */
size_t tango_workspace_size(const tango_shape_t* shape);

/* TANGO block ([TANGO] §2.1 eqs. 2-5, §2.2 eq. 6): out[B,T,d] = h+ for
 * x[B,T,d] = h.  Apply it R times with out == x for the shared-weight stack of
 * §2.3 eq. 11 (the stream is then stored in io_dtype between applications:
 * float32 keeps it unrounded, bfloat16 rounds it once per application). */
int tango_block_fwd(const tango_shape_t* shape, const tango_weights_t* weights,
                    const void* x, void* out, void* workspace, size_t workspace_bytes,
                    void* hip_stream);

/* ---- Stack of TANGO blocks with several parameter sets --------------------
 *
 * The shared-weight stack of [TANGO] §2.3 eq. 11 applies one block R times.
 * The later revision ("TANGO: Treating Tokens as Operators", abstract and
 * Table 2) also trains a variant with three narrower gated-projection sets,
 * one for the first application, one for the middle ones and one for the
 * last.  tango_stack_fwd applies any such schedule: application r uses
 * parameter set schedule[r].
 *
 *   shapes[n_sets], sets[n_sets]: the sizes and parameters of each set.  The
 *       sets must agree on batch, seq_len, d_model, dtype and io_dtype (the
 *       residual stream); d_gate, n_heads, head_dim, rope_base and rms_eps may
 *       differ.  Parameters that the sets share (the three-set model keeps
 *       one W_q, W_k, gain, theta and null bias, and varies W_g, W_v and W_o)
 *       are shared by passing the same pointers.
 *   schedule[n_apps]: set index of each application, 0 <= schedule[r] <
 *       n_sets; n_apps >= 1.  Host memory, read before the call returns.
 *   x -> out: [B, T, d] in io_dtype; out may equal x (in place); after the
 *       first application the stream is carried in out.
 *   workspace: at least tango_stack_workspace_size(shapes, n_sets) bytes (the
 *       largest tango_workspace_size of the sets); 0 is returned there if a
 *       shape is invalid or n_sets < 1.
 * Every argument is checked before the first launch: on an error nothing runs
 * and out is untouched.  Launches are asynchronous on hip_stream. */
size_t tango_stack_workspace_size(const tango_shape_t* shapes, int32_t n_sets);
int tango_stack_fwd(const tango_shape_t* shapes, const tango_weights_t* sets, int32_t n_sets,
                    const int32_t* schedule, int32_t n_apps, const void* x, void* out,
                    void* workspace, size_t workspace_bytes, void* hip_stream);

/* Bytes of workspace wango_block_fwd needs; 0 if the arguments are invalid. */
size_t wango_workspace_size(const tango_shape_t* shape, int32_t window, int32_t phi_dim,
                            int32_t chunk);

/* WANGO block ([TANGO] §2.2 eqs. 7-10): window of `window` positions
 * (counting the destination), feature map of width phi_dim (= head_dim), and
 * the older-prefix running sums carried across chunks of `chunk` positions.
 * The result does not depend on `chunk` except through float rounding. */
int wango_block_fwd(const tango_shape_t* shape, const tango_weights_t* weights,
                    int32_t window, int32_t phi_dim, int32_t chunk,
                    const void* x, void* out, void* workspace, size_t workspace_bytes,
                    void* hip_stream);

/* ---- Autoregressive decode ----------------------------------------------
 *
 * One new token per sequence per call.  A step returns the block output at the
 * token's position p -- row p of the block forward over the sequence's prefix,
 * since no source lies after its destination (eq. 5) -- and advances a state
 * kept between calls.  TANGO's state is every unit key and gate so far (eq. 6
 * sums over the whole prefix).  WANGO's is the running sums S, z of §2.2
 * eq. 10, which take in the key and gate of position p - W as the position p
 * advances, plus the keys and gates of the last window + 1 positions: a state
 * whose size does not depend on the position (§6.1).
 *
 *   shape      batch = B sequences; seq_len = TANGO cache capacity P (positions
 *              0 .. P-1 can be decoded); WANGO ignores seq_len (>= 1).
 *   pos        DEVICE int32 [B]: position of each sequence's new token.  Position
 *              0 starts a sequence afresh (no state needs clearing first); a step
 *              at p > 0 must follow the step at p - 1 of the same sequence on
 *              the same state.  A sequence with pos < 0 (TANGO: or >= P) is
 *              skipped: its out row is NaN and its state is not touched.  (Only
 *              the kernels see pos, so this is not a validation error.)
 *   x, out     [B, d] in io_dtype; out may equal x.
 *   state      DEVICE buffer of *_decode_state_size bytes, kept by the caller
 *              between steps, one per stacked application; never shared by
 *              calls that can run concurrently.  Layout (dtype unless noted):
 *                keys  [B][R][H*d_h] RoPE-rotated keys, stored before the
 *                      unit-length division (the kernels divide by each
 *                      head's norm where they read a key),
 *                gates [B][R][F],
 *                TANGO: R = P, position j in row j;
 *                WANGO: R = window + 1, position j in row j mod R, then
 *                  S [B][H][d_h][F/H] float32 and z [B][2][H][d_h] float32
 *                  (after the step at p, z is in copy p mod 2);
 *              each array starts at a 256-byte boundary.
 *   workspace  per-call scratch of *_decode_workspace_size bytes.
 * Supported shapes: those of the block calls, with n_heads <= 32,
 * (d_gate / n_heads) % 64 == 0 and (WANGO) window <= 2048; the size functions
 * return 0 for anything else.
 */
size_t tango_decode_state_size(const tango_shape_t* shape);
size_t tango_decode_workspace_size(const tango_shape_t* shape);
int tango_decode_step(const tango_shape_t* shape, const tango_weights_t* weights, const int32_t* pos,
                      const void* x, void* out, void* state, size_t state_bytes, void* workspace,
                      size_t workspace_bytes, void* hip_stream);

size_t wango_decode_state_size(const tango_shape_t* shape, int32_t window, int32_t phi_dim);
size_t wango_decode_workspace_size(const tango_shape_t* shape, int32_t window, int32_t phi_dim);
int wango_decode_step(const tango_shape_t* shape, const tango_weights_t* weights, int32_t window,
                      int32_t phi_dim, const int32_t* pos, const void* x, void* out, void* state,
                      size_t state_bytes, void* workspace, size_t workspace_bytes, void* hip_stream);

/* ---- WANGO decode step that allocates nothing ---------------------------
 *
 * For callers that cannot allocate device memory or provide a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, results and errors as wango_decode_step
 * without the workspace: its scratch is a library-owned device array of
 * TANGO_NOALLOC_SCRATCH_BYTES bytes, one per GPU the library runs on, held
 * from the first call on that GPU until the process ends.  The call allocates
 * nothing (no hipMalloc, no allocating library routine).
 *   - A shape whose scratch, wango_decode_workspace_size(shape, window,
 *     phi_dim), exceeds TANGO_NOALLOC_SCRATCH_BYTES is TANGO_ERR_WORKSPACE
 *     before anything runs (at d_model 512 and d_gate 2048: up to 640
 *     sequences per call).
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents.  The step clears what must start at zero (its output
 *     counters) in its own first kernel and writes everything else before
 *     reading it, so calls ordered on one stream are independent; calls that
 *     can overlap on one GPU (unordered streams, or several host threads)
 *     race on the array and must be serialised by the caller.
 *   - The state is the caller's, as for wango_decode_step. */
#define TANGO_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int wango_decode_step_noalloc(const tango_shape_t* shape, const tango_weights_t* weights, int32_t window,
                              int32_t phi_dim, const int32_t* pos, const void* x, void* out, void* state,
                              size_t state_bytes, void* hip_stream);

/* ---- Diagnostics --------------------------------------------------------- */

const char* tango_status_string(int status);  /* static string, never NULL        */
const char* tango_last_error(void);           /* thread-local detail, never NULL  */
int tango_version(void);                      /* TANGO_ABI_VERSION                */

/* ---- Stage entry points (for stage-by-stage parity tests) ---------------
 *
 * They run one kernel (or the kernels of one step) of the block on caller
 * buffers.  Intermediate layouts:
 *   Tp        = seq_len rounded up to a multiple of 128 (rows >= T are padding
 *               that the projection stage writes as zeros);
 *   Fh, Fhp   = d_gate / n_heads, and the padded head width: Fh itself when
 *               it is a multiple of 64; otherwise, for the WANGO stages, Fh
 *               rounded up to a multiple of 64, and for the TANGO stages to a
 *               multiple of 512 if that is at most 1.2 Fh, else of 64;
 *   F'        = n_heads * Fhp: gp and n_old have F' columns, head a's gate
 *               column c at a * Fhp + c, and the projection stages write zeros
 *               into the gates' pad columns c >= Fh;
 *   V         = [B, Tp, d_gate] row-major, not padded: bfloat16 with dtype
 *               bf16 and one operand part (the output stage rounds gbar * v
 *               to bf16 anyway), else float32 (with two parts the output
 *               stage carries gbar * v to about 2^-16, so v is kept
 *               unrounded);
 *   gbar      = [B, Tp, d_gate] row-major, dtype (not padded);
 *   qh, kh    = [B, Tp, H*d_h] row-major, dtype, unit length per head;
 *   gp        = the gates g in the source-packed layout [B][Tp/32][4][F'][8]:
 *               element (b, blk, grp, f, s) holds g[b, t, f] for
 *               t = 32*blk + (s < 4 ? 4*grp + s : 16 + 4*grp + (s - 4));
 *   fk        = phi(sqrt(tau) k) (the WANGO key features of [TANGO] eq. 8) in
 *               the same source-packed layout over the H*d_h feature columns;
 *   fq        = phi(sqrt(tau) q), [B, Tp, H*d_h], with the features of every
 *               group of 32 stored in the order e = 4*grp + s (s < 4) or
 *               16 + 4*grp + (s - 4), at position 8*grp + s of the group;
 *   n_old     = float32 in 16 x 16 blocks [B*Tp/16][F'/16][64][4]: entry
 *               (blk_i, blk_f, l, r) holds row 16*blk_i + l % 16 and column
 *               16*blk_f + 4*(l / 16) + r;
 *   z_old     = [B, Tp, H] float32.
 * The WANGO scan leaves in n_old, z_old the read-out phi(sqrt(tau) q_i)^T S and
 * phi(sqrt(tau) q_i)^T z of the running sums of eq. 10 over the sources before
 * c_i = chunk * floor((i - window) / chunk) (zero for i < window); the band
 * stage adds the older sources c_i <= j <= i - window pairwise.
 */

/* Bytes of scratch the projection stages need for `shape` (the RMSNorm row
 * scales and the dtype parts of the normalised input rows); 0 if the shape is
 * invalid. */
size_t tango_proj_workspace_size(const tango_shape_t* shape);

/* TANGO projections ([TANGO] §2.1 eq. 2 and the head paragraph): RMSNorm,
 * SiLU gate (packed), features, RoPE + unit-norm queries and keys.  workspace:
 * at least tango_proj_workspace_size(shape) bytes of scratch. */
int tango_stage_proj(const tango_shape_t* shape, const tango_weights_t* weights,
                     const void* x, void* gp, void* v, void* qh, void* kh, void* workspace,
                     size_t workspace_bytes, void* hip_stream);

/* WANGO projections: as tango_stage_proj, plus the features fq, fk of eq. 8
 * (needs weights->theta). */
int wango_stage_proj(const tango_shape_t* shape, const tango_weights_t* weights,
                     const void* x, void* gp, void* v, void* qh, void* kh, void* fq, void* fk,
                     void* workspace, size_t workspace_bytes, void* hip_stream);

/* TANGO aggregation ([TANGO] eqs. 4-6): gbar from qh, kh, gp.  Needs the same
 * workspace as tango_block_fwd (it uses the split-sum scratch area). */
int tango_stage_aggregate(const tango_shape_t* shape, const float* theta,
                          const float* null_bias, const void* qh, const void* kh,
                          const void* gp, void* gbar, void* workspace, size_t workspace_bytes,
                          void* hip_stream);

/* Output projection and residual ([TANGO] eq. 3): out = x + (gbar * v) W_o^T. */
int tango_stage_out(const tango_shape_t* shape, const void* w_o, const void* x,
                    const void* gbar, const void* v, void* out, void* hip_stream);

/* WANGO running sums ([TANGO] eqs. 8-10): n_old, z_old as described above.
 * Needs the workspace of wango_block_fwd (segment-state scratch). */
int wango_stage_scan(const tango_shape_t* shape, int32_t window, int32_t chunk,
                     const void* fq, const void* fk, const void* gp, void* n_old, void* z_old,
                     void* workspace, size_t workspace_bytes, void* hip_stream);

/* WANGO window band and joint normalisation ([TANGO] eqs. 5, 7 and the
 * joint-normalisation paragraph of §2.2): gbar from the window exp weights,
 * the pairwise phi weights of the older sources in the chunk next to the
 * window, n_old, z_old and the null term. */
int wango_stage_band(const tango_shape_t* shape, const float* theta, const float* null_bias,
                     int32_t window, int32_t chunk, const void* qh, const void* kh, const void* gp,
                     const float* n_old, const float* z_old, void* gbar, void* hip_stream);

/* ---- Backward pass of the TANGO aggregation --------------------------------
 *
 * The pages train this block in bfloat16 ([TANGO] §3, training recipe); these
 * two calls are the aggregation's part of a training step.  bfloat16 only
 * (TANGO_ERR_UNSUPPORTED for float32).  Layouts as for the stage entry points.
 *
 * tango_aggregate_fwd_train: tango_stage_aggregate that also writes
 *   den [B, Tp, H] float32: the denominator of the ratio of eq. 5 in units of
 *   e^{-tau} (sum_{j<=i} e^{tau (q_i.k_j - 1)} + n_i e^{b - tau}), rows < T;
 *   the backward pass reads it.  Same workspace as tango_stage_aggregate.
 *
 * tango_aggregate_bwd: given the forward's qh, kh, gp, gbar, den and the
 *   incoming gradient dgbar ([B, Tp, d_gate] bf16; rows >= T ignored), writes
 *   the gradients of sum(dgbar * gbar):
 *     dq, dk [B, Tp, H*d_h] float32 with respect to the unit vectors qh, kh
 *            as given (the normalisation and RoPE before them are the caller's
 *            chain rule); rows >= T are written as zeros;
 *     dg     [B, Tp, d_gate] bf16 with respect to the gates (not packed);
 *            rows >= T are not written;
 *     dtheta [H] float32 with respect to theta (zero where theta >= log 20,
 *            the clip of eq. 4);
 *     dnull  [H] float32 with respect to the null bias b of eq. 5 (NULL iff
 *            null_bias is NULL).
 *   Formulas: u_i = dgbar_i / den_i, delta_i = -u_i . gbar_i,
 *   dg_j = sum_{i>=j} w_ij u_i, ds_ij = tau w_ij (u_i . g_j + delta_i),
 *   dq_i = sum_j ds_ij k_j, dk_j = sum_i ds_ij q_i, dtheta = sum ds_ij s_ij,
 *   dnull = sum_i delta_i n_i e^{b - tau}, with w_ij = e^{tau (s_ij - 1)}.
 *   workspace: at least tango_aggregate_bwd_workspace_size(shape) bytes of
 *   scratch (0 is returned for an invalid or unsupported shape).  The call
 *   runs on hip_stream without synchronising; buffers must not overlap. */
int tango_aggregate_fwd_train(const tango_shape_t* shape, const float* theta,
                              const float* null_bias, const void* qh, const void* kh,
                              const void* gp, void* gbar, float* den, void* workspace,
                              size_t workspace_bytes, void* hip_stream);
size_t tango_aggregate_bwd_workspace_size(const tango_shape_t* shape);
int tango_aggregate_bwd(const tango_shape_t* shape, const float* theta, const float* null_bias,
                        const void* qh, const void* kh, const void* gp, const void* gbar,
                        const float* den, const void* dgbar, float* dq, float* dk, void* dg,
                        float* dtheta, float* dnull, void* workspace, size_t workspace_bytes,
                        void* hip_stream);

/* ---- Backward of the WANGO aggregation ------------------------------------
 *
 * Gradients of L = sum(dgbar * gbar) for the WANGO aggregation ([TANGO] §2.2
 * eqs. 7-10; the pages train the block, §3, but print no gradient): window
 * sources i-W < j <= i weighted by exp(tau q_i.k_j), older sources j <= i-W by
 * phi(sqrt(tau) q_i) . phi(sqrt(tau) k_j) (eq. 8), one joint normalisation with
 * the null term.  With p, a the two feature vectors and dm_ij = u_i.g_j +
 * delta_i (u, delta as for TANGO):
 *   ds_ij = tau w_ij dm_ij on window pairs, dP_ij = dm_ij on older pairs,
 *   dq_i = sum_j ds_ij k_j + sqrt(tau) phi'(sqrt(tau) q_i) * sum_j dP_ij a_j,
 *   dk_j alike, dg_j = sum_i (weight_ij) u_i, dtheta through tau in the
 *   window weights and in the features (zero where theta >= log 20).
 * bf16 only; window <= 897 and chunk as for wango_block_fwd.  Shapes, layouts
 * and outputs as for tango_aggregate_bwd, with the gates packed at the WANGO
 * head padding (F' columns as for wango_stage_scan).
 *
 * wango_aggregate_fwd_train: the WANGO aggregation (scan + band) from unit q,
 * k and packed gates, also storing den [B, Tp, H] float32 (e^{-tau} units, rows
 * < T) for the backward; workspace of
 * wango_aggregate_fwd_train_workspace_size bytes.
 * wango_aggregate_bwd: dq, dk [B, Tp, H*d_h] float32, dg [B, Tp, d_gate] bf16,
 * dtheta [H], dnull [H] (or NULL with null_bias NULL); workspace of
 * wango_aggregate_bwd_workspace_size bytes.  Both run on hip_stream without
 * synchronising; buffers must not overlap; 0 sizes for invalid arguments. */
size_t wango_aggregate_fwd_train_workspace_size(const tango_shape_t* shape, int32_t window, int32_t chunk);
int wango_aggregate_fwd_train(const tango_shape_t* shape, int32_t window, int32_t chunk, const float* theta,
                              const float* null_bias, const void* qh, const void* kh, const void* gp,
                              void* gbar, float* den, void* workspace, size_t workspace_bytes,
                              void* hip_stream);
size_t wango_aggregate_bwd_workspace_size(const tango_shape_t* shape, int32_t window, int32_t chunk);
int wango_aggregate_bwd(const tango_shape_t* shape, int32_t window, int32_t chunk, const float* theta,
                        const float* null_bias, const void* qh, const void* kh, const void* gp,
                        const void* gbar, const float* den, const void* dgbar, float* dq, float* dk,
                        void* dg, float* dtheta, float* dnull, void* workspace, size_t workspace_bytes,
                        void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* TANGO_H_ */
