/*
 * kda.h -- C ABI of libkda, the Kimi Delta Attention (KDA) operator for
 * AMD Instinct MI355X (gfx950).
 *
 * The operator (Kimi Linear tech report, section 3, Eq. 1; also
 * "Diagonal-Plus-Low-Rank Matrices and Kimi Delta Attention", section 2):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t                          (read from the updated state)
 *     alpha_t = exp(g_min * sigmoid(z_t)),  g_min < 0   ("KDA Recurrence")
 *
 * with one d_k x d_v state per (batch, head).  Three calls cover the path:
 * chunkwise prefill, one decode token, and the output epilogue; two more
 * run the whole layer (recurrence and epilogue together), one for a prefill
 * and one for a decode token, two take the scalar-gate (Gated DeltaNet)
 * special case, and one gives the recurrence's gradients for training.
 *
 * Conventions shared by every call
 *  - All tensor pointers are DEVICE pointers owned by the caller, contiguous
 *    and row-major in the layouts given below, and 16-byte aligned.  The
 *    library never allocates or frees device memory; scratch space comes
 *    from a caller-provided workspace whose size a query function returns.
 *  - Inputs are never written (the one exception is the decode state,
 *    which is the carry and is updated in place).
 *  - Token tensors use one dtype (KDA_F32 or KDA_BF16) for q, k, v, z,
 *    beta, the gate logits and the outputs o / y.  The recurrent state is
 *    always fp32.
 *  - Supported sizes: d_k, d_v in {64, 128}; chunk == 64; B, H >= 1;
 *    T >= 0 (any T: the last chunk is masked).  Other sizes return
 *    KDA_ERR_UNSUPPORTED.
 *  - Arguments are checked on the host before anything is launched; a bad
 *    argument returns a status and launches nothing.  Work is enqueued on
 *    `stream` (a hipStream_t; NULL means the null stream) and the call
 *    returns without waiting; a launch failure is reported as KDA_ERR_HIP.
 *    Device-side faults surface at the caller's next synchronisation.
 *    Setting the environment variable KDA_DEBUG_SYNC=1 makes every call
 *    synchronise its stream and report execution errors as KDA_ERR_HIP.
 *  - Not checked on the device: beta in [0, 1] and finite inputs (the
 *    "KDA Recurrence" constraints).  g_min must be finite and < 0.
 *  - The library keeps no state between calls and is re-entrant; calls on
 *    different streams may run concurrently if their buffers are disjoint
 *    (kda_chunk_fwd_noalloc excepted: it shares one scratch array per GPU).
 *  - Calls may be captured into a HIP graph (they allocate nothing, record
 *    no memset and never synchronise, unless KDA_DEBUG_SYNC=1).
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,         /* a required pointer is NULL                  */
    KDA_ERR_SHAPE = 2,        /* a size is negative or overflows             */
    KDA_ERR_UNSUPPORTED = 3,  /* d_k / d_v / chunk / dtype not supported     */
    KDA_ERR_ARG = 4,          /* g_min not finite and negative, eps < 0 ...  */
    KDA_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than required     */
    KDA_ERR_ALIGN = 6,        /* a pointer is not 16-byte aligned            */
    KDA_ERR_HIP = 7,          /* a HIP launch or execution error             */
    KDA_ERR_SCRATCH = 8       /* the call needs more scratch than the static */
                              /* array of kda_chunk_fwd_noalloc holds         */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/*
 * Decay bound of the chunkwise kernels.  Inside a 64-token chunk the decay
 * products e^{G_r - G_i} (tech report, appendix B, gamma_{i->r}) are split
 * into per-row and per-column factors around 16-row block references; each
 * factor spans up to eight tokens of decay, at most 8 |g_min| nats, and the
 * factor between two blocks is applied as its square root twice.  For
 * g_min >= KDA_CHUNK_G_MIN_LIMIT every factor is finite in fp32 and bf16 (at
 * most 2^93) and what underflow drops is below 2^-40.  For g_min below it the
 * prefill calls (kda_chunk_fwd, kda_chunk_layer_fwd, kda_gdn_chunk_fwd) run a
 * token-sequential kernel instead: one workgroup per (batch, head) applies
 * alpha_t token by token, exact for any g_min < 0 but latency-bound (about a
 * microsecond per token).  Decode and the backward are token steps already
 * and have no such bound.
 */
#define KDA_CHUNK_G_MIN_LIMIT (-8.0f)

/* Human-readable name of a status code (static string, never NULL). */
const char* kda_status_str(kda_status s);

/* Library build identification (static string). */
const char* kda_version(void);

/*
 * Chunkwise prefill.
 *
 * Computes o_t for t = 0..T-1 and the state after the last token, for every
 * (batch, head), by the chunkwise expansion of Eq. 1 (tech report, section
 * 3.1 and appendix B, Propositions 1-2 / Eqs. 16-19): per 64-token chunk,
 * the decay-weighted key-key and query-key products, the unit-lower
 * triangular solve that yields the WY/UT auxiliaries W and U, and the
 * chunk-to-chunk state propagation.
 *
 *   q, k, z   (B, T, H, dk)  dtype dt   queries, keys, decay logits
 *   v         (B, T, H, dv)  dtype dt   values
 *   beta      (B, T, H)      dtype dt   write strengths
 *   g_min                                lower log-decay bound, < 0
 *   s0        (B, H, dk, dv) fp32       initial state, or NULL for zeros
 *   o         (B, T, H, dv)  dtype dt   output (written)
 *   s_final   (B, H, dk, dv) fp32       final state (written), or NULL to
 *                                        skip; may equal s0 (in place)
 *   workspace, workspace_bytes           device scratch of at least
 *                                        kda_chunk_fwd_workspace_bytes()
 *                                        bytes; may be NULL when that is 0
 * The result is deterministic: identical inputs give identical bits.
 *
 * g_min below KDA_CHUNK_G_MIN_LIMIT runs the token-sequential kernel (see
 * there); it needs no workspace, but the size query does not depend on g_min.
 *
 * Workspace: bf16 sequences split into segments when there are fewer than
 * 256 (batch, head) chains (the per-segment transition P, input term R and
 * entry state, fp32; with dk = dv = 128 also every chunk's
 * T' = (I + A)^-1 diag(beta), 64 x 64 bf16, which the pass that composes
 * the segments hands to the pass that writes the outputs; there the first
 * and last segments of each sequence are expanded directly, without a
 * transition); a single segment needs no workspace.  fp32 sequences also stage the per-chunk products
 * (W, U^T, M, q e^G, (k e^{G_C-G})^T, e^{G_C}).
 */
size_t kda_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk,
                                     kda_dtype dt);
kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const void* z,
                         const void* beta, float g_min, const float* s0, void* o,
                         float* s_final, int B, int T, int H, int dk, int dv, int chunk,
                         kda_dtype dt, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * kda_chunk_fwd without a caller workspace and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.
 *
 * The scratch space kda_chunk_fwd takes from its workspace comes instead from
 * one static device array of KDA_NOALLOC_SCRATCH_BYTES per GPU, which the
 * library holds from its first use on that GPU until the process ends.
 * Arguments and results are exactly those of kda_chunk_fwd (same kernels,
 * bit-identical results).  A call whose kda_chunk_fwd_workspace_bytes()
 * exceeds KDA_NOALLOC_SCRATCH_BYTES returns KDA_ERR_SCRATCH and launches
 * nothing; 176 MiB covers the 32-head, 32768-token bf16 prefill.
 *
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap on one GPU (on different streams, or from
 * different threads) race and must be serialised by the caller.  Nothing in
 * the array needs to start at any value: the kernels write every slot
 * before they read it.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)192 << 20)
kda_status kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* z,
                                 const void* beta, float g_min, const float* s0, void* o,
                                 float* s_final, int B, int T, int H, int dk, int dv, int chunk,
                                 kda_dtype dt, void* stream);

/*
 * One decode token for every (batch, head): the fused recurrent step.
 *
 * Order of the per-token step (agentlenshq blog on KDA, section on the
 * fused recurrent decode kernel; "KDA Recurrence" readout rule): decay the
 * state by alpha, predict p = S'^T k, residual r = beta (v - p), write
 * S = S' + k r^T, read o = S^T q from the updated state.
 *
 *   q, k, z   (B, H, dk)  dtype dt
 *   v         (B, H, dv)  dtype dt
 *   beta      (B, H)      dtype dt
 *   state     (B, H, dk, dv) fp32, read and updated IN PLACE
 *   o         (B, H, dv)  dtype dt (written)
 * The state is read once and written once per call.
 */
kda_status kda_recurrent_step(const void* q, const void* k, const void* v, const void* z,
                              const void* beta, float g_min, float* state, void* o,
                              int B, int H, int dk, int dv, kda_dtype dt, void* stream);

/*
 * Output epilogue ("KDA Recurrence" problem statement and first worked
 * example): per (batch, token, head), RMS normalisation over the d_v values
 * with eps inside the square root and no learnable weight, multiplied by
 * sigmoid(gate); heads concatenated to width H*d_v; then, if w is given,
 * the projection out = y W^T with W of shape (d_model, H*d_v) and no bias.
 *
 *   o, gate   (B, T, H, dv)        dtype dt
 *   eps                             >= 0
 *   w         (d_model, H*dv) bf16, or NULL for no projection
 *   y         (B, T, H*dv) dtype dt when w is NULL,
 *             (B, T, d_model) dtype dt otherwise (written)
 *   workspace kda_out_gate_workspace_bytes() bytes (0 when w is NULL): the
 *             gated activations y and the projection GEMM's scratch
 * With a projection, dt must be KDA_BF16 and d_model a multiple of 16.  The
 * projection is libkda's own GEMM (bf16 MFMA, fp32 accumulation, output
 * rounded to bf16); for up to 1024 rows with d_model a multiple of 128 and
 * H * dv a multiple of 256 it splits the K range in eight and adds the fp32
 * partials in a fixed order, using M * d_model * 32 bytes of the workspace.
 */
size_t kda_out_gate_workspace_bytes(int B, int T, int H, int dv, int d_model, kda_dtype dt,
                                    int with_projection);
kda_status kda_out_gate(const void* o, const void* gate, float eps, const void* w, void* y,
                        int B, int T, int H, int dv, int d_model, kda_dtype dt,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode token of the whole layer of the "KDA Recurrence" problem:
 * the token step of kda_recurrent_step, then the output epilogue of
 * kda_out_gate (RMS normalisation over the d_v values with eps inside the
 * square root, times sigmoid(gate), heads concatenated, then y W^T when w
 * is given).  The normalisation and gate run in the recurrence step's own
 * launch, on the fp32 read-out before any rounding; the projection, when
 * asked for, is a second launch (libkda's GEMM, as in kda_out_gate).
 *
 *   q, k, z   (B, H, dk)  dtype dt
 *   v, gate   (B, H, dv)  dtype dt
 *   beta      (B, H)      dtype dt
 *   g_min, eps            as for kda_recurrent_step and kda_out_gate
 *   state     (B, H, dk, dv) fp32, read and updated IN PLACE
 *   w         (d_model, H*dv) bf16, or NULL for no projection
 *   o         (B, H, dv) dtype dt: the raw read-out S^T q (written), or
 *             NULL to skip it
 *   y         (B, H*dv) dtype dt when w is NULL, (B, d_model) dtype dt
 *             otherwise (written)
 *   workspace kda_recurrent_layer_step_workspace_bytes() bytes (0 when w is
 *             NULL): the gated rows in bf16 and the projection's scratch
 * With a projection, dt must be KDA_BF16 and d_model a multiple of 16.
 * Every other rule is that of kda_recurrent_step and kda_out_gate.
 */
size_t kda_recurrent_layer_step_workspace_bytes(int B, int H, int dv, int d_model, kda_dtype dt,
                                                int with_projection);
kda_status kda_recurrent_layer_step(const void* q, const void* k, const void* v, const void* z,
                                    const void* beta, float g_min, float* state, const void* gate,
                                    float eps, const void* w, void* o, void* y, int B, int H, int dk,
                                    int dv, int d_model, kda_dtype dt, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * The prefill of the whole layer of the "KDA Recurrence" problem:
 * kda_chunk_fwd, then the output epilogue of kda_out_gate (RMS normalisation
 * over each (token, head)'s d_v values with eps inside the square root,
 * times sigmoid(gate), heads concatenated, then y W^T when w is given).
 *
 *   q, k, z, v, beta, g_min, s0, s_final   as for kda_chunk_fwd
 *   gate      (B, T, H, dv)   dtype dt    output-gate logits
 *   eps, w, d_model                        as for kda_out_gate
 *   o         (B, T, H, dv)   dtype dt    the raw outputs (written), or NULL
 *                                          to skip them
 *   y         (B, T, H*dv) dtype dt when w is NULL, (B, T, d_model) dtype dt
 *             otherwise (written)
 *   workspace kda_chunk_layer_fwd_workspace_bytes() bytes: that of
 *             kda_chunk_fwd (256-byte aligned), then room for o where the
 *             epilogue is a launch of its own, then that of kda_out_gate
 * With bf16 tokens, d_k = d_v = 128 and a sequence split into segments
 * (fewer than 256 (batch, head) chains and at least 16 chunks), the
 * normalisation and gate run inside the prefill's last kernel, on the
 * outputs rounded to bf16 (the values kda_out_gate would read back), so o
 * need not be written (the first and last segments' outputs, which that
 * kernel does not gate, go to o, or else to the rows the epilogue writes: y,
 * or with a projection the workspace's gated rows; one more launch gates
 * them); the projection, when asked for, is a launch of its own.  Other sizes run kda_chunk_fwd's kernels and then kda_out_gate's.
 * Every other rule is that of kda_chunk_fwd and kda_out_gate.
 */
size_t kda_chunk_layer_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk,
                                           int d_model, kda_dtype dt, int with_projection);
kda_status kda_chunk_layer_fwd(const void* q, const void* k, const void* v, const void* z,
                               const void* beta, float g_min, const float* s0, const void* gate,
                               float eps, const void* w, void* o, void* y, float* s_final, int B,
                               int T, int H, int dk, int dv, int chunk, int d_model, kda_dtype dt,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * The Gated DeltaNet special case: one decay logit per (token, head), so
 * alpha_t = exp(g_min * sigmoid(z_t)) is a scalar and Diag(alpha_t) =
 * alpha_t I (Kimi Linear tech report, section 3, where KDA refines Gated
 * DeltaNet's scalar gate into a channel-wise one).  Same operator, readout
 * and conventions as kda_chunk_fwd / kda_recurrent_step, except:
 *
 *   z   (B, T, H) for kda_gdn_chunk_fwd, (B, H) for kda_gdn_recurrent_step,
 *       dtype dt
 *
 * The prefill runs on the channel-wise kernels.  With bf16 tokens, d_k =
 * d_v = 128 and g_min >= KDA_CHUNK_G_MIN_LIMIT they read the logit of each
 * (token, head) directly and form its decay factors once per token instead
 * of once per channel; otherwise the logits are first written across the
 * d_k channels of the workspace.  The workspace size
 * kda_gdn_chunk_fwd_workspace_bytes() returns covers both (that of
 * kda_chunk_fwd, rounded up to 256 bytes, plus B*T*H*dk elements).  Decode
 * reads the scalar directly and needs no workspace.  The results equal those
 * of the channel-wise calls given z repeated over the channels, bit for bit.
 */
size_t kda_gdn_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk,
                                         kda_dtype dt);
kda_status kda_gdn_chunk_fwd(const void* q, const void* k, const void* v, const void* z,
                             const void* beta, float g_min, const float* s0, void* o,
                             float* s_final, int B, int T, int H, int dk, int dv, int chunk,
                             kda_dtype dt, void* workspace, size_t workspace_bytes,
                             void* stream);
kda_status kda_gdn_recurrent_step(const void* q, const void* k, const void* v, const void* z,
                                  const void* beta, float g_min, float* state, void* o,
                                  int B, int H, int dk, int dv, kda_dtype dt, void* stream);

/*
 * Gradients of the recurrence of Eq. 1 (with the decay and readout of
 * "KDA Recurrence") for a loss whose gradients with respect to the outputs o
 * and the final state are given: the backward of kda_chunk_fwd, and of a
 * run of kda_recurrent_step.  The pages give no gradient formulas; these are
 * the chain rule through one token, S' = Diag(alpha) S, w = v - S'^T k,
 * S_t = S' + beta k w^T, o = S_t^T q, taken in reverse:
 *   dq = S_t do, dS += q do^T, u = dS^T k, dbeta = u . w, dv = beta u,
 *   dk = beta dS w - beta S' u, dalpha = rowsum(S_{t-1} * (dS - beta k u^T)),
 *   dz = dalpha * alpha * g_min * sigmoid(z) (1 - sigmoid(z)),
 *   dS <- Diag(alpha) (dS - beta k u^T).
 *
 *   q, k, v, z, beta, g_min, s0   the forward's inputs, as for kda_chunk_fwd
 *   grad_o        (B, T, H, dv) dtype dt   gradient with respect to o
 *   grad_s_final  (B, H, dk, dv) fp32      gradient with respect to the final
 *                                           state, or NULL for zeros
 *   grad_q, grad_k, grad_z (B, T, H, dk), grad_v (B, T, H, dv),
 *   grad_beta (B, T, H): fp32 (written)
 *   grad_s0       (B, H, dk, dv) fp32 (written), or NULL to skip
 *   workspace     kda_recurrent_bwd_workspace_bytes() bytes: per (batch,
 *                 head) the state at the start of every 64-token interval
 *                 and one interval's per-token states (min(64, T) of them),
 *                 fp32; none when T == 0
 * Token-sequential: one workgroup per (batch, head) recomputes the states
 * from the stored interval starts and steps back through the tokens; all
 * arithmetic in fp32.  Every other rule is that of kda_chunk_fwd.
 */
size_t kda_recurrent_bwd_workspace_bytes(int B, int T, int H, int dk, int dv);
kda_status kda_recurrent_bwd(const void* q, const void* k, const void* v, const void* z,
                             const void* beta, float g_min, const float* s0, const void* grad_o,
                             const float* grad_s_final, float* grad_q, float* grad_k, float* grad_v,
                             float* grad_z, float* grad_beta, float* grad_s0, int B, int T, int H,
                             int dk, int dv, kda_dtype dt, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * The general diagonal-plus-low-rank (DPLR) recurrence ("Diagonal-Plus-Low-
 * Rank Matrices and Kimi Delta Attention", sections 1 and 3):
 *
 *   S_t = (Diag(alpha_t) - a_t b_t^T) S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t,
 *
 * with two independent directions a_t and b_t, the decay alpha_t =
 * exp(g_min * sigmoid(z_t)) of "KDA Recurrence", and the output read from
 * the updated state.  Section 3's binding a_t = beta_t k_t, b_t = k_t *
 * alpha_t with the write key beta_t k_t gives KDA (kda_chunk_fwd).
 *
 *   q, k, z, a, b   (B, T, H, dk)  dtype dt      (no T for the step)
 *   v               (B, T, H, dv)  dtype dt
 *   g_min           < 0, finite
 *   s0              (B, H, dk, dv) fp32, or NULL for zeros
 *   o               (B, T, H, dv)  dtype dt (written)
 *   s_final         (B, H, dk, dv) fp32 (written), or NULL to skip
 *   state           (B, H, dk, dv) fp32, read and updated IN PLACE (step)
 * Per token, c = S_{t-1}^T b_t is read from the state before the update,
 * S_t = Diag(alpha) S_{t-1} - a c^T + k v^T and o = (Diag(alpha)
 * S_{t-1})^T q - (a . q) c + (k . q) v; all arithmetic in fp32.
 * kda_dplr_fwd is token-sequential, one workgroup per (batch, head) with
 * the state in registers; it needs no workspace, and T may be 0 (then
 * s_final = s0).  kda_dplr_recurrent_step reads the state once and writes it
 * once.  dk, dv in {64, 128}; every pointer 16-byte aligned; B, H at most
 * 65535 for kda_dplr_fwd; other errors as for kda_chunk_fwd.
 */
kda_status kda_dplr_fwd(const void* q, const void* k, const void* v, const void* z, const void* a,
                        const void* b, float g_min, const float* s0, void* o, float* s_final,
                        int B, int T, int H, int dk, int dv, kda_dtype dt, void* stream);
kda_status kda_dplr_recurrent_step(const void* q, const void* k, const void* v, const void* z,
                                   const void* a, const void* b, float g_min, float* state, void* o,
                                   int B, int H, int dk, int dv, kda_dtype dt, void* stream);

/*
 * The same DPLR recurrence by 64-token chunks: per chunk, with G the
 * chunk-local cumulative log-decay (G- the one before each token) and T =
 * (I + L)^{-1},
 *   L_ri = b_r . e^{G-_r - G_i} a_i (i < r),   X = T (B e^{G-}) S + T Mbk V,
 *   O    = (Q e^G) S + Mqk V - Mqa X,
 *   S'   = Diag(e^{G_C}) S + (K e^{G_C - G})^T V - (A e^{G_C - G})^T X,
 * where Mbk, Mqk, Mqa are the decayed products of b with k, q with k and q
 * with a (Mbk strictly, the other two inclusively lower triangular): four
 * decayed products per chunk, evaluated per 16-token block pair around
 * reference rows (section 3's secondary chunking), where KDA's binding needs
 * two.  Arguments as for kda_dplr_fwd, plus:
 *   chunk      64
 *   workspace  kda_dplr_chunk_fwd_workspace_bytes() bytes (per chunk the
 *              products, T-weighted terms and decayed operands in the compute
 *              precision, bf16 for bf16 tokens, else fp32; for sequences of at
 *              least 32 chunks also per 16-chunk segment a d_k x d_k
 *              transition, an input term and an entering state, fp32)
 * For g_min below KDA_CHUNK_G_MIN_LIMIT, and for T == 0, the call runs the
 * token-sequential kernel of kda_dplr_fwd (the workspace is then unused).
 * bf16 tokens: products in bf16 on MFMA with fp32 accumulation, state fp32.
 */
size_t kda_dplr_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk,
                                          kda_dtype dt);
kda_status kda_dplr_chunk_fwd(const void* q, const void* k, const void* v, const void* z,
                              const void* a, const void* b, float g_min, const float* s0, void* o,
                              float* s_final, int B, int T, int H, int dk, int dv, int chunk,
                              kda_dtype dt, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same gradients as kda_recurrent_bwd by 64-token chunks, on MFMA: the
 * chain rule through the chunk form (Kimi Linear tech report, section 3.1
 * and appendix B, Eqs. 16-19) instead of through single tokens.  Per chunk
 * with entering state S and the gradient dS' of the state leaving it:
 *   dV_new = M^T dO + (K e^{G_C - G}) dS',
 *   dS     = e^{G_C} dS' + (Q e^G)^T dO - W^T dV_new   (the chunks in reverse),
 * and the token gradients from dV_new, S, dS' and the chunk's own products
 * (the adjoint of T = (I + A)^{-1} is -T^T dT T^T; every product carrying
 * e^{G_r - G_i} is evaluated per 16-token block pair around reference rows,
 * as in the forward).  Arguments as for kda_recurrent_bwd, plus chunk (64);
 * the workspace, kda_chunk_bwd_workspace_bytes() bytes, holds per chunk the
 * forward operands of both directions, the entering state (fp32), V_new and
 * the reverse pass's products for the per-chunk kernel (fp32).
 * Precision: bf16 tokens run the chunk recurrences on bf16 MFMA with fp32
 * accumulation and state (as kda_chunk_fwd does), so the gradients carry
 * bf16 operand rounding; the per-chunk kernel runs on fp32 MFMA.  fp32 tokens
 * run on fp32 MFMA throughout where d_v = 64; with fp32 tokens and d_v = 128,
 * for g_min below KDA_CHUNK_G_MIN_LIMIT, and for T == 0, the call runs the
 * token-sequential kernel of kda_recurrent_bwd.
 */
size_t kda_chunk_bwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, kda_dtype dt);
kda_status kda_chunk_bwd(const void* q, const void* k, const void* v, const void* z, const void* beta,
                         float g_min, const float* s0, const void* grad_o, const float* grad_s_final,
                         float* grad_q, float* grad_k, float* grad_v, float* grad_z, float* grad_beta,
                         float* grad_s0, int B, int T, int H, int dk, int dv, int chunk, kda_dtype dt,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Measurement helper: x <- s * x in place over n fp32 values (n a multiple
 * of 4, x 16-byte aligned), every byte read once and written once with
 * 16-byte accesses -- the access pattern of the decode step's state.  It
 * gives the read-modify-write rate the GPU's HBM sustains, against which
 * kda_recurrent_step is measured.  variant: bits 0-1 pick 1, 2, 4 or 8 float4
 * in flight per thread, bit 2 non-temporal accesses, bits 3 and up the waves
 * per compute unit of a grid-stride launch (0: one workgroup per slice).
 */
kda_status kda_stream_scale(float* x, size_t n, float s, int variant, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
