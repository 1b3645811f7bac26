/*
 * kda.h -- C ABI of the MI355X (gfx950) gated delta-rule library, libkda.so.
 *
 * The operator is the diagonal-plus-rank-one recurrence of Kimi Delta
 * Attention and its extensions, as described in "Complex KDA: Understanding
 * and Enhancing the Expressivity of Kimi Delta Attention" (summary page,
 * background "diagonal-plus-rank-one transitions" and core method):
 *
 *   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *   o_t = S_t^T q_t
 *
 * per (sequence, head), with state S in R^{dk x dv} read on the key side
 * (Dual DeltaNet abstract). KDA uses a per-channel gate alpha_t in R^{dk};
 * GDN is the scalar-gate case (one alpha per token and head); Complex KDA
 * allows alpha in [-1, 1] (negative and exactly zero gates) and beta in
 * [0, 2]. The gate is applied first, then the rank-one delta term; there is
 * no query scaling and no key normalisation inside the library.
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers (hipMalloc'd or equivalent),
 *    row-major and contiguous, aligned to their element size. The decode
 *    state S and output o, the forward's q, k, v and gate, and any
 *    workspace, must be 16-byte aligned.
 *    The caller owns every buffer.
 *  - Element type of q, k, v, gate and beta is selected by `dtype`:
 *    KDA_BF16 (bfloat16 bits) or KDA_F32. States S0, S_T, S and outputs o
 *    are always fp32.
 *  - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *    and the call returns without synchronising.
 *  - Arguments are validated before any HIP call; nothing is enqueued when
 *    validation fails. Device-side contents (cu_seqlens offsets, NaN/Inf in
 *    inputs) are not checked: NaN/Inf propagate.
 *  - Supported sizes: dk, dv in {16, 32, 64, 128}; chunk in {16, 32, 64}.
 *  - The library never allocates, frees or synchronises device memory in a
 *    compute call: every call that needs scratch space takes a caller-owned
 *    workspace, and a NULL workspace (or a short one) is KDA_EINVAL.
 *  - Calls are re-entrant and keep no state between calls (the compute-unit
 *    count that picks a state walker is queried from the runtime on each
 *    call). Two calls may run concurrently on different streams if they do
 *    not share output or workspace buffers.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define KDA_OK 0
#define KDA_EINVAL (-1)  /* null required pointer, non-positive size, inconsistent counts, short workspace */
#define KDA_ENOTSUP (-2) /* dk, dv, chunk, dtype or gate_kind outside the supported set */
#define KDA_EALIGN (-3)  /* a pointer violates the alignment rules above */
#define KDA_EHIP (-4)    /* a HIP call failed; see kda_last_hip_error() */
#define KDA_EWAIT (-5)   /* from kda_chunk_fwd_status: a bounded wait in the state pass expired */
#define KDA_ESCRATCH (-6) /* kda_chunk_fwd_noalloc: the call needs more than KDA_NOALLOC_SCRATCH_BYTES */

/* dtype */
#define KDA_F32 0
#define KDA_BF16 1

/* gate_kind */
#define KDA_GATE_CHANNEL 0 /* gate [.., dk]: one alpha per key channel (KDA, Complex KDA) */
#define KDA_GATE_SCALAR 1  /* gate [..]: one alpha per token and head (GDN) */

/*
 * Bytes of device workspace kda_chunk_fwd needs for these sizes (0 when the
 * arguments are invalid). For packed variable-length input pass the number
 * of sequences N and has_cu_seqlens = 1; the bound then assumes the worst
 * split of T over N sequences.
 */
size_t kda_chunk_fwd_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, int N,
                                     int has_cu_seqlens, int dtype);

/*
 * Chunkwise-parallel forward over whole sequences (the pages' chunkwise WY
 * training form of this family; Complex KDA summary, background and core
 * method; Gated DeltaNet-2 blurb). Produces exactly the token recurrence above
 * up to floating-point rounding.
 *
 * Layouts (fixed-length batch; cu_seqlens == NULL):
 *   q, k   [B, T, H, dk]      v    [B, T, H, dv]
 *   gate   [B, T, H, dk] (KDA_GATE_CHANNEL) or [B, T, H] (KDA_GATE_SCALAR)
 *   beta   [B, T, H]
 *   o      [B, T, H, dv] fp32 (output; must not alias any input)
 *   S0     [B, H, dk, dv] fp32 initial state, or NULL for zeros
 *   S_T    [B, H, dk, dv] fp32 final state, or NULL; may alias S0
 * Packed variable-length input (cu_seqlens != NULL): B must be 1; cu_seqlens
 * is a DEVICE int32 array of N+1 non-decreasing offsets with cu_seqlens[0] = 0
 * and cu_seqlens[N] = T; sequence s covers tokens [cu_seqlens[s],
 * cu_seqlens[s+1]) and starts from S0[s] (or zeros); S0 and S_T are
 * [N, H, dk, dv]. With cu_seqlens == NULL, N must equal B (or be 0).
 *
 * chunk (16, 32 or 64) sets the block size of the parallel form; results
 * agree across chunk sizes up to rounding. T need not be a multiple of it.
 *
 * workspace: device memory of at least kda_chunk_fwd_workspace_bytes(...)
 * bytes, owned by the caller and not read before it is written (required:
 * NULL or too small is KDA_EINVAL). Its first 4 bytes receive the call's
 * status word once the call's kernels have run: 0 when every bounded wait in
 * the state pass completed. The state pass's waves trade operands through LDS
 * with bounded waits that cannot expire while all waves of a workgroup run;
 * if one ever did, that wave stores neither o nor S_T and sets the status
 * word. The caller may read the word after synchronising with `stream` and
 * map it with kda_chunk_fwd_status().
 *
 * Returns KDA_OK or a negative status.
 */
int kda_chunk_fwd(const void* q, const void* k, const void* v, const void* gate, const void* beta,
                  const float* S0, float* o, float* S_T, int B, int H, int T, int dk, int dv, int chunk,
                  const int32_t* cu_seqlens, int N, int dtype, int gate_kind, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * kda_chunk_fwd for callers that cannot allocate device memory (work recorded
 * under graph capture, allocation-free serving loops, harnesses that forbid
 * hipMalloc): the same arguments and results minus the workspace, which here
 * is a fixed device array of KDA_NOALLOC_SCRATCH_BYTES inside the library,
 * one per GPU, held until the process ends. A call whose workspace would
 * exceed it (kda_chunk_fwd_workspace_bytes(...) > KDA_NOALLOC_SCRATCH_BYTES;
 * about 1,770 (chunk, head) blocks at dk = dv = 128, chunk 64, e.g. H = 16
 * and T = 7,000) returns KDA_ESCRATCH before any HIP call. The call allocates
 * nothing; the first call with a device current looks up the array's address
 * on that device. All calls on one GPU share the array, which keeps the last
 * call's contents (its status word included): calls that overlap on one GPU
 * (concurrent streams, or host threads) race and must be ordered by the
 * caller.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (128u << 20)
int kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* gate, const void* beta,
                          const float* S0, float* o, float* S_T, int B, int H, int T, int dk, int dv, int chunk,
                          const int32_t* cu_seqlens, int N, int dtype, int gate_kind, void* stream);

/*
 * Maps the status word a forward left in the first 4 bytes of its workspace
 * (read by the caller after the call completed) to KDA_OK (0) or KDA_EWAIT.
 * Host-only; touches no device.
 */
int kda_chunk_fwd_status(uint32_t status_word);

/* stage for kda_chunk_fwd_stage */
#define KDA_STAGE_PREP 1  /* in-chunk work: gate products, gated Gram, UT inverse -> workspace */
#define KDA_STAGE_STATE 2 /* sequential state pass over the chunks: reads the workspace, writes o, S_T */
#define KDA_STAGE_ALL 3   /* both, in order (what kda_chunk_fwd does) */

/*
 * kda_chunk_fwd split into its two launches, for callers that schedule or
 * time them separately. Arguments as for kda_chunk_fwd. KDA_STAGE_STATE
 * consumes a workspace that a KDA_STAGE_PREP call with identical arguments
 * filled earlier on the same stream (or with ordering the caller provides).
 * KDA_STAGE_PREP writes neither o nor S_T and clears the status word;
 * KDA_STAGE_STATE only ever sets it.
 */
int kda_chunk_fwd_stage(int stage, const void* q, const void* k, const void* v, const void* gate,
                        const void* beta, const float* S0, float* o, float* S_T, int B, int H, int T, int dk,
                        int dv, int chunk, const int32_t* cu_seqlens, int N, int dtype, int gate_kind,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * One recurrent decode step for N sequences, state updated in place (the
 * pages' recurrent inference form with constant memory per sequence; Gated
 * DeltaNet-2 blurb; Complex KDA summary, background):
 *   S' = Diag(alpha) S;  u = beta (v - S'^T k);  S <- S' + k u^T;  o = S^T q.
 *
 * Layouts: q, k [N, H, dk]; v [N, H, dv]; gate [N, H, dk] or [N, H];
 * beta [N, H]; S [N, H, dk, dv] fp32 (read and written in place);
 * o [N, H, dv] fp32 (must not alias S or the inputs).
 * The state layout equals kda_chunk_fwd's S_T, so a forward's final state
 * feeds decode directly.
 *
 * Returns KDA_OK or a negative status.
 */
int kda_decode_step(const void* q, const void* k, const void* v, const void* gate, const void* beta,
                    float* S, float* o, int N, int H, int dk, int dv, int dtype, int gate_kind,
                    void* stream);

/*
 * Decoupled erase and write gates (Gated DeltaNet-2 blurb: the delta rule's
 * memory update split into a channel-wise erase gate and a channel-wise
 * write gate; the pages name combining them with Complex KDA's gates as
 * future work, Complex KDA summary). The pages give no formula; the form
 * implemented keeps the update rank one along k and gives beta's two roles to
 * two gates:
 *   S_t = (I - k_t (e_t o k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t o v_t)^T
 *   o_t = S_t^T q_t
 * with the erase gate e_t in R^{dk} (per key channel) and the write gate w_t
 * in R^{dv} (per value channel); e_t = w_t = beta_t (every channel) gives the
 * recurrence at the top of this header. Any alpha the forward takes is
 * allowed (channel or scalar gate, signs and zeros included).
 *
 * kda_chunk_fwd_ew: the chunkwise forward of that form. Arguments as for
 * kda_chunk_fwd, with beta replaced by
 *   erase [B, T, H, dk] and write [B, T, H, dv] in the input dtype,
 * both 16-byte aligned; the workspace is kda_chunk_fwd_workspace_bytes(...)
 * bytes (same status word). kda_decode_step_ew: one decode step of it, as
 * kda_decode_step with erase [N, H, dk] and write [N, H, dv].
 * Returns KDA_OK or a negative status.
 */
int kda_chunk_fwd_ew(const void* q, const void* k, const void* v, const void* gate, const void* erase,
                     const void* write, const float* S0, float* o, float* S_T, int B, int H, int T, int dk, int dv,
                     int chunk, const int32_t* cu_seqlens, int N, int dtype, int gate_kind, void* workspace,
                     size_t workspace_bytes, void* stream);
int kda_decode_step_ew(const void* q, const void* k, const void* v, const void* gate, const void* erase,
                       const void* write, float* S, float* o, int N, int H, int dk, int dv, int dtype, int gate_kind,
                       void* stream);

/*
 * Bytes of device workspace kda_chunk_bwd needs for these sizes (0 when the
 * arguments are invalid). Arguments as for kda_chunk_fwd_workspace_bytes.
 */
size_t kda_chunk_bwd_workspace_bytes(int B, int H, int T, int dk, int dv, int N, int has_cu_seqlens);

/*
 * Gradient of kda_chunk_fwd. The pages measure forward-plus-backward
 * training throughput of this family (Complex KDA summary, efficiency) but
 * print no backward; this is the reverse-mode derivative of the token
 * recurrence in the header comment, for the loss
 *   L = sum_t <o_t, dO_t> + sum_seq <S_T, dS_T>,
 * computed in fp32 from the same inputs (the forward states are recomputed
 * from q, k, v, gate, beta and S0; nothing from a forward call is reused).
 *
 * Inputs: q, k, v, gate, beta, S0, cu_seqlens, N, dtype and gate_kind as for
 * kda_chunk_fwd; dO [B, T, H, dv] fp32 (required when T > 0); dS_T
 * [N, H, dk, dv] fp32 or NULL (zero).
 * Outputs (fp32, written in full, must not alias inputs or each other):
 *   grad_q, grad_k [B, T, H, dk]   grad_v [B, T, H, dv]
 *   grad_gate      [B, T, H, dk] (KDA_GATE_CHANNEL) or [B, T, H] (KDA_GATE_SCALAR)
 *   grad_beta      [B, T, H]
 *   grad_S0        [N, H, dk, dv], or NULL when not wanted
 * dO, grad_v, S0, dS_T and grad_S0 must be 16-byte aligned.
 *
 * workspace: at least kda_chunk_bwd_workspace_bytes(...) bytes (state
 * checkpoints every 8 tokens, 4 * dk * dv bytes each per (sequence, head),
 * the per-token residual v - S'^T k, plus per-workgroup partial sums);
 * required (NULL is KDA_EINVAL).
 *
 * Returns KDA_OK or a negative status.
 */
int kda_chunk_bwd(const void* q, const void* k, const void* v, const void* gate, const void* beta,
                  const float* S0, const float* dO, const float* dS_T, float* grad_q, float* grad_k,
                  float* grad_v, float* grad_gate, float* grad_beta, float* grad_S0, int B, int H, int T,
                  int dk, int dv, const int32_t* cu_seqlens, int N, int dtype, int gate_kind,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Gradient of kda_chunk_fwd_ew (decoupled erase and write gates; Gated
 * DeltaNet-2 blurb, and the reading stated at kda_chunk_fwd_ew), by the same
 * token-recurrence method as kda_chunk_bwd: with the read key ke = e o k and
 * u = w o v - S'^T ke, the adjoint of each token reads the state with ke,
 * writes along k, and has no beta. Loss, inputs, dO, dS_T, grad_q, grad_k,
 * grad_v, grad_gate and grad_S0 as for kda_chunk_bwd (erase and write as for
 * kda_chunk_fwd_ew, same dtype as q). Outputs in place of grad_beta (fp32,
 * written in full): grad_erase [B, T, H, dk] and grad_write [B, T, H, dv]
 * (16-byte aligned). workspace: kda_chunk_bwd_ew_workspace_bytes(...) bytes
 * (as for kda_chunk_bwd, with one more partial sum per key channel instead of
 * the partial sums of dbeta); required. Every dk and dv of kda_chunk_fwd.
 * Returns KDA_OK or a negative status.
 */
size_t kda_chunk_bwd_ew_workspace_bytes(int B, int H, int T, int dk, int dv, int N, int has_cu_seqlens);
int kda_chunk_bwd_ew(const void* q, const void* k, const void* v, const void* gate, const void* erase,
                     const void* write, const float* S0, const float* dO, const float* dS_T, float* grad_q,
                     float* grad_k, float* grad_v, float* grad_gate, float* grad_erase, float* grad_write,
                     float* grad_S0, int B, int H, int T, int dk, int dv, const int32_t* cu_seqlens, int N, int dtype,
                     int gate_kind, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same gradient as kda_chunk_bwd (same arguments, outputs and layouts),
 * computed chunk by chunk (the pages' chunkwise algorithm with gate-aware
 * backpropagation for this family; Gated DeltaNet-2 blurb): per 64-token
 * chunk the gated Gram matrices, the UT inverse X = (I + Diag(beta) G)^{-1} and
 * W = X (beta o Gamma o K) in fp32; the state at every chunk start by a
 * forward walk over the chunks and the adjoint at every chunk end by a
 * reverse walk; then every chunk's gradients in parallel, all contractions on
 * fp32 MFMA. The gate gradient uses products of gates only, so exact zero and
 * negative gates have their ordinary derivatives. Supported: dk 64 or 128
 * (KDA_ENOTSUP otherwise), dv in {16, 32, 64, 128}, both dtypes and gate kinds,
 * packed sequences. dO and the workspace must be 16-byte aligned (dO rows are
 * read four values at a time); element alignment suffices for every other
 * pointer. workspace: kda_chunk_bwd_cw_workspace_bytes(...) bytes (per
 * (chunk, head) the chunk's fp32 matrices, the state and adjoint at its
 * boundaries, the chunk's U and dU, and the gradient intermediates);
 * required.
 */
size_t kda_chunk_bwd_cw_workspace_bytes(int B, int H, int T, int dk, int dv, int N, int has_cu_seqlens);
int kda_chunk_bwd_cw(const void* q, const void* k, const void* v, const void* gate, const void* beta,
                     const float* S0, const float* dO, const float* dS_T, float* grad_q, float* grad_k,
                     float* grad_v, float* grad_gate, float* grad_beta, float* grad_S0, int B, int H, int T,
                     int dk, int dv, const int32_t* cu_seqlens, int N, int dtype, int gate_kind,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Gauge transform of Complex KDA onto positive gates (Complex KDA summary,
 * method step 5: the cumulative gate signs are absorbed into queries and
 * keys). Per sequence, head and key channel (per sequence and head for the
 * scalar gate), with s_t = -1 where gate_t < 0 and +1 otherwise (zero and
 * -0.0 included) and c_t = s_1 ... s_t:
 *   q_out_t = c_t q_t,  k_out_t = c_t k_t,  gate_out_t = |gate_t|
 * Running the recurrence on the outputs gives the same o as on the inputs,
 * and a final state whose rows differ by c_T: S_T = Diag(c_T) S~_T.
 * Every output value is an input value with its sign changed or cleared
 * (bit-exact in both dtypes). Layouts, N, cu_seqlens, dtype and gate_kind as
 * for kda_chunk_fwd; outputs have the input layouts and dtype and must not
 * alias the inputs. q, k, their outputs and (channel gate) gate and gate_out
 * must be 16-byte aligned. sign_T: device int8 [N, H, dk] (channel gate) or [N, H]
 * (scalar gate) receiving c_T (+1 / -1), or NULL. workspace: at least
 * kda_gauge_fold_workspace_bytes(...) bytes (required).
 * Returns KDA_OK or a negative status.
 */
size_t kda_gauge_fold_workspace_bytes(int B, int H, int T, int dk, int N, int has_cu_seqlens, int gate_kind);
int kda_gauge_fold(const void* q, const void* k, const void* gate, void* q_out, void* k_out, void* gate_out,
                   int8_t* sign_T, int B, int H, int T, int dk, const int32_t* cu_seqlens, int N, int dtype,
                   int gate_kind, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_fwd computed through the gauge transform: kda_gauge_fold into
 * the workspace, the chunkwise forward on the folded (positive-gate)
 * inputs, then S_T's rows multiplied by c_T. Same arguments, results and
 * tolerances as kda_chunk_fwd; the workspace (required) is
 * kda_chunk_fwd_gauge_workspace_bytes(...) bytes: the forward's own
 * workspace first (so its status word is again the first 4 bytes), then the
 * folded q, k and gate and the fold's scratch.
 */
size_t kda_chunk_fwd_gauge_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, int N,
                                           int has_cu_seqlens, int dtype, int gate_kind);
int kda_chunk_fwd_gauge(const void* q, const void* k, const void* v, const void* gate, const void* beta,
                        const float* S0, float* o, float* S_T, int B, int H, int T, int dk, int dv, int chunk,
                        const int32_t* cu_seqlens, int N, int dtype, int gate_kind, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Static text for a status code (never NULL). */
const char* kda_strerror(int status);

/* hipError_t of the most recent KDA_EHIP on the calling thread (0 if none). */
int kda_last_hip_error(void);

/* Library version, e.g. 100 for 0.1.0. */
int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
