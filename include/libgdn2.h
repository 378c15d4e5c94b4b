/*
 * libgdn2 — Gated DeltaNet-2 core recurrence on AMD Instinct MI355X (gfx950).
 *
 * The operation (per sequence and head; state S is Dk x Dv, rows = key channels):
 *
 *   S_t = (I - k_t (b_t * k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t * v_t)^T
 *   o_t = S_t^T q_t
 *
 * with alpha_t = exp(log_alpha_t) a per-key-channel decay, b_t an erase gate on
 * the key axis and w_t a write gate on the value axis.  Sources: the state
 * update equation of the gist.science summary of arXiv 2605.22791 (technical
 * summary, part "1. Gated Delta Rule-2") and of the zubnet.ai news item (first
 * paragraph); the order decay -> read with b*k -> write, and the query reading
 * the UPDATED state, from the iplexlaw blog digest (section "Decisiones
 * independientes en dos ejes").  No query scale is applied.
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE pointers, allocated and owned by the
 *     caller.  Intermediates live in a caller-supplied device workspace;
 *     the only allocation the library makes is the hipBLASLt handle the
 *     layer calls create on their first call on a device (see below).
 *   - Layouts are dense, row-major, last dimension fastest.  Every tensor
 *     pointer must be 16-byte aligned.
 *   - `io` selects the element type of q, k, v and o (GDN2_BF16 or GDN2_F32).
 *     log_alpha, b, w and all states are always float32.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls enqueue work
 *     and return; results are valid once the stream has been synchronised.
 *     With the environment variable GDN2_DEBUG_SYNC=1 each call synchronises
 *     its stream and reports asynchronous failures as GDN2_ERR_HIP.
 *   - Errors are reported only through the returned status.  Arguments are
 *     validated on the host before anything is launched; on a non-OK status
 *     nothing has been enqueued (except GDN2_ERR_HIP, which reports a failed
 *     launch).  Device faults surface at the caller's next synchronisation.
 *   - Supported head sizes: Dk == Dv, either 64 or 128
 *     (others return GDN2_ERR_UNSUPPORTED).
 *   - Calls keep no state between invocations and are reentrant; two calls
 *     may run concurrently on different streams if they share no outputs or
 *     workspace.  Results are bitwise reproducible for identical inputs.
 */
#ifndef LIBGDN2_H
#define LIBGDN2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn2_status {
    GDN2_OK = 0,
    GDN2_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad size or dtype */
    GDN2_ERR_UNSUPPORTED = 2,      /* valid request the library does not implement */
    GDN2_ERR_WORKSPACE = 3,        /* workspace missing or smaller than required */
    GDN2_ERR_HIP = 4               /* a HIP launch or runtime call failed */
} gdn2_status;

typedef enum gdn2_dtype {
    GDN2_F32 = 0,
    GDN2_BF16 = 1
} gdn2_dtype;

/* Version of this interface; bumped on any incompatible change (2: the
 * workspace layout reports the size with the optional T slot separately). */
int gdn2_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char *gdn2_status_string(int status);

/*
 * The device's compute-unit count and peak engine clock (kHz), as the HIP
 * runtime reports them, for stating peak rates from the part's own figures
 * (a gfx950 CU retires 4096 dense bf16 MFMA flops and 256 fp32 vector flops
 * per clock).  Outputs may be NULL.  Returns GDN2_ERR_HIP when the runtime
 * query fails (no such device), GDN2_OK otherwise.
 */
int gdn2_device_info(int device, int *compute_units, int *peak_clock_khz);

/*
 * Workspace bytes gdn2_chunk_fwd needs for a call with these sizes.
 * varlen != 0 sizes it for a packed call with N sequences and T total tokens
 * (B must then be 1).  Returns 0 for unsupported or invalid sizes.
 */
size_t gdn2_chunk_fwd_workspace_bytes(int N, int B, int T, int H, int Dk, int Dv,
                                      int io, int varlen);

/*
 * Chunk-parallel forward over whole sequences.
 *
 * The sequence is processed in 64-token chunks (the WY chunk form of the
 * iplexlaw digest, section "Procesamiento del token y entrenamiento
 * paralelo", and of the gist.science summary, part "3. Efficient chunkwise
 * parallel training"): per chunk the cumulative log-decay is taken in fp32,
 * the strictly lower-triangular interaction matrix A of the decayed,
 * erase-modulated keys against the keys is formed and T = (I + A)^-1 is
 * solved in fp32, the chunk's auxiliaries (W = T (gamma*b*k), the causal
 * query-key matrix, the decayed queries and keys) are formed with bf16 (or
 * fp32 for io = GDN2_F32) MFMA contractions, and one sequential pass per
 * (sequence, head) carries the fp32 state across chunks and writes o.
 *
 * Dense call (cu_seqlens == NULL): N must equal B; each of the B rows is one
 * sequence of T tokens.
 *   q, k       [B, T, H, Dk]  io dtype        log_alpha, b [B, T, H, Dk] f32
 *   v          [B, T, H, Dv]  io dtype        w            [B, T, H, Dv] f32
 *   o          [B, T, H, Dv]  io dtype (output)
 *   S0         [N, H, Dk, Dv] f32, or NULL for a zero initial state
 *   S_final    [N, H, Dk, Dv] f32 (output), or NULL to skip it; may alias S0.
 * Packed variable-length call (cu_seqlens != NULL): B must be 1 and T is the
 * total token count; cu_seqlens is a DEVICE int32 array of N+1 offsets with
 * cu_seqlens[0] == 0, non-decreasing, cu_seqlens[N] == T.  Sequence n owns
 * tokens [cu_seqlens[n], cu_seqlens[n+1]), starts from S0[n] (or zero), is
 * chunked from its own first token (its last chunk may be shorter than 64)
 * and writes S_final[n].  Offsets are clamped into [0, T] on the device, so
 * malformed offsets give undefined values but no out-of-bounds access.
 *
 * The workspace (device memory, >= gdn2_chunk_fwd_workspace_bytes(...) bytes,
 * 256-byte aligned) holds the per-chunk intermediates; its layout is
 * described by gdn2_chunk_fwd_workspace_layout.  T == 0 or N == 0 is allowed:
 * then S_final = S0 (or zero) and o is untouched; with T == 0 the token
 * pointers (q ... w, o) may be NULL.
 *
 * Precondition on the decay: within one 64-token chunk, the decay of any key
 * channel must stay below about 170 nats (half of it must be representable
 * as an fp32 exponent).  Larger decays overflow the scaled factors.
 */
int gdn2_chunk_fwd(const void *q, const void *k, const void *v,
                   const float *log_alpha, const float *b, const float *w,
                   const float *S0, void *o, float *S_final,
                   const int32_t *cu_seqlens, int N,
                   int B, int T, int H, int Dk, int Dv, int io,
                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn2_chunk_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops and harnesses that forbid allocation): the
 * same computation, arguments and results, but the per-chunk intermediates
 * live in a fixed region of device memory that the library holds itself, one
 * per GPU, from the first call on that GPU until the process ends (128 MiB,
 * 134217728 bytes).  No allocator is called and no workspace is passed.
 *   - A call needing more than that (gdn2_chunk_fwd_workspace_bytes(...) >
 *     134217728; about 1800 chunk-heads at Dk = Dv = 128 in bf16, e.g.
 *     B = 1, H = 16, T = 7168) returns GDN2_ERR_WORKSPACE before anything is
 *     enqueued; gdn2_chunk_fwd with a caller's workspace has no such limit.
 *   - Every call on one GPU shares that GPU's region and leaves its own
 *     intermediates in it: calls that overlap on one GPU (on different
 *     streams, or from several host threads) race and give undefined
 *     results.  Calls enqueued on one stream are ordered and safe.
 *   - GDN2_ERR_HIP if the region's device address cannot be obtained.
 */
int gdn2_chunk_fwd_noalloc(const void *q, const void *k, const void *v,
                           const float *log_alpha, const float *b, const float *w,
                           const float *S0, void *o, float *S_final,
                           const int32_t *cu_seqlens, int N,
                           int B, int T, int H, int Dk, int Dv, int io, void *stream);

/*
 * The stages of gdn2_chunk_fwd, for profiling each kernel on its own and for
 * inspecting the intermediates.  gdn2_chunk_fwd == gdn2_chunk_fwd_stages(...,
 * GDN2_STAGE_ALL).  A later call with the same arguments and workspace may run
 * the remaining stages: the workspace carries the chunk table and the chunk
 * factors between calls.  Running a stage whose inputs were never produced in
 * this workspace gives undefined values (but no out-of-bounds access).
 */
#define GDN2_STAGE_PLAN 1       /* packed calls: build the chunk table on the device */
#define GDN2_STAGE_FACTORS 2    /* per chunk: cumulative decay, A, T = (I+A)^-1, W, U, M, Qhat, Khat */
#define GDN2_STAGE_PROPAGATE 4  /* sequential state propagation: U_eff, o, S_final */
#define GDN2_STAGE_ALL 7
#define GDN2_STAGE_STORE_T 8    /* with FACTORS: also store T in the workspace (inspection only);
                                   the workspace must then hold total_bytes_with_Tinv bytes
                                   (gdn2_chunk_fwd_workspace_layout) */

int gdn2_chunk_fwd_stages(const void *q, const void *k, const void *v,
                          const float *log_alpha, const float *b, const float *w,
                          const float *S0, void *o, float *S_final,
                          const int32_t *cu_seqlens, int N,
                          int B, int T, int H, int Dk, int Dv, int io,
                          void *workspace, size_t workspace_bytes, void *stream, int stages);

/*
 * gdn2_chunk_fwd with bf16 gate inputs.  The gates are the sigmoids of learned
 * projections (iplexlaw digest, section "Decisiones independientes en dos
 * ejes": b and w in (0, 1) per channel), so a layer can hand over the logits
 * and let the chunk kernel take the sigmoid, halving the gate bytes:
 *   log_alpha  [B, T, H, Dk] bf16, log alpha itself (<= 0)
 *   b_logit    [B, T, H, Dk] bf16, b = 1 / (1 + exp(-b_logit))
 *   w_logit    [B, T, H, Dv] bf16, w = 1 / (1 + exp(-w_logit))
 * The sigmoids are taken in fp32.  Everything else (shapes, S0, o, S_final,
 * cu_seqlens, workspace and its size, the decay precondition) is as for
 * gdn2_chunk_fwd.  Only io = GDN2_BF16 is implemented (GDN2_F32 returns
 * GDN2_ERR_UNSUPPORTED).
 */
int gdn2_chunk_fwd_gate_logits(const void *q, const void *k, const void *v,
                               const void *log_alpha, const void *b_logit, const void *w_logit,
                               const float *S0, void *o, float *S_final,
                               const int32_t *cu_seqlens, int N,
                               int B, int T, int H, int Dk, int Dv, int io,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * Where gdn2_chunk_fwd keeps its per-chunk intermediates inside the
 * workspace, for inspection by tests.  total_bytes is what
 * gdn2_chunk_fwd_workspace_bytes returns; total_bytes_with_Tinv also covers
 * the Tinv slot, which lies after every other slot and is used only by
 * calls whose stages include GDN2_STAGE_STORE_T.  Offsets are in bytes from the
 * workspace start; every array is indexed by (chunk id c, head h) as
 * [c][h][...], with chunk ids numbered sequence by sequence (dense: chunk c
 * of row n has id n * ceil(T/64) + c).  Element type is the io dtype unless
 * stated.  For a chunk shorter than 64 tokens, the rows past its length are
 * zero in W, U, M and Qhat, the matching columns of M and KhatT are zero, and
 * T is the identity on those rows and columns.
 *   Tinv   [64][64]  (I + A)^-1, row-major; written only when the stages
 *                    include GDN2_STAGE_STORE_T
 *   W      [64][Dk]  T (gamma * b * k)                  } in fragment order,
 *   Qhat   [64][Dk]  gamma * q                          } see below
 *   KhatT  [Dk][64]  (exp(g_last - g) * k)^T            }
 *   M      [64][64]  lower incl. diagonal, M_ij = sum_c q_i k_j exp(g_i - g_j);
 *                    its fragments wholly above the diagonal (16-row block rb,
 *                    KS-column block kb with kb*KS > 16*rb + 15; for bf16 the
 *                    columns 32..63 of rows 0..31) are not written
 *          Fragment order of an R x K matrix X: X[r][k] is element
 *            ((r/16)*(K/KS) + k/KS)*64*KPL + ((r%16) + 16*((k%KS)/KPL))*KPL + k%KPL
 *          with (KS, KPL) = (32, 8) for bf16 and (4, 1) for f32.
 *   U      [4][Dv/16][64][4]  T (w * v) in MFMA accumulator order: element
 *                    [I][cb][l][r] is U[16 I + 4 (l / 16) + r][16 cb + l % 16]
 *   gamma_last [Dk]  f32, exp(g_last)
 *   plan   int32: for packed calls, [0..N] first chunk id of each sequence
 *          followed by 3 ints (sequence, first token, length) per chunk.
 * Returns GDN2_OK and fills the fields, or an error status.
 */
typedef struct gdn2_workspace_layout {
    size_t total_bytes;
    int max_chunks;          /* chunk-id capacity */
    size_t off_Tinv, off_W, off_Qhat, off_KhatT, off_M, off_U, off_gamma_last, off_plan;
    size_t total_bytes_with_Tinv;
} gdn2_workspace_layout;

int gdn2_chunk_fwd_workspace_layout(int N, int B, int T, int H, int Dk, int Dv,
                                    int io, int varlen, gdn2_workspace_layout *out);

/*
 * Workspace bytes gdn2_chunk_bwd needs for a call with these sizes (same
 * meaning of the arguments as gdn2_chunk_fwd_workspace_bytes).  Returns 0 for
 * unsupported or invalid sizes.
 */
size_t gdn2_chunk_bwd_workspace_bytes(int N, int B, int T, int H, int Dk, int Dv,
                                      int io, int varlen);

/*
 * Gradients of gdn2_chunk_fwd: the gate-aware chunkwise backward (the
 * gist.science summary, part "3. Efficient chunkwise parallel training", item
 * on the backward pass: the channel-wise gates b and w enter the gradients of
 * the chunk's auxiliary matrices; the iplexlaw digest, section "El artículo y
 * su pregunta").  Given the upstream gradients dout = dL/do and dS_final =
 * dL/dS_final, it returns dL/d of every input: the exact chain rule of the
 * recurrence above, taken through the same 64-token chunk form as the forward
 * (the forward is recomputed inside the call; nothing from an earlier
 * gdn2_chunk_fwd is needed).
 *
 * Same sizes, layouts, dense/packed conventions and decay precondition as
 * gdn2_chunk_fwd.  Inputs:
 *   q, k, v, log_alpha, b, w, S0    as for gdn2_chunk_fwd (S0 may be NULL)
 *   dout      [B, T, H, Dv]  io dtype
 *   dS_final  [N, H, Dk, Dv] f32, or NULL for zero
 * Outputs (all written in full; every gradient of a token of the call):
 *   dq, dk    [B, T, H, Dk]  io dtype       dlog_alpha, db [B, T, H, Dk] f32
 *   dv        [B, T, H, Dv]  io dtype       dw             [B, T, H, Dv] f32
 *   dS0       [N, H, Dk, Dv] f32, or NULL to skip it
 * Outputs must not alias each other or any input.  The workspace (>=
 * gdn2_chunk_bwd_workspace_bytes(...) bytes, 256-byte aligned) holds the
 * chunk factors, every chunk's incoming state and state gradient, and the
 * per-chunk partial gradients.  io = GDN2_BF16 runs the fast bf16-MFMA
 * kernels (bf16 factors and intermediates, fp32 accumulation; about 145 KiB
 * of workspace per chunk-head at Dk = 128); io = GDN2_F32
 * computes every product and intermediate in fp32 (fp32 MFMA), the precision
 * reference of the same chain rule, with a larger workspace (about 1 MiB per
 * chunk-head at Dk = 128).
 */
int gdn2_chunk_bwd(const void *q, const void *k, const void *v,
                   const float *log_alpha, const float *b, const float *w,
                   const float *S0, const void *dout, const float *dS_final,
                   void *dq, void *dk, void *dv,
                   float *dlog_alpha, float *db, float *dw, float *dS0,
                   const int32_t *cu_seqlens, int N,
                   int B, int T, int H, int Dk, int Dv, int io,
                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * A training step's forward and backward without recomputing the forward in
 * the backward (the same chain rule as gdn2_chunk_bwd, same citations): the
 * forward keeps, in a workspace the caller holds until the backward, what
 * gdn2_chunk_bwd would otherwise rebuild first -- the chunk table, the chunk
 * factors with their transposes and every chunk's incoming state.  This
 * trades HBM (about 184.5 KiB per chunk-head at Dk = 128, 1.55 GB for
 * B = 8, H = 16, T = 4096) for the recomputation.  bf16 I/O only
 * (io = GDN2_F32 returns GDN2_ERR_UNSUPPORTED; gdn2_*_workspace_bytes
 * returns 0 for it).
 *
 * gdn2_chunk_train_workspace_bytes: bytes of that workspace for a call with
 * these sizes (arguments as for gdn2_chunk_fwd_workspace_bytes).
 *
 * gdn2_chunk_fwd_train: gdn2_chunk_fwd (same arguments, outputs and results,
 * bitwise) on such a workspace (>= gdn2_chunk_train_workspace_bytes(...)
 * bytes, 256-byte aligned), which it also fills for the backward.
 *
 * gdn2_chunk_bwd_saved: gdn2_chunk_bwd's gradients (bitwise the same) from a
 * workspace a gdn2_chunk_fwd_train call filled, with the same q, k, v,
 * log_alpha, b, w, cu_seqlens and sizes (S0 entered through the saved
 * states, so it is not passed; the library cannot check that the inputs
 * match, and gradients of other inputs are meaningless).  Its other
 * arguments are those of gdn2_chunk_bwd.  It writes only the backward's own
 * slots of the workspace, so the saved data stay valid: several backward
 * calls may follow one forward.
 */
size_t gdn2_chunk_train_workspace_bytes(int N, int B, int T, int H, int Dk, int Dv,
                                        int io, int varlen);

int gdn2_chunk_fwd_train(const void *q, const void *k, const void *v,
                         const float *log_alpha, const float *b, const float *w,
                         const float *S0, void *o, float *S_final,
                         const int32_t *cu_seqlens, int N, int B, int T, int H,
                         int Dk, int Dv, int io, void *workspace,
                         size_t workspace_bytes, void *stream);

int gdn2_chunk_bwd_saved(const void *q, const void *k, const void *v,
                         const float *log_alpha, const float *b, const float *w,
                         const void *dout, const float *dS_final,
                         void *dq, void *dk, void *dv,
                         float *dlog_alpha, float *db, float *dw, float *dS0,
                         const int32_t *cu_seqlens, int N,
                         int B, int T, int H, int Dk, int Dv, int io,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * One recurrent decode token for B independent sequences (constant-memory
 * decoding: the gist.science summary, "Problem statement").  The state is
 * read once and written once, in place:
 *   r = sum_c alpha_c b_c k_c S[c,:],  p = sum_c alpha_c q_c S[c,:]
 *   o = p + (q . k) (w*v - r),         S[c,:] <- alpha_c S[c,:] + k_c (w*v - r)
 * which equals the update above followed by o = S_t^T q_t.
 *   q, k   [B, H, Dk] io dtype      log_alpha, b [B, H, Dk] f32
 *   v      [B, H, Dv] io dtype      w            [B, H, Dv] f32
 *   S      [B, H, Dk, Dv] f32, updated in place
 *   o      [B, H, Dv] io dtype (output); must not alias S or any input.
 */
int gdn2_step(const void *q, const void *k, const void *v,
              const float *log_alpha, const float *b, const float *w,
              float *S, void *o, int B, int H, int Dk, int Dv, int io,
              void *stream);

/*
 * Token-mixer layer forward around the core (the iplexlaw digest, section
 * "Procesamiento del token y entrenamiento paralelo"; gates as in section
 * "Decisiones independientes en dos ejes"), for x [B, T, D] bf16:
 *   P = x W_in^T split into the blocks q | k | v | alpha | gate | b | w
 *   q, k, v = SiLU(causal depthwise conv_L(P_q, P_k, P_v))
 *   q, k   /= sqrt(|.|^2 + 1e-6) per head (L2 normalisation over Dk)
 *   log alpha = logsigmoid(P_alpha + alpha_bias), b = sigmoid(P_b), w = sigmoid(P_w)
 *   o, S_final = the core recurrence (gdn2_chunk_fwd_gate_logits)
 *   z = o / sqrt(mean_c(o^2) + norm_eps) * norm_w * sigmoid(P_gate)   per head over Dv
 *   y = z W_o^T
 * The convolution reads conv_w[c][j] * x_{t-L+1+j} for taps j < L, with
 * zeros before the first token of each sequence.  Readings where the page is
 * silent: no projection biases; the decay is a logsigmoid gate with a
 * per-channel bias; one RMS weight vector [Dv] shared by the heads; the
 * output gate is a sigmoid.
 *
 * Weights (device pointers, row-major, caller-owned, 16-byte aligned):
 *   W_in        bf16 [7 * H * Dk, D]  (blocks of H*Dk rows in the order above)
 *   conv_w      f32  [3 * H * Dk, conv_len]  (q, k, v channels; tap j = 0 oldest)
 *   alpha_bias  f32  [H * Dk]
 *   norm_w      f32  [Dv]
 *   W_o         bf16 [D, H * Dv]
 * Activations: x, y bf16 [B, T, D] (y must not alias x or any weight); S0,
 * S_final, cu_seqlens, N, B, T as for gdn2_chunk_fwd.  Requirements: Dk == Dv
 * in {64, 128}; D > 0 and a multiple of 8; 1 <= conv_len <= 8; norm_eps >= 0.
 *
 * The projections are bf16 GEMMs with fp32 accumulation run by hipBLASLt; the
 * first call on a device creates that device's hipBLASLt handle and caches
 * the chosen GEMM algorithm per shape (both kept until the process ends).
 * All intermediates live in the caller's workspace (at least
 * gdn2_layer_fwd_workspace_bytes, 0 on invalid sizes; varlen != 0 for packed
 * calls).  Only bf16 is implemented.
 */
typedef struct gdn2_layer_weights {
    const void *W_in;
    const float *conv_w;
    const float *alpha_bias;
    const float *norm_w;
    const void *W_o;
} gdn2_layer_weights;

size_t gdn2_layer_fwd_workspace_bytes(int N, int B, int T, int H, int Dk, int Dv, int D,
                                      int varlen);

int gdn2_layer_fwd(const void *x, const gdn2_layer_weights *weights, int conv_len,
                   float norm_eps, const float *S0, void *y, float *S_final,
                   const int32_t *cu_seqlens, int N, int B, int T, int H, int Dk, int Dv,
                   int D, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Sliding-window softmax attention, forward: the hybrid model's local
 * attention layer core (iplexlaw digest, section "Condiciones de
 * comparación": a 2K sliding window; gist.science summary, part
 * "4. Architecture": SWA interleaved with the mixer).  Per sequence and head,
 * query i attends to the keys j of the same sequence with i - window < j <= i:
 *   o_i = sum_j softmax_j(scale * q_i . k_j) v_j,
 *   lse_i = log sum_j exp(scale * q_i . k_j)      (natural log)
 * One key/value head per query head; no positional encoding is applied here.
 *   q, k, v, o  [B, T, H, D] bf16 (o must not alias an input)
 *   lse         [B, H, T] f32, or NULL (not written)
 *   cu_seqlens / N / B / T as for gdn2_chunk_fwd (packed: B == 1, T = total tokens)
 *   window >= 1 (the 1.3B hybrid uses 2048), scale > 0 (1/sqrt(D) is usual)
 *   D = 64 or 128.  Packed calls need a workspace of
 *   gdn2_swa_fwd_workspace_bytes(N, 1) bytes (256-byte aligned); dense calls
 *   need none (workspace may be NULL).
 * bf16 inputs, fp32 scores, softmax statistics and accumulation (the
 * probabilities enter the second product as bf16).
 */
size_t gdn2_swa_fwd_workspace_bytes(int N, int varlen);

int gdn2_swa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                 const int32_t *cu_seqlens, int N, int B, int T, int H, int D, int window,
                 float scale, void *workspace, size_t workspace_bytes, void *stream);

/*
 * The hybrid model's sliding-window attention layer around gdn2_swa_fwd:
 *   [q | k | v] = x W_qkv^T,  o = gdn2_swa_fwd(q, k, v),  y = o W_o^T
 * with no biases, positional encoding, normalisation or gate (the pages name
 * only the 2K window; iplexlaw digest, "Condiciones de comparación").
 *   x, y     [B, T, Dm] bf16 (y must not alias x or a weight)
 *   W_qkv    [3 * H * D, Dm] bf16, row blocks q | k | v
 *   W_o      [Dm, H * D] bf16
 *   lse      [B, H, T] f32 or NULL; cu_seqlens, N, B, T, window, scale and D
 *            as for gdn2_swa_fwd; Dm > 0 and a multiple of 8.
 * The projections are hipBLASLt bf16 GEMMs (fp32 accumulation), as in
 * gdn2_layer_fwd (same handle and algorithm cache).  Intermediates live in the
 * caller's workspace (gdn2_swa_layer_fwd_workspace_bytes).
 */
size_t gdn2_swa_layer_fwd_workspace_bytes(int N, int B, int T, int H, int D, int Dm, int varlen);

int gdn2_swa_layer_fwd(const void *x, const void *W_qkv, const void *W_o, void *y, float *lse,
                       const int32_t *cu_seqlens, int N, int B, int T, int H, int D, int Dm,
                       int window, float scale, void *workspace, size_t workspace_bytes,
                       void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBGDN2_H */
