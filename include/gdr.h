/*
 * gdr.h -- C ABI of libgdr, the MI355X (gfx950) gated delta-rule forward pass.
 *
 * The operation (one independent recurrence per sequence and head), with the
 * state S a d_k x d_v fp32 matrix (row i = key channel i, d_v contiguous, the
 * orientation of the Kaczmarz page, gist.science "Kaczmarz Linear Attention",
 * section "Derivazione Teorica"):
 *
 *   S~  = D_t S_{t-1}         D_t = exp(g_t) I (Gated DeltaNet) or
 *                             Diag(exp(g_t)) over key channels (KDA);
 *                             blog summary on the DeltaNet family, sections
 *                             "Gated DeltaNet" and "Kimi Delta Attention"; g is
 *                             the stored log-decay, DPLR subsection
 *   e_t = v_t - S~^T k_t      predict after the forget step (same sections)
 *   S_t = S~ + beta_t k_t e_t^T
 *   o_t = scale * S_t^T q_t   read after the write (the token sees its own
 *                             write: blog summary, KDA step 5 and the chunked
 *                             output subsection)
 *
 * with beta_t given, or the Kaczmarz step beta_t = eta_t / (||k_t||^2 + eps)
 * (Kaczmarz page, "La Regola di Aggiornamento KLA").
 *
 * With delta_mode = GDR_DELTA_OFF the prediction and the residual drop out
 * and the write is the plain additive one, S_t = D_t S_{t-1} + k_t v_t^T,
 * o_t = scale * S_t^T q_t: linear attention (D_t = I, g = 0), RetNet /
 * Mamba-2 (scalar decay) and GLA (per-channel decay), the rows of the
 * textbook page's update table whose transition is the decay alone.  No beta
 * scales that write; beta_or_eta, beta_mode and eps are then ignored.
 *
 * Two schedules of the same recurrence (blog summary, "Kernel Triton
 * recurrente fusionado" and "Pipeline Triton por chunks"): a chunked prefill
 * (gdr_chunk_fwd) and a fused single-token decode step (gdr_recurrent_step).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers (hipMalloc'd or equivalent) and
 *    are owned by the caller.  The library allocates nothing, frees nothing,
 *    never synchronises, and keeps no global state: it is reentrant.  The one
 *    exception is gdr_chunk_fwd_noalloc, which takes its workspace from a
 *    fixed device array of the library (see there).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  A
 *    GDR_OK return means the work is ENQUEUED on that stream, not finished.
 *  - Every argument is validated on the host before any HIP call.  A bad
 *    argument returns a negative gdr_status synchronously and nothing is
 *    enqueued.  A failed kernel launch returns GDR_E_HIP.  Nothing is printed.
 *  - Values are not checked: g should be finite and <= 0, beta / eta finite and
 *    >= 0 (beta is never clamped; the Kaczmarz beta exceeds 1 for short keys),
 *    and keys are used as given (the caller normalises them if it wants to).
 *  - Alignment: q, k, v, o, s0, s_final, state and workspace must be 16-byte
 *    aligned; g and beta_or_eta 4-byte aligned (16-byte for per-channel g).
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDR_ABI_VERSION 2

/* decay_mode */
#define GDR_DECAY_SCALAR 0       /* g is [.., H]: one log-decay per token and head */
#define GDR_DECAY_PER_CHANNEL 1  /* g is [.., H, Dk]: one log-decay per key channel */
/* beta_mode */
#define GDR_BETA_GIVEN 0         /* beta_or_eta holds beta_t */
#define GDR_BETA_KACZMARZ 1      /* beta_or_eta holds eta_t; beta_t = eta_t / (||k_t||^2 + eps) */
/* delta_mode */
#define GDR_DELTA_RULE 0         /* the (gated) delta rule above */
#define GDR_DELTA_OFF 1          /* additive write S = D S + k v^T (no prediction, no beta) */
/* dtypes of q, k, v (qkv_dtype) and of o (o_dtype) */
#define GDR_F32 0
#define GDR_BF16 1
/* algo: which kernels run the chunked path */
#define GDR_ALGO_AUTO 0          /* the matrix-core kernels (GDR_ALGO_MATRIX) */
#define GDR_ALGO_VECTOR 1        /* fp32 vector-ALU kernels (any dtype, any mode) */
#define GDR_ALGO_MATRIX 2        /* matrix-core kernels: bf16 MFMA (bf16 operands split hi/lo, fp32
                                    accumulation) for bf16 q/k/v at Dk = Dv = 128; fp32 MFMA tiles
                                    (fp32 operands and accumulation) for every other dtype and width */

typedef enum gdr_status {
    GDR_OK = 0,
    GDR_E_NULL = -1,         /* a required pointer is NULL */
    GDR_E_SHAPE = -2,        /* a size is negative or the element count overflows */
    GDR_E_UNSUPPORTED = -3,  /* Dk/Dv not in {64,128}, chunk != 64, algo not available */
    GDR_E_ALIGN = -4,        /* a pointer is misaligned */
    GDR_E_WORKSPACE = -5,    /* workspace missing or smaller than the queried size */
    GDR_E_HIP = -6,          /* a HIP launch failed */
    GDR_E_ALIAS = -7,        /* outputs overlap inputs (s_final == s0 exactly is allowed) */
    GDR_E_MODE = -8          /* bad enum value, negative/non-finite eps, non-finite scale */
} gdr_status;

/* Problem descriptor.  All fields are plain integers / floats. */
typedef struct gdr_desc {
    int32_t B;           /* sequences (batch); for gdr_recurrent_step: N sequences */
    int32_t T;           /* tokens per sequence; ignored by gdr_recurrent_step (= 1) */
    int32_t H;           /* heads (q, k and v share H) */
    int32_t Dk;          /* key width, 64 or 128 */
    int32_t Dv;          /* value width, 64 or 128 */
    int32_t chunk;       /* chunk length C of the chunked path, must be 64 */
    int32_t qkv_dtype;   /* GDR_F32 or GDR_BF16 */
    int32_t o_dtype;     /* GDR_F32 or GDR_BF16 */
    int32_t decay_mode;  /* GDR_DECAY_* */
    int32_t beta_mode;   /* GDR_BETA_* */
    int32_t algo;        /* GDR_ALGO_*; gdr_recurrent_step ignores it */
    int32_t delta_mode;  /* GDR_DELTA_*; 0 (the delta rule) in descriptors of ABI version 1 */
    float eps;           /* Kaczmarz stabiliser (>= 0); ignored for GDR_BETA_GIVEN and GDR_DELTA_OFF */
    float scale;         /* output scale; 1 = the plain read, 1/sqrt(Dk) = KDA's read */
} gdr_desc;

/* Version of this ABI (GDR_ABI_VERSION). */
int gdr_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char *gdr_status_string(int status);

/*
 * Bytes of device workspace gdr_chunk_fwd needs for `desc`, written to *bytes.
 * Host-only; returns a gdr_status (the same validation of desc as
 * gdr_chunk_fwd, pointers aside).
 */
int gdr_chunk_fwd_workspace_size(const gdr_desc *desc, size_t *bytes);

/*
 * Chunked forward pass over whole sequences (prefill).
 *
 * The chunked algebra is the blog summary's section "KDA por chunks": within
 * a chunk of C tokens the corrected writes solve a unit lower-triangular
 * system (I + R) E = Ebar, one per value channel; the chunk-end state is
 * S_{c+1} = D_{0:C-1} S_c + (K^end)^T E; the in-chunk outputs add a causal
 * read matrix (diagonal included) to the read of the entering state.  The
 * Kaczmarz page states that only the diagonal beta matrix changes for KLA.
 *
 *   q, k        [B, T, H, Dk]  qkv_dtype, contiguous
 *   v           [B, T, H, Dv]  qkv_dtype, contiguous
 *   g           [B, T, H] (scalar decay) or [B, T, H, Dk] (per channel), fp32
 *   beta_or_eta [B, T, H] fp32 (may be NULL with GDR_DELTA_OFF)
 *   s0          [B, H, Dk, Dv] fp32 initial state, or NULL for zero
 *   o           [B, T, H, Dv]  o_dtype (written)
 *   s_final     [B, H, Dk, Dv] fp32 final state (written), or NULL; may be
 *               the same pointer as s0 (in-place state update)
 *   workspace   device scratch of at least gdr_chunk_fwd_workspace_size bytes;
 *               its contents on entry do not matter and are clobbered
 * T may be any value >= 0 (the last chunk may be partial); with T == 0 only
 * s_final is written (s0, or zero).  B == 0 or H == 0 is a no-op.
 * q, k, v, g and beta_or_eta must not overlap o, s_final or workspace.
 */
int gdr_chunk_fwd(const gdr_desc *desc,
                  const void *q, const void *k, const void *v,
                  const float *g, const float *beta_or_eta,
                  const float *s0, void *o, float *s_final,
                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * Chunked forward pass over a packed batch of sequences of different lengths
 * (serving: prefills of several requests in one call; blog summary, "Pipeline
 * Triton por chunks", on the chunk mode for prefill next to the recurrent one
 * for decode).  desc->B is the number of sequences N and desc->T the number of
 * tokens of all of them; sequence n holds tokens [cu_seqlens[n],
 * cu_seqlens[n+1]) of the packed tensors and has its own state.
 *
 *   cu_seqlens  [N + 1] int32 in DEVICE memory, 0 = cu[0] <= ... <= cu[N] = T
 *   q, k        [T, H, Dk]  qkv_dtype, contiguous
 *   v           [T, H, Dv]  qkv_dtype, contiguous
 *   g           [T, H] or [T, H, Dk] fp32
 *   beta_or_eta [T, H] fp32 (may be NULL with GDR_DELTA_OFF)
 *   s0, s_final [N, H, Dk, Dv] fp32 (as for gdr_chunk_fwd: s0 may be NULL,
 *               s_final may be NULL or equal s0)
 *   o           [T, H, Dv]  o_dtype (written for the tokens of the sequences)
 *   workspace   at least gdr_chunk_fwd_varlen_workspace_size bytes
 * Every sequence gives the results gdr_chunk_fwd gives for it alone.  The
 * library does not read cu_seqlens on the host.  On the device, entries
 * outside the form above never address memory out of bounds: each is clamped
 * to [0, T] and raised to the largest entry before it (tokens outside every
 * sequence are then not written).  Empty sequences are allowed (their final
 * state is their initial one).  Long sequences are walked in one piece (no
 * time segments).  cu_seqlens must not overlap o, s_final or the workspace.
 */
int gdr_chunk_fwd_varlen_workspace_size(const gdr_desc *desc, size_t *bytes);
int gdr_chunk_fwd_varlen(const gdr_desc *desc, const int32_t *cu_seqlens,
                         const void *q, const void *k, const void *v,
                         const float *g, const float *beta_or_eta,
                         const float *s0, void *o, float *s_final,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * Backward pass of gdr_chunk_fwd (training): the gradients of a loss L with
 * respect to every input, given dL/do and dL/ds_final.  The pages derive no
 * backward pass (the blog summary, "Pipeline Triton por chunks", calls the
 * chunked mode the training mode); it is reverse-mode differentiation of the
 * chunk algebra of gdr_chunk_fwd, with the chunk-entering states recomputed.
 * Products on matrix-core tiles: bf16 with fp32 operands split into hi + lo
 * (the forward's arithmetic) for bf16 q/k/v at Dk = Dv = 128 with scalar
 * decay, fp32 otherwise; fp32 accumulation and gradients; fixed-length
 * batches (packed ones: gdr_chunk_bwd_varlen below); desc->algo and
 * desc->o_dtype are ignored.  With GDR_DELTA_OFF
 * (the additive write) beta_or_eta and dbeta are ignored and may be NULL.
 *
 *   q, k, v, g, beta_or_eta, s0   as for gdr_chunk_fwd (s0 may be NULL)
 *   d_o       [B, T, H, Dv] fp32, dL/do
 *   ds_final  [B, H, Dk, Dv] fp32, dL/ds_final, or NULL for zero
 *   dq, dk    [B, T, H, Dk] fp32 (written)
 *   dv        [B, T, H, Dv] fp32 (written)
 *   dg        shaped as g, fp32 (written)
 *   dbeta     [B, T, H] fp32 (written): dL/dbeta, or dL/deta for the
 *             Kaczmarz step size (not written with GDR_DELTA_OFF)
 *   ds0       [B, H, Dk, Dv] fp32 (written), or NULL
 *   workspace at least gdr_chunk_bwd_workspace_size bytes (per chunk and
 *             head: the entering state and its gradient, 2 Dk Dv fp32, and
 *             about 80 KiB of per-chunk matrices; with per-channel decay or
 *             fp32 q, k also the decayed keys and queries, 3 x 64 x Dk fp32)
 * Outputs must not overlap inputs, each other or the workspace.  With
 * T == 0 only ds0 is written (= ds_final, or zero).
 */
int gdr_chunk_bwd_workspace_size(const gdr_desc *desc, size_t *bytes);
int gdr_chunk_bwd(const gdr_desc *desc,
                  const void *q, const void *k, const void *v,
                  const float *g, const float *beta_or_eta, const float *s0,
                  const float *d_o, const float *ds_final,
                  float *dq, float *dk, float *dv, float *dg, float *dbeta,
                  float *ds0, void *workspace, size_t workspace_bytes,
                  void *stream);

/*
 * Backward pass of gdr_chunk_fwd_varlen: a packed batch of N = desc->B
 * sequences of different lengths, desc->T tokens in all, sequence n holding
 * tokens [cu_seqlens[n], cu_seqlens[n+1]) and its own state (training on
 * packed sequences).  Tensors as for gdr_chunk_fwd_varlen: token tensors
 * [T, H, ..] (q, k, v, g, beta_or_eta, d_o in; dq, dk, dv, dg, dbeta out),
 * states [N, H, Dk, Dv] (s0 and ds_final in, may be NULL; ds0 out, may be
 * NULL); cu_seqlens [N + 1] int32 in device memory, read on the device only,
 * with entries clamped as gdr_chunk_fwd_varlen clamps them (gradients of
 * tokens outside every sequence are not written).  Every sequence gets the
 * gradients gdr_chunk_bwd gives for it alone.  The workspace holds the
 * sequence table and the per-chunk records of floor((T + 63 N) / 64) chunks
 * per head; cu_seqlens must not overlap an output or the workspace.
 */
int gdr_chunk_bwd_varlen_workspace_size(const gdr_desc *desc, size_t *bytes);
int gdr_chunk_bwd_varlen(const gdr_desc *desc, const int32_t *cu_seqlens,
                         const void *q, const void *k, const void *v,
                         const float *g, const float *beta_or_eta, const float *s0,
                         const float *d_o, const float *ds_final,
                         float *dq, float *dk, float *dv, float *dg, float *dbeta,
                         float *ds0, void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * One stage of gdr_chunk_fwd, with the same arguments.  The chunked path is a
 * pipeline of two kernels (blog summary, "Pipeline Triton por chunks": an
 * intra-chunk kernel builds the in-chunk interaction matrices and the WY-like
 * form of the corrected writes; the state kernel is the only walk across
 * chunks and produces the outputs):
 *   stage 0 (GDR_STAGE_INTRA): every chunk in parallel; reads q, k, v, g,
 *            beta_or_eta and writes the workspace only.
 *   stage 1 (GDR_STAGE_STATE): walks the chunks of each sequence in order;
 *            reads q, k, v, g, beta_or_eta, s0 and the workspace written by
 *            stage 0 with the same arguments, and writes o and s_final.
 * Stage 0 followed by stage 1 on one stream is exactly gdr_chunk_fwd.  The
 * split exists so that callers (profilers, benchmarks) can time each kernel;
 * validation is identical to gdr_chunk_fwd.
 */
#define GDR_STAGE_INTRA 0
#define GDR_STAGE_STATE 1
int gdr_chunk_fwd_stage(int stage, const gdr_desc *desc,
                        const void *q, const void *k, const void *v,
                        const float *g, const float *beta_or_eta,
                        const float *s0, void *o, float *s_final,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdr_chunk_fwd_stage with the stage's kernel time recorded, for measurement:
 * start_event and stop_event are hipEvent_t handles created by the caller
 * with timing enabled (both required, else GDR_E_NULL).  On the matrix-core
 * path the stage's first kernel records start_event when it begins and its
 * last kernel records stop_event when it ends (hipExtLaunchKernelGGL), so
 * hipEventElapsedTime gives the kernels' time without the launch gap before
 * them; on the other paths the events are recorded on the stream before and
 * after the stage's launches.  Everything else (arguments, validation,
 * results) is exactly gdr_chunk_fwd_stage.  The events are only written.
 */
int gdr_chunk_fwd_stage_timed(int stage, const gdr_desc *desc,
                              const void *q, const void *k, const void *v,
                              const float *g, const float *beta_or_eta,
                              const float *s0, void *o, float *s_final,
                              void *workspace, size_t workspace_bytes, void *stream,
                              void *start_event, void *stop_event);

/*
 * One fused recurrent step for B = N independent sequences (decode): the
 * seven steps above for a single token, with the state read once and written
 * once (blog summary, "Kernel Triton recurrente fusionado": decay, predict,
 * residual, rank-1 write and read fused in one pass).
 *
 *   q, k        [N, H, Dk]  qkv_dtype
 *   v           [N, H, Dv]  qkv_dtype
 *   g           [N, H] or [N, H, Dk] fp32
 *   beta_or_eta [N, H] fp32 (may be NULL with GDR_DELTA_OFF)
 *   state       [N, H, Dk, Dv] fp32, read and updated in place
 *   o           [N, H, Dv] o_dtype (written)
 * desc->T and desc->chunk are ignored.  q, k, v, g, beta_or_eta must not
 * overlap state or o.
 */
int gdr_recurrent_step(const gdr_desc *desc,
                       const void *q, const void *k, const void *v,
                       const float *g, const float *beta_or_eta,
                       float *state, void *o, void *stream);

/*
 * gdr_recurrent_step with its kernel time recorded, for measurement: the
 * step's kernel records start_event (a caller-created hipEvent_t with timing
 * enabled) when it begins and stop_event when it ends (hipExtLaunchKernelGGL);
 * both are required (else GDR_E_NULL).  With nothing to launch (B = 0 or
 * H = 0) both are recorded on the stream.  Everything else is exactly
 * gdr_recurrent_step.
 */
int gdr_recurrent_step_timed(const gdr_desc *desc,
                             const void *q, const void *k, const void *v,
                             const float *g, const float *beta_or_eta,
                             float *state, void *o, void *stream,
                             void *start_event, void *stop_event);

/*
 * The fused recurrent schedule over desc->T tokens of B sequences (short
 * prefills, several decode tokens at once): token after token as in
 * gdr_recurrent_step, with the state read once before the first token and
 * written once after the last (blog summary, "Kernel Triton recurrente
 * fusionado", which puts the recurrent mode in charge of decode and short
 * sequences).
 *
 *   q, k        [B, T, H, Dk]  qkv_dtype
 *   v           [B, T, H, Dv]  qkv_dtype
 *   g           [B, T, H] or [B, T, H, Dk] fp32
 *   beta_or_eta [B, T, H] fp32 (may be NULL with GDR_DELTA_OFF)
 *   state       [B, H, Dk, Dv] fp32, read and updated in place
 *   o           [B, T, H, Dv] o_dtype (written)
 * desc->chunk and desc->algo are ignored; T == 0, B == 0 or H == 0 is a
 * no-op.  The same results as gdr_chunk_fwd with s0 = s_final = state, to
 * rounding; the work is sequential in T, so long sequences belong on the
 * chunked path.  Inputs must not overlap state or o.
 */
int gdr_recurrent_fwd(const gdr_desc *desc,
                      const void *q, const void *k, const void *v,
                      const float *g, const float *beta_or_eta,
                      float *state, void *o, void *stream);

/*
 * gdr_recurrent_fwd over a packed batch (serving: a few tokens of each of N
 * requests of different lengths in one call).  desc->B = N sequences,
 * desc->T = tokens of all of them; sequence n is tokens [cu_seqlens[n],
 * cu_seqlens[n+1]) of q, k, v [T, H, ..], g, beta_or_eta [T, H(, Dk)] and o
 * [T, H, Dv], and owns state [n] of state [N, H, Dk, Dv] (updated in place).
 * cu_seqlens [N + 1] int32 in device memory, read on the device only: each
 * offset is clamped to [0, T] and raised to the largest one before it, so
 * no entry addresses memory out of bounds (an empty sequence keeps its
 * state; outputs of tokens outside every sequence are not written).
 * cu_seqlens must not overlap state or o.
 */
int gdr_recurrent_fwd_varlen(const gdr_desc *desc, const int32_t *cu_seqlens,
                             const void *q, const void *k, const void *v,
                             const float *g, const float *beta_or_eta,
                             float *state, void *o, void *stream);

/*
 * gdr_chunk_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same pass, kernels, arithmetic and validation as gdr_chunk_fwd, with
 * the workspace taken from a fixed scratch array of GDR_NOALLOC_SCRATCH_BYTES
 * (128 MiB) that the library holds on each GPU it runs on until the process
 * ends, instead of from the caller.  The caller still passes every input and
 * output.  The call allocates and frees nothing.
 *
 *   Arguments as for gdr_chunk_fwd, without workspace and workspace_bytes.
 *   Returns GDR_E_WORKSPACE (before any HIP call, nothing enqueued) when
 *   gdr_chunk_fwd_workspace_size(desc) exceeds GDR_NOALLOC_SCRATCH_BYTES: it
 *   covers for example B4 H16 T4096 d128 with scalar decay (98 MiB), or
 *   about 5,300 (sequence, head, chunk) records on the matrix-core path with
 *   scalar decay, 1,000 with per-channel decay.
 *
 * The scratch array of the calling thread's current device is used; `stream`
 * must belong to that device.  Its device address is looked up on the first
 * call on each device (hipGetSymbolAddress), so make that first call outside
 * graph capture.  Every call on one GPU shares that GPU's array and the array
 * keeps the last call's contents (the pass does not depend on them): calls
 * that can overlap on one GPU (on different streams without ordering between
 * them, or from several threads) race on it and must be serialised by the
 * caller.
 */
#define GDR_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int gdr_chunk_fwd_noalloc(const gdr_desc *desc,
                          const void *q, const void *k, const void *v,
                          const float *g, const float *beta_or_eta,
                          const float *s0, void *o, float *s_final, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */
