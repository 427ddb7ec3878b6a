/*
 * gdr.h -- C ABI of the gated delta-rule library for AMD Instinct MI355X (gfx950).
 *
 * The library computes the delta-rule linear-attention recurrence, written
 * key-major (the state S has d_k rows and d_v columns):
 *
 *     S_t = (I - beta_t k_t k_t^T) diag(a_t) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = S_t^T q_t,                       a_t = exp(log_a_t).
 *
 * Sources: "Moonshot AI's New Attention Architecture: Key Innovations
 * Explained", §2 Core Operator (DeltaNet update; scalar-gated update; per-channel
 * gated update) and §3 Hardware-Friendly Algorithm (chunkwise form: state passed
 * between chunks, correction terms W and U, causally masked intra-chunk
 * product); "OSDN: Improving Delta Rule with Provable Online Preconditioning in
 * Linear Attention", Technical Summary §1 (the delta rule as one gradient step
 * on 0.5*||S k - v||^2).  Without a gate (a_t = 1) this is DeltaNet; a scalar
 * a_t gives Gated DeltaNet; a vector a_t over key channels gives the per-channel
 * (KDA-style) gate.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument is a DEVICE pointer except `desc` (and the size
 *    out-parameter of gdr_chunk_fwd_workspace_size), which are host pointers
 *    used during the call only.  The caller owns every buffer, scratch
 *    included; the library allocates no device memory, keeps no mutable global
 *    state and is safe to call from several host threads.  The one exception is
 *    gdr_chunk_fwd_noalloc, whose scratch is a static device array per GPU.
 *  - Work is enqueued asynchronously on `stream` (0 = the null stream).  The
 *    library never synchronises; the caller synchronises before reading results.
 *  - All tensors are dense, contiguous and row-major in the layouts given
 *    below.  Pointers to q, k, v, o and to the fp32 states must be 16-byte
 *    aligned; beta and log_a must be aligned to their element size.
 *  - q, k, v, beta, log_a and o share the I/O dtype (`io`): GDR_F32 or GDR_BF16.
 *    Recurrent states (S0, S_T, S, S_new) are always fp32.  bf16 outputs are
 *    rounded to nearest even.
 *  - Every argument check runs before anything is enqueued; on error nothing
 *    is enqueued, the status is returned and a message is available from
 *    gdr_last_error() on the calling thread.  No C++ exception crosses the ABI
 *    and the library never aborts.
 */
#ifndef GDR_H_
#define GDR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDR_OK = 0,
  GDR_ERR_INVALID_ARG = 1,   /* null pointer, bad size, bad enum, forbidden alias */
  GDR_ERR_UNSUPPORTED = 2,   /* valid but not implemented (d_k, d_v, chunk) */
  GDR_ERR_ALIGNMENT = 3,     /* pointer not aligned as required */
  GDR_ERR_WORKSPACE = 4,     /* workspace missing (NULL) or smaller than its size query returns */
  GDR_ERR_HIP = 5            /* the HIP runtime reported an error at launch */
} gdr_status;

typedef enum { GDR_F32 = 0, GDR_BF16 = 1 } gdr_dtype;

typedef enum {
  GDR_GATE_NONE = 0,     /* a_t = 1; log_a must be NULL                        */
  GDR_GATE_SCALAR = 1,   /* one log-gate per (token, head): log_a [B, T, H]    */
  GDR_GATE_CHANNEL = 2   /* one per key channel: log_a [B, T, H, d_k]          */
} gdr_gate;

/* Where the decay sits relative to the erase.  GDR_FORM_PAGE (default) decays
 * first and erases from the decayed state, S_t = (I - b k k^T) D S + b k v^T, as
 * both gated updates of "Moonshot AI's New Attention Architecture", §2 print it.
 * GDR_FORM_LITERAL erases from the undecayed state, S_t = (D - b k k^T) S + b k v^T.
 * The two coincide without a gate. */
typedef enum { GDR_FORM_PAGE = 0, GDR_FORM_LITERAL = 1 } gdr_form;

/* Problem descriptor.  All fields are read by value during the call. */
typedef struct {
  int64_t B;       /* sequences (batch); for a decode step: independent sequences */
  int64_t T;       /* tokens per sequence (>= 0); must be 1 for a decode step     */
  int64_t H;       /* heads                                                       */
  int64_t d_k;     /* key / query width: 64 or 128                                 */
  int64_t d_v;     /* value width: 64 or 128                                       */
  int32_t chunk;   /* chunk length of the chunkwise form: 64 (0 selects 64).  The
                      result does not depend on it beyond rounding.               */
  int32_t io;      /* gdr_dtype */
  int32_t gate;    /* gdr_gate  */
  int32_t form;    /* gdr_form  */
} gdr_desc;

/*
 * gdr_chunk_fwd_workspace_size -- device scratch that gdr_chunk_fwd needs.
 *
 * Writes to *bytes the size of the workspace for a forward described by desc.
 * Per (sequence, head, chunk) it holds what the chunk contributes independently
 * of the state ("Moonshot AI's New Attention Architecture", §3): the inverse
 * (I + A)^{-1} of the chunk's unit lower triangular system (its WY correction
 * terms are that solve applied to the keys and values) and room for the
 * causally masked query-key score matrix, each as the ten 16 x 16 blocks of a
 * 64 x 64 triangle in the I/O dtype, plus six rows of 64 fp32 per-token gate
 * factors.  With bf16 I/O and a per-channel gate each record also holds the
 * chunk's three decayed key/query operands (64 x d_k bf16 each), formed once per
 * chunk rather than once per d_v tile.  That is B * H * ceil(T / 64) *
 * (5120 * elem + 1536) bytes, plus B * H * ceil(T / 64) * 384 * d_k bytes for
 * bf16 with a per-channel gate (0 when T == 0).  Returns the same errors as
 * gdr_chunk_fwd's descriptor checks; *bytes is 0 on error.
 */
gdr_status gdr_chunk_fwd_workspace_size(const gdr_desc* desc, size_t* bytes);

/*
 * gdr_chunk_fwd -- forward over whole sequences with the chunkwise-parallel form.
 *
 * Defined by the recurrence above, run token by token from S0 for each (b, h)
 * independently; computed chunk by chunk as in "Moonshot AI's New Attention
 * Architecture", §3 (per-chunk cumulative log-gate, intra-chunk WY correction
 * terms from a unit-lower-triangular solve, sequential state pass between
 * chunks, output as a state read plus a causally masked intra-chunk product).
 *
 *   q      [B, T, H, d_k]  io dtype
 *   k      [B, T, H, d_k]  io dtype
 *   v      [B, T, H, d_v]  io dtype
 *   beta   [B, T, H]       io dtype (any finite value; workloads use (0, 1))
 *   log_a  NULL for GDR_GATE_NONE; [B, T, H] (scalar) or [B, T, H, d_k]
 *          (channel), io dtype, finite (log of a decay in (0, 1] for workloads).
 *          Any finite decay is handled: with a per-channel gate, a chunk in which
 *          some channel decays by more than e^-64 within one 16-token block has its
 *          triangular solve and score matrix formed by a slower generic kernel
 *          (every decay one exponential), the rest by the split-factor transform.
 *   S0     [B, H, d_k, d_v] fp32, or NULL for a zero initial state
 *   o      [B, T, H, d_v]  io dtype, written (may be NULL only when T == 0)
 *   S_T    [B, H, d_k, d_v] fp32 final state, or NULL to skip it.  S_T may be
 *          the same pointer as S0 (updated in place) but must not otherwise
 *          overlap any argument.
 *   o must not overlap any input or S_T.
 *   workspace        device scratch of at least gdr_chunk_fwd_workspace_size()
 *                    bytes, 16-byte aligned, overlapping no other argument (may
 *                    be NULL when T == 0).  Its contents on entry do not matter
 *                    and are overwritten; it may be reused once the call's work
 *                    on `stream` has finished (or by later work on the same
 *                    stream).  Calls that overlap in time need separate ones.
 *   workspace_bytes  its size in bytes.
 *
 * Supported: d_k, d_v in {64, 128} with every gate and form for bf16 I/O; fp32 I/O
 * with every gate at d_k = 64 and without a gate or with a scalar gate at
 * d_k = 128 (an fp32 per-channel gate at d_k = 128 returns GDR_ERR_UNSUPPORTED).
 *
 * Two kernels run in order on `stream`: the per-chunk transform (cumulative
 * log-gate, the gated Gram blocks of the keys, (I + A)^{-1}, the masked score
 * matrix) for all chunks at once, then the sequential state pass with the output
 * (with a per-channel gate a third one between them re-forms the chunks whose
 * decay leaves the transform's range; it exits at once when there are none).
 *
 * T == 0 writes S_T = S0 (or zeros).  T need not be a multiple of the chunk.
 */
gdr_status gdr_chunk_fwd(const gdr_desc* desc, const void* q, const void* k, const void* v,
                         const void* beta, const void* log_a, const float* S0, void* o,
                         float* S_T, void* workspace, size_t workspace_bytes,
                         void* stream /* hipStream_t */);

/*
 * gdr_chunk_fwd_noalloc -- gdr_chunk_fwd without a caller workspace and without
 * any device allocation, for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, semantics, kernels and errors as gdr_chunk_fwd minus the
 * workspace: the per-chunk records live in a static device array of 256 MiB
 * (268435456 bytes) that every GPU the library runs on holds from its first use
 * until the process ends.  A forward whose gdr_chunk_fwd_workspace_size exceeds
 * that returns GDR_ERR_WORKSPACE with nothing enqueued (for example the scalar
 * gate at d_k = 128 fits B * H * ceil(T / 64) <= 22795 chunk records; the
 * per-channel gate at d_k = 128, 4405).  The first call on a device looks the
 * array's address up (GDR_ERR_HIP if that fails).  The array keeps the last call's
 * contents, which the next call overwrites before reading.  Every call on one GPU
 * shares that GPU's array: calls whose work overlaps in time on one GPU (on
 * different streams, or from several host threads at once) race and give
 * undefined results; calls on one stream are ordered and safe.
 */
gdr_status gdr_chunk_fwd_noalloc(const gdr_desc* desc, const void* q, const void* k, const void* v,
                                 const void* beta, const void* log_a, const float* S0, void* o, float* S_T,
                                 void* stream /* hipStream_t */);

/*
 * gdr_chunk_fwd_varlen_workspace_size -- workspace of gdr_chunk_fwd_varlen.
 *
 * desc describes the packed tensors (desc->B must be 1, desc->T = total
 * tokens); n_seq >= 1 is the number of sequences.  Sequence i's chunks use
 * record slots from floor(cu_seqlens[i] / 64) + i on, so H * (ceil(T / 64) +
 * n_seq) records of the size given under gdr_chunk_fwd_workspace_size cover
 * any split of the T tokens; then 4 * n_seq bytes (rounded up to 16) hold the
 * order, longest sequence first, in which the bf16 state pass takes the sequences
 * (the fp32 one, which serves parity, takes them in order).  Both dtypes, with the
 * configurations of gdr_chunk_fwd.
 */
gdr_status gdr_chunk_fwd_varlen_workspace_size(const gdr_desc* desc, int64_t n_seq, size_t* bytes);

/*
 * gdr_chunk_fwd_varlen -- gdr_chunk_fwd over variable-length sequences packed
 * along T (one prefill batch of prompts of different lengths).
 *
 * The recurrence runs independently on each sequence i = tokens
 * cu_seqlens[i] .. cu_seqlens[i+1] - 1 of the packed tensors, from S0[i]; a
 * sequence boundary is an independent restart of the same operator, so the
 * result for each sequence equals gdr_chunk_fwd on that sequence alone.
 *
 *   cu_seqlens  device int32 [n_seq + 1], 0 = cu[0] <= cu[1] <= ... <= cu[n_seq]
 *               = T (not checked by the library: the kernels clamp each entry to
 *               [0, T] and each length to >= 0, so a malformed table cannot make
 *               them read or write outside the tensors, but its results are
 *               undefined).  Empty sequences are allowed (S_T[i] = S0[i]).
 *   q, k   [1, T, H, d_k] bf16   v, o [1, T, H, d_v] bf16   beta [1, T, H] bf16
 *   log_a  NULL / [1, T, H] / [1, T, H, d_k] bf16
 *   S0     [n_seq, H, d_k, d_v] fp32 or NULL;  S_T [n_seq, H, d_k, d_v] fp32 or NULL
 *   workspace  at least gdr_chunk_fwd_varlen_workspace_size() bytes.
 * Other rules (alignment, aliasing, errors) as for gdr_chunk_fwd; desc->B must be
 * 1 and desc->io GDR_BF16.
 */
gdr_status gdr_chunk_fwd_varlen(const gdr_desc* desc, const int32_t* cu_seqlens, int64_t n_seq,
                                const void* q, const void* k, const void* v, const void* beta,
                                const void* log_a, const float* S0, void* o, float* S_T,
                                void* workspace, size_t workspace_bytes, void* stream /* hipStream_t */);

/*
 * gdr_recurrent_step -- one decode token for B independent sequences.
 *
 * One step of the recurrence above with a constant-size state ("Moonshot AI's
 * New Attention Architecture", §1: linear layers decode with a fixed-size state
 * instead of a growing key-value cache).  desc->T must be 1; desc->chunk is
 * ignored.
 *
 *   q, k   [B, H, d_k]  io dtype        v, o  [B, H, d_v]  io dtype
 *   beta   [B, H]       io dtype        log_a NULL / [B, H] / [B, H, d_k]
 *   S      [B, H, d_k, d_v] fp32 state before the token
 *   S_new  [B, H, d_k, d_v] fp32 state after the token; may equal S (in place)
 *          but must not otherwise overlap S.
 *   o must not overlap any other argument.
 */
gdr_status gdr_recurrent_step(const gdr_desc* desc, const void* q, const void* k, const void* v,
                              const void* beta, const void* log_a, const float* S, float* S_new,
                              void* o, void* stream /* hipStream_t */);

/* Static description of a status code. */
const char* gdr_status_string(gdr_status status);

/* Message describing the last error returned on the calling thread ("" if none). */
const char* gdr_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int gdr_version(void);

/*
 * gdr_chunk_fwd_wkey / gdr_recurrent_step_wkey -- the delta rule with a separate
 * write key ("OSDN: Improving Delta Rule with Provable Online Preconditioning in
 * Linear Attention", §2.1: right-preconditioning the delta-rule step by
 * diag(d_t) is the same as writing along the scaled key kw_t = d_t * k_t while
 * the residual still reads along k_t; the chunkwise pipeline is unchanged with
 * kw in place of k on the write side; §4 runs it on DeltaNet, gated DeltaNet and
 * per-channel gated backbones).  Key-major, per token, with the decay
 * D_t = diag(a_t) of the gate (identity without one) applied first:
 *
 *     S_t = (I - beta_t kw_t k_t^T) D_t S_{t-1} + beta_t kw_t v_t^T,    o_t = S_t^T q_t
 *
 * (GDR_FORM_LITERAL: the residual reads the undecayed state, as for
 * gdr_chunk_fwd).  kw = k is gdr_chunk_fwd / gdr_recurrent_step.  The caller
 * forms kw (the pages' preconditioner scan is gdr_precond_scan).
 *
 *   kw     same shape, dtype and alignment rules as k ([B, T, H, d_k] for the
 *          forward, [B, H, d_k] for the step); may alias k or q (it is only read).
 *   log_a  as for gdr_chunk_fwd / gdr_recurrent_step (NULL without a gate).
 * Every other argument, the workspace (gdr_chunk_fwd_workspace_size of the same
 * descriptor) and the errors are as for gdr_chunk_fwd / gdr_recurrent_step.  The
 * forward takes bf16 I/O only, and d_k = 128 with a per-channel gate; the step
 * takes both dtypes and every gate.
 */
gdr_status gdr_chunk_fwd_wkey(const gdr_desc* desc, const void* q, const void* k, const void* kw,
                              const void* v, const void* beta, const void* log_a, const float* S0, void* o,
                              float* S_T, void* workspace, size_t workspace_bytes, void* stream /* hipStream_t */);
gdr_status gdr_recurrent_step_wkey(const gdr_desc* desc, const void* q, const void* k, const void* kw,
                                   const void* v, const void* beta, const void* log_a, const float* S,
                                   float* S_new, void* o, void* stream /* hipStream_t */);

/*
 * gdr_chunk_fwd_varlen_wkey -- gdr_chunk_fwd_wkey over variable-length sequences
 * packed along T (phase 2 of the preconditioned rule on packed prompts).
 *
 * Every argument as for gdr_chunk_fwd_varlen, plus kw ([1, T, H, d_k] bf16) as for
 * gdr_chunk_fwd_wkey; the workspace is gdr_chunk_fwd_varlen_workspace_size's.
 * Supported and errors as for both calls.
 */
gdr_status gdr_chunk_fwd_varlen_wkey(const gdr_desc* desc, const int32_t* cu_seqlens, int64_t n_seq, const void* q,
                                     const void* k, const void* kw, const void* v, const void* beta,
                                     const void* log_a, const float* S0, void* o, float* S_T, void* workspace,
                                     size_t workspace_bytes, void* stream /* hipStream_t */);

/*
 * gdr_precond_scan -- the preconditioner scan that produces the write keys of the
 * preconditioned delta rule ("OSDN: Improving Delta Rule with Provable Online
 * Preconditioning in Linear Attention", §2.2: a first phase over the keys alone;
 * each token's write key is the diagonal preconditioner d_t times the key, then
 * d takes one online-gradient step on the closed-form surrogate
 * h_t(d) = ((1 - beta_t <d, k_t^2>)^2 - 1) / (2 ||k_t||^2); §2.3: adaptive
 * preconditioner forgetting multiplies d by a per-token, per-head retention r_t).
 * For each (b, h) independently, token by token from d_0:
 *
 *     kw_t    = d_t * k_t                                  (elementwise)
 *     d_{t+1} = r_t d_t + eta beta_t (1 - beta_t <d_t, k_t^2>) k_t^2 / ||k_t||^2
 *
 * a descent step on h_t (a zero key adds nothing; r_t = 1 without forgetting).
 * The kw it writes is the write key of gdr_chunk_fwd_wkey / gdr_recurrent_step_wkey.
 *
 * desc: B, T (>= 0), H, d_k (64 or 128) and io are read; d_v, chunk, gate and
 * form are ignored.
 *   k     [B, T, H, d_k]  io dtype, 16-byte aligned
 *   beta  [B, T, H]       io dtype
 *   r     [B, T, H]       io dtype retention (> 0; the kernels take its log), or
 *         NULL for no forgetting
 *   eta   step size, finite
 *   d0    [B, H, d_k] fp32 preconditioner before token 0, or NULL (all ones)
 *   kw    [B, T, H, d_k]  io dtype, written, 16-byte aligned (k, beta and kw may
 *         be NULL only when T == 0)
 *   d_T   [B, H, d_k] fp32 preconditioner after the last token, or NULL to skip
 *         it; may be the same pointer as d0 (updated in place)
 * kw and d_T overlap no other argument (except d_T == d0).  T == 0 writes
 * d_T = d0 (or ones).  (T + 128) * H * d_k * elem_size may not exceed 2^31 - 1
 * bytes (GDR_ERR_UNSUPPORTED): offsets within one sequence are 32-bit.  bf16 runs the chunkwise form (bf16 products with fp32
 * accumulation for the key Gram matrix and the per-token preconditioners; the
 * preconditioner carried between chunks in fp32); fp32 runs token by token in fp32.
 */
gdr_status gdr_precond_scan(const gdr_desc* desc, const void* k, const void* beta, const void* r, float eta,
                            const float* d0, void* kw, float* d_T, void* stream /* hipStream_t */);

/*
 * gdr_precond_scan_bwd_workspace_size -- device scratch for gdr_precond_scan_bwd:
 * B * H * T * (d_k + 2) * 4 bytes (the preconditioner before every token and two
 * fp32 sums per token).  Returns gdr_precond_scan_bwd's descriptor errors; *bytes is
 * 0 on error.
 */
gdr_status gdr_precond_scan_bwd_workspace_size(const gdr_desc* desc, size_t* bytes);

/*
 * gdr_precond_scan_bwd -- gradients of the preconditioner scan (training the
 * preconditioned delta rule, "OSDN: Improving Delta Rule with Provable Online
 * Preconditioning in Linear Attention", §2.2 and §4: the write keys of phase 1
 * feed phase 2, so the gradient of phase 2's write key flows back through the scan).
 *
 * For the scan gdr_precond_scan(desc, k, beta, r, eta, d0) with outputs kw and d_T,
 * returns the gradients of L = <dkw, kw> + <dd_T, d_T> with respect to k, beta, r
 * and d0 -- the reverse-mode derivatives of the scan's update, taken token by token
 * (the pages print no gradients; a zero key, which leaves d unchanged, passes only
 * dkw_t * d_t to k_t).
 *
 *   desc, k, beta, r, eta, d0   as for gdr_precond_scan (desc->d_v is not read)
 *   dkw    [B, T, H, d_k] io dtype gradient of kw, or NULL (zero)
 *   dd_T   [B, H, d_k] fp32 gradient of d_T, or NULL (zero)
 *   dk     [B, T, H, d_k] io dtype, written (non-NULL when T > 0)
 *   dbeta  [B, T, H] io dtype, written (non-NULL when T > 0)
 *   dr     [B, T, H] io dtype, written; NULL to skip it; must be NULL when r is NULL
 *   dd0    [B, H, d_k] fp32, written, or NULL to skip it; may equal dd_T
 *   workspace / workspace_bytes  at least gdr_precond_scan_bwd_workspace_size bytes,
 *          16-byte aligned, overwritten
 *
 * Each (sequence, head) runs the scan forward in fp32, keeping each token's
 * preconditioner in the workspace, then walks the tokens back in fp32: bf16 I/O in
 * blocks of 16 tokens (the key products on fp32 MFMA, one scalar chain per block),
 * fp32 I/O token by token.
 * T == 0 writes dd0 = dd_T (or zeros).  Errors as for gdr_precond_scan, plus
 * GDR_ERR_WORKSPACE for a missing or short workspace and the alias checks of the
 * outputs against every other buffer.
 */
gdr_status gdr_precond_scan_bwd(const gdr_desc* desc, const void* k, const void* beta, const void* r, float eta,
                                const float* d0, const void* dkw, const float* dd_T, void* dk, void* dbeta, void* dr,
                                float* dd0, void* workspace, size_t workspace_bytes, void* stream /* hipStream_t */);

/*
 * gdr_chunk_bwd_workspace_size -- device scratch that gdr_chunk_bwd needs.
 *
 * Writes to *bytes: the per-chunk records of the forward's workspace (see
 * gdr_chunk_fwd_workspace_size) plus two bf16 d_k x d_v matrices per (sequence,
 * head, chunk), that is B * H * ceil(T / 64) * (R + 4 * d_k * d_v) bytes with the
 * bf16 record size R = 11776 (no gate, scalar gate) or 11776 + 384 * d_k
 * (per-channel gate: the three decayed operands), 0 when T == 0.  Returns
 * gdr_chunk_bwd's descriptor errors; *bytes is 0 on error.
 */
gdr_status gdr_chunk_bwd_workspace_size(const gdr_desc* desc, size_t* bytes);

/*
 * gdr_chunk_bwd -- gradients of the chunk forward (training).
 *
 * For the forward gdr_chunk_fwd(desc, q, k, v, beta, log_a, S0) with output o and
 * final state S_T, returns the gradients of the scalar L = <dO, o> + <dS_T, S_T>
 * with respect to q, k, v, beta, log_a and S0.  The pages print no gradients;
 * these are the reverse-mode derivatives of the recurrence ("Moonshot AI's New
 * Attention Architecture", §2) taken through its chunk form (§3): the states
 * entering each chunk are recomputed in order, the gradients of the states
 * leaving each chunk are carried in reverse order, and then every chunk forms its
 * token gradients independently (the transposes of the forward's products and of
 * its triangular solve).  The forward's outputs are not needed: the call
 * recomputes what it uses from the inputs.
 *
 * Supported: bf16 I/O; GDR_GATE_NONE or GDR_GATE_SCALAR with d_k, d_v in {64, 128},
 * GDR_GATE_CHANNEL (a gate per key channel, "Moonshot AI's New Attention
 * Architecture", §2) with d_k = 128 and d_v in {64, 128}; either gdr_form;
 * fixed-length batches here, packed sequences through gdr_chunk_bwd_varlen.
 * Anything else returns GDR_ERR_UNSUPPORTED.
 *
 *   q, k, v, beta, log_a, S0   the forward's inputs, as for gdr_chunk_fwd (log_a
 *                              NULL for GDR_GATE_NONE; S0 NULL = zero state)
 *   dO     [B, T, H, d_v] bf16  gradient of o
 *   dS_T   [B, H, d_k, d_v] fp32 gradient of S_T, or NULL (zero)
 *   dq, dk [B, T, H, d_k] bf16  written
 *   dv     [B, T, H, d_v] bf16  written
 *   dbeta  [B, T, H]      bf16  written
 *   dlog_a [B, T, H] (GDR_GATE_SCALAR) or [B, T, H, d_k] (GDR_GATE_CHANNEL) bf16
 *          written; must be NULL for GDR_GATE_NONE
 *   dS0    [B, H, d_k, d_v] fp32 written, or NULL (not computed); may equal dS_T
 *          (overwritten in place), no other alias is allowed
 *   workspace / workspace_bytes  scratch of at least gdr_chunk_bwd_workspace_size
 *          bytes, 16-byte aligned, overwritten
 *
 * Precision: bf16 products with fp32 accumulation, the carried state and state
 * gradient in fp32 (stored per chunk in bf16, the precision the products read
 * them in); reductions over tokens (dbeta, dlog_a) in fp32.  With a per-channel
 * gate the per-chunk gradient sums split each decay at 16-token blocks with one
 * factor of up to 16 tokens' decay inverted, so the gate must not decay by more
 * than e^-80 within 16 tokens of one channel (the forward has no such bound);
 * past it that chunk's gradients are not finite.
 * T == 0 writes dS0 =
 * dS_T (or zeros).  Errors as for gdr_chunk_fwd; besides, one sequence's chunk
 * states must stay below 2^31 bytes (ceil(T / 64) * d_k * d_v * 2).
 */
gdr_status gdr_chunk_bwd(const gdr_desc* desc, const void* q, const void* k, const void* v, const void* beta,
                         const void* log_a, const float* S0, const void* dO, const float* dS_T, void* dq, void* dk,
                         void* dv, void* dbeta, void* dlog_a, float* dS0, void* workspace, size_t workspace_bytes,
                         void* stream /* hipStream_t */);

/*
 * gdr_chunk_bwd_wkey -- gradients of gdr_chunk_fwd_wkey (training the
 * preconditioned delta rule).
 *
 * For the forward gdr_chunk_fwd_wkey(desc, q, k, kw, v, beta, log_a, S0) -- the
 * erase reads the state along k and the write goes along the separate write key
 * kw ("OSDN: Improving Delta Rule with Provable Online Preconditioning in Linear
 * Attention", §2.1) -- returns the gradients of L = <dO, o> + <dS_T, S_T> with
 * respect to q, k, kw, v, beta, log_a and S0, the reverse mode of that recurrence
 * through its chunk form (the column side of the Gram and score matrices, the
 * state write and its gradient take kw; the residual and the rows of the Gram
 * matrix take k).  dk is the gradient through the read side only and dkw the one
 * through the write side; with kw == k their sum is gdr_chunk_bwd's dk.
 *
 * Supported: bf16 I/O; GDR_GATE_NONE or GDR_GATE_SCALAR with d_k, d_v in {64, 128};
 * either gdr_form; fixed-length batches.  GDR_GATE_CHANNEL returns
 * GDR_ERR_UNSUPPORTED.
 *
 *   kw     [B, T, H, d_k] bf16  the write key (non-NULL when T > 0)
 *   dkw    [B, T, H, d_k] bf16  written (non-NULL when T > 0)
 *   every other argument as for gdr_chunk_bwd; the workspace is that of
 *   gdr_chunk_bwd_workspace_size for the same descriptor.
 *
 * Precision and errors as for gdr_chunk_bwd; kw and dkw take part in the alias
 * checks like the other token tensors.
 */
gdr_status gdr_chunk_bwd_wkey(const gdr_desc* desc, const void* q, const void* k, const void* kw, const void* v,
                              const void* beta, const void* log_a, const float* S0, const void* dO, const float* dS_T,
                              void* dq, void* dk, void* dkw, void* dv, void* dbeta, void* dlog_a, float* dS0,
                              void* workspace, size_t workspace_bytes, void* stream /* hipStream_t */);

/*
 * gdr_chunk_bwd_varlen_wkey -- gdr_chunk_bwd_wkey over variable-length sequences
 * packed along T (training the preconditioned rule on packed sequences).
 *
 * The gradients of gdr_chunk_fwd_varlen_wkey's forward; every argument as for
 * gdr_chunk_bwd_varlen, plus kw and dkw ([1, T, H, d_k] bf16) as for
 * gdr_chunk_bwd_wkey.  Supported, precision and errors as for both calls.
 */
gdr_status gdr_chunk_bwd_varlen_wkey(const gdr_desc* desc, const int32_t* cu_seqlens, int64_t n_seq, const void* q,
                                     const void* k, const void* kw, const void* v, const void* beta,
                                     const void* log_a, const float* S0, const void* dO, const float* dS_T, void* dq,
                                     void* dk, void* dkw, void* dv, void* dbeta, void* dlog_a, float* dS0,
                                     void* workspace, size_t workspace_bytes, void* stream /* hipStream_t */);

/*
 * gdr_chunk_bwd_varlen_workspace_size -- scratch for gdr_chunk_bwd_varlen.
 *
 * The records of gdr_chunk_fwd_varlen (H * (ceil(T / 64) + n_seq) slots of R
 * bytes, R as under gdr_chunk_bwd_workspace_size) plus two bf16 d_k x d_v matrices
 * per slot (0 when T == 0).  Returns the
 * descriptor and n_seq errors of gdr_chunk_bwd_varlen; *bytes is 0 on error.
 */
gdr_status gdr_chunk_bwd_varlen_workspace_size(const gdr_desc* desc, int64_t n_seq, size_t* bytes);

/*
 * gdr_chunk_bwd_varlen -- gdr_chunk_bwd over variable-length sequences packed
 * along T (training with packed sequences).
 *
 * The gradients of L = <dO, o> + <dS_T, S_T> for the forward
 * gdr_chunk_fwd_varlen(desc, cu_seqlens, n_seq, q, k, v, beta, log_a, S0): sequence
 * i is tokens cu_seqlens[i] .. cu_seqlens[i+1] - 1 of the packed tensors and
 * starts from S0[i]; its gradients are those of that sequence alone.  Layouts as
 * for gdr_chunk_fwd_varlen: desc->B == 1, desc->T the total token count, token
 * tensors [1, T, H, .] (dO, dq, dk, dv like v, q, k; dbeta, dlog_a like beta);
 * S0, dS_T, dS0 [n_seq, H, d_k, d_v] fp32.  cu_seqlens is the device int32 table
 * of gdr_chunk_fwd_varlen, with the same requirements and the same behaviour on
 * a malformed table (no access outside the tensors; results undefined).
 * Supported and precision as for gdr_chunk_bwd; errors as for both calls.
 */
gdr_status gdr_chunk_bwd_varlen(const gdr_desc* desc, const int32_t* cu_seqlens, int64_t n_seq, const void* q,
                                const void* k, const void* v, const void* beta, const void* log_a, const float* S0,
                                const void* dO, const float* dS_T, void* dq, void* dk, void* dv, void* dbeta,
                                void* dlog_a, float* dS0, void* workspace, size_t workspace_bytes,
                                void* stream /* hipStream_t */);

/*
 * gdr_chunk_fwd_save -- the chunk forward of a training step: gdr_chunk_fwd (with
 * cu_seqlens: gdr_chunk_fwd_varlen; with kw: the _wkey forms) that also leaves in
 * its workspace what gdr_chunk_bwd would otherwise recompute, for a later
 * gdr_chunk_bwd_saved.
 *
 * The backward of the chunk form ("Moonshot AI's New Attention Architecture", §3)
 * needs the state entering every chunk and the per-chunk transform (T and the
 * gate factors); the forward forms both on its way.  This call writes them into
 * a workspace laid out as gdr_chunk_bwd's: the transform's records, then the
 * chunk-start states in bf16 (the precision the backward's products read them
 * in), then room the backward uses.  o and S_T are those of gdr_chunk_fwd, bit
 * for bit.
 *
 *   cu_seqlens, n_seq   NULL and 0 for fixed-length batches; else packed
 *                       sequences as for gdr_chunk_fwd_varlen (desc->B == 1)
 *   kw                  NULL, or the write key as for gdr_chunk_fwd_wkey (no
 *                       gate or a scalar gate)
 *   workspace / workspace_bytes  at least gdr_chunk_bwd_workspace_size (packed:
 *                       gdr_chunk_bwd_varlen_workspace_size) bytes, 16-byte
 *                       aligned; written, and to be passed unchanged to
 *                       gdr_chunk_bwd_saved
 *   every other argument as for gdr_chunk_fwd
 *
 * Supported: the configurations of gdr_chunk_bwd (bf16 I/O), with a write key
 * those of gdr_chunk_bwd_wkey; else GDR_ERR_UNSUPPORTED.  Errors as for
 * gdr_chunk_fwd (GDR_ERR_WORKSPACE for a missing or short workspace), and
 * GDR_ERR_INVALID_ARG for n_seq != 0 without cu_seqlens.
 */
gdr_status gdr_chunk_fwd_save(const gdr_desc* desc, const int32_t* cu_seqlens, int64_t n_seq, const void* q,
                              const void* k, const void* kw, const void* v, const void* beta, const void* log_a,
                              const float* S0, void* o, float* S_T, void* workspace, size_t workspace_bytes,
                              void* stream /* hipStream_t */);

/*
 * gdr_chunk_bwd_saved -- gdr_chunk_bwd (with cu_seqlens: _varlen; with kw and dkw:
 * _wkey) that takes the transform's records and the chunk-start states from the
 * workspace of an earlier gdr_chunk_fwd_save instead of recomputing them, so
 * only the reverse pass over the chunks and the per-chunk gradients run.
 *
 * The descriptor, cu_seqlens, n_seq, q, k, kw, v, beta and log_a must be those of
 * that gdr_chunk_fwd_save call, unchanged since, and the workspace must hold what
 * it wrote (no check is possible: otherwise the gradients are undefined, and no
 * access leaves the buffers).  S0 is not read (its chunk-start state is in the
 * workspace) and may be NULL.  The workspace is overwritten past the records and
 * the states only, so one saved forward can serve several backward calls.  kw and dkw: both NULL, or both given (dk is then the read side's
 * gradient, as for gdr_chunk_bwd_wkey).  Outputs, precision, supported
 * configurations and errors as for gdr_chunk_bwd and its _varlen and _wkey forms.
 */
gdr_status gdr_chunk_bwd_saved(const gdr_desc* desc, const int32_t* cu_seqlens, int64_t n_seq, const void* q,
                               const void* k, const void* kw, const void* v, const void* beta, const void* log_a,
                               const float* S0, const void* dO, const float* dS_T, void* dq, void* dk, void* dkw,
                               void* dv, void* dbeta, void* dlog_a, float* dS0, void* workspace,
                               size_t workspace_bytes, void* stream /* hipStream_t */);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H_ */
