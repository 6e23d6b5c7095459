/*
 * gdn.h -- C ABI of the MI355X (gfx950) Gated DeltaNet mixer: prologue, forward,
 * decode, verify and backward.
 *
 * The operation (Atomic-GDN2 model card, section 2.1 "Gated DeltaNet-2"), for
 * every batch row b and head h independently, token by token:
 *
 *   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *   o_t = S_t^T q_t                              (read after the write)
 *   alpha_t = exp(g_t)
 *
 * S_t is a K x V fp32 matrix (keys on the rows, values on the columns).  The
 * library receives the log-decay g and exponentiates it itself (same section).
 * g is either one value per head-token (GDN_GATE_HEAD: the scalar retention
 * gate) or one value per key channel (GDN_GATE_CHANNEL: the per-key-channel
 * gate of GDN-2 / KDA).  No 1/sqrt(K) scale is applied to q; the caller
 * normalises q and k, applies the sigmoid to beta and the clamp to g.
 *
 * The two entry points are the two execution modes that compute this same
 * mathematics (MindPattern "Gated DeltaNet" page, finding of 2026-07-29):
 * a chunkwise mode for prefill/training and a fused recurrent mode for decode.
 * The recurrent state is the fixed-size fp32 S (the state-memory accounting of
 * "Hybrid layouts: three DeltaNet, one attention", 01 Concept), and the initial
 * state is a first-class input (the S0-tuning finding on the MindPattern page).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers, owned by the caller, contiguous
 *    row-major in the layouts given, aligned to their element size.  The
 *    streamed operands need 16 bytes: q, k, v, o and a per-channel g of
 *    gdn_chunk_fwd, and S of gdn_recurrent_step.  The library allocates nothing
 *    and keeps no state between calls (gdn_chunk_bwd and gdn_chunk_fwd_ws take
 *    a caller-provided workspace).
 *  - q, k, v and o share one storage type (gdn_dtype).  g, beta and every state
 *    tensor are fp32.  Arithmetic is fp32 with fp32 accumulation; for
 *    GDN_BF16 the matrix products take bf16 operands on the MFMA units.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and
 *    the call returns without waiting.  Faults inside a kernel surface at the
 *    caller's next synchronisation of that stream.
 *  - Arguments are checked on the host before anything is enqueued.  A call that
 *    returns an error has enqueued nothing and written nothing.
 *  - Preconditions that are NOT checked per element: g <= 0; for
 *    GDN_GATE_CHANNEL, g in [-5, 0] (the configured domain of the card's
 *    section 2.1); finite inputs.  Outside them results are unspecified.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 7

#if defined(__GNUC__)
#define GDN_API __attribute__((visibility("default")))
#else
#define GDN_API
#endif

typedef enum {
    GDN_OK = 0,
    GDN_EINVAL = 1,   /* null / misaligned / aliasing pointer, negative size, bad enum */
    GDN_ENOTSUP = 2,  /* valid request this build has no kernel for (K, V, chunk) */
    GDN_EHIP = 3      /* the HIP runtime rejected a launch */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;
typedef enum { GDN_GATE_HEAD = 0, GDN_GATE_CHANNEL = 1 } gdn_gate;
typedef enum { GDN_ACT_NONE = 0, GDN_ACT_SILU = 1 } gdn_act;

/*
 * Chunkwise forward over a whole sequence batch.
 *
 *   q, k  [B, T, H, K]   dtype        v  [B, T, H, V]   dtype
 *   g     [B, T, H] (GDN_GATE_HEAD) or [B, T, H, K] (GDN_GATE_CHANNEL), fp32 log-decay
 *   beta  [B, T, H]      fp32
 *   S0    [B, H, K, V]   fp32 initial state, or NULL for zeros
 *   o     [B, T, H, V]   dtype output, or NULL to compute the final state only
 *   S_T   [B, H, K, V]   fp32 final state, or NULL.  May equal S0 (updated in
 *                        place); must not partially overlap any other buffer.
 *
 * K and V: 64 or 128 (GDN_F32: K = 64; fp32 with K = 128 is GDN_ENOTSUP, since one
 * chunk's fp32 operand tiles would not fit the 160 KB of LDS a workgroup may
 * use).  chunk: 64 (tokens per chunk).  64 rows
 * of H * max(K, V) fp32 values must stay below 2^31 bytes (H < 65536 at 128;
 * GDN_ENOTSUP otherwise: the kernels address a chunk with 32-bit offsets).  Any
 * T >= 0: a partial last chunk behaves as if padded with identity tokens
 * (beta = 0, g = 0), whose outputs are not written.  B, T or H equal to 0 is a
 * valid call: with T = 0, S_T receives S0 (or zeros).  At least one of o, S_T
 * must be non-NULL.  o must not alias any input.
 */
GDN_API gdn_status gdn_chunk_fwd(const void *q, const void *k, const void *v,
                         const float *g, const float *beta, const float *S0,
                         void *o, float *S_T,
                         int B, int T, int H, int K, int V, int chunk,
                         gdn_dtype dtype, gdn_gate gate, void *stream);

/*
 * Bytes of device workspace that gdn_chunk_fwd_ws uses for these sizes (written
 * to *bytes); want_o != 0 when o will be requested.  0 means the call runs as
 * gdn_chunk_fwd does and needs no workspace.  Same size and type rules as
 * gdn_chunk_fwd.
 */
GDN_API gdn_status gdn_chunk_fwd_workspace_size(int B, int T, int H, int K, int V, int chunk,
                                                gdn_dtype dtype, gdn_gate gate, int want_o,
                                                size_t *bytes);

/*
 * gdn_chunk_fwd with a caller-provided workspace, which lets a long call run
 * the sequence-parallel form: each (b, h) sequence is cut into segments of
 * whole chunks that run at the same time, every segment after the first
 * reduced to the affine map S -> M S + N it applies to the state (each chunk is
 * such a map and maps compose associatively: the recurrence of the Atomic-GDN2
 * model card, section 2.1, whose kernel benchmark, section 5.1, is against an
 * associative scan of it), and the maps of a sequence are then applied in
 * order to the state from the first segment (fp32).  A call that also writes o
 * keeps the state entering each segment and then runs the chunk kernel on
 * every segment at once from it.  The form is used with bf16 operands,
 * GDN_GATE_CHANNEL and K = V = 128 when B * H is too small to fill the device;
 * with o it also needs S_T non-NULL and not S0 itself (otherwise the call runs
 * sequentially, and the workspace goes unused).  Every other call runs as
 * gdn_chunk_fwd.
 *
 *   arguments as gdn_chunk_fwd, plus
 *   workspace        device memory of at least
 *                    gdn_chunk_fwd_workspace_size(..., o != NULL, ...) bytes,
 *                    256-byte aligned, owned by the caller, not overlapping any
 *                    input or output; may be NULL when that size is 0.  Its
 *                    contents on entry do not matter; on return they are
 *                    unspecified.  Calls sharing one workspace must not run
 *                    concurrently.
 *
 * Results equal gdn_chunk_fwd's to rounding (the segment maps add one fp32
 * product per segment boundary), not bit for bit.  S_T may equal S0.
 */
GDN_API gdn_status gdn_chunk_fwd_ws(const void *q, const void *k, const void *v,
                                    const float *g, const float *beta, const float *S0,
                                    void *o, float *S_T, void *workspace, size_t workspace_bytes,
                                    int B, int T, int H, int K, int V, int chunk,
                                    gdn_dtype dtype, gdn_gate gate, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): gdn_chunk_fwd_ws with
 * the segment maps in a static device buffer that the library owns instead of a
 * caller's workspace.  Arguments as gdn_chunk_fwd; the call runs exactly as
 * gdn_chunk_fwd_ws does with a large enough workspace (same kernels, same
 * segments, the same results bit for bit).
 *
 * The buffer holds GDN_NOALLOC_SCRATCH_BYTES (64 MiB) on every GPU the library
 * runs on, from the module load until the process ends.  A call whose segment
 * maps would need more (gdn_chunk_fwd_workspace_size(..., o != NULL, ...) >
 * GDN_NOALLOC_SCRATCH_BYTES) returns GDN_ENOTSUP and enqueues nothing; use
 * gdn_chunk_fwd_ws for it.  Every call on one GPU shares that GPU's buffer, so
 * calls that overlap on one GPU (concurrent streams, threads) race; each call
 * writes every map it reads, so nothing needs clearing between calls.  The
 * stream must belong to the current device.  No hipMalloc, hipFree or other
 * allocation happens in the call.
 */
#define GDN_NOALLOC_SCRATCH_BYTES (64ull << 20)
GDN_API gdn_status gdn_chunk_fwd_noalloc(const void *q, const void *k, const void *v,
                                         const float *g, const float *beta, const float *S0,
                                         void *o, float *S_T,
                                         int B, int T, int H, int K, int V, int chunk,
                                         gdn_dtype dtype, gdn_gate gate, void *stream);

/*
 * One fused recurrent (decode) step for N sequences, updating S in place.
 *
 *   q, k  [N, H, K]   dtype          v  [N, H, V]   dtype
 *   g     [N, H] or [N, H, K] fp32   beta [N, H]    fp32
 *   S     [N, H, K, V] fp32, read and overwritten with S' (in place)
 *   o     [N, H, V]   dtype output, or NULL
 *
 * K and V: 64 or 128.  N or H equal to 0 is a valid empty call.  Each (n, h)
 * slice is owned by one workgroup, so the in-place update is race-free.
 */
GDN_API gdn_status gdn_recurrent_step(const void *q, const void *k, const void *v,
                              const float *g, const float *beta,
                              float *S, void *o,
                              int N, int H, int K, int V,
                              gdn_dtype dtype, gdn_gate gate, void *stream);

/*
 * Decoupled erase and write gates.  The MindPattern "Gated DeltaNet" page (its
 * finding of 2026-05-22) names a variant that replaces the single scalar beta,
 * which both removes the old association of k and writes the new one, by
 * separate gates; it prints no formula.  These entry points compute the reading
 *
 *   S_t = (I - e_t k_t k_t^T) Diag(alpha_t) S_{t-1} + w_t k_t v_t^T,  o_t = S_t^T q_t
 *
 * with the erase gate e in beta's place in the removal term and the write gate
 * w in its place in the write term; e = w = beta gives the calls above.
 *
 *   erase, write  [B, T, H] (prefill) or [N, H] (decode) fp32, both required
 *                 when there is at least one token; any real values (the
 *                 sigmoid-like range (0, 1) is the caller's choice).
 *
 * Every other argument, layout, check and error is that of gdn_chunk_fwd
 * (prefill: o and S_T outputs, S_T may equal S0) and gdn_recurrent_step
 * (decode: S updated in place); neither output may overlap `write`.  The
 * prefill runs the sequential chunk kernels for every storage type, gate and
 * K (fp32: K = 64), never the sequence-parallel form: bf16 on the
 * warp-specialised kernels, fp32 on the plain chunk kernel.
 */
GDN_API gdn_status gdn_chunk_fwd_decoupled(const void *q, const void *k, const void *v,
                                           const float *g, const float *erase, const float *write,
                                           const float *S0, void *o, float *S_T,
                                           int B, int T, int H, int K, int V, int chunk,
                                           gdn_dtype dtype, gdn_gate gate, void *stream);
GDN_API gdn_status gdn_recurrent_step_decoupled(const void *q, const void *k, const void *v,
                                                const float *g, const float *erase,
                                                const float *write, float *S, void *o,
                                                int N, int H, int K, int V,
                                                gdn_dtype dtype, gdn_gate gate, void *stream);

/*
 * M tokens of each of N sequences, applied in order from one state: the
 * verification step of speculative decoding (M draft tokens scored from the
 * state of the accepted prefix: the chained multi-token-prediction speculative
 * decoding behind the single-card decode figure on the MindPattern "Gated
 * DeltaNet" page, finding of 2026-08-18).  Each token is
 * one step of the recurrence above, computed as gdn_recurrent_step computes it,
 * so M = 1 gives gdn_recurrent_step's results.
 *
 *   q, k    [N, M, H, K]   dtype        v  [N, M, H, V]   dtype
 *   g       [N, M, H] or [N, M, H, K] fp32          beta [N, M, H] fp32
 *   S0      [N, H, K, V]   fp32 state before the first token, or NULL for zeros
 *   o       [N, M, H, V]   dtype output of every token, or NULL
 *   S_T     [N, H, K, V]   fp32 state after the last token, or NULL.  May equal
 *                          S0 (updated in place).
 *   S_hist  [N, M, H, K, V] fp32 state after every token (S_hist[n, j] is the
 *                          state after token j: rolling back to an accepted
 *                          prefix of j + 1 tokens is taking it), or NULL.
 *
 * At least one of o, S_T, S_hist must be non-NULL.  No output may overlap an
 * input or another output (except S_T == S0).  q, k, v, o need their element
 * alignment, g and beta 4 bytes, S0, S_T and S_hist 16 bytes.  K and V: 64 or
 * 128.  N, M or H equal to 0 is a valid call (with M = 0, S_T receives S0).
 * The state is read once and S_T written once whatever M is; S_hist adds M
 * state writes.
 */
GDN_API gdn_status gdn_recurrent_steps(const void *q, const void *k, const void *v,
                               const float *g, const float *beta, const float *S0,
                               void *o, float *S_T, float *S_hist,
                               int N, int M, int H, int K, int V,
                               gdn_dtype dtype, gdn_gate gate, void *stream);

/*
 * Bytes of device workspace that gdn_chunk_bwd needs for these sizes (written
 * to *bytes).  Same argument rules as gdn_chunk_bwd; 0 for an empty problem.
 */
GDN_API gdn_status gdn_chunk_bwd_workspace_size(int B, int T, int H, int K, int V, int chunk,
                                                size_t *bytes);

/*
 * Chunkwise backward: the gradients of a loss L through gdn_chunk_fwd's
 * operation, given dL/do and dL/dS_T (the card's kernel benchmark, section 5.1
 * of the Atomic-GDN2 model card, times forward and backward together; training
 * runs the chunk mode).  Same inputs as the forward; the forward's outputs are
 * not needed (the states are recomputed).
 *
 *   q, k, v, g, beta, S0   as for gdn_chunk_fwd (S0 may be NULL = zeros)
 *   d_o   [B, T, H, V]   dtype    dL/do
 *   dS_T  [B, H, K, V]   fp32     dL/dS_T, or NULL for zeros
 *   dq, dk [B, T, H, K]  dtype    outputs
 *   dv    [B, T, H, V]   dtype    output
 *   dg    shaped as g,   fp32     dL/dg (the log-decay)
 *   dbeta [B, T, H]      fp32
 *   dS0   [B, H, K, V]   fp32     dL/dS0, or NULL if not wanted
 *   workspace            device memory of at least workspace_bytes >=
 *                        gdn_chunk_bwd_workspace_size(...) bytes, 256-byte
 *                        aligned, owned by the caller; its contents on entry
 *                        do not matter and on return are unspecified.
 *
 * K and V: 64 or 128; chunk: 64; dtype GDN_F32 or GDN_BF16 (the arithmetic is
 * fp32 for both).  q, k, v, d_o, a per-channel g, S0 and dS_T need 16-byte
 * alignment, every other pointer its element alignment.  No output may
 * overlap an input, another output or the workspace.  B, T or H equal to 0 is a
 * valid call (T = 0: dS0 receives dS_T, or zeros).  Calls that share one
 * workspace must not run concurrently.  B H ceil(T / 64) must stay below 2^23
 * chunks (one workgroup of up to 512 threads per chunk; GDN_ENOTSUP beyond).
 */
GDN_API gdn_status gdn_chunk_bwd(const void *q, const void *k, const void *v, const float *g,
                                 const float *beta, const float *S0, const void *d_o,
                                 const float *dS_T, void *dq, void *dk, void *dv, float *dg,
                                 float *dbeta, float *dS0, void *workspace,
                                 size_t workspace_bytes, int B, int T, int H, int K, int V,
                                 int chunk, gdn_dtype dtype, gdn_gate gate, void *stream);

/*
 * The prologue: the steps between the layer's projections and the recurrence,
 * for a whole chunk-mode call, in one launch.  Per token:
 *   q, k, v  <- causal depthwise 4-tap convolution over time, per channel (the
 *               kernel-4 convolution of the DeltaNet layers: "Hybrid layouts:
 *               three DeltaNet, one attention", 01 Concept): channel c of token
 *               t is sum_j w[c][j] * raw[t - 3 + j][c], the tokens before the
 *               sequence taken from the carried state
 *            <- SiLU if act == GDN_ACT_SILU
 *   q, k     <- divided by max(L2 norm over the K channels of the head, 1e-12)
 *   g        <- -min(softplus(g_raw), g_cap)  (g_cap = 5 on the Atomic-GDN2
 *   beta     <- sigmoid(b_raw)                 card, section 2.1)
 * so that the outputs feed gdn_chunk_fwd / gdn_chunk_bwd directly.
 *
 *   q_raw, k_raw [B, T, H, K]  dtype      v_raw [B, T, H, V]  dtype
 *   g_raw   shaped as g of gdn_chunk_fwd, fp32      b_raw [B, T, H] fp32
 *   w_q, w_k [H*K, 4] fp32, w_v [H*V, 4] fp32: the taps of channel c = h*K + x
 *   cs_q, cs_k [B, 3, H*K], cs_v [B, 3, H*V]  dtype: the raw inputs of the three
 *           tokens before the sequence (row j = token j - 3), or NULL for zeros
 *   q, k, v, g, beta   outputs in the layouts of gdn_chunk_fwd's inputs
 *   cs_*_out  the raw inputs of the last three tokens (older rows from cs_* when
 *           T < 3), or NULL.  Each may be its own input exactly (updated in place).
 *
 * K and V: 64 or 128.  g_cap > 0 (+inf: no cap); with GDN_GATE_CHANNEL at most 5
 * (GDN_ENOTSUP otherwise: the per-channel chunk kernels that take these outputs
 * need g >= -5).  q_raw, k_raw, v_raw, q, k, v,
 * the taps, the carried states and a per-channel g_raw / g need 16-byte
 * alignment; b_raw, beta and a scalar g 4 bytes.  No output may overlap an input
 * or another output, except a state output that is its own input.  B, T or H
 * equal to 0 is a valid call (with T = 0 the states pass through).
 */
GDN_API gdn_status gdn_prologue(const void *q_raw, const void *k_raw, const void *v_raw,
                                const float *g_raw, const float *b_raw, const float *w_q,
                                const float *w_k, const float *w_v, const void *cs_q,
                                const void *cs_k, const void *cs_v, void *q, void *k, void *v,
                                float *g, float *beta, void *cs_q_out, void *cs_k_out,
                                void *cs_v_out, int B, int T, int H, int K, int V, float g_cap,
                                gdn_act act, gdn_dtype dtype, gdn_gate gate, void *stream);

/*
 * The prologue and the chunkwise forward in one launch: the raw projections in,
 * o and S_T out, with the transformed q, k, v, g and beta never written to HBM
 * (the chunk kernel applies the prologue of gdn_prologue in its load stage, to
 * each chunk's rows and the three raw rows before them).  Results are those of
 * gdn_prologue followed by gdn_chunk_fwd, up to the rounding order of the
 * convolution and the norm.
 *
 *   q_raw .. w_v, cs_q .. cs_v, g_cap, act  as gdn_prologue
 *   cs_*_out  the carried states after the sequence as gdn_prologue writes them,
 *             or NULL; here never the incoming state (EINVAL if any overlap)
 *   S0, o, S_T, B .. chunk, dtype, gate      as gdn_chunk_fwd
 *
 * Checks and errors are those of gdn_chunk_fwd (with q_raw .. b_raw in the
 * places of q .. beta) and of gdn_prologue.  The call takes the chunk kernel of
 * gdn_chunk_fwd_decoupled for every storage type, gate and K (fp32: K = 64).
 */
GDN_API gdn_status gdn_chunk_fwd_prologue(const void *q_raw, const void *k_raw, const void *v_raw,
                                          const float *g_raw, const float *b_raw,
                                          const float *w_q, const float *w_k, const float *w_v,
                                          const void *cs_q, const void *cs_k, const void *cs_v,
                                          void *cs_q_out, void *cs_k_out, void *cs_v_out,
                                          const float *S0, void *o, float *S_T,
                                          int B, int T, int H, int K, int V, int chunk,
                                          float g_cap, gdn_act act, gdn_dtype dtype,
                                          gdn_gate gate, void *stream);

/*
 * One decode token of N sequences from the raw projections: the prologue above
 * and gdn_recurrent_step in one kernel (S updated in place, o written).
 *
 *   q_raw, k_raw [N, H, K], v_raw [N, H, V] dtype; g_raw [N, H] or [N, H, K] and
 *   b_raw [N, H] fp32; w_* as for gdn_prologue; cs_* [N, 3, H*K] / [N, 3, H*V]
 *   dtype or NULL (zeros); cs_*_out the states after this token, or NULL.  A
 *   state output must not overlap any state input (the value blocks of a head
 *   all read the incoming q/k state): keep two state buffers and alternate.
 *   S [N, H, K, V] fp32 in place; o [N, H, V] dtype or NULL.
 *
 * K and V: 64 or 128.  The taps and S need 16-byte alignment, every other
 * pointer its element alignment.
 */
GDN_API gdn_status gdn_recurrent_step_prologue(const void *q_raw, const void *k_raw,
                                               const void *v_raw, const float *g_raw,
                                               const float *b_raw, const float *w_q,
                                               const float *w_k, const float *w_v,
                                               const void *cs_q, const void *cs_k,
                                               const void *cs_v, void *cs_q_out, void *cs_k_out,
                                               void *cs_v_out, float *S, void *o, int N, int H,
                                               int K, int V, float g_cap, gdn_act act,
                                               gdn_dtype dtype, gdn_gate gate, void *stream);

/* Static English text for a status code (never NULL). */
GDN_API const char *gdn_status_str(gdn_status s);

/* GDN_ABI_VERSION of the library that is loaded. */
GDN_API int gdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
