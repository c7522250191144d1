/*
 * glahybrid.h -- C ABI of the MI355X (gfx950) hybrid gated-linear + sliding-window
 * attention library.
 *
 * The layer is the hybrid attention of Lizard ("Lizard" technical summary,
 * gist.science paper 2507.09025, Methodology section A; Lizard abstract on
 * chatpaper.ai):
 *
 *   gated linear attention (Methodology A.1):
 *     phi(x)  = [softmax(x Wphi), softmax(-x Wphi)]     Hedgehog map, non-negative
 *                                                        (Methodology C)
 *     Gamma_t = sigmoid(g_t)        g_t = W_gamma x_t, supplied by the caller
 *     S_t     = diag(Gamma_t) S_{t-1} + phi(k_t)^T v_t   f x d_v state, fp32
 *     o_gla,t = phi(q_t) S_t
 *   sliding-window attention with meta-memory sinks (Methodology A.2):
 *     s_tj    = scale * q_t . k_j      for j in [t-w+1, t]
 *     o_swa,t = sum_j e^{s_tj} v_j / (sum_j e^{s_tj} + sum_m e^{t_m})
 *   hybrid:  o_t = o_gla,t + o_swa,t
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers (hipMalloc / torch CUDA memory) unless
 *    stated otherwise; the caller owns every buffer.  The library never allocates
 *    or frees memory and never synchronises the stream.
 *  - All tensors are dense, C-contiguous, row-major:
 *      q, k            [B][H][L][d_qk]        (decode: [B][H][d_qk])
 *      v, o            [B][H][L][d_v]         (decode: [B][H][d_v])
 *      gate            [B][H][L][f]           (decode: [B][H][f])
 *      wphi_q, wphi_k  [H][d_qk][f/2]         Hedgehog projections, per head
 *      meta            [H][n_meta]            fp32 sink logits t_m
 *      state           [B][H][f][d_v]         fp32
 *      kcache, vcache  [B][H][window][d_qk|d_v]  ring: token p lives in slot p % window
 *    The element type of q, k, v, gate, wphi_*, o and the caches is desc->dtype;
 *    meta and state are always fp32.  Every pointer must be 16-byte aligned.
 *  - Work is enqueued on `stream` (0 = the null stream) and returns immediately.
 *  - Argument errors are reported synchronously, before anything is launched;
 *    no entry point throws.  GLAH_EHIP means a HIP launch error was reported.
 *  - Outputs must not alias inputs, except state_in == state_out (prefill).
 */
#ifndef GLAHYBRID_H
#define GLAHYBRID_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *glah_stream_t; /* = hipStream_t */

typedef enum {
  GLAH_OK = 0,
  GLAH_EINVAL = 1,     /* null required pointer, bad size, misaligned pointer */
  GLAH_ENOTSUP = 2,    /* valid but unsupported combination of sizes/dtype   */
  GLAH_EWORKSPACE = 3, /* workspace missing or smaller than required         */
  GLAH_EHIP = 4        /* the HIP runtime reported an error                  */
} glah_status;

typedef enum { GLAH_BF16 = 0, GLAH_F32 = 1 } glah_dtype;

/* Gate layouts.  The first two give one gate per feature channel; the last two
 * are the scalar-decay variants (a per-token scalar as in Mamba-2, a fixed
 * per-head decay as in RetNet: "LT2" technical summary, 2.1 architecture
 * variants; "systematic analysis of hybrid linear attention", evaluated models),
 * run through the same kernels as a log-gate broadcast over the features. */
typedef enum {
  GLAH_GATE_LOGITS = 0,    /* gate [B][H][L][f] holds g = W_gamma x; Gamma = sigmoid(g) */
  GLAH_GATE_LOG = 1,       /* gate [B][H][L][f] holds log Gamma <= 0 (-inf allowed)     */
  GLAH_GATE_LOG_TOKEN = 2, /* gate [B][H][L] holds one log Gamma <= 0 per token, the
                              same for every feature (decode: [B][H])                 */
  GLAH_GATE_LOG_HEAD = 3   /* gate [H] holds one fixed log Gamma <= 0 per head, the same
                              for every token and feature (decode: [H])               */
} glah_gate_kind;

typedef struct glah_desc {
  int32_t B, H, L;      /* batch, heads, tokens (L is ignored by the decode step)  */
  int32_t d_qk, d_v, f; /* q/k head dim, value dim, feature dim (f even)            */
  int32_t chunk;        /* token chunk of the chunkwise prefill: 16, 32, 64 or 128;
                           0 = 64.  The result does not depend on it beyond
                           rounding; the bf16 MFMA path (d = f = d_v = 128)
                           blocks at 64 tokens (fold references per 16-token
                           tile) for every value, the other paths are
                           token-recurrent and ignore it                      */
  int32_t window;       /* SWA window w >= 1 (keys including the query's own);
                           gla_decode_step: 0 = no window part                      */
  int32_t n_meta;       /* number of meta-memory sink scalars per head, >= 0        */
  float scale;          /* SWA score scale; <= 0 selects 1/sqrt(d_qk)               */
  int32_t dtype;        /* glah_dtype                                               */
  int32_t gate_kind;    /* glah_gate_kind                                           */
} glah_desc;

/* Human-readable name of a status code (static storage). */
const char *glah_status_str(int status);

/* Library version, (major << 16) | minor. */
int glah_version(void);

/* Bytes of device workspace that gla_prefill / hybrid_layer_fwd need for `desc`
 * on the current device (segment states of the parallel state pass).  0 means
 * none.  Returns (size_t)-1 when `desc` is invalid. */
size_t glah_workspace_bytes(const glah_desc *desc);

/*
 * gla_prefill -- gated linear attention over whole sequences (Methodology A.1 and
 * C): chunkwise-parallel form with the cumulative log-gates folded into phi(q)
 * and phi(k), an fp32 inter-chunk state pass, o = o_gla.
 *   state_in   nullable; [B][H][f][d_v] fp32 state before token 0 (0 if NULL)
 *   state_out  nullable; receives S_{L-1} (L = 0: the state before the sequence,
 *              state_in or zeros); may equal state_in
 *   ws         device workspace of ws_bytes >= glah_workspace_bytes(desc)
 */
glah_status gla_prefill(const glah_desc *desc, const void *q, const void *k,
                        const void *v, const void *gate, const void *wphi_q,
                        const void *wphi_k, const float *state_in,
                        float *state_out, void *o, void *ws, size_t ws_bytes,
                        glah_stream_t stream);

/*
 * swa_meta_attn -- sliding-window softmax attention with meta-memory sinks
 * (Methodology A.2), o = o_swa.  meta is [H][n_meta] fp32 and may be NULL only
 * when n_meta == 0.  Positions start at 0 (no keys before the sequence).
 * bf16 at d_qk = d_v = 128 runs on the matrix cores for any window: one pass
 * over the band for window <= 64, an online softmax over 64-key chunks
 * (started from the sinks) beyond that.
 */
glah_status swa_meta_attn(const glah_desc *desc, const void *q, const void *k,
                          const void *v, const float *meta, void *o,
                          glah_stream_t stream);

/*
 * hybrid_layer_fwd -- the whole hybrid layer in one pass over q, k, v and gate:
 * o = o_gla + o_swa (Lizard abstract: gated linear attention for global context
 * plus meta-memory window attention for local detail).
 *   state_in/state_out  as in gla_prefill (state_in continues the gated part only;
 *                       the window part starts at token 0 of this call)
 *   kcache_out/vcache_out  nullable; receive the ring of the last `window` keys and
 *                       values (slot p % window holds token p; slots of tokens
 *                       before 0 are zero-filled), ready for gla_decode_step
 * bf16 at d_qk = f = d_v = 128: window <= 64 runs both parts in one fused pass;
 * a wider window runs the gated part in the same chunked kernels and then the
 * window part (online softmax over 64-key chunks), which adds its result to o
 * (bf16 o is then rounded twice: at most one more bf16 ulp).  Other sizes and
 * fp32 run the token-recurrent kernels (window <= 4096, n_meta <= 64).
 */
glah_status hybrid_layer_fwd(const glah_desc *desc, const void *q, const void *k,
                             const void *v, const void *gate, const void *wphi_q,
                             const void *wphi_k, const float *meta,
                             const float *state_in, float *state_out,
                             void *kcache_out, void *vcache_out, void *o,
                             void *ws, size_t ws_bytes, glah_stream_t stream);

/*
 * hybrid_layer_fwd_noalloc -- hybrid_layer_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments and results as hybrid_layer_fwd
 * without the workspace: the state pass keeps its segment states in a static
 * device array of the library, GLAH_NOALLOC_SCRATCH_BYTES on every device the
 * library runs on, held until the process ends.  The call allocates and frees
 * nothing (the array's address is looked up once per device, on the first call
 * with that device current).
 *   - A call whose segment states need more than GLAH_NOALLOC_SCRATCH_BYTES
 *     returns GLAH_EWORKSPACE before launching anything (the need is
 *     glah_workspace_bytes(desc); on a 256-CU MI355X it is at most about 34 MB
 *     for any size, since the plan cuts the sequences into at most two slices
 *     per compute unit).
 *   - Every call on one device shares the array and leaves it holding that
 *     call's segment states; nothing in it has to start at zero.  Calls that
 *     overlap on one device (concurrent streams, or host threads enqueueing on
 *     different streams) race on it: order them on one stream or with events.
 */
#define GLAH_NOALLOC_SCRATCH_BYTES ((size_t)40 << 20)
glah_status hybrid_layer_fwd_noalloc(const glah_desc *desc, const void *q, const void *k,
                                     const void *v, const void *gate, const void *wphi_q,
                                     const void *wphi_k, const float *meta,
                                     const float *state_in, float *state_out,
                                     void *kcache_out, void *vcache_out, void *o,
                                     glah_stream_t stream);

/*
 * gla_decode_step -- one token of constant-memory recurrent inference
 * (Methodology A.1: the state is updated token by token instead of keeping a KV
 * cache; A.2 for the window part).  For every (b, h):
 *   S <- diag(Gamma) S + phi(k_t)^T v_t   in place in `state`
 *   ring slot pos[b] % window <- (k_t, v_t)       (when window > 0)
 *   o_t = phi(q_t) S + window attention over positions [pos-w+1, pos] and sinks
 *   pos     DEVICE int32 [B]: tokens already consumed by sequence b (= the new
 *           token's position); read only, the caller advances it
 *   kcache, vcache  may be NULL only when desc->window == 0
 */
glah_status gla_decode_step(const glah_desc *desc, const void *q_t,
                            const void *k_t, const void *v_t, const void *gate_t,
                            const void *wphi_q, const void *wphi_k,
                            const float *meta, float *state, void *kcache,
                            void *vcache, const int32_t *pos, void *o_t,
                            glah_stream_t stream);

/*
 * hybrid_layer_bwd -- gradient of hybrid_layer_fwd, for training the layer's
 * parameters (the two-stage training of the Lizard summary, Methodology B, fits
 * the gate, the Hedgehog feature maps and the meta-memory scalars; the layer is
 * Methodology A.1, A.2 and C).  For the scalar loss
 *     L = sum o . d_o + sum S_{L-1} . dstate_out
 * it writes dL/dx for every input x of the forward:
 *   dq, dk      [B][H][L][d_qk]   desc->dtype
 *   dv          [B][H][L][d_v]    desc->dtype
 *   dgate       the layout and dtype of `gate` (logits, log-gates, per token or
 *               per head: [H], summed over the batch and every token)
 *   dwphi_q, dwphi_k  [H][d_qk][f/2] fp32, summed over the batch
 *   dmeta       [H][n_meta] fp32 (may be NULL only when n_meta == 0)
 *   dstate_in   nullable, [B][H][f][d_v] fp32: gradient of state_in
 * Inputs are those of the forward call (same descriptor, same tensors), plus
 *   d_o         [B][H][L][d_v] desc->dtype, the gradient of o
 *   dstate_out  nullable, [B][H][f][d_v] fp32, the gradient of the final state
 *               (NULL = zero)
 *   ws          device workspace of ws_bytes bytes, at least the workspace of one
 *               batch row and one head (glah_bwd_workspace_bytes of this
 *               descriptor with B = H = 1; else GLAH_EWORKSPACE).  The gradient
 *               of every (batch row, head) is independent of the others, so a
 *               workspace below the whole call's runs the call as the fewest
 *               sub-problems that fit it (blocks of whole batch rows, else one
 *               row and a block of heads), in order on `stream`, the per-head
 *               sums over the batch added up across them.
 * glah_bwd_workspace_bytes reports the whole call's workspace when it is at
 * most 1.5e9 bytes, else that of the largest sub-problem within that (at 32K
 * tokens, 32 heads of 128: blocks of 16 heads, 1.42 GB; the whole call takes
 * 2.78 GB); (size_t)-1 for an invalid descriptor, 0 when the sizes are not
 * supported.
 * Supported: d_qk, d_v <= 128 and multiples of 4; f <= 128, a multiple of 4 with
 * f/2 a power of two; window <= 1024; n_meta <= 64 (otherwise GLAH_ENOTSUP).
 * Arithmetic: bf16 with d_qk = f = d_v = 128 runs on the matrix cores (bf16
 * operands, split into high and low bf16 halves where the gate gradient needs
 * more, fp32 accumulation; one part's dq, dk, dv are rounded to bf16 before the
 * other's are added to them; log-gates are floored at -10 as in the forward);
 * other sizes and fp32 run token-recurrent fp32 kernels.  With one gate per
 * feature and the window part on the matrix cores (window <= 64), the parts'
 * gradients meet in the output rows: dq, dk, dv are written more than once
 * during the call and hold the gradient only when it has finished.
 * Reductions over tokens and batch rows run in a fixed order, so results are
 * bitwise repeatable for a given ws_bytes.
 * Streams: that path (bf16, d_qk = f = d_v = 128, one gate per feature, window
 * <= 64) runs on `stream` alone.  In the other cases the window part runs
 * on a side stream of the library (one per device, with two events, created on
 * the first such call and kept until the process ends), forked from `stream`
 * at the call and joined back into it before the call's last kernels, so all
 * of the call's work is ordered on `stream` as usual.  When `stream` is being
 * captured into a graph before the side stream exists, the call uses `stream`
 * alone.
 */
size_t glah_bwd_workspace_bytes(const glah_desc *desc);
/* The workspace with which hybrid_layer_bwd runs the whole call at once (no
 * sub-problems; the fastest plan, for callers with the memory to spare);
 * (size_t)-1 for an invalid descriptor, 0 when the sizes are not supported. */
size_t glah_bwd_workspace_bytes_whole(const glah_desc *desc);
glah_status hybrid_layer_bwd(const glah_desc *desc, const void *q, const void *k,
                             const void *v, const void *gate, const void *wphi_q,
                             const void *wphi_k, const float *meta,
                             const float *state_in, const void *d_o,
                             const float *dstate_out, void *dq, void *dk, void *dv,
                             void *dgate, float *dwphi_q, float *dwphi_k,
                             float *dmeta, float *dstate_in, void *ws,
                             size_t ws_bytes, glah_stream_t stream);

/*
 * hybrid_layer_fwd_cont -- hybrid_layer_fwd for sequences that continue: this
 * call's L tokens sit at positions start .. start+L-1 of sequences that have
 * already consumed `start` tokens (the same count for every batch row), as in
 * a prefill cut into pieces or a prompt appended after decoding.  The gated
 * part continues from state_in; the window of the query at position P covers
 * keys [P-window+1, P] (Methodology A.2), those before `start` read from the
 * input ring.  The result equals the matching rows of one hybrid_layer_fwd
 * over the whole sequence.
 *   start       host int32 >= 0
 *   state_in    nullable; [B][H][f][d_v] fp32 state after token start-1
 *   kcache_in, vcache_in  [B][H][window][d] ring after token start-1 (slot p %
 *               window holds token p, as hybrid_layer_fwd and gla_decode_step
 *               leave it); may be NULL only when start == 0
 *   kcache_out, vcache_out  nullable; the ring after this call (same layout,
 *               global positions); may be the same buffers as the input ring
 *   other arguments as hybrid_layer_fwd
 * Supported: window <= 64 and n_meta <= 64 (else GLAH_ENOTSUP).  The first
 * window-1 queries get their window term corrected in fp32 after the layer
 * kernels (the difference between the softmax over ring and call keys and the
 * one over call keys alone), so for bf16 output they are rounded twice.
 */
glah_status hybrid_layer_fwd_cont(const glah_desc *desc, int32_t start,
                                  const void *q, const void *k, const void *v,
                                  const void *gate, const void *wphi_q,
                                  const void *wphi_k, const float *meta,
                                  const float *state_in, const void *kcache_in,
                                  const void *vcache_in, float *state_out,
                                  void *kcache_out, void *vcache_out, void *o,
                                  void *ws, size_t ws_bytes,
                                  glah_stream_t stream);

/*
 * glah_output_gate -- output-gate epilogue o <- o * sigmoid(g), elementwise, in
 * place (the attention-output gate of the "LT2" technical summary, 2605.20670,
 * contributions: it keeps activations from growing across loop iterations).
 *   o, g        [B][H][L][d_v], desc->dtype; g holds the gate logits (W_o x)
 * Reads B, H, L, d_v and dtype of the descriptor.
 */
glah_status glah_output_gate(const glah_desc *desc, void *o, const void *g,
                             glah_stream_t stream);

/*
 * gdn_prefill -- the gated delta rule (Gated DeltaNet), the token mixer that
 * "systematic analysis of hybrid linear attention" (2507.06457, findings and
 * recommendations) and the "LT2" summary (2605.20670, hybrid designs) pair
 * with attention: an error-correcting write into the state with gated
 * forgetting.  The pages give it in words only; this is the published
 * recurrence, per (b, h), with the state M kept as d_v rows of d_qk:
 *     k^ = k_t / sqrt(|k_t|^2 + 1e-6),  q^ = q_t / sqrt(|q_t|^2 + 1e-6)
 *     M_t = alpha_t M_{t-1} (I - beta_t k^ k^T) + beta_t v_t k^T,  alpha_t = e^{a_t}
 *     o_t = M_t q^
 *   q, k        [B][H][L][d_qk]  desc->dtype
 *   v, o        [B][H][L][d_v]   desc->dtype
 *   log_alpha   [B][H][L]        desc->dtype, a_t <= 0 (-inf allowed: alpha = 0)
 *   beta        [B][H][L]        desc->dtype, write strength in [0, 1]
 *   state_in    nullable; [B][H][d_v][d_qk] fp32 state before token 0 (0 if NULL)
 *   state_out   nullable; [B][H][d_v][d_qk] fp32, receives M_{L-1} (L = 0: the
 *               state before the sequence); may equal state_in
 *   ws          device workspace of ws_bytes >= gdn_workspace_bytes(desc)
 *               (may be NULL when that is 0), owned by the caller; the call
 *               overwrites it
 * Reads B, H, L, d_qk, d_v and dtype of the descriptor; the other fields are
 * ignored.  Supported: d_qk in {32, 64, 128}, any d_v >= 1 (else
 * GLAH_ENOTSUP); GLAH_EWORKSPACE when ws is missing or too small.  bf16 with
 * d_qk = 128, d_v a multiple of 16 and L >= 64 runs the chunkwise form on the
 * matrix cores (bf16 operands, fp32 accumulation and state); every other case
 * the token-recurrent fp32 form.  Both are bitwise repeatable.
 */
glah_status gdn_prefill(const glah_desc *desc, const void *q, const void *k,
                        const void *v, const void *log_alpha, const void *beta,
                        const float *state_in, float *state_out, void *o,
                        void *ws, size_t ws_bytes, glah_stream_t stream);

/* Bytes of device workspace gdn_prefill needs for `desc`: per 64-token chunk
 * of every (b, h), 13568 bytes on the chunkwise path; 0 on the
 * token-recurrent one.  Returns (size_t)-1 when `desc` is invalid. */
size_t gdn_workspace_bytes(const glah_desc *desc);

/*
 * gdn_decode_step -- one token of the gated delta rule for every (b, h): the
 * same update as gdn_prefill with L = 1, the state updated in place.
 *   q_t, k_t    [B][H][d_qk]; v_t, o_t [B][H][d_v]; log_alpha_t, beta_t [B][H]
 *   state       [B][H][d_v][d_qk] fp32, in/out
 */
glah_status gdn_decode_step(const glah_desc *desc, const void *q_t,
                            const void *k_t, const void *v_t,
                            const void *log_alpha_t, const void *beta_t,
                            float *state, void *o_t, glah_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* GLAHYBRID_H */
