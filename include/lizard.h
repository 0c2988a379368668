/*
 * lizard.h -- C ABI of the MI355X (gfx950) hybrid-attention library.
 *
 * The hybrid layer (source: "Lizard: An Efficient Linearization Framework for
 * Large Language Models", gist.science technical summary, section 2(a) "Hybrid
 * attention architecture") adds two branches that read the same q, k, v:
 *
 *   GLA branch    S_t = diag(alpha_t) S_{t-1} + k_t^T v_t,   o_gla,t = q_t S_t
 *                 (the section's constant-memory state update; phi is applied
 *                 by the caller, alpha_t = exp(log_alpha_t) per key channel)
 *   window branch one softmax over the keys j in [t-w+1, t] and M meta-memory
 *                 key/value slots (the section's anchor window whose learnable
 *                 meta tokens sit in the softmax denominator)
 *   combine       o_t = o_gla,t + mix * o_swa,t   (the section's weighted sum;
 *                 the page calls the weight alpha, here it is `mix`)
 *
 * Section 2(c) "Hardware-aware algorithm" of the same page absorbs the
 * cumulative gate into q and k in log space so that the chunk work is a plain
 * matrix product.  The kernels behind this ABI do that per 64-token chunk with
 * bf16 matrix-core products and fp32 log-space gates.
 *
 * Conventions for every entry point
 *   - Tensors are dense, row-major, device memory owned by the caller:
 *       q, k        [B, H, T, dk]      dtype of desc->dtype
 *       v, o        [B, H, T, dv]      dtype of desc->dtype
 *       gate        [B, H, T, dk]      the per-channel decay, as desc->gate says:
 *                                      LIZARD_GATE_LOG_ALPHA: float32 log alpha,
 *                                      finite, <= 0;  LIZARD_GATE_LOGIT: bf16
 *                                      logits x, alpha = sigmoid(x) (the
 *                                      section's learnable sigmoid gate), half
 *                                      the bytes, log-sigmoid taken in-kernel.
 *                                      A log alpha below -15 ln 2 (alpha <
 *                                      2^-15, a state all but reset at that
 *                                      token) is taken as -15 ln 2 in every
 *                                      entry point: the gated operands stay
 *                                      inside the fp32/bf16 exponent range, and
 *                                      the older state then enters with a
 *                                      weight of at most 2^-15 instead of
 *                                      alpha; for such a token the gate
 *                                      gradient is taken at the floored value
 *                                      and passed through the floor unchanged
 *                                      (not zeroed)
 *       meta_k      [H, M, dk]         dtype of desc->dtype (shared by the batch)
 *       meta_v      [H, M, dv]         dtype of desc->dtype
 *       state/h0/hT [B, H, dk, dv]     float32 (row = key channel)
 *       ring_k      [B, H, w, dk]      dtype; slot p mod w holds token p
 *       ring_v      [B, H, w, dv]      dtype
 *       lse         [B, H, T]          float32, natural-log sum of exp of the logits
 *   - The library never allocates, frees or keeps a pointer after a call returns.
 *     Scratch memory comes from the caller through (ws, ws_bytes); size it with
 *     lizard_workspace_bytes.
 *   - Work is enqueued asynchronously on `stream` (NULL = the default stream).
 *     There is no global mutable state: calls on different streams may overlap
 *     as long as their buffers do not.  Results are deterministic (no float
 *     atomics; fixed reduction orders).
 *   - Arguments are checked on the host before anything is enqueued; a failed
 *     check returns a non-zero status and enqueues nothing.  A launch failure
 *     returns LIZARD_E_HIP.  NaN/Inf inputs propagate to the outputs.
 *   - With LIZARD_SYNC_DEBUG=1 in the environment (read once per process),
 *     every call waits for its work on `stream` to finish and returns
 *     LIZARD_E_HIP if that work failed, so an asynchronous fault is reported
 *     by the call that caused it (for debugging; it serialises the stream).
 *   - Supported in this version: dk == dv, dk in {64, 128}, chunk == 64,
 *     window >= 1, 0 <= M <= 16, T >= 0 with T*dk*4 < 2^31, B*H <= 65535;
 *     dtype BF16 or F32 for dk in {64, 128}.  Output gradients dq, dk, dv use
 *     desc->dtype; every other output is float32.
 */
#ifndef LIZARD_H
#define LIZARD_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LIZARD_OK = 0,
  LIZARD_E_NULL = 1,        /* a required pointer is NULL                         */
  LIZARD_E_SHAPE = 2,       /* a size is negative, zero where it must not be, or inconsistent */
  LIZARD_E_DTYPE = 3,       /* unknown dtype code                                 */
  LIZARD_E_UNSUPPORTED = 4, /* valid but not built (e.g. dk = 96)                   */
  LIZARD_E_WORKSPACE = 5,   /* ws_bytes smaller than lizard_workspace_bytes()     */
  LIZARD_E_HIP = 6,         /* a HIP launch or query failed                       */
  LIZARD_E_SCRATCH = 7      /* needs more scratch than LIZARD_STATIC_SCRATCH_BYTES */
} lizard_status_t;

typedef enum { LIZARD_F32 = 0, LIZARD_BF16 = 1 } lizard_dtype_t;

/* Format of the gate input (desc->gate). */
typedef enum { LIZARD_GATE_LOG_ALPHA = 0, LIZARD_GATE_LOGIT = 1 } lizard_gate_t;

typedef enum {
  LIZARD_OP_GLA_FWD = 0,
  LIZARD_OP_SWA_FWD = 1,
  LIZARD_OP_HYBRID_FWD = 2,
  LIZARD_OP_HYBRID_BWD = 3,
  LIZARD_OP_DECODE = 4
} lizard_op_t;

/* Problem description shared by every call. */
typedef struct {
  int32_t B, H, T;   /* batch, heads, sequence length (T ignored by decode)          */
  int32_t dk, dv;    /* key/query and value head sizes                               */
  int32_t chunk;     /* GLA chunk length; must be 64                                 */
  int32_t window;    /* w: keys t-w+1 .. t are visible to query t (w >= 1)            */
  int32_t n_meta;    /* M: always-visible meta-memory slots (0..16)                   */
  float scale;       /* softmax logit scale; <= 0 selects 1/sqrt(dk)                 */
  float mix;         /* weight of the window branch in the combine                   */
  int32_t dtype;     /* lizard_dtype_t of q, k, v, o, meta, ring, dq, dk, dv          */
  int32_t gate;      /* lizard_gate_t of the gate input; LIZARD_GATE_LOGIT needs BF16 */
} lizard_desc_t;

/* Bytes of scratch memory `op` needs for `desc` (0 if none).  Never fails: an
 * invalid desc yields 0, and the call itself then reports the problem.
 * LIZARD_OP_GLA_FWD / LIZARD_OP_HYBRID_FWD: per-segment GLA states, at most
 * 15 * B*H * (dk*dv + dk) * 4 bytes and independent of T once T >= 1024.
 * LIZARD_OP_HYBRID_BWD: 64 chunk states per head in the element type plus one
 * fp32 state per head, and per-segment meta-gradient partials; it does not
 * depend on T at all (the backward walks a sequence in blocks of 2048 tokens).
 * The workspace holds no state between calls. */
size_t lizard_workspace_bytes(const lizard_desc_t* desc, int32_t op);

/* Chunked gated linear attention forward (GLA branch alone): the gated state
 * update of "Lizard: An Efficient Linearization Framework for Large Language
 * Models" (gist.science summary, section 2(a)), computed chunk by chunk with the
 * log-space gate absorption of its section 2(c):
 *   o_t = q_t S_t with S_t = diag(exp(log_alpha_t)) S_{t-1} + k_t^T v_t, S_{-1} = h0.
 * h0 (nullable, NULL = zeros) is read; o is written; hT (nullable) receives S_{T-1}
 * (h0, or zeros, when T == 0).  ws must hold lizard_workspace_bytes(desc,
 * LIZARD_OP_GLA_FWD) bytes (it may be NULL when that is 0). */
lizard_status_t lizard_gla_fwd(const lizard_desc_t* desc, const void* q, const void* k,
                               const void* v, const void* gate, const float* h0,
                               void* o, float* hT, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/* Sliding-window + meta-memory softmax attention forward (window branch alone):
 * the anchor window of "Lizard: An Efficient Linearization Framework for Large
 * Language Models" (gist.science summary, section 2(a)), one softmax over the
 * keys t-w+1 .. t and the M learnable meta-memory slots (which the section puts
 * in the softmax denominator), scaled by desc->scale.  o receives o_swa (no mix
 * applied); lse (nullable) receives the natural log-sum-exp of each query's
 * logits.  Needs no workspace. */
lizard_status_t lizard_swa_fwd(const lizard_desc_t* desc, const void* q, const void* k,
                               const void* v, const void* meta_k, const void* meta_v,
                               void* o, float* lse, hipStream_t stream);

/* Hybrid forward: o = o_gla + mix * o_swa.  Optional outputs (each nullable):
 * lse and o_swa (needed by lizard_hybrid_bwd), hT = final GLA state, and the
 * window cache ring_k/ring_v for a prefill -> decode handoff (slot p mod w holds
 * token p for the last min(T, w) tokens; slots no token reached are zeroed).
 * q_w, k_w [B,H,T,dk] (desc->dtype; both NULL, or both given, else
 * LIZARD_E_NULL): the window branch's own queries and keys, for models whose
 * gated branch reads feature-mapped q, k ("Lizard: An Efficient Linearization
 * Framework for Large Language Models", gist.science summary, section 2(a));
 * NULL means the window branch reads q, k.  The window cache holds k_w.
 * ws must hold lizard_workspace_bytes(desc, LIZARD_OP_HYBRID_FWD) bytes. */
lizard_status_t lizard_hybrid_fwd(const lizard_desc_t* desc, const void* q, const void* k,
                                  const void* v, const void* gate, const void* meta_k,
                                  const void* meta_v, const float* h0, void* o, float* lse,
                                  void* o_swa, float* hT, void* ring_k, void* ring_v,
                                  const void* q_w, const void* k_w, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/* Hybrid forward over a packed batch of sequences of different lengths (serving
 * prefill).  q, k, v, gate, o (and q_w, k_w) are [H, n_tokens, d]: sequence b
 * holds tokens cu_seqlens[b] .. cu_seqlens[b+1]-1 of every head.  cu_seqlens is
 * a device array of B+1 int32 with 0 = cu[0] <= cu[1] <= ... <= cu[B] =
 * n_tokens, and desc->T must be at least the longest length (it sizes the
 * work split and the workspace); the kernels clamp entries into [0, n_tokens]
 * and lengths to desc->T.  h0, hT [B,H,dk,dv] and ring_k/ring_v [B,H,w,d] are
 * per sequence, as in lizard_hybrid_fwd, so lizard_decode_step continues
 * every sequence from pos[b] = its length.  Each sequence's outputs equal those
 * of lizard_hybrid_fwd on that sequence alone (the state of "Lizard: An
 * Efficient Linearization Framework for Large Language Models", gist.science
 * summary, section 2(a), starts from h0 at each sequence's first token, and no
 * window reaches into another sequence).  Inference outputs only (no lse,
 * o_swa); BF16 and F32, desc->T >= 1 (else LIZARD_E_UNSUPPORTED).  ws must
 * hold lizard_workspace_bytes(desc, LIZARD_OP_HYBRID_FWD) bytes. */
lizard_status_t lizard_hybrid_fwd_varlen(const lizard_desc_t* desc, const int32_t* cu_seqlens,
                                         int32_t n_tokens, const void* q, const void* k,
                                         const void* v, const void* gate, const void* meta_k,
                                         const void* meta_v, const float* h0, void* o, float* hT,
                                         void* ring_k, void* ring_v, const void* q_w,
                                         const void* k_w, void* ws, size_t ws_bytes,
                                         hipStream_t stream);

/* Hybrid backward for the loss sum(dO * o) + sum(dhT * hT).  Reads the forward
 * inputs plus the o_swa and lse that lizard_hybrid_fwd saved.  Writes dq, dk, dv
 * (desc->dtype), dgate [B,H,T,dk] (the gradient with respect to the gate input:
 * d log_alpha, or d x = d log_alpha * sigmoid(-x) for logits), dmeta_k [H,M,dk], dmeta_v [H,M,dv] (all
 * float32 except dq/dk/dv).  Every output is fully overwritten.  h0 (nullable) as
 * in the forward.  dhT [B,H,dk,dv] float32 (nullable = zero) is the gradient of
 * the final state hT; dh0 [B,H,dk,dv] float32 (nullable = not written) receives
 * the gradient of the initial state; dmix (one float32, nullable = not written)
 * receives the gradient of the mix weight, sum(dO * o_swa), summed in a fixed
 * order.  A sequence run in segments (hT of one
 * segment as h0 of the next, the window branch given its own inputs) is
 * differentiated by chaining dh0 of a segment into dhT of the one before, the
 * constant-size state of "Lizard: An Efficient Linearization Framework for Large
 * Language Models" (gist.science summary, sections 2(a) and 4).  ws must hold
 * lizard_workspace_bytes(desc, LIZARD_OP_HYBRID_BWD) bytes, which do not grow
 * with T: the gated branch is differentiated in blocks of 32 chunks, last block
 * first, recomputing each block's chunk states from the state entering it;
 * those block-entry states (and per-token scratch of the window branch) are
 * kept in dgate's own rows until the rows are written, so dgate must not
 * overlap any input.  q_w, k_w, dq_w, dk_w
 * (all four NULL, or all four given, else LIZARD_E_NULL): the window branch's
 * own queries and keys as passed to lizard_hybrid_fwd, and their gradients
 * [B,H,T,dk] (desc->dtype, overwritten); dq, dk then hold the gated branch's
 * gradients alone.  With them NULL, dq and dk hold both branches' gradients.
 * Supported for BF16 and F32 with dk = dv in {64, 128}. */
lizard_status_t lizard_hybrid_bwd(const lizard_desc_t* desc, const void* q, const void* k,
                                  const void* v, const void* gate, const void* meta_k,
                                  const void* meta_v, const float* h0, const void* o_swa,
                                  const float* lse, const void* dO, void* dq, void* dk,
                                  void* dv, float* dgate, float* dmeta_k, float* dmeta_v,
                                  const float* dhT, float* dh0, float* dmix, const void* q_w,
                                  const void* k_w, void* dq_w, void* dk_w, void* ws,
                                  size_t ws_bytes, hipStream_t stream);

/* Segment-wise runs of a long sequence (training over contexts far longer than
 * one call should hold, e.g. 32k-64k tokens): the sequence is cut into segments
 * run one after another, the gated branch chained through its constant-size
 * state (hT of a segment as h0 of the next, dh0 of a segment as dhT of the one
 * before), which is what the constant-memory claims of "Lizard: An Efficient
 * Linearization Framework for Large Language Models" (gist.science summary,
 * sections 2(a), 3 and 4 "Efficiency") rest on.  The window branch of a segment
 * also needs the w-1 keys and values before its first token, its halo:
 *   halo_k, halo_v [B, H, halo_len, d] (desc->dtype): the halo_len tokens just
 *     before the segment, oldest first (keys in the window branch's key space:
 *     k_w when given, else k); 0 <= halo_len <= w-1, both non-NULL when
 *     halo_len > 0 (else LIZARD_E_NULL; a halo_len out of range:
 *     LIZARD_E_SHAPE).  halo_len = min(w-1, tokens before the segment) makes
 *     every output equal that of one call on the whole sequence.
 * lizard_hybrid_fwd_segment: lizard_hybrid_fwd with a halo (no window cache
 *   output; the other arguments and outputs as there).
 * lizard_hybrid_bwd_segment: lizard_hybrid_bwd with the same halo, plus
 *   dhalo_k, dhalo_v [B, H, halo_len, d] float32 (both or neither; nullable):
 *     receive the loss gradient with respect to the halo keys and values;
 *   tail_dk, tail_dv [B, H, tail_len, d] float32: gradients with respect to
 *     this segment's last tail_len window keys and values coming from the next
 *     segment (that segment's dhalo), added into dk (or dk_w) and dv;
 *     0 <= tail_len <= min(w-1, T), both non-NULL when tail_len > 0.
 * Segments run last to first in the backward, passing dh0 -> dhT and
 * dhalo -> tail; the meta-memory gradients of the segments add up. */
lizard_status_t lizard_hybrid_fwd_segment(const lizard_desc_t* desc, const void* q,
                                          const void* k, const void* v, const void* gate,
                                          const void* meta_k, const void* meta_v,
                                          const float* h0, void* o, float* lse, void* o_swa,
                                          float* hT, const void* q_w, const void* k_w,
                                          const void* halo_k, const void* halo_v,
                                          int32_t halo_len, void* ws, size_t ws_bytes,
                                          hipStream_t stream);
lizard_status_t lizard_hybrid_bwd_segment(
    const lizard_desc_t* desc, const void* q, const void* k, const void* v, const void* gate,
    const void* meta_k, const void* meta_v, const float* h0, const void* o_swa,
    const float* lse, const void* dO, void* dq, void* dk, void* dv, float* dgate,
    float* dmeta_k, float* dmeta_v, const float* dhT, float* dh0, float* dmix, const void* q_w,
    const void* k_w, void* dq_w, void* dk_w, const void* halo_k, const void* halo_v,
    int32_t halo_len, float* dhalo_k, float* dhalo_v, const float* tail_dk,
    const float* tail_dv, int32_t tail_len, void* ws, size_t ws_bytes, hipStream_t stream);

/* Decode window cache after a prefill run in segments (a chunked prefill that
 * continues into generation; the anchor window of section 2(a) and the
 * constant-memory generation of section 4 "Efficiency" of "Lizard: An
 * Efficient Linearization Framework for Large Language Models", gist.science
 * summary): ring_k, ring_v [B, H, w, d] (desc->dtype, overwritten) receive the
 * cache lizard_hybrid_fwd returns for a whole prefill -- slot p mod w holds
 * token p for the last min(w, pos0 + T) positions p, zeros in the other
 * slots -- so that lizard_decode_step continues the sequence (pos = pos0 + T,
 * state = the last segment's hT).
 *   k, v [B, H, T, d]: the last segment's window keys (k_w when the window
 *     branch has its own) and values, positions pos0 .. pos0 + T - 1;
 *   halo_k, halo_v [B, H, halo_len, d]: the halo_len tokens before it,
 *     positions pos0 - halo_len .. pos0 - 1, oldest first (both non-NULL when
 *     halo_len > 0);
 *   0 <= halo_len <= min(w, pos0), and when T < w at least the min(pos0, w - T)
 *   tokens before the segment that the cache keeps (else LIZARD_E_SHAPE; the
 *   segment run's own halo of min(w - 1, pos0) tokens is enough unless T = 0).
 * desc: B, H, T, dk = dv, window and dtype are read (the rest must still be a
 * valid descriptor).  A copy: no workspace, inputs read once. */
lizard_status_t lizard_window_cache_fill(const lizard_desc_t* desc, const void* k, const void* v,
                                         const void* halo_k, const void* halo_v,
                                         int32_t halo_len, int64_t pos0, void* ring_k,
                                         void* ring_v, hipStream_t stream);

/* One constant-memory generation step for B sequences (desc->T is ignored): the
 * recurrent form of both branches, as the constant-memory inference of "Lizard:
 * An Efficient Linearization Framework for Large Language Models" (gist.science
 * summary, sections 2(a) and 4 "Efficiency") needs it: the fp32 state is
 * updated in place and the window branch reads only a ring of the last w keys
 * and values, so the memory per sequence does not grow with its length.
 * q, k [B,H,dk], v [B,H,dv] in desc->dtype; gate [B,H,dk] as desc->gate says.
 * pos [B] int64 (device): tokens already seen by each sequence.  The call
 * updates state in place, writes (k, v) to ring slot pos mod w, attends over the
 * min(pos+1, w) filled slots plus the M meta slots, writes o [B,H,dv] and then
 * increments every pos[b] by one.  |pos[b]| must stay below 2^39; while the
 * call runs, pos[b] holds intermediate values (the heads of a sequence count
 * their completion in its high bits), so it must not be read or written by
 * other work until the call has finished.  q_w, k_w [B,H,dk] (both NULL, or
 * both given, else LIZARD_E_NULL): the window branch's own query and key, as
 * in lizard_hybrid_fwd; k_w (else k) goes into the ring, q_w (else q) attends. */
lizard_status_t lizard_decode_step(const lizard_desc_t* desc, const void* q, const void* k,
                                   const void* v, const void* gate, float* state,
                                   void* ring_k, void* ring_v, int64_t* pos,
                                   const void* meta_k, const void* meta_v, const void* q_w,
                                   const void* k_w, void* o, hipStream_t stream);

/* Size of the fixed per-device scratch array behind lizard_hybrid_fwd_static. */
#define LIZARD_STATIC_SCRATCH_BYTES ((size_t)17 << 20)

/* lizard_hybrid_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid allocation.  Arguments, outputs and errors are those of
 * lizard_hybrid_fwd; the scratch memory is a fixed array of
 * LIZARD_STATIC_SCRATCH_BYTES that the library holds on every device it runs on
 * until the process ends, so the call itself allocates and frees nothing.  A
 * problem whose lizard_workspace_bytes(desc, LIZARD_OP_HYBRID_FWD) exceeds that
 * size returns LIZARD_E_SCRATCH (no shape this version accepts does).  The array
 * of the current device (hipGetDevice) is used; its device address is looked up
 * on the first call on each device (LIZARD_E_HIP if that fails).  All calls on
 * one device share the array and nothing in it carries over between calls (no
 * part of it must start at zero), but two such calls that overlap in time on one
 * device, on different streams or threads, race on it: serialise them. */
lizard_status_t lizard_hybrid_fwd_static(const lizard_desc_t* desc, const void* q, const void* k,
                                         const void* v, const void* gate, const void* meta_k,
                                         const void* meta_v, const float* h0, void* o,
                                         float* lse, void* o_swa, float* hT, void* ring_k,
                                         void* ring_v, const void* q_w, const void* k_w,
                                         hipStream_t stream);

/* Static description of a status code. */
const char* lizard_status_str(lizard_status_t status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t lizard_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LIZARD_H */
