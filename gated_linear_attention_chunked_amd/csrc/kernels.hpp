// Internal launcher interface between the C ABI host layer and the kernels.
// Launchers assume the host layer has validated every argument.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lz {

struct Shape {
  int B, H, T, dk, dv, window, n_meta;
  float scale;  // resolved (> 0)
  float mix;
  int dtype;    // 0 = f32, 1 = bf16
  int gate;     // gate input: 0 = float log alpha, 1 = bf16 logit x (alpha = sigmoid(x))
  // packed batches (single-pass forward only): tensors [H, n_tokens, d], sequence b
  // = tokens cu[b] .. cu[b+1]-1 (device array of B+1), T = the longest length
  const int* cu = nullptr;
  int n_tokens = 0;
  // window halo (segment-wise runs): the hlen keys and values [B, H, hlen, d]
  // just before the segment's first token, in order (the window branch's key
  // space); the backward returns their gradients (dhk, dhv, fp32, nullable) and
  // adds tdk, tdv [B, H, tlen, d] (fp32: the next segment's halo gradients) to
  // the gradients of the segment's last tlen keys and values
  const void* hk = nullptr;
  const void* hv = nullptr;
  int hlen = 0;
  float* dhk = nullptr;
  float* dhv = nullptr;
  const float* tdk = nullptr;
  const float* tdv = nullptr;
  int tlen = 0;
};

// GLA branch: o = o_gla; hT (optional) = final state.  ws holds
// gla_fwd_workspace_bytes(s) bytes (segment states; independent of T once
// T >= 16 chunks).
size_t gla_fwd_workspace_bytes(const Shape& s);
hipError_t launch_gla_fwd(const Shape& s, const void* q, const void* k, const void* v,
                          const void* la, const float* h0, void* o, float* hT, void* ws,
                          hipStream_t st);

// State pass of the GLA branch alone (bf16, dk = dv in {64, 128}): the local end
// states and decays of the (G-1) m pieces of segments 0..G-2 into ws (pieces of
// cps / m 64-token chunks, in order; m = 1 gives launch_gla_fwd's layout); G
// segments of cps 64-token chunks each.
hipError_t launch_gla_state(const Shape& s, const void* k, const void* v, const void* la,
                            void* ws, int* G, int* cps, int* m, hipStream_t st);

// Both branches' outputs in one pass after launch_gla_state: o = o_gla + mix *
// o_swa, hT (optional), the decode window cache (optional) and, with save, the
// training outputs o_swa and lse (each optional).  Only for the shapes
// hybrid_fused_ok accepts.
bool hybrid_fused_ok(const Shape& s, bool save);
// qw, kw: the window branch's queries and keys (both null: q, k).
hipError_t launch_hybrid_fused(const Shape& s, const void* q, const void* k, const void* qw,
                               const void* kw, const void* v, const void* la, const void* mk,
                               const void* mv, const float* h0, void* o, float* hT, void* ring_k,
                               void* ring_v, void* o_swa, float* lse, void* ws, hipStream_t st);

// Window + meta branch.  o = out_scale * o_swa (or o += out_scale * o_swa when
// accumulate != 0); o_swa and lse are optional extra outputs.
// ring_k / ring_v (nullable): also fill the decode window cache (slot p mod w <- token p
// for the last min(T, w) tokens, zero elsewhere).
hipError_t launch_swa_fwd(const Shape& s, const void* q, const void* k, const void* v,
                          const void* mk, const void* mv, void* o, float out_scale,
                          int accumulate, void* o_swa, float* lse, void* ring_k, void* ring_v,
                          hipStream_t st);

// Window cache after a prefill (slot p mod w <- token p for the last min(T,w) tokens).
hipError_t launch_ring_fill(const Shape& s, const void* k, const void* v, void* ring_k,
                            void* ring_v, hipStream_t st);

// Window cache from the last segment of a sequence prefilled in segments: its
// T tokens k, v [B, H, T, d] are positions pos0.., the hlen halo tokens hk, hv
// [B, H, hlen, d] the positions just before (the host checks that they cover
// what the cache keeps).
hipError_t launch_cache_from_segment(const Shape& s, const void* k, const void* v,
                                     const void* hk, const void* hv, int hlen, long long pos0,
                                     void* ring_k, void* ring_v, hipStream_t st);

// hT <- h0 (or zeros) for T == 0.
hipError_t launch_state_copy(const Shape& s, const float* h0, float* hT, hipStream_t st);

// qw, kw: the window branch's query and key (pass q, k when they are shared).
hipError_t launch_decode(const Shape& s, const void* q, const void* k, const void* qw,
                         const void* kw, const void* v, const void* la, float* state,
                         void* ring_k, void* ring_v, int64_t* pos, const void* mk, const void* mv,
                         void* o, hipStream_t st);

// Backward (bf16 or fp32, dk = dv = 64 or 128).  The workspace (owned by
// hybrid_bwd, gla_bwd and swa_bwd) does not depend on T.  qw, kw, dqw, dkw:
// separate window queries and keys and their gradients (all null: shared).
bool bwd_supported(const Shape& s);
size_t bwd_workspace_bytes(const Shape& s);
hipError_t launch_hybrid_bwd(const Shape& s, const void* q, const void* k, const void* v,
                             const void* la, const void* mk, const void* mv, const float* h0,
                             const void* o_swa, const float* lse, const void* dO, void* dq,
                             void* dk, void* dv, float* dla, float* dmk, float* dmv,
                             const float* dhT, float* dh0, float* dmix, const void* qw,
                             const void* kw, void* dqw, void* dkw, void* ws, hipStream_t st);

}  // namespace lz
