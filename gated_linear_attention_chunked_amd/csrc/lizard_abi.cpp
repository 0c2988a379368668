// C ABI host layer: argument checks, workspace sizing and dispatch.
// Every check runs before anything is enqueued; no C++ exception leaves a call.
#include "../../include/lizard.h"

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>

#include "kernels.hpp"

namespace {

using lz::Shape;

constexpr int32_t kVersion = 10200;  // 1.2.0: lizard_window_cache_fill

lizard_status_t check_desc(const lizard_desc_t* d, bool need_T) {
  if (!d) return LIZARD_E_NULL;
  if (d->dtype != LIZARD_F32 && d->dtype != LIZARD_BF16) return LIZARD_E_DTYPE;
  if (d->gate != LIZARD_GATE_LOG_ALPHA && d->gate != LIZARD_GATE_LOGIT) return LIZARD_E_DTYPE;
  if (d->B < 0 || d->H < 0 || (need_T && d->T < 0)) return LIZARD_E_SHAPE;
  if (d->dk <= 0 || d->dv <= 0 || d->chunk <= 0 || d->window < 1 || d->n_meta < 0)
    return LIZARD_E_SHAPE;
  if (!std::isfinite(d->scale) || !std::isfinite(d->mix)) return LIZARD_E_SHAPE;
  if (d->chunk != 64) return LIZARD_E_UNSUPPORTED;
  if (d->dk != d->dv) return LIZARD_E_UNSUPPORTED;
  if (d->dk != 64 && d->dk != 128) return LIZARD_E_UNSUPPORTED;
  if (d->gate == LIZARD_GATE_LOGIT && d->dtype != LIZARD_BF16) return LIZARD_E_UNSUPPORTED;
  if (d->n_meta > 16) return LIZARD_E_UNSUPPORTED;
  const long long bh = (long long)d->B * d->H;
  if (bh > 65535) return LIZARD_E_UNSUPPORTED;  // work-group grid limit of the prefill kernels
  // per-head slices are addressed with 32-bit byte offsets
  if (need_T && (long long)d->T * d->dk * 4 >= (1LL << 31)) return LIZARD_E_UNSUPPORTED;
  return LIZARD_OK;
}

Shape to_shape(const lizard_desc_t* d) {
  Shape s;
  s.B = d->B;
  s.H = d->H;
  s.T = d->T;
  s.dk = d->dk;
  s.dv = d->dv;
  s.window = d->window;
  s.n_meta = d->n_meta;
  s.scale = d->scale > 0.f ? d->scale : 1.0f / std::sqrt((float)d->dk);
  s.mix = d->mix;
  s.dtype = d->dtype;
  s.gate = d->gate;
  return s;
}

bool has_tokens(const lizard_desc_t* d) { return (long long)d->B * d->H * d->T > 0; }

// LIZARD_SYNC_DEBUG=1 in the environment (read once): every call waits for its
// work on the stream to finish and reports an asynchronous failure of it as
// LIZARD_E_HIP, so a fault is tied to the call that caused it.
bool sync_debug() {
  static const bool on = [] {
    const char* v = std::getenv("LIZARD_SYNC_DEBUG");
    return v && v[0] && v[0] != '0';
  }();
  return on;
}

lizard_status_t hip_status(hipError_t e, hipStream_t stream) {
  if (e == hipSuccess && sync_debug()) {
    e = hipStreamSynchronize(stream);
    if (e == hipSuccess) e = hipGetLastError();
  }
  return e == hipSuccess ? LIZARD_OK : LIZARD_E_HIP;
}

}  // namespace

extern "C" {

const char* lizard_status_str(lizard_status_t status) {
  // A C caller may pass any int; its bytes are read as an int, since loading an
  // out-of-range value through the enum type is undefined in C++.
  int s;
  static_assert(sizeof(s) == sizeof(status), "the status enum is int-sized");
  std::memcpy(&s, &status, sizeof s);
  switch (s) {
    case LIZARD_OK: return "ok";
    case LIZARD_E_NULL: return "a required pointer is NULL";
    case LIZARD_E_SHAPE: return "invalid size or parameter";
    case LIZARD_E_DTYPE: return "unknown dtype";
    case LIZARD_E_UNSUPPORTED: return "configuration not supported in this version";
    case LIZARD_E_WORKSPACE: return "workspace too small";
    case LIZARD_E_HIP: return "HIP launch failed";
    case LIZARD_E_SCRATCH: return "problem needs more than the static scratch array holds";
  }
  return "unknown status";
}

int32_t lizard_version(void) { return kVersion; }

size_t lizard_workspace_bytes(const lizard_desc_t* desc, int32_t op) {
  if (op == LIZARD_OP_SWA_FWD || op == LIZARD_OP_DECODE) return 0;
  if (check_desc(desc, true) != LIZARD_OK) return 0;
  if (op == LIZARD_OP_GLA_FWD || op == LIZARD_OP_HYBRID_FWD)
    return lz::gla_fwd_workspace_bytes(to_shape(desc));
  if (op == LIZARD_OP_HYBRID_BWD) return lz::bwd_workspace_bytes(to_shape(desc));
  return 0;
}

lizard_status_t lizard_gla_fwd(const lizard_desc_t* desc, const void* q, const void* k,
                               const void* v, const void* gate, const float* h0, void* o,
                               float* hT, void* ws, size_t ws_bytes, hipStream_t stream) {
  lizard_status_t st = check_desc(desc, true);
  if (st != LIZARD_OK) return st;
  if (has_tokens(desc) && (!q || !k || !v || !gate || !o)) return LIZARD_E_NULL;
  const size_t need = lz::gla_fwd_workspace_bytes(to_shape(desc));
  if (ws_bytes < need) return LIZARD_E_WORKSPACE;
  if (need > 0 && !ws) return LIZARD_E_NULL;
  if ((long long)desc->B * desc->H == 0) return LIZARD_OK;
  return hip_status(lz::launch_gla_fwd(to_shape(desc), q, k, v, gate, h0, o, hT, ws, stream), stream);
}

lizard_status_t lizard_swa_fwd(const lizard_desc_t* desc, const void* q, const void* k,
                               const void* v, const void* meta_k, const void* meta_v, void* o,
                               float* lse, hipStream_t stream) {
  lizard_status_t st = check_desc(desc, true);
  if (st != LIZARD_OK) return st;
  if (has_tokens(desc) && (!q || !k || !v || !o)) return LIZARD_E_NULL;
  if (desc->n_meta > 0 && desc->H > 0 && (!meta_k || !meta_v)) return LIZARD_E_NULL;
  if (!has_tokens(desc)) return LIZARD_OK;
  return hip_status(
      lz::launch_swa_fwd(to_shape(desc), q, k, v, meta_k, meta_v, o, 1.0f, 0, nullptr, lse,
                         nullptr, nullptr, stream), stream);
}

}  // extern "C"

namespace lz {
// Host checks of lizard_hybrid_fwd other than the workspace's.
lizard_status_t hybrid_fwd_args(const lizard_desc_t* desc, const void* q, const void* k,
                                const void* v, const void* gate, const void* meta_k,
                                const void* meta_v, const void* o, const void* ring_k,
                                const void* ring_v, const void* q_w, const void* k_w) {
  lizard_status_t st = check_desc(desc, true);
  if (st != LIZARD_OK) return st;
  if (has_tokens(desc) && (!q || !k || !v || !gate || !o)) return LIZARD_E_NULL;
  if ((q_w == nullptr) != (k_w == nullptr)) return LIZARD_E_NULL;
  if (desc->n_meta > 0 && desc->H > 0 && (!meta_k || !meta_v)) return LIZARD_E_NULL;
  if ((ring_k == nullptr) != (ring_v == nullptr)) return LIZARD_E_NULL;
  return LIZARD_OK;
}
}  // namespace lz

namespace {
// A window halo (segment-wise runs): halo_len in [0, w - 1], both buffers given
// when it is positive.
lizard_status_t check_halo(const lizard_desc_t* d, const void* hk, const void* hv, int32_t hlen) {
  if (hlen < 0 || hlen > d->window - 1) return LIZARD_E_SHAPE;
  if (hlen > 0 && (!hk || !hv)) return LIZARD_E_NULL;
  return LIZARD_OK;
}

lizard_status_t hybrid_fwd_impl(const lizard_desc_t* desc, const void* q, const void* k,
                                const void* v, const void* gate, const void* meta_k,
                                const void* meta_v, const float* h0, void* o, float* lse,
                                void* o_swa, float* hT, void* ring_k, void* ring_v,
                                const void* q_w, const void* k_w, const void* halo_k,
                                const void* halo_v, int32_t halo_len, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  lizard_status_t st =
      lz::hybrid_fwd_args(desc, q, k, v, gate, meta_k, meta_v, o, ring_k, ring_v, q_w, k_w);
  if (st != LIZARD_OK) return st;
  st = check_halo(desc, halo_k, halo_v, halo_len);
  if (st != LIZARD_OK) return st;
  // the window branch's queries and keys (the same as the GLA branch's by default)
  const void* qw = q_w ? q_w : q;
  const void* kw = k_w ? k_w : k;
  Shape s = to_shape(desc);
  s.hk = halo_k;
  s.hv = halo_v;
  s.hlen = halo_len;
  const size_t need = lz::gla_fwd_workspace_bytes(s);
  if (ws_bytes < need) return LIZARD_E_WORKSPACE;
  if (need > 0 && !ws) return LIZARD_E_NULL;
  if ((long long)desc->B * desc->H == 0) return LIZARD_OK;
  hipError_t e = hipSuccess;
  if (desc->T > 0 && lz::hybrid_fused_ok(s, lse || o_swa)) {
    // state pass, then both branches in one output pass (o written once)
    e = lz::launch_hybrid_fused(s, q, k, q_w, k_w, v, gate, meta_k, meta_v, h0, o, hT,
                                ring_k, ring_v, o_swa, lse, ws, stream);
  } else if (desc->T > 0) {
    // GLA branch writes o = o_gla; the window branch then adds mix * o_swa in place
    e = lz::launch_gla_fwd(s, q, k, v, gate, h0, o, hT, ws, stream);
    if (e == hipSuccess)
      e = lz::launch_swa_fwd(s, qw, kw, v, meta_k, meta_v, o, s.mix, 1, o_swa, lse, ring_k,
                             ring_v, stream);
  } else {
    if (hT) e = lz::launch_state_copy(s, h0, hT, stream);
    if (e == hipSuccess && ring_k) e = lz::launch_ring_fill(s, kw, v, ring_k, ring_v, stream);
  }
  return hip_status(e, stream);
}
}  // namespace

extern "C" {

lizard_status_t lizard_hybrid_fwd(const lizard_desc_t* desc, const void* q, const void* k,
                                  const void* v, const void* gate, const void* meta_k,
                                  const void* meta_v, const float* h0, void* o, float* lse,
                                  void* o_swa, float* hT, void* ring_k, void* ring_v,
                                  const void* q_w, const void* k_w, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  return hybrid_fwd_impl(desc, q, k, v, gate, meta_k, meta_v, h0, o, lse, o_swa, hT, ring_k,
                         ring_v, q_w, k_w, nullptr, nullptr, 0, ws, ws_bytes, stream);
}

lizard_status_t lizard_hybrid_fwd_segment(const lizard_desc_t* desc, const void* q,
                                          const void* k, const void* v, const void* gate,
                                          const void* meta_k, const void* meta_v,
                                          const float* h0, void* o, float* lse, void* o_swa,
                                          float* hT, const void* q_w, const void* k_w,
                                          const void* halo_k, const void* halo_v,
                                          int32_t halo_len, void* ws, size_t ws_bytes,
                                          hipStream_t stream) {
  return hybrid_fwd_impl(desc, q, k, v, gate, meta_k, meta_v, h0, o, lse, o_swa, hT, nullptr,
                         nullptr, q_w, k_w, halo_k, halo_v, halo_len, ws, ws_bytes, stream);
}

lizard_status_t lizard_hybrid_fwd_varlen(const lizard_desc_t* desc, const int32_t* cu_seqlens,
                                         int32_t n_tokens, const void* q, const void* k,
                                         const void* v, const void* gate, const void* meta_k,
                                         const void* meta_v, const float* h0, void* o, float* hT,
                                         void* ring_k, void* ring_v, const void* q_w,
                                         const void* k_w, void* ws, size_t ws_bytes,
                                         hipStream_t stream) {
  lizard_status_t st = check_desc(desc, true);
  if (st != LIZARD_OK) return st;
  if (n_tokens < 0) return LIZARD_E_SHAPE;
  if ((q_w == nullptr) != (k_w == nullptr)) return LIZARD_E_NULL;
  if ((ring_k == nullptr) != (ring_v == nullptr)) return LIZARD_E_NULL;
  if (desc->n_meta > 0 && desc->H > 0 && (!meta_k || !meta_v)) return LIZARD_E_NULL;
  Shape s = to_shape(desc);
  // the longest length bounds the kernels' grids
  if (desc->T < 1) return LIZARD_E_UNSUPPORTED;
  // per-head token rows are addressed with 32-bit byte offsets
  if ((long long)n_tokens * desc->dk * 4 >= (1LL << 31)) return LIZARD_E_UNSUPPORTED;
  const size_t need = lz::gla_fwd_workspace_bytes(s);
  if (ws_bytes < need) return LIZARD_E_WORKSPACE;
  if (need > 0 && !ws) return LIZARD_E_NULL;
  if ((long long)desc->B * desc->H == 0) return LIZARD_OK;
  if (!cu_seqlens) return LIZARD_E_NULL;
  if (n_tokens > 0 && (!q || !k || !v || !gate || !o)) return LIZARD_E_NULL;
  s.cu = cu_seqlens;
  s.n_tokens = n_tokens;
  if (lz::hybrid_fused_ok(s, false))
    return hip_status(lz::launch_hybrid_fused(s, q, k, q_w, k_w, v, gate, meta_k, meta_v, h0, o,
                                              hT, ring_k, ring_v, nullptr, nullptr, ws, stream),
                      stream);
  // other shapes: the GLA branch writes o, the window branch adds mix * o_swa
  hipError_t e = lz::launch_gla_fwd(s, q, k, v, gate, h0, o, hT, ws, stream);
  if (e == hipSuccess)
    e = lz::launch_swa_fwd(s, q_w ? q_w : q, k_w ? k_w : k, v, meta_k, meta_v, o, s.mix, 1,
                           nullptr, nullptr, ring_k, ring_v, stream);
  return hip_status(e, stream);
}

}  // extern "C"

namespace {
lizard_status_t hybrid_bwd_impl(const lizard_desc_t* desc, const void* q, const void* k,
                                const void* v, const void* gate, const void* meta_k,
                                const void* meta_v, const float* h0, const void* o_swa,
                                const float* lse, const void* dO, void* dq, void* dk, void* dv,
                                float* dgate, float* dmeta_k, float* dmeta_v, const float* dhT,
                                float* dh0, float* dmix, const void* q_w, const void* k_w,
                                void* dq_w, void* dk_w, const void* halo_k, const void* halo_v,
                                int32_t halo_len, float* dhalo_k, float* dhalo_v,
                                const float* tail_dk, const float* tail_dv, int32_t tail_len,
                                void* ws, size_t ws_bytes, hipStream_t stream) {
  lizard_status_t st = check_desc(desc, true);
  if (st != LIZARD_OK) return st;
  // separate window queries and keys come with their gradient outputs: all four or none
  const int n_sep = !!q_w + !!k_w + !!dq_w + !!dk_w;
  if (n_sep != 0 && n_sep != 4) return LIZARD_E_NULL;
  const bool meta = desc->n_meta > 0 && desc->H > 0;
  if (has_tokens(desc) && (!q || !k || !v || !gate || !o_swa || !lse || !dO || !dq || !dk ||
                           !dv || !dgate))
    return LIZARD_E_NULL;
  if (meta && (!meta_k || !meta_v || !dmeta_k || !dmeta_v)) return LIZARD_E_NULL;
  st = check_halo(desc, halo_k, halo_v, halo_len);
  if (st != LIZARD_OK) return st;
  if ((dhalo_k == nullptr) != (dhalo_v == nullptr)) return LIZARD_E_NULL;
  if (tail_len < 0 || tail_len > desc->window - 1 || tail_len > desc->T) return LIZARD_E_SHAPE;
  if (tail_len > 0 && (!tail_dk || !tail_dv)) return LIZARD_E_NULL;
  Shape s = to_shape(desc);
  if (!lz::bwd_supported(s)) return LIZARD_E_UNSUPPORTED;
  const size_t need = lz::bwd_workspace_bytes(s);
  if (ws_bytes < need) return LIZARD_E_WORKSPACE;
  if (need > 0 && !ws) return LIZARD_E_NULL;
  if ((long long)desc->B * desc->H == 0) return LIZARD_OK;
  s.hk = halo_k;
  s.hv = halo_v;
  s.hlen = halo_len;
  s.dhk = halo_len > 0 ? dhalo_k : nullptr;
  s.dhv = halo_len > 0 ? dhalo_v : nullptr;
  s.tdk = tail_dk;
  s.tdv = tail_dv;
  s.tlen = tail_len;
  return hip_status(lz::launch_hybrid_bwd(s, q, k, v, gate, meta_k, meta_v, h0, o_swa, lse,
                                          dO, dq, dk, dv, dgate, dmeta_k, dmeta_v, dhT, dh0,
                                          dmix, q_w, k_w, dq_w, dk_w, ws, stream), stream);
}
}  // namespace

extern "C" {

lizard_status_t lizard_hybrid_bwd(const lizard_desc_t* desc, const void* q, const void* k,
                                  const void* v, const void* gate, const void* meta_k,
                                  const void* meta_v, const float* h0, const void* o_swa,
                                  const float* lse, const void* dO, void* dq, void* dk, void* dv,
                                  float* dgate, float* dmeta_k, float* dmeta_v,
                                  const float* dhT, float* dh0, float* dmix, const void* q_w,
                                  const void* k_w, void* dq_w, void* dk_w, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  return hybrid_bwd_impl(desc, q, k, v, gate, meta_k, meta_v, h0, o_swa, lse, dO, dq, dk, dv,
                         dgate, dmeta_k, dmeta_v, dhT, dh0, dmix, q_w, k_w, dq_w, dk_w, nullptr,
                         nullptr, 0, nullptr, nullptr, nullptr, nullptr, 0, ws, ws_bytes, stream);
}

lizard_status_t lizard_hybrid_bwd_segment(
    const lizard_desc_t* desc, const void* q, const void* k, const void* v, const void* gate,
    const void* meta_k, const void* meta_v, const float* h0, const void* o_swa,
    const float* lse, const void* dO, void* dq, void* dk, void* dv, float* dgate,
    float* dmeta_k, float* dmeta_v, const float* dhT, float* dh0, float* dmix, const void* q_w,
    const void* k_w, void* dq_w, void* dk_w, const void* halo_k, const void* halo_v,
    int32_t halo_len, float* dhalo_k, float* dhalo_v, const float* tail_dk,
    const float* tail_dv, int32_t tail_len, void* ws, size_t ws_bytes, hipStream_t stream) {
  return hybrid_bwd_impl(desc, q, k, v, gate, meta_k, meta_v, h0, o_swa, lse, dO, dq, dk, dv,
                         dgate, dmeta_k, dmeta_v, dhT, dh0, dmix, q_w, k_w, dq_w, dk_w, halo_k,
                         halo_v, halo_len, dhalo_k, dhalo_v, tail_dk, tail_dv, tail_len, ws,
                         ws_bytes, stream);
}

lizard_status_t lizard_window_cache_fill(const lizard_desc_t* desc, const void* k,
                                         const void* v, const void* halo_k, const void* halo_v,
                                         int32_t halo_len, int64_t pos0, void* ring_k,
                                         void* ring_v, hipStream_t stream) {
  lizard_status_t st = check_desc(desc, true);
  if (st != LIZARD_OK) return st;
  if (pos0 < 0 || halo_len < 0 || halo_len > desc->window || halo_len > pos0)
    return LIZARD_E_SHAPE;
  // positions before the segment that the cache keeps (the last w of pos0 + T)
  const long long keep =
      desc->T >= desc->window ? 0 : std::min<long long>(pos0, (long long)desc->window - desc->T);
  if (halo_len < keep) return LIZARD_E_SHAPE;
  if ((long long)desc->B * desc->H == 0) return LIZARD_OK;
  if (!ring_k || !ring_v) return LIZARD_E_NULL;
  if (desc->T > 0 && (!k || !v)) return LIZARD_E_NULL;
  if (halo_len > 0 && (!halo_k || !halo_v)) return LIZARD_E_NULL;
  return hip_status(lz::launch_cache_from_segment(to_shape(desc), k, v, halo_k, halo_v, halo_len,
                                                  pos0, ring_k, ring_v, stream),
                    stream);
}

lizard_status_t lizard_decode_step(const lizard_desc_t* desc, const void* q, const void* k,
                                   const void* v, const void* gate, float* state,
                                   void* ring_k, void* ring_v, int64_t* pos, const void* meta_k,
                                   const void* meta_v, const void* q_w, const void* k_w, void* o,
                                   hipStream_t stream) {
  lizard_status_t st = check_desc(desc, false);
  if (st != LIZARD_OK) return st;
  if (!q_w != !k_w) return LIZARD_E_NULL;  // window query and key: both or neither
  if ((long long)desc->B * desc->H == 0) return LIZARD_OK;
  if (!q || !k || !v || !gate || !state || !ring_k || !ring_v || !pos || !o)
    return LIZARD_E_NULL;
  if (desc->n_meta > 0 && (!meta_k || !meta_v)) return LIZARD_E_NULL;
  // the window softmax keeps w + M logits in LDS
  if ((long long)desc->window + desc->n_meta > 16384) return LIZARD_E_UNSUPPORTED;
  // the heads of a sequence count their completion in bits 40.. of pos[b]
  if (desc->H >= (1 << 22)) return LIZARD_E_UNSUPPORTED;
  return hip_status(lz::launch_decode(to_shape(desc), q, k, q_w ? q_w : q, k_w ? k_w : k, v,
                                      gate, state, ring_k, ring_v, pos, meta_k, meta_v, o,
                                      stream), stream);
}

}  // extern "C"
