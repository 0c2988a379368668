// Hybrid forward as one output pass: the launch side.  The kernel (its design
// and the pages' passages it follows) is in hybrid_fwd.hpp; the d = 128
// instances are built here and the d = 64 ones in hybrid_fwd_d64.hip.
#include "hybrid_fwd.hpp"

namespace lz {

void launch_fused_d64(const Shape& s, bool sep, const void* q, const void* k, const void* qw,
                      const void* kw, const void* v, const void* la, const void* mk,
                      const void* mv, const float* h0, const float* ws_state,
                      const float* ws_gamma, void* o, float* hT, void* ring_k, void* ring_v,
                      void* o_swa, float* lse, int cps, int G, int m, hipStream_t st);

// bf16 with d_k = d_v in {64, 128} (with or without the training outputs o_swa
// and lse), a window the five-chunk ring holds, at most 16 meta slots, no halo.
bool hybrid_fused_ok(const Shape& s, bool save) {
  (void)save;
  return s.dtype == 1 && (s.dk == 64 || s.dk == 128) && s.dv == s.dk && s.window >= 1 &&
         s.window <= max_window(5) && s.n_meta <= 16 && s.T > 0 && s.hlen == 0;
}

hipError_t launch_hybrid_fused(const Shape& s, const void* q, const void* k, const void* qw,
                               const void* kw, const void* v, const void* la, const void* mk,
                               const void* mv, const float* h0, void* o, float* hT, void* ring_k,
                               void* ring_v, void* o_swa, float* lse, void* ws, hipStream_t st) {
  if (s.B * s.H == 0) return hipSuccess;
  int G = 1, cps = 1, m = 1;
  hipError_t e = launch_gla_state(s, k, v, la, ws, &G, &cps, &m, st);
  if (e != hipSuccess) return e;
  const int BH = s.B * s.H;
  const float* ws_state = (const float*)ws;
  const float* ws_gamma = ws_state ? ws_state + (size_t)BH * (G - 1) * m * s.dk * s.dk : nullptr;
  const bool sep = qw != nullptr;
  const void* qw_ = sep ? qw : q;
  const void* kw_ = sep ? kw : k;
  if (s.dk == 128 && (o_swa || lse))
    launch_fused_ring<128, 5, true>(s, sep, q, k, qw_, kw_, v, la, mk, mv, h0, ws_state, ws_gamma, o,
                                    hT, ring_k, ring_v, o_swa, lse, cps, G, m, st);
  else if (s.dk == 128)
    launch_fused_ring<128, 5>(s, sep, q, k, qw_, kw_, v, la, mk, mv, h0, ws_state, ws_gamma, o, hT,
                              ring_k, ring_v, nullptr, nullptr, cps, G, m, st);
  else
    launch_fused_d64(s, sep, q, k, qw_, kw_, v, la, mk, mv, h0, ws_state, ws_gamma, o, hT, ring_k,
                     ring_v, o_swa, lse, cps, G, m, st);
  return hipGetLastError();
}

}  // namespace lz
