// The d = 64 instances of the single-pass hybrid forward (hybrid_fwd.hpp), in a
// translation unit of their own so that they take their own build flags (the
// scheduling strategy in build.py) while the d = 128 instances keep theirs.
#include "hybrid_fwd.hpp"

namespace lz {

void launch_fused_d64(const Shape& s, bool sep, const void* q, const void* k, const void* qw,
                      const void* kw, const void* v, const void* la, const void* mk,
                      const void* mv, const float* h0, const float* ws_state,
                      const float* ws_gamma, void* o, float* hT, void* ring_k, void* ring_v,
                      void* o_swa, float* lse, int cps, int G, int m, hipStream_t st) {
  if (s.window <= max_window(3))
    launch_fused_ring<64, 3>(s, sep, q, k, qw, kw, v, la, mk, mv, h0, ws_state, ws_gamma, o, hT,
                             ring_k, ring_v, o_swa, lse, cps, G, m, st);
  else
    launch_fused_ring<64, 5>(s, sep, q, k, qw, kw, v, la, mk, mv, h0, ws_state, ws_gamma, o, hT,
                             ring_k, ring_v, o_swa, lse, cps, G, m, st);
}

}  // namespace lz
