// Hybrid backward orchestration: the window branch writes dq, dk, dv, then the
// GLA branch adds its gradients to them (read-modify-write in its grad kernel).
#include "common.hpp"
#include "kernels.hpp"

namespace lz {

size_t gla_bwd_workspace_bytes(const Shape& s);
size_t swa_bwd_workspace_bytes(const Shape& s);
hipError_t launch_gla_bwd_scans(const Shape& s, const void* q, const void* k, const void* v,
                                const float* la, const float* h0, const float* dhT, float* dh0,
                                const void* dO, void* ws, hipStream_t st);
hipError_t launch_gla_bwd_grads(const Shape& s, const void* q, const void* k, const void* v,
                                const float* la, const void* dO, void* dq, void* dk, void* dv,
                                float* dla, const void* ws, hipStream_t st);
hipError_t launch_swa_bwd(const Shape& s, const void* q, const void* k, const void* v,
                          const void* mk, const void* mv, const void* o_swa, const float* lse,
                          const void* dO, void* dq, void* dk, void* dv, float* dmk, float* dmv,
                          void* ws, hipStream_t st);

namespace {
size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

__global__ void zero_kernel(float* p, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

}  // namespace

bool bwd_supported(const Shape& s) { return s.dtype == 1 && s.dk == 64 && s.dv == 64; }

size_t bwd_workspace_bytes(const Shape& s) {
  if (!bwd_supported(s)) return 0;
  return align256(gla_bwd_workspace_bytes(s)) + align256(swa_bwd_workspace_bytes(s));
}

hipError_t launch_hybrid_bwd(const Shape& s, const void* q, const void* k, const void* v,
                             const float* la, const void* mk, const void* mv, const float* h0,
                             const void* o_swa, const float* lse, const void* dO, void* dq,
                             void* dk, void* dv, float* dla, float* dmk, float* dmv,
                             const float* dhT, float* dh0, void* ws, hipStream_t st) {
  if (s.T == 0 || s.B == 0) {
    // no tokens: the meta-memory gradients are zero, dh0 = dhT (or zero)
    const size_t n = (size_t)s.H * s.n_meta * s.dk;
    if (n > 0) {
      hipLaunchKernelGGL(zero_kernel, dim3((n + 255) / 256), dim3(256), 0, st, dmk, n);
      hipLaunchKernelGGL(zero_kernel, dim3((n + 255) / 256), dim3(256), 0, st, dmv, n);
    }
    if (dh0) {
      const hipError_t e = launch_state_copy(s, dhT, dh0, st);
      if (e != hipSuccess) return e;
    }
    return hipGetLastError();
  }
  char* w = (char*)ws;
  char* wswa = w + align256(gla_bwd_workspace_bytes(s));
  // The window branch writes dq, dk, dv; the GLA grad kernel (after the scans
  // that produce its states) adds its gradients to them.
  hipError_t e = launch_gla_bwd_scans(s, q, k, v, la, h0, dhT, dh0, dO, w, st);
  if (e != hipSuccess) return e;
  e = launch_swa_bwd(s, q, k, v, mk, mv, o_swa, lse, dO, dq, dk, dv, dmk, dmv, wswa, st);
  if (e != hipSuccess) return e;
  return launch_gla_bwd_grads(s, q, k, v, la, dO, dq, dk, dv, dla, w, st);
}

}  // namespace lz
