// Hybrid backward orchestration: the window branch writes dq, dk, dv, then the
// GLA branch adds its gradients to them (read-modify-write in its grad kernel).
// With separate window queries and keys (qw, kw) the window branch writes dqw,
// dkw, dv instead, and the GLA branch writes dq, dk and adds to dv.
// The mix weight of "Lizard: An Efficient Linearization Framework for Large
// Language Models" (gist.science summary, section 2(a), final weighted sum)
// enters only o = o_gla + mix * o_swa, so dmix = sum(dO * o_swa).
#include "common.hpp"
#include "kernels.hpp"

namespace lz {

size_t gla_bwd_workspace_bytes(const Shape& s);
size_t swa_bwd_workspace_bytes(const Shape& s);
hipError_t launch_gla_bwd_scans(const Shape& s, const void* q, const void* k, const void* v,
                                const void* la, const float* h0, const float* dhT, float* dh0,
                                const void* dO, void* ws, hipStream_t st);
hipError_t launch_gla_bwd_grads(const Shape& s, const void* q, const void* k, const void* v,
                                const void* la, const void* dO, void* dq, void* dk, void* dv,
                                float* dla, const void* ws, bool add_qk, hipStream_t st);
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

// dmix = sum(dO * o_swa), in a fixed order: kMixBlocks work-groups each add a
// fixed strided set of 8-element granules, then one work-group adds the
// partials; a work-group's sum is a butterfly inside each wave, then the four
// wave sums in order, so repeated calls agree bit for bit.
constexpr int kMixBlocks = 256;

__device__ __forceinline__ float block_sum256(float x, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(256) void dmix_partial(const bf16* __restrict__ dO,
                                                    const bf16* __restrict__ os, size_t n8,
                                                    float* __restrict__ part) {
  __shared__ float red[4];
  float acc = 0.f;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (size_t)kMixBlocks * 256) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(dO + 8 * i);
    const u32x4 b = *reinterpret_cast<const u32x4*>(os + 8 * i);
#pragma unroll
    for (int c = 0; c < 8; ++c) acc += bf_at(a, c) * bf_at(b, c);
  }
  const float s = block_sum256(acc, red);
  if (threadIdx.x == 0) part[blockIdx.x] = s;
}

__global__ __launch_bounds__(256) void dmix_final(const float* __restrict__ part,
                                                  float* __restrict__ dmix) {
  __shared__ float red[4];
  const float s = block_sum256(part[threadIdx.x], red);
  if (threadIdx.x == 0) *dmix = s;
}

}  // namespace

bool bwd_supported(const Shape& s) { return s.dtype == 1 && s.dk == 64 && s.dv == 64; }

size_t bwd_workspace_bytes(const Shape& s) {
  if (!bwd_supported(s)) return 0;
  return align256(gla_bwd_workspace_bytes(s)) + align256(swa_bwd_workspace_bytes(s)) +
         align256(kMixBlocks * sizeof(float));
}

hipError_t launch_hybrid_bwd(const Shape& s, const void* q, const void* k, const void* v,
                             const void* la, const void* mk, const void* mv, const float* h0,
                             const void* o_swa, const float* lse, const void* dO, void* dq,
                             void* dk, void* dv, float* dla, float* dmk, float* dmv,
                             const float* dhT, float* dh0, float* dmix, const void* qw,
                             const void* kw, void* dqw, void* dkw, void* ws, hipStream_t st) {
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
    if (dmix) hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(64), 0, st, dmix, (size_t)1);
    return hipGetLastError();
  }
  char* w = (char*)ws;
  char* wswa = w + align256(gla_bwd_workspace_bytes(s));
  // The window branch writes dq, dk, dv; the GLA grad kernel (after the scans
  // that produce its states) adds its gradients to them.
  hipError_t e = launch_gla_bwd_scans(s, q, k, v, la, h0, dhT, dh0, dO, w, st);
  if (e != hipSuccess) return e;
  const bool sep = qw != nullptr;
  e = launch_swa_bwd(s, sep ? qw : q, sep ? kw : k, v, mk, mv, o_swa, lse, dO, sep ? dqw : dq,
                     sep ? dkw : dk, dv, dmk, dmv, wswa, st);
  if (e != hipSuccess) return e;
  if (dmix) {
    float* part = (float*)(wswa + align256(swa_bwd_workspace_bytes(s)));
    const size_t n8 = (size_t)s.B * s.H * s.T * s.dv / 8;  // dv is a multiple of 8
    hipLaunchKernelGGL(dmix_partial, dim3(kMixBlocks), dim3(256), 0, st, (const bf16*)dO,
                       (const bf16*)o_swa, n8, part);
    hipLaunchKernelGGL(dmix_final, dim3(1), dim3(256), 0, st, (const float*)part, dmix);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_gla_bwd_grads(s, q, k, v, la, dO, dq, dk, dv, dla, w, !sep, st);
}

}  // namespace lz
