// Hybrid backward orchestration: the window branch writes dq, dk, dv, then the
// GLA branch adds its gradients to them (read-modify-write in its grad kernel).
// With separate window queries and keys (qw, kw) the window branch writes dqw,
// dkw, dv instead, and the GLA branch writes dq, dk and adds to dv.
// The mix weight of "Lizard: An Efficient Linearization Framework for Large
// Language Models" (gist.science summary, section 2(a), final weighted sum)
// enters only o = o_gla + mix * o_swa, so dmix = sum(dO * o_swa).
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace lz {

size_t swa_bwd_workspace_bytes(const Shape& s);
hipError_t launch_swa_bwd(const Shape& s, const void* q, const void* k, const void* v,
                          const void* mk, const void* mv, const void* o_swa, const float* lse,
                          const void* dO, void* dq, void* dk, void* dv, float* dmk, float* dmv,
                          float* Dws, void* ws, MetaReduceArgs* defer, hipStream_t st);
hipError_t launch_gla_checkpoints(const Shape& s, const void* k, const void* v, const void* la,
                                  const float* h0, float* region, int cps, int nb,
                                  hipStream_t st);
hipError_t launch_gla_bwd_block(const Shape& s, const void* q, const void* k, const void* v,
                                const void* la, const void* dO, const float* fstart,
                                size_t fstride, const float* rstart, float* rend, void* dq,
                                void* dk, void* dv, float* dla, void* S_ws, void* dS_ws,
                                bool add_qk, int c0, int c1, int L, const MetaReduceArgs& meta,
                                hipStream_t st);
hipError_t launch_gla_bwd_block_gen(const Shape& s, const void* q, const void* k, const void* v,
                                    const void* la, const void* dO, const float* fstart,
                                    size_t fstride, const float* rstart, float* rend, void* dq,
                                    void* dk, void* dv, float* dla, void* S_ws, void* dS_ws,
                                    bool add_qk, int c0, int c1, int L, hipStream_t st);

namespace {
constexpr int kC = 64;
// The GLA backward walks each head in blocks of kBlk chunks, last block first,
// so its per-chunk state buffers hold kBlk states per head whatever T is.
constexpr int kBlk = 32;

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

template <typename T>
__global__ __launch_bounds__(256) void dmix_partial(const T* __restrict__ dO,
                                                    const T* __restrict__ os, size_t n8,
                                                    float* __restrict__ part) {
  __shared__ float red[4];
  float acc = 0.f;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (size_t)kMixBlocks * 256) {
    const typename Frag<T>::type a = ld8<T>(dO + 8 * i);
    const typename Frag<T>::type b = ld8<T>(os + 8 * i);
#pragma unroll
    for (int c = 0; c < 8; ++c) acc += to_f(a[c]) * to_f(b[c]);
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

size_t elem_bytes(const Shape& s) { return s.dtype == 1 ? 2 : 4; }

// per head: kBlk chunk states S_c and kBlk gradients dS_{c+1} in the element
// type, then one fp32 state for the reverse carry between blocks
size_t gla_bwd_workspace_bytes(const Shape& s) {
  const size_t bh = (size_t)s.B * s.H, dd = (size_t)s.dk * s.dv;
  return align256(2 * bh * kBlk * dd * elem_bytes(s)) + align256(bh * dd * sizeof(float));
}

}  // namespace

bool bwd_supported(const Shape& s) {
  if (s.dk != s.dv) return false;
  return s.dk == 64 || s.dk == 128;
}

size_t bwd_workspace_bytes(const Shape& s) {
  if (!bwd_supported(s)) return 0;
  return gla_bwd_workspace_bytes(s) + align256(swa_bwd_workspace_bytes(s)) +
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
    // no queries see the halo
    const size_t nh = (size_t)s.B * s.H * s.hlen * s.dk;
    if (s.dhk && nh > 0) {
      hipLaunchKernelGGL(zero_kernel, dim3((nh + 255) / 256), dim3(256), 0, st, s.dhk, nh);
      hipLaunchKernelGGL(zero_kernel, dim3((nh + 255) / 256), dim3(256), 0, st, s.dhv, nh);
    }
    return hipGetLastError();
  }
  const size_t bh = (size_t)s.B * s.H, dd = (size_t)s.dk * s.dv;
  const size_t es = elem_bytes(s);
  char* w = (char*)ws;
  char* S_ws = w;
  char* dS_ws = w + bh * kBlk * dd * es;
  float* carry = (float*)(w + align256(2 * bh * kBlk * dd * es));
  char* wswa = w + gla_bwd_workspace_bytes(s);
  float* part = (float*)(wswa + align256(swa_bwd_workspace_bytes(s)));
  // 1. the window branch writes dq, dk, dv (its per-token D_t scratch is the
  //    first B*H*T floats of dla, which the GLA branch overwrites below)
  //    With the tuned GLA kernels (bf16, d = 64) the window branch's
  //    meta-gradient reduction, if it leaves it, runs inside the first scans
  //    launch.
  const bool sep = qw != nullptr;
  const bool tuned = s.dtype == 1 && s.dk == 64;
  MetaReduceArgs meta;
  hipError_t e = launch_swa_bwd(s, sep ? qw : q, sep ? kw : k, v, mk, mv, o_swa, lse, dO,
                                sep ? dqw : dq, sep ? dkw : dk, dv, dmk, dmv, dla, wswa,
                                tuned ? &meta : nullptr, st);
  if (e != hipSuccess) return e;
  if (dmix) {
    const size_t n8 = (size_t)s.B * s.H * s.T * s.dv / 8;  // dv is a multiple of 8
    if (s.dtype == 1)
      hipLaunchKernelGGL(dmix_partial<bf16>, dim3(kMixBlocks), dim3(256), 0, st, (const bf16*)dO,
                         (const bf16*)o_swa, n8, part);
    else
      hipLaunchKernelGGL(dmix_partial<float>, dim3(kMixBlocks), dim3(256), 0, st,
                         (const float*)dO, (const float*)o_swa, n8, part);
    hipLaunchKernelGGL(dmix_final, dim3(1), dim3(256), 0, st, (const float*)part, dmix);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // 2. the GLA branch in blocks of kBlk chunks, last block first.  The state
  //    entering block b >= 1 is parked in the rows of block b-1 of dla (see
  //    launch_gla_checkpoints), which block b-1's own gradients overwrite only
  //    after block b has used it; the reverse scan carries the state gradient
  //    from block to block.
  const int nc = (s.T + kC - 1) / kC;
  const int nb = (nc + kBlk - 1) / kBlk;
  e = launch_gla_checkpoints(s, k, v, la, h0, dla, kBlk, nb, st);
  if (e != hipSuccess) return e;
  for (int b = nb - 1; b >= 0; --b) {
    const int c0 = b * kBlk, c1 = std::min(nc, c0 + kBlk);
    const float* fstart = b == 0 ? h0 : dla + (size_t)(b - 1) * kBlk * kC * s.dk + dd + s.dk;
    const size_t fstride = b == 0 ? dd : (size_t)s.T * s.dk;
    const float* rstart = b == nb - 1 ? dhT : carry;
    float* rend = b == 0 ? dh0 : carry;
    if (tuned)
      e = launch_gla_bwd_block(s, q, k, v, la, dO, fstart, fstride, rstart, rend, dq, dk, dv, dla,
                               S_ws, dS_ws, !sep, c0, c1, kBlk,
                               b == nb - 1 ? meta : MetaReduceArgs(), st);
    else
      e = launch_gla_bwd_block_gen(s, q, k, v, la, dO, fstart, fstride, rstart, rend, dq, dk, dv,
                                   dla, S_ws, dS_ws, !sep, c0, c1, kBlk, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace lz
