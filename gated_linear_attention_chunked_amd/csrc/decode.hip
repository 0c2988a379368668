// Constant-memory decode step and the prefill -> decode window cache, gfx950.
//
// "Lizard: An Efficient Linearization Framework for Large Language Models"
// (gist.science summary, section 2(a) and section 4 "Efficiency") keeps a fixed
// size hidden state instead of a growing KV cache.  One step for token p of a
// sequence: S <- diag(alpha) S + k^T v; o_gla = q S; the window cache keeps the
// last w keys/values in slot (position mod w); the window softmax runs over the
// min(p+1, w) filled slots plus the M meta slots; o = o_gla + mix * o_swa.  The
// window branch may read a query and key of its own (qw, kw; else q, k); the
// window cache then holds kw.
//
// One work-group per (batch, head).  The fp32 state (64 KiB at d = 128) is
// streamed once in and once out with 16-byte accesses; it dominates the bytes
// of a step, so the kernel is bound by HBM bandwidth.
#include "common.hpp"
#include "kernels.hpp"

namespace lz {
namespace {

template <typename T, int D, typename G>
__global__ __launch_bounds__(256, 8) void decode_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ qw,
    const T* __restrict__ kw, const T* __restrict__ v,
    const G* __restrict__ la, float* __restrict__ state, T* __restrict__ ring_k,
    T* __restrict__ ring_v, int64_t* __restrict__ pos, const T* __restrict__ mk,
    const T* __restrict__ mv, T* __restrict__ o, int H, int W, int M, float scale_log2,
    float mix) {
  constexpr int CQ = D / 4;        // threads per state row (4 columns each)
  constexpr int RG = 256 / CQ;     // row groups
  constexpr int LPR = 16;          // lanes per key row in the logit pass
  constexpr int EPL = D / LPR;     // elements per lane in the logit pass
  extern __shared__ float logit[];  // W + M floats
  __shared__ __attribute__((aligned(16))) float sq[D], sk[D], sv[D], sa[D], swq[D], swk[D];
  __shared__ __attribute__((aligned(16))) f32x4 red[RG][CQ];
  __shared__ __attribute__((aligned(16))) float wred[8];

  const int tid = threadIdx.x;
  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  // While the heads of sequence b run, pos[b] = position + (heads done) * 2^40
  // (see the end of the kernel); the position is the low 40 bits, sign-extended.
  const int64_t pv = (int64_t)((uint64_t)pos[b] << 24) >> 24;
  const int64_t p = pv < 0 ? 0 : pv;  // negative positions count as 0
  const int slot = (int)(p % W);
  const int n = (int)((p + 1 < W) ? p + 1 : W);
  const int nk = n + M;

  if (tid < D) {
    const size_t off = (size_t)bh * D + tid;
    sq[tid] = to_f(q[off]);
    sk[tid] = to_f(k[off]);
    sv[tid] = to_f(v[off]);
    sa[tid] = exp2_fast(gate_log2(to_f(la[off]), G()));
    swq[tid] = to_f(qw[off]);
    swk[tid] = to_f(kw[off]);
  }
  __syncthreads();

  // ---- GLA: S <- a*S + k v^T (in place), o_gla = q S
  const int cq = tid % CQ, rg = tid / CQ;
  float* Sb = state + (size_t)bh * D * D;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const f32x4 v4 = {sv[4 * cq], sv[4 * cq + 1], sv[4 * cq + 2], sv[4 * cq + 3]};
#pragma unroll 4
  for (int r = rg; r < D; r += RG) {
    f32x4* ptr = reinterpret_cast<f32x4*>(Sb + (size_t)r * D + 4 * cq);
    f32x4 s4 = *ptr;
    s4 = s4 * sa[r] + v4 * sk[r];
    *ptr = s4;
    acc += s4 * sq[r];
  }
  red[rg][cq] = acc;

  // ---- new token into its ring slot
  if (tid < D) {
    const size_t roff = ((size_t)bh * W + slot) * D + tid;
    ring_k[roff] = to_t<T>(swk[tid]);
    ring_v[roff] = to_t<T>(sv[tid]);
  }

  // ---- window + meta logits (16 lanes per key row)
  {
    const int part = tid % LPR;
    float qv[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[e] = swq[part * EPL + e];
    // loads are unconditional (the slot row's value is replaced by the new key
    // from LDS afterwards) so that several passes' loads are in flight at once
#pragma unroll 3
    for (int base = 0; base < nk; base += 256 / LPR) {
      const int row = base + tid / LPR;
      float dot = 0.f;
      if (row < nk) {
        const T* kp = (row < n) ? ring_k + ((size_t)bh * W + row) * D
                                : mk + ((size_t)h * M + (row - n)) * D;
        float kv[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) kv[e] = to_f(kp[part * EPL + e]);
        if (row == slot)
#pragma unroll
          for (int e = 0; e < EPL; ++e) kv[e] = swk[part * EPL + e];
#pragma unroll
        for (int e = 0; e < EPL; ++e) dot += qv[e] * kv[e];
      }
#pragma unroll
      for (int off = 1; off < LPR; off <<= 1) dot += __shfl_xor(dot, off);
      if (part == 0 && row < nk) logit[row] = dot * scale_log2;
    }
  }
  __syncthreads();

  // ---- softmax over nk logits
  float mx = -INFINITY;
  for (int i = tid; i < nk; i += 256) mx = fmaxf(mx, logit[i]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if ((tid & 63) == 0) wred[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3]));
  float sum = 0.f;
  for (int i = tid; i < nk; i += 256) {
    const float e = exp2_fast(logit[i] - mx);
    logit[i] = e;
    sum += e;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  __syncthreads();
  if ((tid & 63) == 0) wred[4 + (tid >> 6)] = sum;
  __syncthreads();
  sum = wred[4] + wred[5] + wred[6] + wred[7];

  // ---- o_swa = sum p_s val_s, with the same (row group, 4 columns) layout
  f32x4 ow = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int row = rg; row < nk; row += RG) {
    const T* vp = (row < n) ? ring_v + ((size_t)bh * W + row) * D
                            : mv + ((size_t)h * M + (row - n)) * D;
    f32x4 val = ld4f<T>(vp + 4 * cq);
    if (row == slot) val = v4;  // the new token, from LDS
    ow += val * logit[row];
  }
  __syncthreads();  // red (GLA partials) complete; reuse red for o_swa after reading
  f32x4 og = {0.f, 0.f, 0.f, 0.f};
  if (rg == 0) {
#pragma unroll 1
    for (int r = 0; r < RG; ++r) og += red[r][cq];
  }
  __syncthreads();
  red[rg][cq] = ow;
  __syncthreads();
  if (rg == 0) {
    f32x4 os = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int r = 0; r < RG; ++r) os += red[r][cq];
    const f32x4 out = og + os * (mix / sum);
    st4<T>(o + (size_t)bh * D + 4 * cq, out);
  }
  // This head is done (every thread read pos[b] before the first barrier): add
  // 2^40; the last of the H heads of sequence b turns the H arrivals into the
  // step, pos[b] + 1.  No head reads pos[b] after its own arrival.
  if (tid == 0) {
    const int64_t old = (int64_t)atomicAdd(reinterpret_cast<unsigned long long*>(&pos[b]), 1ull << 40);
    if (((old - pv) >> 40) == H - 1)
      atomicAdd(reinterpret_cast<unsigned long long*>(&pos[b]),
                (unsigned long long)(1 - ((int64_t)H << 40)));
  }
}


template <typename T>
__global__ void ring_fill_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                 T* __restrict__ rk, T* __restrict__ rv, int T_arg, int W, int D,
                                 const int* __restrict__ cu, int N, int H) {
  const int slot = blockIdx.x, bh = blockIdx.y;
  const T* x = blockIdx.z ? v : k;  // z = 0: keys, z = 1: values
  T* ring = blockIdx.z ? rv : rk;
  const SeqRows sr = seq_rows(cu, N, T_arg, H, bh);
  const int T_len = sr.len;
  // the position p = slot (mod W) inside [T - W, T), if any
  long base = (long)T_len - W;
  long p = base + ((((long)slot - base) % W) + W) % W;
  T* dst = ring + ((size_t)bh * W + slot) * D;
  for (int d = threadIdx.x; d < D; d += blockDim.x)
    dst[d] = (p >= 0) ? x[(sr.row0 + p) * D + d] : to_t<T>(0.f);
}

// Window cache of a sequence prefilled in segments, from its last segment: the
// segment's T_arg tokens are positions pos0 .. pos0+T_arg-1 and the halo's hlen
// tokens positions pos0-hlen .. pos0-1 (the host has checked that the halo
// holds every earlier position the cache keeps).  Slot p mod W <- token p for
// the last min(W, pos0 + T_arg) positions, zero where no position lands.
template <typename T>
__global__ void cache_from_segment_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                          const T* __restrict__ hk, const T* __restrict__ hv,
                                          T* __restrict__ rk, T* __restrict__ rv, int T_arg,
                                          int hlen, long long pos0, int W, int D) {
  const int slot = blockIdx.x, bh = blockIdx.y;
  const bool val = blockIdx.z != 0;  // z = 0: keys, z = 1: values
  const long long N = pos0 + T_arg, base = N - W;
  // the position p = slot (mod W) inside [N - W, N)
  const long long p = base + ((((long long)slot - base) % W) + W) % W;
  const T* src = nullptr;
  if (p >= pos0)
    src = (val ? v : k) + ((size_t)bh * T_arg + (size_t)(p - pos0)) * D;
  else if (p >= 0)
    src = (val ? hv : hk) + ((size_t)bh * hlen + (size_t)(p - (pos0 - hlen))) * D;
  T* dst = (val ? rv : rk) + ((size_t)bh * W + slot) * D;
  for (int d = threadIdx.x; d < D; d += blockDim.x) dst[d] = src ? src[d] : to_t<T>(0.f);
}

template <typename T, int D, typename G>
hipError_t launch_decode_typed(const Shape& s, const void* q, const void* k, const void* qw,
                               const void* kw, const void* v, const void* la, float* state,
                               void* ring_k, void* ring_v, int64_t* pos, const void* mk,
                               const void* mv, void* o, hipStream_t st) {
  const size_t lds = sizeof(float) * (size_t)(s.window + s.n_meta);
  hipLaunchKernelGGL((decode_kernel<T, D, G>), dim3(s.B * s.H), dim3(256), lds, st, (const T*)q,
                     (const T*)k, (const T*)qw, (const T*)kw, (const T*)v, (const G*)la, state,
                     (T*)ring_k, (T*)ring_v, pos,
                     (const T*)mk, (const T*)mv, (T*)o, s.H, s.window, s.n_meta,
                     s.scale * kLog2e, s.mix);
  return hipGetLastError();
}

template <typename T>
hipError_t ring_fill_typed(const Shape& s, const void* k, const void* v, void* rk, void* rv,
                           hipStream_t st) {
  dim3 grid(s.window, s.B * s.H, 2);  // dk == dv
  hipLaunchKernelGGL(ring_fill_kernel<T>, grid, dim3(64), 0, st, (const T*)k, (const T*)v,
                     (T*)rk, (T*)rv, s.T, s.window, s.dk, s.cu, s.n_tokens, s.H);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_cache_from_segment(const Shape& s, const void* k, const void* v,
                                     const void* hk, const void* hv, int hlen, long long pos0,
                                     void* ring_k, void* ring_v, hipStream_t st) {
  if (s.B * s.H == 0) return hipSuccess;
  const dim3 grid(s.window, s.B * s.H, 2);  // dk == dv
  if (s.dtype == 1)
    hipLaunchKernelGGL(cache_from_segment_kernel<bf16>, grid, dim3(64), 0, st, (const bf16*)k,
                       (const bf16*)v, (const bf16*)hk, (const bf16*)hv, (bf16*)ring_k,
                       (bf16*)ring_v, s.T, hlen, pos0, s.window, s.dk);
  else
    hipLaunchKernelGGL(cache_from_segment_kernel<float>, grid, dim3(64), 0, st, (const float*)k,
                       (const float*)v, (const float*)hk, (const float*)hv, (float*)ring_k,
                       (float*)ring_v, s.T, hlen, pos0, s.window, s.dk);
  return hipGetLastError();
}

hipError_t launch_decode(const Shape& s, const void* q, const void* k, const void* qw,
                         const void* kw, const void* v, const void* la, float* state,
                         void* ring_k, void* ring_v, int64_t* pos, const void* mk, const void* mv,
                         void* o, hipStream_t st) {
  if (s.B * s.H == 0) return hipSuccess;
  if (s.dtype == 1) {
    if (s.gate == 1) {
      if (s.dk == 128)
        return launch_decode_typed<bf16, 128, bf16>(s, q, k, qw, kw, v, la, state, ring_k, ring_v,
                                                     pos, mk, mv, o, st);
      return launch_decode_typed<bf16, 64, bf16>(s, q, k, qw, kw, v, la, state, ring_k, ring_v,
                                                  pos, mk, mv, o, st);
    }
    if (s.dk == 128)
      return launch_decode_typed<bf16, 128, float>(s, q, k, qw, kw, v, la, state, ring_k, ring_v,
                                                    pos, mk, mv, o, st);
    return launch_decode_typed<bf16, 64, float>(s, q, k, qw, kw, v, la, state, ring_k, ring_v,
                                                 pos, mk, mv, o, st);
  }
  if (s.dk == 128)
    return launch_decode_typed<float, 128, float>(s, q, k, qw, kw, v, la, state, ring_k, ring_v,
                                                  pos, mk, mv, o, st);
  return launch_decode_typed<float, 64, float>(s, q, k, qw, kw, v, la, state, ring_k, ring_v, pos,
                                               mk, mv, o, st);
}

hipError_t launch_ring_fill(const Shape& s, const void* k, const void* v, void* ring_k,
                            void* ring_v, hipStream_t st) {
  if (s.B * s.H == 0) return hipSuccess;
  if (s.dtype == 1) return ring_fill_typed<bf16>(s, k, v, ring_k, ring_v, st);
  return ring_fill_typed<float>(s, k, v, ring_k, ring_v, st);
}

}  // namespace lz
