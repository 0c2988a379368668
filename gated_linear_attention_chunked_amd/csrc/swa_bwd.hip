// Sliding-window + meta-memory attention backward for gfx950.
//
// Reverse mode of the window branch ("Lizard: An Efficient Linearization
// Framework for Large Language Models", gist.science summary, section 2(a):
// anchor window with meta-memory tokens in one softmax), for dO_swa = mix * dO:
//   p = exp(logit - lse_t),  D_t = dO_swa,t . o_swa,t,  ds = p (dO_swa . v - D_t)
//   dq_t += scale sum_j ds_tj key_j,  dk_j += scale sum_t ds_tj q_t,
//   dv_j += sum_t p_tj dO_swa,t,       meta grads summed over batch and time.
// The forward's saved lse and o_swa make every probability recomputable tile by
// tile, so nothing of size T x T is ever formed.
//
// Kernels (deterministic, no float atomics):
//   1. dq   per (head, 64-query tile): D_t, dq, and the tile's meta-gradient
//           partial sums
//   2. dkdv per (head, 64-key tile):   dk, dv
// This branch runs first and writes dq, dk, dv; the GLA branch adds to them.
//   3. meta reduction per head over (batch, tile) in a fixed order
#include "common.hpp"
#include "kernels.hpp"

namespace lz {
namespace {

constexpr int kT = 64;       // tile (queries or keys)
constexpr int kD = 64;       // head size supported by the backward
constexpr int kDP = kD + 8;
constexpr int kTP = kT + 8;
constexpr int kThreads = 256;

// ------------------------------------------------------------------- 1. dq
template <typename T>
__global__ __launch_bounds__(kThreads) void swa_bwd_dq(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ mk, const T* __restrict__ mv, const T* __restrict__ o_swa,
    const float* __restrict__ lse, const T* __restrict__ dO, T* __restrict__ dq,
    float* __restrict__ Dws, float* __restrict__ metap, int T_len, int H, int W, int M,
    float scale, float mix) {
  typedef typename Frag<T>::type F;
  __shared__ __attribute__((aligned(16))) T skt[kT][kDP];   // key tile, row-major
  __shared__ __attribute__((aligned(16))) T svt[kT][kDP];   // value tile, row-major
  __shared__ __attribute__((aligned(16))) T skT[kD][kTP];   // key tile, transposed
  __shared__ __attribute__((aligned(16))) T smk[16][kDP];
  __shared__ __attribute__((aligned(16))) T smv[16][kDP];
  __shared__ __attribute__((aligned(16))) T smkT[kD][40];   // meta keys transposed (slots 16..31 zero)
  __shared__ __attribute__((aligned(16))) T sqT[kD][kTP];   // this tile's queries, transposed
  __shared__ __attribute__((aligned(16))) T sdoT[kD][kTP];  // this tile's dO, transposed
  __shared__ __attribute__((aligned(16))) float slse[kT], sD[kT];
  __shared__ __attribute__((aligned(16))) float red[kD * 2][17];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int ntile = gridDim.x;
  const int logical = xcd_remap(blockIdx.y * ntile + blockIdx.x, ntile * gridDim.y);
  const int bh = logical / ntile, h = bh % H;
  const int tile = logical % ntile;
  const int t0 = tile * kT;
  const int tq = t0 + 16 * wave + r16;  // this lane's query (column of S^T tiles)
  const size_t off = (size_t)bh * T_len * kD;
  const u32 nb = (u32)((size_t)T_len * kD * sizeof(T));
  const Buf bq(q + off, nb), bk(k + off, nb), bv(v + off, nb), bo(o_swa + off, nb),
      bdo(dO + off, nb);
  const float sl2 = scale * kLog2e;

  // per-wave fragments of q and dO (also used as A fragments: same layout)
  F qf[2], df[2];
  float dot = 0.f;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int tl = min(tq, T_len - 1);
    qf[p] = ld8<T>(q + off + (size_t)tl * kD + 32 * p + 8 * g);
    df[p] = ld8<T>(dO + off + (size_t)tl * kD + 32 * p + 8 * g);
    const F of = ld8<T>(o_swa + off + (size_t)tl * kD + 32 * p + 8 * g);
#pragma unroll
    for (int e = 0; e < 8; ++e) dot += to_f(df[p][e]) * to_f(of[e]);
  }
  const float Dt = mix * wave_sum16(dot);
  const float lse2 = (tq < T_len ? lse[(size_t)bh * T_len + tq] : 0.f) * kLog2e;
  if (g == 0) {
    slse[16 * wave + r16] = lse2;
    sD[16 * wave + r16] = Dt;
    if (tq < T_len) Dws[(size_t)bh * T_len + tq] = Dt;
  }

  f32x4 dqT[kD / 16];
#pragma unroll
  for (int ct = 0; ct < kD / 16; ++ct) dqT[ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- meta slots
  if (M > 0) {
    const Buf bmk(mk + (size_t)h * M * kD, (u32)(M * kD * sizeof(T)));
    const Buf bmv(mv + (size_t)h * M * kD, (u32)(M * kD * sizeof(T)));
    stage_rows<T>(&smk[0][0], kDP, bmk, 0, kD, 16, tid, kThreads);
    stage_rows<T>(&smv[0][0], kDP, bmv, 0, kD, 16, tid, kThreads);
    stage_cols<T>(&smkT[0][0], 40, bmk, 0, kD, 32, tid, kThreads);
    stage_cols<T>(&sqT[0][0], kTP, bq, t0, kD, kT, tid, kThreads);
    stage_cols<T>(&sdoT[0][0], kTP, bdo, t0, kD, kT, tid, kThreads);
    __syncthreads();
    // transposed orientation (lane <-> query) for dq
    f32x4 s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      mma(s, ld8<T>(&smk[r16][32 * p + 8 * g]), qf[p]);
      mma(dp, ld8<T>(&smv[r16][32 * p + 8 * g]), df[p]);
    }
    f32x4 ds;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = 4 * g + r < M;
      const float pr = ok ? exp2_fast(s[r] * sl2 - lse2) : 0.f;
      ds[r] = pr * (mix * dp[r] - Dt);
    }
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ct = 0; ct < kD / 16; ++ct)
      mma(dqT[ct], ld4x2<T>(&smkT[16 * ct + r16][4 * g]), pack_acc<T>(ds, zero));
    // slot orientation (lane <-> slot) for the meta gradients of this wave's queries
    f32x4 s2 = {0.f, 0.f, 0.f, 0.f}, dp2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      mma(s2, qf[p], ld8<T>(&smk[r16][32 * p + 8 * g]));
      mma(dp2, df[p], ld8<T>(&smv[r16][32 * p + 8 * g]));
    }
    f32x4 p2, ds2;  // rows t = 16 wave + 4g + r, column slot r16
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tl = 16 * wave + 4 * g + r;
      const bool ok = (r16 < M) && (t0 + tl < T_len);
      p2[r] = ok ? exp2_fast(s2[r] * sl2 - slse[tl]) : 0.f;
      ds2[r] = p2[r] * (mix * dp2[r] - sD[tl]);
    }
    f32x4 mkT[kD / 16], mvT[kD / 16];  // [c = 16ct + 4g + r][slot r16]
#pragma unroll
    for (int ct = 0; ct < kD / 16; ++ct) {
      mkT[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      mvT[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      F aq, ao;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        aq[e] = sqT[16 * ct + r16][16 * wave + 4 * g + e];
        ao[e] = sdoT[16 * ct + r16][16 * wave + 4 * g + e];
        aq[e + 4] = to_t<T>(0.f);
        ao[e + 4] = to_t<T>(0.f);
      }
      mma(mkT[ct], aq, pack_acc<T>(ds2, zero));
      mma(mvT[ct], ao, pack_acc<T>(p2, zero));
    }
    // reduce the four waves' partials in a fixed order: red[c or D + j][slot]
    for (int wv = 0; wv < 4; ++wv) {
      if (wave == wv) {
#pragma unroll
        for (int ct = 0; ct < kD / 16; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int cc = 16 * ct + 4 * g + r;
            const float a = scale * mkT[ct][r], b = mix * mvT[ct][r];
            red[cc][r16] = (wv == 0 ? 0.f : red[cc][r16]) + a;
            red[kD + cc][r16] = (wv == 0 ? 0.f : red[kD + cc][r16]) + b;
          }
      }
      __syncthreads();
    }
    // partial layout per (bh, tile): [M][kD] for meta_k then [M][kD] for meta_v
    float* mp = metap + ((size_t)bh * ntile + tile) * (size_t)M * 2 * kD;
    for (int e = tid; e < M * 2 * kD; e += kThreads) {
      const int which = e / (M * kD), rem = e % (M * kD), i = rem / kD, cc = rem % kD;
      mp[e] = red[which * kD + cc][i];
    }
  }

  // ---- key tiles overlapping [t0 - W + 1, t0 + 63]
  const int first_key = max(0, t0 - W + 1);
  const int last_key = min(T_len - 1, t0 + kT - 1);
  const int tq0 = t0 + 16 * wave;
  for (int kt0 = (first_key / kT) * kT; kt0 <= last_key; kt0 += kT) {
    __syncthreads();
    stage_rows<T>(&skt[0][0], kDP, bk, kt0, kD, kT, tid, kThreads);
    stage_rows<T>(&svt[0][0], kDP, bv, kt0, kD, kT, tid, kThreads);
    stage_cols<T>(&skT[0][0], kTP, bk, kt0, kD, kT, tid, kThreads);
    __syncthreads();
    f32x4 ds[4];
    bool act[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int s_lo = kt0 + 16 * b;
      act[b] = (s_lo + 15 >= tq0 - W + 1) && (s_lo <= tq0 + 15) && (s_lo < T_len);
      ds[b] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (act[b]) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          mma(s, ld8<T>(&skt[16 * b + r16][32 * p + 8 * g]), qf[p]);
          mma(dp, ld8<T>(&svt[16 * b + r16][32 * p + 8 * g]), df[p]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int sk = s_lo + 4 * g + r;
          const bool ok = (sk <= tq) && (sk > tq - W) && (tq < T_len);
          const float pr = ok ? exp2_fast(s[r] * sl2 - lse2) : 0.f;
          ds[b][r] = pr * (mix * dp[r] - Dt);
        }
      }
    }
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      if (act[2 * pp] || act[2 * pp + 1]) {
        const F bf = pack_acc<T>(ds[2 * pp], ds[2 * pp + 1]);
#pragma unroll
        for (int ct = 0; ct < kD / 16; ++ct)
          mma(dqT[ct], ld4x2<T>(&skT[16 * ct + r16][32 * pp + 4 * g]), bf);
      }
    }
  }
  // ---- dq[t][c] = scale * dq^T[c][t]
  if (tq < T_len) {
#pragma unroll
    for (int ct = 0; ct < kD / 16; ++ct)
      st4<T>(dq + off + (size_t)tq * kD + 16 * ct + 4 * g, dqT[ct] * scale);
  }
}

// ----------------------------------------------------------------- 2. dk, dv
template <typename T>
__global__ __launch_bounds__(kThreads) void swa_bwd_dkdv(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ lse, const T* __restrict__ dO, const float* __restrict__ Dws,
    T* __restrict__ dk, T* __restrict__ dv, int T_len, int W, float scale, float mix) {
  typedef typename Frag<T>::type F;
  __shared__ __attribute__((aligned(16))) T sq[kT][kDP];
  __shared__ __attribute__((aligned(16))) T sdo[kT][kDP];
  __shared__ __attribute__((aligned(16))) T sqT[kD][kTP];
  __shared__ __attribute__((aligned(16))) T sdoT[kD][kTP];
  __shared__ __attribute__((aligned(16))) float slse[kT], sD[kT];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int ntile = gridDim.x;
  const int logical = xcd_remap(blockIdx.y * ntile + blockIdx.x, ntile * gridDim.y);
  const int bh = logical / ntile;
  const int s0 = (logical % ntile) * kT;
  const int sk0 = s0 + 16 * wave;      // first key of this wave
  const int sk = sk0 + r16;            // this lane's key (column of the S tiles)
  const size_t off = (size_t)bh * T_len * kD;
  const u32 nb = (u32)((size_t)T_len * kD * sizeof(T));
  const Buf bq(q + off, nb), bdo(dO + off, nb);
  const float sl2 = scale * kLog2e;

  F kf[2], vf[2];
  const int skl = min(sk, T_len - 1);
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    kf[p] = ld8<T>(k + off + (size_t)skl * kD + 32 * p + 8 * g);
    vf[p] = ld8<T>(v + off + (size_t)skl * kD + 32 * p + 8 * g);
  }
  f32x4 dkT[kD / 16], dvT[kD / 16];  // [c or j = 16ct + 4g + r][key r16]
#pragma unroll
  for (int ct = 0; ct < kD / 16; ++ct) {
    dkT[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    dvT[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int last_q = min(T_len - 1, s0 + kT - 1 + W - 1);
  for (int qt0 = s0; qt0 <= last_q; qt0 += kT) {
    __syncthreads();
    stage_rows<T>(&sq[0][0], kDP, bq, qt0, kD, kT, tid, kThreads);
    stage_rows<T>(&sdo[0][0], kDP, bdo, qt0, kD, kT, tid, kThreads);
    stage_cols<T>(&sqT[0][0], kTP, bq, qt0, kD, kT, tid, kThreads);
    stage_cols<T>(&sdoT[0][0], kTP, bdo, qt0, kD, kT, tid, kThreads);
    if (tid < kT) {
      const int t = qt0 + tid;
      slse[tid] = t < T_len ? lse[(size_t)bh * T_len + t] * kLog2e : 0.f;
      sD[tid] = t < T_len ? Dws[(size_t)bh * T_len + t] : 0.f;
    }
    __syncthreads();
    f32x4 P[4], dS[4];
    bool act[4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const int t_lo = qt0 + 16 * qb;
      act[qb] = (t_lo + 15 >= sk0) && (t_lo <= sk0 + 15 + W - 1) && (t_lo < T_len);
      P[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
      dS[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (act[qb]) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          mma(s, ld8<T>(&sq[16 * qb + r16][32 * p + 8 * g]), kf[p]);
          mma(dp, ld8<T>(&sdo[16 * qb + r16][32 * p + 8 * g]), vf[p]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tl = 16 * qb + 4 * g + r, t = qt0 + tl;
          const bool ok = (sk <= t) && (t < sk + W) && (t < T_len) && (sk < T_len);
          const float pr = ok ? exp2_fast(s[r] * sl2 - slse[tl]) : 0.f;
          P[qb][r] = pr;
          dS[qb][r] = pr * (mix * dp[r] - sD[tl]);
        }
      }
    }
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      if (act[2 * pp] || act[2 * pp + 1]) {
        const F bp = pack_acc<T>(P[2 * pp], P[2 * pp + 1]);
        const F bs = pack_acc<T>(dS[2 * pp], dS[2 * pp + 1]);
#pragma unroll
        for (int ct = 0; ct < kD / 16; ++ct) {
          mma(dvT[ct], ld4x2<T>(&sdoT[16 * ct + r16][32 * pp + 4 * g]), bp);
          mma(dkT[ct], ld4x2<T>(&sqT[16 * ct + r16][32 * pp + 4 * g]), bs);
        }
      }
    }
  }
  if (sk < T_len) {
#pragma unroll
    for (int ct = 0; ct < kD / 16; ++ct) {
      st4<T>(dk + off + (size_t)sk * kD + 16 * ct + 4 * g, dkT[ct] * scale);
      st4<T>(dv + off + (size_t)sk * kD + 16 * ct + 4 * g, dvT[ct] * mix);
    }
  }
}

// ----------------------------------------------------------- 3. meta reduce
// Meta gradients: sum of the per-(sequence, query tile) partials, in a fixed
// order (deterministic).  A block takes 64 consecutive entries of one head;
// its 16 thread groups sum interleaved sixteenths of the partials (coalesced,
// up to 16 loads in flight per thread), then a fixed tree adds the 16 sums.
constexpr int kMetaGroups = 16;
__global__ __launch_bounds__(64 * kMetaGroups) void swa_meta_reduce(
    const float* __restrict__ metap, float* __restrict__ dmk, float* __restrict__ dmv, int B,
    int H, int ntiles, int M) {
  const int h = blockIdx.x;
  const int n = M * kD;
  const int i = threadIdx.x & 63;
  const int e = blockIdx.y * 64 + i;
  const int grp = threadIdx.x >> 6;
  const int np = B * ntiles;  // partials of this head: p = b * ntiles + tile
  float s = 0.f;
  if (e < 2 * n) {
    auto at = [&](int p) {
      const int b = p / ntiles, tl = p - b * ntiles;
      return metap[(((size_t)(b * H + h)) * ntiles + tl) * 2 * n + e];
    };
    constexpr int G = kMetaGroups;
    int p = grp;
    for (; p + 15 * G < np; p += 16 * G) {
      float x[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) x[u] = at(p + G * u);
#pragma unroll
      for (int u = 0; u < 16; ++u) s += x[u];
    }
    for (; p < np; p += G) s += at(p);
  }
  __shared__ float part[kMetaGroups][64];
  part[grp][i] = s;
  __syncthreads();
#pragma unroll
  for (int w = kMetaGroups / 2; w >= 1; w >>= 1) {
    if (grp < w) part[grp][i] += part[grp + w][i];
    __syncthreads();
  }
  if (grp == 0 && e < 2 * n) {
    if (e < n) dmk[(size_t)h * n + e] = part[0][i];
    else dmv[(size_t)h * n + e - n] = part[0][i];
  }
}

}  // namespace

size_t swa_bwd_workspace_bytes(const Shape& s) {
  const size_t bh = (size_t)s.B * s.H;
  const size_t nqt = (size_t)(s.T + kT - 1) / kT;
  return bh * s.T * sizeof(float) + bh * nqt * s.n_meta * 2 * kD * sizeof(float);
}

hipError_t launch_swa_bwd(const Shape& s, const void* q, const void* k, const void* v,
                          const void* mk, const void* mv, const void* o_swa, const float* lse,
                          const void* dO, void* dq, void* dk, void* dv, float* dmk, float* dmv,
                          void* ws, hipStream_t st) {
  typedef bf16 T;
  const int BH = s.B * s.H;
  const int nqt = (s.T + kT - 1) / kT;
  float* Dws = (float*)ws;
  float* metap = Dws + (size_t)BH * s.T;
  if (nqt > 0 && BH > 0) {
    hipLaunchKernelGGL(swa_bwd_dq<T>, dim3(nqt, BH), dim3(kThreads), 0, st, (const T*)q,
                       (const T*)k, (const T*)v, (const T*)mk, (const T*)mv, (const T*)o_swa, lse,
                       (const T*)dO, (T*)dq, Dws, metap, s.T, s.H, s.window, s.n_meta, s.scale,
                       s.mix);
    hipLaunchKernelGGL(swa_bwd_dkdv<T>, dim3(nqt, BH), dim3(kThreads), 0, st, (const T*)q,
                       (const T*)k, (const T*)v, lse, (const T*)dO, Dws, (T*)dk, (T*)dv, s.T,
                       s.window, s.scale, s.mix);
  }
  if (s.n_meta > 0 && s.H > 0)
    hipLaunchKernelGGL(swa_meta_reduce, dim3(s.H, (2 * s.n_meta * kD + 63) / 64),
                       dim3(64 * kMetaGroups), 0, st,
                       metap, dmk, dmv, s.B, s.H, nqt, s.n_meta);
  return hipGetLastError();
}

}  // namespace lz
