// Gated linear attention backward, generic form: bf16 at d = 128 and fp32 at
// d = 64 and 128 (bf16 at d = 64 has its own tuned kernels in gla_bwd.hip).
//
// Same mathematics as gla_bwd.hip (reverse mode of the chunked recurrence of
// "Lizard: An Efficient Linearization Framework for Large Language Models",
// gist.science summary, section 2(a), state update; log2-space chunk form with
// 16-token sub-block references): per 64-token chunk c with S_c the state
// entering it, dS_{c+1} the gradient of the state leaving it and b_t the
// in-chunk log2-gate cumsum,
//   dq_t  = (dO_t S_c^T) 2^{b_t} + sum_{s<=t} (dO_t . v_s) k_s 2^{b_t - b_s}
//   dk_s  = (V dS_{c+1}^T)_s 2^{b_last - b_s} + sum_{t>=s} (dO_t . v_s) q_t 2^{b_t - b_s}
//   dv_s  = K^_s dS_{c+1} + sum_{t>=s} A_ts dO_t,   K^_s = k_s 2^{b_last - b_s}
// and the chunk-local gate gradient (see gla_bwd.hip).  The kernels here stage
// their tiles with plain element-wise stores (no lane-pair packing), read the
// two states as row-major rows straight from the workspace, and so work for any
// element type; the scans gate one channel per thread.
#include "common.hpp"
#include "kernels.hpp"

namespace lz {
namespace {

constexpr int kC = 64;
constexpr int kThreads = 256;
constexpr float kFastLog2 = 64.f;  // single-reference bound on the chunk decay (log2)

__host__ __device__ constexpr int pair_of(int i, int j) { return i * (i - 1) / 2 + j; }

// Four consecutive elements of a token row, as floats.
template <typename T> struct Row4;
template <> struct Row4<bf16> {
  u32x2 w;
  __device__ __forceinline__ void load(const Buf& b, u32 elem) { w = ld64v(b, elem * 2); }
  __device__ __forceinline__ float at(int r) const {
    const u32 x = w[r >> 1];
    return (r & 1) ? bf_hi(x) : bf_lo(x);
  }
};
template <> struct Row4<float> {
  u32x4 w;
  __device__ __forceinline__ void load(const Buf& b, u32 elem) { w = b.ld128(elem * 4); }
  __device__ __forceinline__ float at(int r) const { return as_f(w[r]); }
};

template <typename T>
__device__ __forceinline__ f32x4 row4_f(const Row4<T>& x) {
  return f32x4{x.at(0), x.at(1), x.at(2), x.at(3)};
}

// ------------------------------------------------------------------ scans
// Work-groups 0..BH-1 scan one head's chunks c0..c1-1 forward from fstart,
// writing S_c (the state entering chunk c) to slot c - c0; work-groups
// BH..2BH-1 scan them in reverse from rstart, writing dS_{c+1} (the state
// gradient leaving chunk c), and store the gradient entering chunk c0 at rend:
//   S_{c+1} = D_c S_c + K^_c^T V_c,   dS_c = D_c dS_{c+1} + Q^_c^T dO_c,
// D_c = diag(2^{b_last}), K^_s = k_s 2^{b_last - b_s}, Q^_t = q_t 2^{b_t}.
// States are fp32 in registers (16 x 16 tiles spread over the four waves) and
// stored row-major [c][j] in T.  Thread c < D gates channel c of the chunk
// (a serial scan over its 64 tokens); threads D..2D-1 copy value column j.
template <typename T, int D>
struct ScanGenSmem {
  static constexpr int TP = kC + 8;
  T xT[D][TP];  // gated k (or q), transposed [c][t]
  T yT[D][TP];  // v (or dO), transposed [j][t]
  float dec[D];
};

template <typename T, int D, typename GT>
__global__ __launch_bounds__(kThreads) void gla_bwd_scan_gen(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const GT* __restrict__ la, const T* __restrict__ dO, const float* __restrict__ fstart,
    size_t fstride, const float* __restrict__ rstart, float* __restrict__ rend,
    T* __restrict__ S_ws, T* __restrict__ dS_ws, int BH, int T_len, int c0, int c1, int L) {
  constexpr int NB = D / 16;             // 16-row blocks per side
  constexpr int NTW = NB * NB / 4;       // state tiles per wave
  constexpr int KP = kC / 32;
  typedef typename Frag<T>::type F;
  __shared__ __attribute__((aligned(16))) ScanGenSmem<T, D> sm;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int r16 = lane & 15, g = lane >> 4;
  const bool rev = (int)blockIdx.x >= BH;
  const int bh = rev ? blockIdx.x - BH : blockIdx.x;
  const size_t off = (size_t)bh * T_len * D;
  const T* x = (rev ? q : k) + off;
  const T* y = (rev ? dO : v) + off;
  const GT* lg = la + off;

  // tile m of this wave: n = w + 4m, rows 16 (n / NB).., columns 16 (n % NB)..
  f32x4 acc[NTW];
  const float* st = rev ? rstart : fstart;
  const size_t sstride = rev ? (size_t)D * D : fstride;
#pragma unroll
  for (int m = 0; m < NTW; ++m) {
    const int n = w + 4 * m, cb = n / NB, jb = n % NB;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      acc[m][r] = st ? st[(size_t)bh * sstride + (size_t)(16 * cb + 4 * g + r) * D + 16 * jb + r16]
                     : 0.f;
  }
  for (int n = 0; n < c1 - c0; ++n) {
    const int ch = rev ? c1 - 1 - n : c0 + n;
    const int t0 = ch * kC;
    // the state at the chunk boundary, before this chunk's update
    T* dst = (rev ? dS_ws : S_ws) + ((size_t)bh * L + (ch - c0)) * D * D;
#pragma unroll
    for (int m = 0; m < NTW; ++m) {
      const int nn = w + 4 * m, cb = nn / NB, jb = nn % NB;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        dst[(size_t)(16 * cb + 4 * g + r) * D + 16 * jb + r16] = to_t<T>(acc[m][r]);
    }
    if (tid < D) {
      const int c = tid;
      float l2[kC];
      float tot = 0.f;
#pragma unroll
      for (int t = 0; t < kC; ++t) {
        const bool ok = t0 + t < T_len;
        l2[t] = ok ? gate_log2(to_f(lg[(size_t)(t0 + t) * D + c]), GT()) : 0.f;
        tot += l2[t];
      }
      float b = 0.f;
#pragma unroll
      for (int t = 0; t < kC; ++t) {
        b += l2[t];
        const float xv = t0 + t < T_len ? to_f(x[(size_t)(t0 + t) * D + c]) : 0.f;
        sm.xT[c][t] = to_t<T>(xv * exp2_fast(rev ? b : tot - b));
      }
      sm.dec[c] = exp2_fast(tot);
    } else if (tid < 2 * D) {
      const int j = tid - D;
#pragma unroll 8
      for (int t = 0; t < kC; ++t)
        sm.yT[j][t] = t0 + t < T_len ? y[(size_t)(t0 + t) * D + j] : to_t<T>(0.f);
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < NTW; ++m) {
      const int nn = w + 4 * m, cb = nn / NB, jb = nn % NB;
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sm.dec[16 * cb + 4 * g]);
      acc[m] *= d4;
#pragma unroll
      for (int p = 0; p < KP; ++p)
        mma(acc[m], ld8<T>(&sm.xT[16 * cb + r16][32 * p + 8 * g]),
            ld8<T>(&sm.yT[16 * jb + r16][32 * p + 8 * g]));
    }
    __syncthreads();
  }
  // the reverse scan ends with the gradient entering chunk c0
  if (rev && rend) {
#pragma unroll
    for (int m = 0; m < NTW; ++m) {
      const int n = w + 4 * m, cb = n / NB, jb = n % NB;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        rend[(size_t)bh * D * D + (size_t)(16 * cb + 4 * g + r) * D + 16 * jb + r16] = acc[m][r];
    }
  }
}

// --------------------------------------------------- per-chunk gradients
// fp32 at D = 128 ("lean"): the ungated operands (dO and v rows, dO^T, dS^T)
// are read from global memory (L2) instead of LDS, so the gated tiles fit.
template <typename T, int D>
constexpr bool kLean = sizeof(T) == 4 && D == 128;

template <typename T, int D>
struct GenSmem {
  static constexpr int TL = kC * D;  // elements of a [64][D] (or [D][64]) tile
  static constexpr int TU = kLean<T, D> ? 8 : TL;  // the tiles a lean kernel does not keep
  T qg[TL];    // q~ rows [t][c] = q_t 2^{b_t - R_i}
  T kg[TL];    // k~ rows [s][c] = k_s 2^{R_j - b_s}
  T dor[TU];   // dO rows [t][j]
  T vr[TU];    // v rows [s][j]
  T qgT[TL];   // q~ transposed [c][split_pos(t)]
  T kgT[TL];   // k~ transposed [c][split_pos(s)]
  T doT[TU];   // dO transposed [j][split_pos(t)]
  T dST[kLean<T, D> ? 8 : D * D];  // dS_{c+1} transposed [j][c]
  float tot_sx[4][D];  // per-block gate totals; later the suffix totals of dlog_alpha
  float R_sy[4][D];    // sub-block midpoints; later the prefix totals of dlog_alpha
  float Ru[4][D];      // references in use: the midpoints, or 0 on the single-reference path
  float eR[4][D];      // 2^{R_i}
  float elR[4][D];     // 2^{b_last - R_i}
  float vij[6][D];     // 2^{R_i - R_j}, i > j, index pair_of(i, j)
  float bl[D];         // chunk total b_last
  float st[D];         // state term 2^{b_last} sum_j dS_{c+1}[c][j] S_c[c][j]
};

template <int D>
__device__ __forceinline__ int at_r(int row, int col) { return swz_at<D / 8>(row, col); }
__device__ __forceinline__ int at_t(int row, int col) { return swz_at<8>(row, col); }

template <typename T, int D>
__device__ __forceinline__ float pair_factor(const GenSmem<T, D>& sm, int i, int j, int c) {
  return i > j ? sm.vij[pair_of(i, j)][c] : (i == j ? 1.f : 0.f);
}

template <typename T>
__device__ __forceinline__ typename Frag<T>::type scale_halves(typename Frag<T>::type f, float f0,
                                                               float f1) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[e] = to_t<T>(to_f(f[e]) * f0);
    f[e + 4] = to_t<T>(to_f(f[e + 4]) * f1);
  }
  return f;
}

// One work-group per (chunk c0 + blockIdx.x, head): dq, dk (added to what they
// hold when kAddQK, else written), dv (added) and dlog_alpha of the GLA branch.
// Wave w owns token block w in both roles (query for dq, key for dk and dv);
// lane (r16, g) owns token t = 16w + r16 and channels 16ct + 4g + r, the
// accumulator layout of every output tile.
template <bool kAddQK, typename T, int D, typename GT>
__global__ __launch_bounds__(kThreads, 1) void gla_bwd_chunk_gen(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const GT* __restrict__ la, const T* __restrict__ dO, const T* __restrict__ S_ws,
    const T* __restrict__ dS_ws, T* __restrict__ dq, T* __restrict__ dk, T* __restrict__ dv,
    float* __restrict__ dla, int T_len, int c0, int L) {
  constexpr int NCT = D / 16, KP = D / 32;
  typedef typename Frag<T>::type F;
  __shared__ __attribute__((aligned(16))) GenSmem<T, D> sm;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int ch = c0 + blockIdx.x, bh = blockIdx.y;
  const int t0 = ch * kC;
  const size_t off = (size_t)bh * T_len * D;
  const u32 nb = (u32)((size_t)T_len * D * sizeof(T));
  const Buf bq(q + off, nb), bk(k + off, nb), bv(v + off, nb), bdo(dO + off, nb);
  const Buf bla(la + off, (u32)((size_t)T_len * D * sizeof(GT)));
  const T* Sg = S_ws + ((size_t)bh * L + blockIdx.x) * D * D;
  const T* dSg = dS_ws + ((size_t)bh * L + blockIdx.x) * D * D;
  const int t = 16 * w + r16;
  const bool live = t0 + t < T_len;
  const u32 rowe = (u32)(t0 + t) * D;  // element offset of this lane's token row
  const int ts = split_pos(t);
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  constexpr bool lean = kLean<T, D>;
  // fragments of the ungated operands: from LDS, or (lean) from global memory
  // through the buffer views (rows past T read as zero)
  auto gfrag = [&](const Buf& b, int row, int col) {  // 8 fp32 elements of row `row` of the chunk
    F f{};
    if constexpr (lean) {
      const u32 off = (u32)((t0 + row) * D + col) * 4u;
      const u32x4 a = b.ld128(off), c = b.ld128(off + 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[e] = as_f(a[e]);
        f[e + 4] = as_f(c[e]);
      }
    }
    return f;
  };
  auto frag_dor = [&](int row, int col) {
    if constexpr (lean) return gfrag(bdo, row, col);
    else return ld8<T>(&sm.dor[at_r<D>(row, col)]);
  };
  auto frag_vr = [&](int row, int col) {
    if constexpr (lean) return gfrag(bv, row, col);
    else return ld8<T>(&sm.vr[at_r<D>(row, col)]);
  };
  // dO^T[j][tokens at split positions col..col+7]
  auto frag_doT = [&](int j, int col) {
    if constexpr (lean) {
      F f{};
      const int tb = (col & ~31) + 4 * ((col >> 3) & 3);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        f[e] = as_f(bdo.ld32((u32)((t0 + tb + (e & 3) + 16 * (e >> 2)) * D + j) * 4u));
      return f;
    } else {
      return ld8<T>(&sm.doT[at_t(j, col)]);
    }
  };
  // dS_{c+1}^T[j][c..c+7] = dS_{c+1}[c..c+7][j]
  auto frag_dST = [&](int j, int c) {
    if constexpr (lean) {
      F f{};
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = to_f(dSg[(size_t)(c + e) * D + j]);
      return f;
    } else {
      return ld8<T>(&sm.dST[at_r<D>(j, c)]);
    }
  };

  // ---- 0. this lane's token row: gates, q, k; dO and v into their tiles
  float b[NCT][4];
  Row4<T> q4[NCT], k4[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const u32 e = rowe + 16 * ct + 4 * g;
    Gate4<GT> g4;
    g4.load(bla, e);
#pragma unroll
    for (int r = 0; r < 4; ++r) b[ct][r] = gate_row<GT>(g4.log2_at(r), live);
    q4[ct].load(bq, e);
    k4[ct].load(bk, e);
    Row4<T> d4, v4;
    d4.load(bdo, e);
    v4.load(bv, e);
    if constexpr (!lean) {
      const int c = 16 * ct + 4 * g;
      st4<T>(&sm.dor[at_r<D>(t, c)], row4_f(d4));
      st4<T>(&sm.vr[at_r<D>(t, c)], row4_f(v4));
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.doT[at_t(c + r, ts)] = to_t<T>(d4.at(r));
    }
  }
  // dS_{c+1} transposed into LDS: row c of the workspace state, 8 columns at a time
  if constexpr (!lean) {
    for (int e = tid; e < D * D / 8; e += kThreads) {
      const int c = e / (D / 8), j0 = 8 * (e % (D / 8));
      const F x = ld8<T>(dSg + (size_t)c * D + j0);
#pragma unroll
      for (int i = 0; i < 8; ++i) sm.dST[at_r<D>(j0 + i, c)] = x[i];
    }
  }

  // ---- 1. gate cumsum within each 16-token block
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) b[ct][r] += dpp_shr<1>(b[ct][r]);
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) b[ct][r] += dpp_shr<2>(b[ct][r]);
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) b[ct][r] += dpp_shr<4>(b[ct][r]);
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) b[ct][r] += dpp_shr<8>(b[ct][r]);
  if (r16 == 15)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
      *reinterpret_cast<f32x4*>(&sm.tot_sx[w][16 * ct + 4 * g]) =
          f32x4{b[ct][0], b[ct][1], b[ct][2], b[ct][3]};
  __syncthreads();

  // ---- 2. chunk-wide cumsum, references
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    f32x4 pre = zero;
    for (int j = 0; j < w; ++j) pre += *reinterpret_cast<const f32x4*>(&sm.tot_sx[j][16 * ct + 4 * g]);
#pragma unroll
    for (int r = 0; r < 4; ++r) b[ct][r] += pre[r];
    if (r16 == 7)
      *reinterpret_cast<f32x4*>(&sm.R_sy[w][16 * ct + 4 * g]) = f32x4{b[ct][0], b[ct][1], b[ct][2], b[ct][3]};
    if (w == 3 && r16 == 15)
      *reinterpret_cast<f32x4*>(&sm.bl[16 * ct + 4 * g]) = f32x4{b[ct][0], b[ct][1], b[ct][2], b[ct][3]};
  }
  __syncthreads();

  // ---- 3. factor tables; gated q, k tiles (rows and transposes)
  // Single reference (the chunk start) when every channel's chunk decay stays
  // above 2^-kFastLog2; the choice is uniform over the work-group.
  bool slow = false;
  for (int c = lane; c < D; c += 64) slow |= sm.bl[c] < -kFastLog2;
  const bool fast = !__any(slow);
  for (int e = tid; e < 4 * D; e += kThreads) {
    const int c = e % D, x = e / D;
    const float Rx = fast ? 0.f : sm.R_sy[x][c], blc = sm.bl[c];
    sm.Ru[x][c] = Rx;
    sm.eR[x][c] = exp2_fast(Rx);
    sm.elR[x][c] = exp2_fast(blc - Rx);
  }
  for (int e = tid; e < 6 * D; e += kThreads) {
    const int c = e % D, pr = e / D;
    const int pi = pr == 0 ? 1 : pr < 3 ? 2 : 3, pj = pr - pi * (pi - 1) / 2;
    sm.vij[pr][c] = fast ? 1.f : exp2_fast(sm.R_sy[pi][c] - sm.R_sy[pj][c]);
  }
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int c = 16 * ct + 4 * g;
    const f32x4 R4 = fast ? zero : *reinterpret_cast<const f32x4*>(&sm.R_sy[w][c]);
    f32x4 qx, kx;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float fq = b[ct][r] - R4[r];
      qx[r] = q4[ct].at(r) * exp2_fast(fq);
      kx[r] = k4[ct].at(r) * exp2_fast(-fq);
    }
    st4<T>(&sm.qg[at_r<D>(t, c)], qx);
    st4<T>(&sm.kg[at_r<D>(t, c)], kx);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sm.qgT[at_t(c + r, ts)] = to_t<T>(qx[r]);
      sm.kgT[at_t(c + r, ts)] = to_t<T>(kx[r]);
    }
  }
  __syncthreads();

  float X[NCT][4], Y[NCT][4];  // dlog_alpha items: suffix-summed X, prefix-summed Y
  // ---- 4. dq: wave w is query block w
  {
    F dof[KP];
#pragma unroll
    for (int p = 0; p < KP; ++p) dof[p] = frag_dor(t, 32 * p + 8 * g);
    f32x4 dAT[4];  // dA^T[s = 16j + 4g + r][t], strictly s < t
    float dAtt = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dAT[j] = zero;
      if (j <= w) {
#pragma unroll
        for (int p = 0; p < KP; ++p)
          mma(dAT[j], frag_vr(16 * j + r16, 32 * p + 8 * g), dof[p]);
        if (j == w) {
          dAtt = __shfl(dAT[j][r16 & 3], 16 * (r16 >> 2) + r16);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (4 * g + r >= r16) dAT[j][r] = 0.f;
        }
      }
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4 inter = zero, intra = zero;
      const int cl = 16 * ct + r16;
#pragma unroll
      for (int p = 0; p < KP; ++p) mma(inter, ld8<T>(Sg + (size_t)cl * D + 32 * p + 8 * g), dof[p]);
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        if (2 * pp <= w) {
          F af = ld8<T>(&sm.kgT[at_t(cl, 32 * pp + 8 * g)]);
          if (!fast) af = scale_halves<T>(af, pair_factor(sm, w, 2 * pp, cl), pair_factor(sm, w, 2 * pp + 1, cl));
          mma(intra, af, pack_acc<T>(dAT[2 * pp], dAT[2 * pp + 1]));
        }
      }
      const int c = 16 * ct + 4 * g;
      const f32x4 eR4 = *reinterpret_cast<const f32x4*>(&sm.eR[w][c]);
      const f32x4 R4 = *reinterpret_cast<const f32x4*>(&sm.Ru[w][c]);
      f32x4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float od = exp2_fast(b[ct][r] - R4[r]) * (eR4[r] * inter[r] + intra[r]);
        o[r] = od + dAtt * k4[ct].at(r);
        X[ct][r] = q4[ct].at(r) * od;
      }
      if (live) {
        T* dst = dq + off + rowe + c;
        if (kAddQK) o += ld4f<T>(dst);
        st4<T>(dst, o);
      }
    }
  }
  // state term (wave 0)
  if (w == 0) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int cl = 16 * ct + r16;
      float pc = 0.f;
#pragma unroll
      for (int p = 0; p < KP; ++p) {
        const F s8 = ld8<T>(Sg + (size_t)cl * D + 32 * p + 8 * g);
        const F d8 = ld8<T>(dSg + (size_t)cl * D + 32 * p + 8 * g);
#pragma unroll
        for (int e = 0; e < 8; ++e) pc += to_f(s8[e]) * to_f(d8[e]);
      }
      pc += __shfl_xor(pc, 16);
      pc += __shfl_xor(pc, 32);
      if (g == 0) sm.st[cl] = pc * exp2_fast(sm.bl[cl]);
    }
  }
  // ---- 5. dk, dv: wave w is key block w
  {
    F vf[KP], kf[KP];
#pragma unroll
    for (int p = 0; p < KP; ++p) {
      vf[p] = frag_vr(t, 32 * p + 8 * g);
      kf[p] = ld8<T>(&sm.kg[at_r<D>(t, 32 * p + 8 * g)]);
    }
    f32x4 dA[4], Ab[4];  // [t = 16i + 4g + r][s]; dA strictly t > s, A with t >= s
    float dAss = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dA[i] = zero;
      Ab[i] = zero;
      if (i >= w) {
#pragma unroll
        for (int p = 0; p < KP; ++p) {
          mma(dA[i], frag_dor(16 * i + r16, 32 * p + 8 * g), vf[p]);
          F af = ld8<T>(&sm.qg[at_r<D>(16 * i + r16, 32 * p + 8 * g)]);
          if (i > w && !fast) {
            const float* f = &sm.vij[pair_of(i, w)][32 * p + 8 * g];
#pragma unroll
            for (int e = 0; e < 8; ++e) af[e] = to_t<T>(to_f(af[e]) * f[e]);
          }
          mma(Ab[i], af, kf[p]);
        }
        if (i == w) {
          dAss = __shfl(dA[i][r16 & 3], 16 * (r16 >> 2) + r16);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (4 * g + r <= r16) dA[i][r] = 0.f;
            if (4 * g + r < r16) Ab[i][r] = 0.f;
          }
        }
      }
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4 intra = zero, inter = zero;
      const int cl = 16 * ct + r16;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        if (2 * pp + 1 >= w) {
          F af = ld8<T>(&sm.qgT[at_t(cl, 32 * pp + 8 * g)]);
          if (!fast) af = scale_halves<T>(af, pair_factor(sm, 2 * pp, w, cl), pair_factor(sm, 2 * pp + 1, w, cl));
          mma(intra, af, pack_acc<T>(dA[2 * pp], dA[2 * pp + 1]));
        }
      }
#pragma unroll
      for (int p = 0; p < KP; ++p) mma(inter, ld8<T>(dSg + (size_t)cl * D + 32 * p + 8 * g), vf[p]);
      const int c = 16 * ct + 4 * g;
      const f32x4 bl4 = *reinterpret_cast<const f32x4*>(&sm.bl[c]);
      const f32x4 R4 = *reinterpret_cast<const f32x4*>(&sm.Ru[w][c]);
      f32x4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float kv = k4[ct].at(r);
        const float di = exp2_fast(R4[r] - b[ct][r]) * intra[r];
        const float de = exp2_fast(bl4[r] - b[ct][r]) * inter[r];
        o[r] = di + de + dAss * q4[ct].at(r);
        X[ct][r] -= kv * di;
        Y[ct][r] = kv * de;
      }
      if (live) {
        T* dst = dk + off + rowe + c;
        if (kAddQK) o += ld4f<T>(dst);
        st4<T>(dst, o);
      }
    }
    // K^_s = k~_s 2^{b_last - R_w}
    F kh[KP];
#pragma unroll
    for (int p = 0; p < KP; ++p) {
      const float* f = &sm.elR[w][32 * p + 8 * g];
#pragma unroll
      for (int e = 0; e < 8; ++e) kh[p][e] = to_t<T>(to_f(kf[p][e]) * f[e]);
    }
#pragma unroll
    for (int jt = 0; jt < NCT; ++jt) {
      f32x4 acc = zero;
      const int jl = 16 * jt + r16;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
        if (2 * pp + 1 >= w)
          mma(acc, frag_doT(jl, 32 * pp + 8 * g), pack_acc<T>(Ab[2 * pp], Ab[2 * pp + 1]));
#pragma unroll
      for (int p = 0; p < KP; ++p) mma(acc, frag_dST(jl, 32 * p + 8 * g), kh[p]);
      if (live) {
        T* dst = dv + off + rowe + 16 * jt + 4 * g;
        st4<T>(dst, acc + ld4f<T>(dst));
      }
    }
  }
  // ---- 6. dlog_alpha: suffix sums of X and exclusive prefix sums of Y over
  // the chunk, plus the state term
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float xs = X[ct][r], yi = Y[ct][r];
      xs += dpp_shl<1>(xs);
      yi += dpp_shr<1>(yi);
      xs += dpp_shl<2>(xs);
      yi += dpp_shr<2>(yi);
      xs += dpp_shl<4>(xs);
      yi += dpp_shr<4>(yi);
      xs += dpp_shl<8>(xs);
      yi += dpp_shr<8>(yi);
      X[ct][r] = xs;
      Y[ct][r] = yi - Y[ct][r];  // exclusive
      if (r16 == 0) sm.tot_sx[w][16 * ct + 4 * g + r] = xs;
      if (r16 == 15) sm.R_sy[w][16 * ct + 4 * g + r] = yi;
    }
  __syncthreads();
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int c = 16 * ct + 4 * g;
    f32x4 add = *reinterpret_cast<const f32x4*>(&sm.st[c]);
    for (int j = w + 1; j < 4; ++j) add += *reinterpret_cast<const f32x4*>(&sm.tot_sx[j][c]);
    for (int j = 0; j < w; ++j) add += *reinterpret_cast<const f32x4*>(&sm.R_sy[j][c]);
    f32x4 o;
    if constexpr (sizeof(GT) == 2) {
      // with logit gates, d logit = d log(alpha) * sigmoid(-logit)
      Gate4<GT> g4;
      g4.load(bla, rowe + c);
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = (X[ct][r] + Y[ct][r] + add[r]) * gate_dlog(g4.raw_at(r), GT());
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = X[ct][r] + Y[ct][r] + add[r];
    }
    if (live) *reinterpret_cast<f32x4*>(dla + off + rowe + c) = o;
  }
}

template <typename T, int D, typename GT>
void launch_gen(const Shape& s, const void* q, const void* k, const void* v, const void* la,
                const void* dO, const float* fstart, size_t fstride, const float* rstart,
                float* rend, void* dq, void* dk, void* dv, float* dla, void* S_ws, void* dS_ws,
                bool add_qk, int c0, int c1, int L, hipStream_t st) {
  const int BH = s.B * s.H;
  hipLaunchKernelGGL((gla_bwd_scan_gen<T, D, GT>), dim3(2 * BH), dim3(kThreads), 0, st,
                     (const T*)q, (const T*)k, (const T*)v, (const GT*)la, (const T*)dO, fstart,
                     fstride, rstart, rend, (T*)S_ws, (T*)dS_ws, BH, s.T, c0, c1, L);
  auto kern = add_qk ? gla_bwd_chunk_gen<true, T, D, GT> : gla_bwd_chunk_gen<false, T, D, GT>;
  hipLaunchKernelGGL(kern, dim3(c1 - c0, BH), dim3(kThreads), 0, st, (const T*)q, (const T*)k,
                     (const T*)v, (const GT*)la, (const T*)dO, (const T*)S_ws, (const T*)dS_ws,
                     (T*)dq, (T*)dk, (T*)dv, dla, s.T, c0, L);
}

}  // namespace

// Chunks c0..c1-1 of every head: both scans (forward from fstart, per-head
// stride fstride floats, or zero; reverse from rstart or zero, ending in rend
// when given), then the per-chunk gradients.  S_ws and dS_ws hold L states per
// head in the problem's element type.
hipError_t launch_gla_bwd_block_gen(const Shape& s, const void* q, const void* k, const void* v,
                                    const void* la, const void* dO, const float* fstart,
                                    size_t fstride, const float* rstart, float* rend, void* dq,
                                    void* dk, void* dv, float* dla, void* S_ws, void* dS_ws,
                                    bool add_qk, int c0, int c1, int L, hipStream_t st) {
  if (s.dtype == 1) {
    if (s.gate == 1)
      launch_gen<bf16, 128, bf16>(s, q, k, v, la, dO, fstart, fstride, rstart, rend, dq, dk, dv,
                                  dla, S_ws, dS_ws, add_qk, c0, c1, L, st);
    else
      launch_gen<bf16, 128, float>(s, q, k, v, la, dO, fstart, fstride, rstart, rend, dq, dk, dv,
                                   dla, S_ws, dS_ws, add_qk, c0, c1, L, st);
  } else if (s.dk == 128) {
    launch_gen<float, 128, float>(s, q, k, v, la, dO, fstart, fstride, rstart, rend, dq, dk, dv,
                                  dla, S_ws, dS_ws, add_qk, c0, c1, L, st);
  } else {
    launch_gen<float, 64, float>(s, q, k, v, la, dO, fstart, fstride, rstart, rend, dq, dk, dv,
                                 dla, S_ws, dS_ws, add_qk, c0, c1, L, st);
  }
  return hipGetLastError();
}

}  // namespace lz
