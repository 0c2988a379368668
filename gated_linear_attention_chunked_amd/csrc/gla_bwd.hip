// Gated linear attention backward for gfx950 (loss = sum(dO * o_gla)).
//
// Reverse mode of the chunked recurrence of "Lizard: An Efficient
// Linearization Framework for Large Language Models" (gist.science summary,
// section 2(a), state update), in the same log2-space chunk form as the
// forward.  With S_c the state entering chunk c, dS_{c+1} the gradient of the
// state leaving it, b_t the in-chunk log2-gate cumsum and D = diag(2^{b_last}):
//   dq_t  = (dO_t S_c^T) * 2^{b_t} + sum_{s<=t} (dO_t . v_s) k_s * 2^{b_t - b_s}
//   dk_s  = (V dS_{c+1}^T)_s * 2^{b_last - b_s} + sum_{t>=s} (dO_t . v_s) q_t * 2^{b_t - b_s}
//   dv_s  = K^_s dS_{c+1} + sum_{t>=s} A_ts dO_t,   K^_s = k_s * 2^{b_last - b_s}
//   dS_c  = D dS_{c+1} + Q^^T dO,                  Q^_t = q_t * 2^{b_t}
// The gate gradient is alpha_u * rowsum(G_u * S_{u-1}) with G_u the state
// gradient after token u.  Expanding G_u and S_{u-1} inside the chunk gives,
// for token u and channel c, only in-chunk sums (no sum over the whole
// sequence, so no large terms that cancel):
//   dlog_alpha_u = sum_{t>=u} q_t (dq_t^inter + dq_t^intra,s<t)
//                - sum_{t>=u} k_t dk_t^intra,t>s
//                + sum_{s<u}  k_s dk_s^inter
//                + 2^{b_last} sum_j dS_{c+1}[c][j] S_c[c][j]
// where "intra,s<t" leaves out the diagonal pair s = t (it cancels exactly and
// is never formed).
//
// Kernels:
//   1. state scan    (per head, forward)  S_c for every chunk  -> workspace
//   2. dstate scan   (per head, reverse)  dS_{c+1} per chunk   -> workspace
//   3. dq            (per head x chunk)   dq, and the q-side and state terms of
//                                          dlog_alpha
//   4. dk, dv        (per head x chunk)   dk, dv, and the k-side terms
// Intra-chunk factors use the forward's 16-token sub-block midpoints R_i.
#include "common.hpp"
#include "kernels.hpp"

namespace lz {
namespace {

constexpr int kC = 64;
constexpr int kD = 64;          // head size supported by the backward
constexpr int kDP = kD + 8;     // padded row (elements)
constexpr int kTP = kC + 8;     // padded token row
constexpr int kThreads = 256;

__host__ __device__ constexpr int pair_of(int i, int j) { return i * (i - 1) / 2 + j; }

// b[t][c] = log2-gate cumsum over rows 0..t of the chunk (rows past T add 0).
// Thread (c, quarter) scans 16 rows; quarter totals are exchanged through tot.
__device__ __forceinline__ void gate_table(float (*bt)[kD + 4], float (*tot)[kD], const Buf& bla,
                                           int t0, int tid) {
  const int c = tid % kD, qtr = tid / kD;
  float loc[16];
  float run = 0.f;
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    const u32 off = (u32)(((t0 + 16 * qtr + rr) * kD + c) * 4);
    run += __builtin_bit_cast(float, bla.ld32(off)) * kLog2e;
    loc[rr] = run;
  }
  tot[qtr][c] = run;
  lds_barrier();
  float pre = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) pre += (j < qtr) ? tot[j][c] : 0.f;
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) bt[16 * qtr + rr][c] = loc[rr] + pre;
}

template <typename T>
__device__ __forceinline__ void scale_run16(T* p, float f0, const float* bcol, float sgn,
                                            float ref) {
  // p[0..15] *= 2^{sgn * (b[t] - ref)} (b read with stride kD + 4)
  typedef typename Frag<T>::type F;
  F a = *reinterpret_cast<F*>(p), b = *reinterpret_cast<F*>(p + 8);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = to_t<T>(to_f(a[e]) * exp2_fast(sgn * (bcol[e * (kD + 4)] - ref)) * f0);
    b[e] = to_t<T>(to_f(b[e]) * exp2_fast(sgn * (bcol[(e + 8) * (kD + 4)] - ref)) * f0);
  }
  *reinterpret_cast<F*>(p) = a;
  *reinterpret_cast<F*>(p + 8) = b;
}

// ---------------------------------------------------------------- 1. states
template <typename T>
__global__ __launch_bounds__(kThreads) void gla_bwd_state_scan(
    const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ la,
    const float* __restrict__ h0, T* __restrict__ S_all, int T_len) {
  typedef typename Frag<T>::type F;
  __shared__ __attribute__((aligned(16))) float bt[kC][kD + 4];
  __shared__ __attribute__((aligned(16))) float tot[4][kD];
  __shared__ __attribute__((aligned(16))) T khT[kD][kTP];
  __shared__ __attribute__((aligned(16))) T vT[kD][kTP];
  __shared__ __attribute__((aligned(16))) float decay[kD];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int c = tid % kD, qtr = tid / kD;
  const int bh = blockIdx.x;
  const size_t off = (size_t)bh * T_len * kD;
  const u32 nb = (u32)((size_t)T_len * kD * sizeof(T));
  const Buf bk(k + off, nb), bv(v + off, nb), bla(la + off, (u32)((size_t)T_len * kD * 4));
  const int nc = (T_len + kC - 1) / kC;
  f32x4 S[kD / 16];
#pragma unroll
  for (int cb = 0; cb < kD / 16; ++cb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      S[cb][r] = h0 ? h0[(size_t)bh * kD * kD + (16 * cb + 4 * g + r) * kD + 16 * wave + r16] : 0.f;
  for (int ch = 0; ch < nc; ++ch) {
    T* dst = S_all + ((size_t)bh * nc + ch) * kD * kD;
#pragma unroll
    for (int cb = 0; cb < kD / 16; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(16 * cb + 4 * g + r) * kD + 16 * wave + r16] = to_t<T>(S[cb][r]);
    stage_cols<T>(&khT[0][0], kTP, bk, ch * kC, kD, kC, tid, kThreads);
    stage_cols<T>(&vT[0][0], kTP, bv, ch * kC, kD, kC, tid, kThreads);
    gate_table(bt, tot, bla, ch * kC, tid);
    lds_barrier();
    const float blast = bt[kC - 1][c];
    scale_run16<T>(&khT[c][16 * qtr], 1.f, &bt[16 * qtr][c], -1.f, blast);
    if (qtr == 0) decay[c] = exp2_fast(blast);
    lds_barrier();
#pragma unroll
    for (int cb = 0; cb < kD / 16; ++cb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) S[cb][r] *= decay[16 * cb + 4 * g + r];
#pragma unroll
      for (int p = 0; p < 2; ++p)
        mma(S[cb], ld8<T>(&khT[16 * cb + r16][32 * p + 8 * g]), ld8<T>(&vT[16 * wave + r16][32 * p + 8 * g]));
    }
    lds_barrier();
  }
}

// --------------------------------------------------------------- 2. dstates
template <typename T>
__global__ __launch_bounds__(kThreads) void gla_bwd_dstate_scan(
    const T* __restrict__ q, const T* __restrict__ dO, const float* __restrict__ la,
    T* __restrict__ dS_all, int T_len) {
  __shared__ __attribute__((aligned(16))) float bt[kC][kD + 4];
  __shared__ __attribute__((aligned(16))) float tot[4][kD];
  __shared__ __attribute__((aligned(16))) T qhT[kD][kTP];
  __shared__ __attribute__((aligned(16))) T dOT[kD][kTP];
  __shared__ __attribute__((aligned(16))) float decay[kD];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int c = tid % kD, qtr = tid / kD;
  const int bh = blockIdx.x;
  const size_t off = (size_t)bh * T_len * kD;
  const u32 nb = (u32)((size_t)T_len * kD * sizeof(T));
  const Buf bq(q + off, nb), bdo(dO + off, nb), bla(la + off, (u32)((size_t)T_len * kD * 4));
  const int nc = (T_len + kC - 1) / kC;
  f32x4 dS[kD / 16];  // dS[16cb + 4g + r][16 wave + r16]
#pragma unroll
  for (int cb = 0; cb < kD / 16; ++cb) dS[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int ch = nc - 1; ch >= 0; --ch) {
    T* dst = dS_all + ((size_t)bh * nc + ch) * kD * kD;
#pragma unroll
    for (int cb = 0; cb < kD / 16; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(16 * cb + 4 * g + r) * kD + 16 * wave + r16] = to_t<T>(dS[cb][r]);
    stage_cols<T>(&qhT[0][0], kTP, bq, ch * kC, kD, kC, tid, kThreads);
    stage_cols<T>(&dOT[0][0], kTP, bdo, ch * kC, kD, kC, tid, kThreads);
    gate_table(bt, tot, bla, ch * kC, tid);
    lds_barrier();
    scale_run16<T>(&qhT[c][16 * qtr], 1.f, &bt[16 * qtr][c], 1.f, 0.f);
    if (qtr == 0) decay[c] = exp2_fast(bt[kC - 1][c]);
    lds_barrier();
#pragma unroll
    for (int cb = 0; cb < kD / 16; ++cb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) dS[cb][r] *= decay[16 * cb + 4 * g + r];
#pragma unroll
      for (int p = 0; p < 2; ++p)
        mma(dS[cb], ld8<T>(&qhT[16 * cb + r16][32 * p + 8 * g]), ld8<T>(&dOT[16 * wave + r16][32 * p + 8 * g]));
    }
    lds_barrier();
  }
}

// Shared per-chunk quantities: midpoints R_i = b[16i+7], pair factors 2^{R_i - R_j}.
struct ChunkRefs {
  float R[4][kD];
  float vij[6][kD];
};

__device__ __forceinline__ void chunk_refs(ChunkRefs& cr, float (*bt)[kD + 4], int tid) {
  const int c = tid % kD, qtr = tid / kD;
  cr.R[qtr][c] = bt[16 * qtr + 7][c];
  // pairs (1,0) (2,0) (2,1) (3,0) (3,1) (3,2) -> indices 0..5; quarter qtr computes qtr and qtr+4
  const int pi[6] = {1, 2, 2, 3, 3, 3}, pj[6] = {0, 0, 1, 0, 1, 2};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int p = qtr + 4 * h;
    if (p < 6) cr.vij[p][c] = exp2_fast(bt[16 * pi[p] + 7][c] - bt[16 * pj[p] + 7][c]);
  }
}

// factor 2^{R_i - R_j} for query block i and key block j (1 on the diagonal, 0 above)
__device__ __forceinline__ float pair_factor(const ChunkRefs& cr, int i, int j, int c) {
  return i > j ? cr.vij[pair_of(i, j)][c] : (i == j ? 1.f : 0.f);
}

// ---------------------------------------------------------------------- 3. dq
template <typename T>
__global__ __launch_bounds__(kThreads) void gla_bwd_dq(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ la, const T* __restrict__ dO, const T* __restrict__ S_all,
    const T* __restrict__ dS_all, T* __restrict__ dq, float* __restrict__ dla, int T_len) {
  typedef typename Frag<T>::type F;
  __shared__ __attribute__((aligned(16))) T sdo[kC][kDP];
  __shared__ __attribute__((aligned(16))) T sv[kC][kDP];
  __shared__ __attribute__((aligned(16))) T sS[kD][kDP];
  __shared__ __attribute__((aligned(16))) T sq[kC][kDP];
  __shared__ __attribute__((aligned(16))) T kgT[kD][kTP];
  __shared__ __attribute__((aligned(16))) T sk[kC][kDP];
  __shared__ __attribute__((aligned(16))) T sdS[kD][kDP];
  __shared__ __attribute__((aligned(16))) float bt[kC][kD + 4];
  __shared__ __attribute__((aligned(16))) float dbt[kC][kD + 4];
  __shared__ __attribute__((aligned(16))) float tot[4][kD];
  __shared__ __attribute__((aligned(16))) ChunkRefs cr;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int c = tid % kD, qtr = tid / kD;
  const int ch = blockIdx.x, bh = blockIdx.y;
  const int nc = gridDim.x, t0 = ch * kC;
  const size_t off = (size_t)bh * T_len * kD;
  const u32 nb = (u32)((size_t)T_len * kD * sizeof(T));
  const Buf bq(q + off, nb), bk(k + off, nb), bv(v + off, nb), bdo(dO + off, nb);
  const Buf bla(la + off, (u32)((size_t)T_len * kD * 4));
  const Buf bS(S_all + ((size_t)bh * nc + ch) * kD * kD, (u32)(kD * kD * sizeof(T)));
  const Buf bdS(dS_all + ((size_t)bh * nc + ch) * kD * kD, (u32)(kD * kD * sizeof(T)));
  stage_rows<T>(&sk[0][0], kDP, bk, t0, kD, kC, tid, kThreads);
  stage_rows<T>(&sdS[0][0], kDP, bdS, 0, kD, kD, tid, kThreads);
  stage_rows<T>(&sdo[0][0], kDP, bdo, t0, kD, kC, tid, kThreads);
  stage_rows<T>(&sv[0][0], kDP, bv, t0, kD, kC, tid, kThreads);
  stage_rows<T>(&sq[0][0], kDP, bq, t0, kD, kC, tid, kThreads);
  stage_rows<T>(&sS[0][0], kDP, bS, 0, kD, kD, tid, kThreads);
  stage_cols<T>(&kgT[0][0], kTP, bk, t0, kD, kC, tid, kThreads);
  gate_table(bt, tot, bla, t0, tid);
  lds_barrier();
  // kg^T[c][s] = k_s 2^{R_j - b_s}, j = block of s (= qtr for this thread's rows)
  scale_run16<T>(&kgT[c][16 * qtr], 1.f, &bt[16 * qtr][c], -1.f, bt[16 * qtr + 7][c]);
  chunk_refs(cr, bt, tid);
  lds_barrier();

  const int w = wave;  // query block
  f32x4 dAT[4];        // dA^T[s = 16j + 4g + r][t = 16w + r16], strictly s < t
  float dAtt = 0.f;    // diagonal dA[t][t] of this lane's query
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    dAT[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (j <= w) {
#pragma unroll
      for (int p = 0; p < 2; ++p)
        mma(dAT[j], ld8<T>(&sv[16 * j + r16][32 * p + 8 * g]), ld8<T>(&sdo[16 * w + r16][32 * p + 8 * g]));
      if (j == w) {
        // lane (col r16, group r16/4) holds the diagonal at element r16 % 4
        dAtt = __shfl(dAT[j][r16 & 3], 16 * (r16 >> 2) + r16);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * g + r >= r16) dAT[j][r] = 0.f;
      }
    }
  }
  const int t = 16 * w + r16;
#pragma unroll
  for (int ct = 0; ct < kD / 16; ++ct) {
    f32x4 inter = {0.f, 0.f, 0.f, 0.f}, intra = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < 2; ++p)
      mma(inter, ld8<T>(&sS[16 * ct + r16][32 * p + 8 * g]), ld8<T>(&sdo[16 * w + r16][32 * p + 8 * g]));
    const int cl = 16 * ct + r16;  // A-fragment row (channel)
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      if (2 * pp <= w) {
        F af = ld4x2<T>(&kgT[cl][32 * pp + 4 * g]);
        const float f0 = pair_factor(cr, w, 2 * pp, cl), f1 = pair_factor(cr, w, 2 * pp + 1, cl);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          af[e] = to_t<T>(to_f(af[e]) * f0);
          af[e + 4] = to_t<T>(to_f(af[e + 4]) * f1);
        }
        mma(intra, af, pack_acc<T>(dAT[2 * pp], dAT[2 * pp + 1]));
      }
    }
    // lane holds rows c = 16ct + 4g + r of dq^T at column t
    const int c0 = 16 * ct + 4 * g;
    const f32x4 b4 = *reinterpret_cast<const f32x4*>(&bt[t][c0]);
    const f32x4 R4 = *reinterpret_cast<const f32x4*>(&cr.R[w][c0]);
    const f32x4 q4 = ld4f<T>(&sq[t][c0]);
    const f32x4 k4 = ld4f<T>(&sk[t][c0]);
    f32x4 dqv, db;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float off_diag = exp2_fast(b4[r] - R4[r]) * (exp2_fast(R4[r]) * inter[r] + intra[r]);
      dqv[r] = off_diag + dAtt * k4[r];
      db[r] = q4[r] * off_diag;
    }
    if (t0 + t < T_len) st4<T>(dq + off + (size_t)(t0 + t) * kD + c0, dqv);
    *reinterpret_cast<f32x4*>(&dbt[t][c0]) = db;
  }
  lds_barrier();
  // ---- dlog_alpha, q side: in-chunk suffix sums plus the state term
  {
    float st = 0.f;
    for (int j = 0; j < kD; ++j) st += to_f(sdS[c][j]) * to_f(sS[c][j]);
    st *= exp2_fast(bt[kC - 1][c]);
    float loc[16];
    float run = 0.f;
#pragma unroll
    for (int rr = 15; rr >= 0; --rr) {
      run += dbt[16 * qtr + rr][c];
      loc[rr] = run;
    }
    tot[qtr][c] = run;
    lds_barrier();
    float post = st;
#pragma unroll
    for (int j = 0; j < 4; ++j) post += (j > qtr) ? tot[j][c] : 0.f;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int tt = t0 + 16 * qtr + rr;
      if (tt < T_len) dla[off + (size_t)tt * kD + c] = loc[rr] + post;
    }
  }
}

// ------------------------------------------------------------------ 4. dk, dv
template <typename T>
__global__ __launch_bounds__(kThreads) void gla_bwd_dkdv(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ la, const T* __restrict__ dO, const T* __restrict__ dS_all,
    T* __restrict__ dk, T* __restrict__ dv, float* __restrict__ dla, int T_len) {
  typedef typename Frag<T>::type F;
  __shared__ __attribute__((aligned(16))) T sdo[kC][kDP];
  __shared__ __attribute__((aligned(16))) T dOT[kD][kTP];
  __shared__ __attribute__((aligned(16))) T sv[kC][kDP];
  __shared__ __attribute__((aligned(16))) T qg[kC][kDP];
  __shared__ __attribute__((aligned(16))) T qgT[kD][kTP];
  __shared__ __attribute__((aligned(16))) T kg[kC][kDP];
  __shared__ __attribute__((aligned(16))) T sk[kC][kDP];
  __shared__ __attribute__((aligned(16))) T sdS[kD][kDP];
  __shared__ __attribute__((aligned(16))) T dST[kD][kDP];
  __shared__ __attribute__((aligned(16))) float bt[kC][kD + 4];
  __shared__ __attribute__((aligned(16))) T sq[kC][kDP];
  __shared__ __attribute__((aligned(16))) float dbs[kC][kD + 4];  // k dk^intra, t > s
  __shared__ __attribute__((aligned(16))) float dbp[kC][kD + 4];  // k dk^inter
  __shared__ __attribute__((aligned(16))) float tot[4][kD];
  __shared__ __attribute__((aligned(16))) float tot2[4][kD];
  __shared__ __attribute__((aligned(16))) float elR[4][kD];  // 2^{b_last - R_j}
  __shared__ __attribute__((aligned(16))) ChunkRefs cr;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int c = tid % kD, qtr = tid / kD;
  const int ch = blockIdx.x, bh = blockIdx.y;
  const int nc = gridDim.x, t0 = ch * kC;
  const size_t off = (size_t)bh * T_len * kD;
  const u32 nb = (u32)((size_t)T_len * kD * sizeof(T));
  const Buf bq(q + off, nb), bk(k + off, nb), bv(v + off, nb), bdo(dO + off, nb);
  const Buf bla(la + off, (u32)((size_t)T_len * kD * 4));
  const Buf bdS(dS_all + ((size_t)bh * nc + ch) * kD * kD, (u32)(kD * kD * sizeof(T)));
  stage_rows<T>(&sdo[0][0], kDP, bdo, t0, kD, kC, tid, kThreads);
  stage_cols<T>(&dOT[0][0], kTP, bdo, t0, kD, kC, tid, kThreads);
  stage_rows<T>(&sv[0][0], kDP, bv, t0, kD, kC, tid, kThreads);
  stage_rows<T>(&qg[0][0], kDP, bq, t0, kD, kC, tid, kThreads);
  stage_rows<T>(&sq[0][0], kDP, bq, t0, kD, kC, tid, kThreads);
  stage_cols<T>(&qgT[0][0], kTP, bq, t0, kD, kC, tid, kThreads);
  stage_rows<T>(&kg[0][0], kDP, bk, t0, kD, kC, tid, kThreads);
  stage_rows<T>(&sk[0][0], kDP, bk, t0, kD, kC, tid, kThreads);
  stage_rows<T>(&sdS[0][0], kDP, bdS, 0, kD, kD, tid, kThreads);
  stage_cols<T>(&dST[0][0], kDP, bdS, 0, kD, kD, tid, kThreads);
  gate_table(bt, tot, bla, t0, tid);
  lds_barrier();
  {
    const float Rq = bt[16 * qtr + 7][c];
    const float blast = bt[kC - 1][c];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int t = 16 * qtr + rr;
      const float d = bt[t][c] - Rq;
      qg[t][c] = to_t<T>(to_f(qg[t][c]) * exp2_fast(d));
      kg[t][c] = to_t<T>(to_f(kg[t][c]) * exp2_fast(-d));
    }
    scale_run16<T>(&qgT[c][16 * qtr], 1.f, &bt[16 * qtr][c], 1.f, Rq);
    elR[qtr][c] = exp2_fast(blast - Rq);
    chunk_refs(cr, bt, tid);
  }
  lds_barrier();

  const int w = wave;  // key block
  f32x4 dA[4], Ab[4];  // [t = 16i + 4g + r][s = 16w + r16]; dA strictly t > s
  float dAss = 0.f;    // diagonal dA[s][s] of this lane's key
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dA[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    Ab[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (i >= w) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        mma(dA[i], ld8<T>(&sdo[16 * i + r16][32 * p + 8 * g]), ld8<T>(&sv[16 * w + r16][32 * p + 8 * g]));
        F af = ld8<T>(&qg[16 * i + r16][32 * p + 8 * g]);
        if (i > w) {
          const float* f = &cr.vij[pair_of(i, w)][32 * p + 8 * g];
#pragma unroll
          for (int e = 0; e < 8; ++e) af[e] = to_t<T>(to_f(af[e]) * f[e]);
        }
        mma(Ab[i], af, ld8<T>(&kg[16 * w + r16][32 * p + 8 * g]));
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
  const int s = 16 * w + r16;  // this lane's key (column of the accumulators)
  // ---- dk^T[c][s]
#pragma unroll
  for (int ct = 0; ct < kD / 16; ++ct) {
    f32x4 intra = {0.f, 0.f, 0.f, 0.f}, inter = {0.f, 0.f, 0.f, 0.f};
    const int cl = 16 * ct + r16;
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      if (2 * pp + 1 >= w) {
        F af = ld4x2<T>(&qgT[cl][32 * pp + 4 * g]);
        const float f0 = pair_factor(cr, 2 * pp, w, cl), f1 = pair_factor(cr, 2 * pp + 1, w, cl);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          af[e] = to_t<T>(to_f(af[e]) * f0);
          af[e + 4] = to_t<T>(to_f(af[e + 4]) * f1);
        }
        mma(intra, af, pack_acc<T>(dA[2 * pp], dA[2 * pp + 1]));
      }
    }
#pragma unroll
    for (int p = 0; p < 2; ++p)
      mma(inter, ld8<T>(&sdS[cl][32 * p + 8 * g]), ld8<T>(&sv[16 * w + r16][32 * p + 8 * g]));
    const int c0 = 16 * ct + 4 * g;
    const f32x4 b4 = *reinterpret_cast<const f32x4*>(&bt[s][c0]);
    const f32x4 R4 = *reinterpret_cast<const f32x4*>(&cr.R[w][c0]);
    const f32x4 k4 = ld4f<T>(&sk[s][c0]);
    const f32x4 q4 = ld4f<T>(&sq[s][c0]);
    f32x4 dkv, bs, bp;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float bl = bt[kC - 1][c0 + r];
      const float di = exp2_fast(R4[r] - b4[r]) * intra[r];
      const float de = exp2_fast(bl - b4[r]) * inter[r];
      dkv[r] = di + de + dAss * q4[r];
      bs[r] = k4[r] * di;
      bp[r] = k4[r] * de;
    }
    if (t0 + s < T_len) st4<T>(dk + off + (size_t)(t0 + s) * kD + c0, dkv);
    *reinterpret_cast<f32x4*>(&dbs[s][c0]) = bs;
    *reinterpret_cast<f32x4*>(&dbp[s][c0]) = bp;
  }
  // ---- dv^T[j][s]
#pragma unroll
  for (int jt = 0; jt < kD / 16; ++jt) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int jl = 16 * jt + r16;
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
      if (2 * pp + 1 >= w) mma(acc, ld4x2<T>(&dOT[jl][32 * pp + 4 * g]), pack_acc<T>(Ab[2 * pp], Ab[2 * pp + 1]));
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      F bf = ld8<T>(&kg[16 * w + r16][32 * p + 8 * g]);
      const float* f = &elR[w][32 * p + 8 * g];
#pragma unroll
      for (int e = 0; e < 8; ++e) bf[e] = to_t<T>(to_f(bf[e]) * f[e]);
      mma(acc, ld8<T>(&dST[jl][32 * p + 8 * g]), bf);
    }
    if (t0 + s < T_len) st4<T>(dv + off + (size_t)(t0 + s) * kD + 16 * jt + 4 * g, acc);
  }
  lds_barrier();
  // ---- dlog_alpha, k side: minus the suffix sums of dbs, plus the exclusive
  // prefix sums of dbp, added to the q-side terms already in dlog_alpha
  {
    float suf[16], pre[16];
    float rs = 0.f, rp = 0.f;
#pragma unroll
    for (int rr = 15; rr >= 0; --rr) {
      rs += dbs[16 * qtr + rr][c];
      suf[rr] = rs;
    }
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      pre[rr] = rp;
      rp += dbp[16 * qtr + rr][c];
    }
    tot[qtr][c] = rs;
    tot2[qtr][c] = rp;
    lds_barrier();
    float after = 0.f, before = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      after += (j > qtr) ? tot[j][c] : 0.f;
      before += (j < qtr) ? tot2[j][c] : 0.f;
    }
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int t = t0 + 16 * qtr + rr;
      if (t < T_len) {
        float* p = dla + off + (size_t)t * kD + c;
        *p = *p - (suf[rr] + after) + (pre[rr] + before);
      }
    }
  }
}

}  // namespace

size_t gla_bwd_workspace_bytes(const Shape& s) {
  const size_t nc = (size_t)(s.T + kC - 1) / kC;
  const size_t bh = (size_t)s.B * s.H;
  return 2 * bh * nc * kD * kD * sizeof(bf16);
}

hipError_t launch_gla_bwd(const Shape& s, const void* q, const void* k, const void* v,
                          const float* la, const float* h0, const void* dO, void* dq, void* dk,
                          void* dv, float* dla, void* ws, hipStream_t st) {
  typedef bf16 T;
  const int nc = (s.T + kC - 1) / kC;
  const int BH = s.B * s.H;
  if (nc == 0 || BH == 0) return hipSuccess;
  T* S_all = (T*)ws;
  T* dS_all = S_all + (size_t)BH * nc * kD * kD;
  hipLaunchKernelGGL(gla_bwd_state_scan<T>, dim3(BH), dim3(kThreads), 0, st, (const T*)k,
                     (const T*)v, la, h0, S_all, s.T);
  hipLaunchKernelGGL(gla_bwd_dstate_scan<T>, dim3(BH), dim3(kThreads), 0, st, (const T*)q,
                     (const T*)dO, la, dS_all, s.T);
  hipLaunchKernelGGL(gla_bwd_dq<T>, dim3(nc, BH), dim3(kThreads), 0, st, (const T*)q, (const T*)k,
                     (const T*)v, la, (const T*)dO, (const T*)S_all, (const T*)dS_all, (T*)dq,
                     dla, s.T);
  hipLaunchKernelGGL(gla_bwd_dkdv<T>, dim3(nc, BH), dim3(kThreads), 0, st, (const T*)q,
                     (const T*)k, (const T*)v, la, (const T*)dO, (const T*)dS_all, (T*)dk, (T*)dv,
                     dla, s.T);
  return hipGetLastError();
}

}  // namespace lz
