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
//   0. bf16, d = 64, w <= 65: one streaming pass per (head, segment) for dq,
//      dk, dv and the segment's meta-gradient partial sums
//   otherwise (bf16 or fp32, d = 64 or 128)
//   1. dq   per (head, segment of 64-query tiles): D_t, dq, and the segment's
//           meta-gradient partial sums
//   2. dkdv per (head, 64-key tile):   dk, dv
// This branch runs first and writes dq, dk, dv; the GLA branch adds to them.
//   3. meta reduction per head over (batch, segment) in a fixed order
// Segments, not tiles, carry the meta partials, so the scratch memory does not
// grow with T; D_t goes to caller memory that is overwritten afterwards.
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>
#include <type_traits>

namespace lz {
namespace {

constexpr int kT = 64;       // tile (queries or keys)
constexpr int kD = 64;       // head size of the streaming kernel
constexpr int kThreads = 256;

// ------------------------------------------------------------------- 1. dq
// One work-group per (head, segment of whole 64-query tiles), walking its
// tiles in order; D = 64 or 128 channels, T = bf16 or float.  Per tile: the
// tile's D_t (kept for the dk/dv kernel in Dws), the meta-slot terms of dq and
// of the meta gradients (summed over the segment's tiles in LDS), then dq over
// the key tiles that the window reaches.
// fp32 at D = 128 does not fit with every tile apart: there the query tiles
// (used only by the meta-slot terms, before the key loop) share their LDS with
// the key and value rows (used only in the key loop), and rows are padded less.
template <typename T, int D>
struct DqSmem {
  static constexpr bool kShare = sizeof(T) == 4 && D == 128;
  static constexpr int DP = D + 8, TP = kT + (kShare ? 4 : 8);
  struct KeyRows {
    T skt[kT][DP];   // key tile, row-major
    T svt[kT][DP];   // value tile, row-major
  };
  struct QueryCols {
    T sqT[D][TP];    // this tile's queries, transposed
    T sdoT[D][TP];   // this tile's dO, transposed
  };
  struct Apart {
    KeyRows kr;
    QueryCols qc;
  };
  union Shared {
    KeyRows kr;
    QueryCols qc;
  };
  typename std::conditional<kShare, Shared, Apart>::type u;
  T skT[D][TP];    // key tile, transposed
  T smk[16][DP];
  T smv[16][DP];
  T smkT[D][40];   // meta keys transposed (slots 16..31 zero)
  float slse[kT], sD[kT];
  float red[2 * D][17];  // meta-gradient sums of the segment: [c or D + j][slot]
};

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void swa_bwd_dq(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ mk, const T* __restrict__ mv, const T* __restrict__ o_swa,
    const float* __restrict__ lse, const T* __restrict__ dO, T* __restrict__ dq,
    float* __restrict__ Dws, float* __restrict__ metap, int T_len, int H, int W, int M,
    float scale, float mix, int per, const T* __restrict__ hk, const T* __restrict__ hv,
    int hlen) {
  constexpr int KP = D / 32, NCT = D / 16;
  constexpr int DP = DqSmem<T, D>::DP, TP = DqSmem<T, D>::TP;
  typedef typename Frag<T>::type F;
  __shared__ __attribute__((aligned(16))) DqSmem<T, D> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int nseg = gridDim.x;
  const int logical = xcd_remap(blockIdx.y * nseg + blockIdx.x, nseg * gridDim.y);
  const int bh = logical / nseg, h = bh % H;
  const int seg = logical % nseg;
  const int ntiles = (T_len + kT - 1) / kT;
  const int i0 = seg * per, i1 = min(ntiles, i0 + per);
  const size_t off = (size_t)bh * T_len * D;
  const u32 nb = (u32)((size_t)T_len * D * sizeof(T));
  const Buf bq(q + off, nb), bk(k + off, nb), bv(v + off, nb), bdo(dO + off, nb);
  const float sl2 = scale * kLog2e;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  if (M > 0) {
    const Buf bmk(mk + (size_t)h * M * D, (u32)(M * D * sizeof(T)));
    const Buf bmv(mv + (size_t)h * M * D, (u32)(M * D * sizeof(T)));
    stage_rows<T>(&sm.smk[0][0], DP, bmk, 0, D, 16, tid, kThreads);
    stage_rows<T>(&sm.smv[0][0], DP, bmv, 0, D, 16, tid, kThreads);
    stage_cols<T>(&sm.smkT[0][0], 40, bmk, 0, D, 32, tid, kThreads);
    for (int e = tid; e < 2 * D * 17; e += kThreads) (&sm.red[0][0])[e] = 0.f;
  }

  for (int tile = i0; tile < i1; ++tile) {
    const int t0 = tile * kT;
    const int tq = t0 + 16 * wave + r16;  // this lane's query (column of S^T tiles)
    // per-wave fragments of q and dO (also used as A fragments: same layout)
    F qf[KP], df[KP];
    float dot = 0.f;
#pragma unroll
    for (int p = 0; p < KP; ++p) {
      const int tl = min(tq, T_len - 1);
      qf[p] = ld8<T>(q + off + (size_t)tl * D + 32 * p + 8 * g);
      df[p] = ld8<T>(dO + off + (size_t)tl * D + 32 * p + 8 * g);
      const F of = ld8<T>(o_swa + off + (size_t)tl * D + 32 * p + 8 * g);
#pragma unroll
      for (int e = 0; e < 8; ++e) dot += to_f(df[p][e]) * to_f(of[e]);
    }
    const float Dt = mix * wave_sum16(dot);
    const float lse2 = (tq < T_len ? lse[(size_t)bh * T_len + tq] : 0.f) * kLog2e;
    __syncthreads();  // the previous tile's LDS reads are done
    if (g == 0) {
      sm.slse[16 * wave + r16] = lse2;
      sm.sD[16 * wave + r16] = Dt;
      if (tq < T_len) Dws[(size_t)bh * T_len + tq] = Dt;
    }

    f32x4 dqT[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) dqT[ct] = zero;

    // ---- meta slots
    if (M > 0) {
      stage_cols<T>(&sm.u.qc.sqT[0][0], TP, bq, t0, D, kT, tid, kThreads);
      stage_cols<T>(&sm.u.qc.sdoT[0][0], TP, bdo, t0, D, kT, tid, kThreads);
      __syncthreads();
      // transposed orientation (lane <-> query) for dq
      f32x4 sc = zero, dp = zero;
#pragma unroll
      for (int p = 0; p < KP; ++p) {
        mma(sc, ld8<T>(&sm.smk[r16][32 * p + 8 * g]), qf[p]);
        mma(dp, ld8<T>(&sm.smv[r16][32 * p + 8 * g]), df[p]);
      }
      f32x4 ds;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = 4 * g + r < M;
        const float pr = ok ? exp2_fast(sc[r] * sl2 - lse2) : 0.f;
        ds[r] = pr * (mix * dp[r] - Dt);
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        mma(dqT[ct], ld4x2<T>(&sm.smkT[16 * ct + r16][4 * g]), pack_acc<T>(ds, zero));
      // slot orientation (lane <-> slot) for the meta gradients of this wave's queries
      f32x4 s2 = zero, dp2 = zero;
#pragma unroll
      for (int p = 0; p < KP; ++p) {
        mma(s2, qf[p], ld8<T>(&sm.smk[r16][32 * p + 8 * g]));
        mma(dp2, df[p], ld8<T>(&sm.smv[r16][32 * p + 8 * g]));
      }
      f32x4 p2, ds2;  // rows t = 16 wave + 4g + r, column slot r16
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tl = 16 * wave + 4 * g + r;
        const bool ok = (r16 < M) && (t0 + tl < T_len);
        p2[r] = ok ? exp2_fast(s2[r] * sl2 - sm.slse[tl]) : 0.f;
        ds2[r] = p2[r] * (mix * dp2[r] - sm.sD[tl]);
      }
      // add the four waves' partials to the segment's sums in a fixed order
      for (int wv = 0; wv < 4; ++wv) {
        if (wave == wv) {
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            f32x4 mkT = zero, mvT = zero;  // [c = 16ct + 4g + r][slot r16]
            F aq, ao;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              aq[e] = sm.u.qc.sqT[16 * ct + r16][16 * wave + 4 * g + e];
              ao[e] = sm.u.qc.sdoT[16 * ct + r16][16 * wave + 4 * g + e];
              aq[e + 4] = to_t<T>(0.f);
              ao[e + 4] = to_t<T>(0.f);
            }
            mma(mkT, aq, pack_acc<T>(ds2, zero));
            mma(mvT, ao, pack_acc<T>(p2, zero));
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int cc = 16 * ct + 4 * g + r;
              sm.red[cc][r16] += scale * mkT[r];
              sm.red[D + cc][r16] += mix * mvT[r];
            }
          }
        }
        __syncthreads();
      }
    }

    // ---- key tiles overlapping [t0 - W + 1, t0 + 63]: first the halo's (rows
    // r at position r - hlen, for queries that reach before the segment), then
    // the segment's own
    const int tq0 = t0 + 16 * wave;
    const int nhalo = (hlen > 0 && t0 < W - 1) ? (hlen - (max(0, t0 - W + 1 + hlen) / kT) * kT + kT - 1) / kT : 0;
    const int first_key = max(0, t0 - W + 1);
    const int last_key = min(T_len - 1, t0 + kT - 1);
    const int kbeg = (first_key / kT) * kT;
    const int nmain = last_key >= kbeg ? (last_key - kbeg) / kT + 1 : 0;
    const Buf bhk(hk + (size_t)bh * hlen * D, (u32)((size_t)hlen * D * sizeof(T)));
    const Buf bhv(hv + (size_t)bh * hlen * D, (u32)((size_t)hlen * D * sizeof(T)));
    const int hbeg = (max(0, t0 - W + 1 + hlen) / kT) * kT;
    for (int it = 0; it < nhalo + nmain; ++it) {
      const bool halo = it < nhalo;
      const int kt0 = halo ? hbeg + it * kT : kbeg + (it - nhalo) * kT;
      __syncthreads();
      stage_rows<T>(&sm.u.kr.skt[0][0], DP, halo ? bhk : bk, kt0, D, kT, tid, kThreads);
      stage_rows<T>(&sm.u.kr.svt[0][0], DP, halo ? bhv : bv, kt0, D, kT, tid, kThreads);
      stage_cols<T>(&sm.skT[0][0], TP, halo ? bhk : bk, kt0, D, kT, tid, kThreads);
      __syncthreads();
      // key positions of this tile's rows (halo rows sit before position 0)
      const int pos0 = halo ? kt0 - hlen : kt0;
      const int rows = halo ? hlen : T_len;
      f32x4 ds[4];
      bool act[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int s_lo = pos0 + 16 * b;
        act[b] = (s_lo + 15 >= tq0 - W + 1) && (s_lo <= tq0 + 15) && (kt0 + 16 * b < rows);
        ds[b] = zero;
        if (act[b]) {
          f32x4 sc = zero, dp = zero;
#pragma unroll
          for (int p = 0; p < KP; ++p) {
            mma(sc, ld8<T>(&sm.u.kr.skt[16 * b + r16][32 * p + 8 * g]), qf[p]);
            mma(dp, ld8<T>(&sm.u.kr.svt[16 * b + r16][32 * p + 8 * g]), df[p]);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int sk = s_lo + 4 * g + r;
            const bool ok = (sk <= tq) && (sk > tq - W) && (tq < T_len) &&
                            (kt0 + 16 * b + 4 * g + r < rows);
            const float pr = ok ? exp2_fast(sc[r] * sl2 - lse2) : 0.f;
            ds[b][r] = pr * (mix * dp[r] - Dt);
          }
        }
      }
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        if (act[2 * pp] || act[2 * pp + 1]) {
          const F bf = pack_acc<T>(ds[2 * pp], ds[2 * pp + 1]);
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct)
            mma(dqT[ct], ld4x2<T>(&sm.skT[16 * ct + r16][32 * pp + 4 * g]), bf);
        }
      }
    }
    // ---- dq[t][c] = scale * dq^T[c][t]
    if (tq < T_len) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        st4<T>(dq + off + (size_t)tq * D + 16 * ct + 4 * g, dqT[ct] * scale);
    }
  }
  // ---- the segment's meta partials: [M][D] for meta_k then [M][D] for meta_v
  if (M > 0) {
    __syncthreads();
    float* mp = metap + ((size_t)bh * nseg + seg) * (size_t)M * 2 * D;
    for (int e = tid; e < M * 2 * D; e += kThreads) {
      const int which = e / (M * D), rem = e % (M * D), i = rem / D, cc = rem % D;
      mp[e] = sm.red[which * D + cc][i];
    }
  }
}

// ----------------------------------------------------------------- 2. dk, dv
// Keys are rows of k, v [B*H, nrows, D] at positions row + kpos (kpos = 0 for
// the segment's own keys, -hlen for the halo); queries are the segment's.  OT is
// the output type (the problem's for the segment, fp32 for the halo).  tdk, tdv
// (nullable, [B*H, tlen, D] fp32) are added to the gradients of the last tlen
// rows.
template <typename T, int D, typename OT = T>
__global__ __launch_bounds__(kThreads) void swa_bwd_dkdv(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ lse, const T* __restrict__ dO, const float* __restrict__ Dws,
    OT* __restrict__ dk, OT* __restrict__ dv, int T_len, int W, float scale, float mix,
    int nrows, int kpos, const float* __restrict__ tdk, const float* __restrict__ tdv, int tlen) {
  constexpr int KP = D / 32, NCT = D / 16;
  constexpr int DP = D + 8, TP = kT + 8;
  typedef typename Frag<T>::type F;
  __shared__ __attribute__((aligned(16))) T sq[kT][DP];
  __shared__ __attribute__((aligned(16))) T sdo[kT][DP];
  __shared__ __attribute__((aligned(16))) T sqT[D][TP];
  __shared__ __attribute__((aligned(16))) T sdoT[D][TP];
  __shared__ __attribute__((aligned(16))) float slse[kT], sD[kT];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int ntile = gridDim.x;
  const int logical = xcd_remap(blockIdx.y * ntile + blockIdx.x, ntile * gridDim.y);
  const int bh = logical / ntile;
  const int s0 = (logical % ntile) * kT + kpos;  // position of the tile's first key
  const int sk0 = s0 + 16 * wave;      // first key of this wave
  const int sk = sk0 + r16;            // this lane's key (column of the S tiles)
  const int krow = sk - kpos;          // its row in k, v
  const size_t off = (size_t)bh * T_len * D;
  const size_t koff = (size_t)bh * nrows * D;
  const u32 nb = (u32)((size_t)T_len * D * sizeof(T));
  const Buf bq(q + off, nb), bdo(dO + off, nb);
  const float sl2 = scale * kLog2e;

  F kf[KP], vf[KP];
  const int skl = min(krow, nrows - 1);
#pragma unroll
  for (int p = 0; p < KP; ++p) {
    kf[p] = ld8<T>(k + koff + (size_t)skl * D + 32 * p + 8 * g);
    vf[p] = ld8<T>(v + koff + (size_t)skl * D + 32 * p + 8 * g);
  }
  f32x4 dkT[NCT], dvT[NCT];  // [c or j = 16ct + 4g + r][key r16]
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    dkT[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    dvT[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int last_q = min(T_len - 1, s0 + kT - 1 + W - 1);
  for (int qt0 = max(s0, 0); qt0 <= last_q; qt0 += kT) {
    __syncthreads();
    stage_rows<T>(&sq[0][0], DP, bq, qt0, D, kT, tid, kThreads);
    stage_rows<T>(&sdo[0][0], DP, bdo, qt0, D, kT, tid, kThreads);
    stage_cols<T>(&sqT[0][0], TP, bq, qt0, D, kT, tid, kThreads);
    stage_cols<T>(&sdoT[0][0], TP, bdo, qt0, D, kT, tid, kThreads);
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
        f32x4 sc = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < KP; ++p) {
          mma(sc, ld8<T>(&sq[16 * qb + r16][32 * p + 8 * g]), kf[p]);
          mma(dp, ld8<T>(&sdo[16 * qb + r16][32 * p + 8 * g]), vf[p]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tl = 16 * qb + 4 * g + r, t = qt0 + tl;
          const bool ok = (sk <= t) && (t < sk + W) && (t < T_len) && (krow < nrows);
          const float pr = ok ? exp2_fast(sc[r] * sl2 - slse[tl]) : 0.f;
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
        for (int ct = 0; ct < NCT; ++ct) {
          mma(dvT[ct], ld4x2<T>(&sdoT[16 * ct + r16][32 * pp + 4 * g]), bp);
          mma(dkT[ct], ld4x2<T>(&sqT[16 * ct + r16][32 * pp + 4 * g]), bs);
        }
      }
    }
  }
  if (krow < nrows) {
    const int trow = krow - (nrows - tlen);  // row of the added gradients, if >= 0
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4 gk = dkT[ct] * scale, gv = dvT[ct] * mix;
      if (tdk && trow >= 0) {
        const size_t to = ((size_t)bh * tlen + trow) * D + 16 * ct + 4 * g;
        gk += *reinterpret_cast<const f32x4*>(tdk + to);
        gv += *reinterpret_cast<const f32x4*>(tdv + to);
      }
      st4<OT>(dk + koff + (size_t)krow * D + 16 * ct + 4 * g, gk);
      st4<OT>(dv + koff + (size_t)krow * D + 16 * ct + 4 * g, gv);
    }
  }
}

// --------------------------------------------- 0. streaming form (w <= 65)
// With w <= 65 the keys of query tile i lie in key tiles i-1 and i, so one
// work-group can walk the key tiles of a segment in order and meet every
// (query, key) pair of the band exactly once.  Step i takes key tile i against
// query tiles i (block A, on and below the diagonal) and i+1 (block B, above
// it): dk_i and dv_i are then complete; dq_i is complete once block A is added
// to what block B of step i-1 left.  A segment starting at tile i0 > 0 first
// runs key tile i0-1 for that carry only.
// Eight waves: wave w owns keys 16(w & 3).. of the key tile (rows in registers,
// one key per lane) against query rows 32(w >> 2).. of both blocks, so every
// wave meets at most three of the 16x16 (query, key) blocks that reach the
// band.  The two waves of a key block swap partial sums through LDS: the first
// completes dk, the second dv.  dS of both blocks passes through LDS for dq,
// which wave w computes for query rows 16(w & 3).. of tile i (waves of group
// i & 1) or tile i+1 (the other group): query tile j's dq is thus made by group
// j & 1 in both steps that touch it, and its block-B part stays in registers.
// Query tiles sit in a two-slot LDS ring (tile j in slot j & 1), loaded one
// step ahead; K^T goes to LDS.
constexpr int kTE = kT * kD;  // elements of one 64 x 64 tile
constexpr int kStreamThreads = 512;

// Tiles use swz64 (64-element rows); a fragment of rows 16a..16a+15 at
// columns 32p + 8g.. is read at 1024 a + fb[p] with fb the lane's base.
struct StreamSmem {
  bf16 qr[2][kTE];   // query rows [t][c]
  bf16 qT[2][kTE];   // queries transposed [c][split_pos(t)]
  bf16 dor[2][kTE];  // dO rows [t][j]
  bf16 doT[2][kTE];  // dO transposed [j][split_pos(t)]
  float lse2[2][kT];  // lse * log2(e)
  float Dt[2][kT];    // mix * (dO . o_swa)
  bf16 kT[kTE];       // key tile transposed [c][s]
  bf16 dsA[kTE];      // dS of block A as [t][s]
  bf16 dsB[kTE];      // dS of block B as [t][s]
  bf16 mkr[16 * kD];  // meta keys [m][c] (rows >= M zero)
  bf16 mvr[16 * kD];  // meta values [m][j]
  bf16 mkT[kD * 16];  // meta keys transposed [c][m], plain
  union {
    f32x4 x[2][4][4][64];  // dk (0) / dv (1) partials: [key block][channel block][lane]
    float red[2 * kD][17];  // final meta-gradient sums
  } u;
};

__global__ __launch_bounds__(kStreamThreads) void swa_bwd_stream(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ mk, const bf16* __restrict__ mv, const bf16* __restrict__ o_swa,
    const float* __restrict__ lse, const bf16* __restrict__ dO, bf16* __restrict__ dq,
    bf16* __restrict__ dk, bf16* __restrict__ dv, float* __restrict__ metap, int T_len, int H,
    int W, int M, float scale, float mix, int per) {
  __shared__ __attribute__((aligned(16))) StreamSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int grp = w >> 2, wl = w & 3;  // query half and key block of this wave
  const int r16 = lane & 15, g = lane >> 4, odd = tid & 1;
  const int seg = blockIdx.x, nseg = gridDim.x, bh = blockIdx.y, h = bh % H;
  const int ntiles = (T_len + kT - 1) / kT;
  const int i0 = seg * per, i1 = min(ntiles, i0 + per);
  const size_t off = (size_t)bh * T_len * kD;
  const u32 nb = (u32)((size_t)T_len * kD * sizeof(bf16));
  const Buf bq(q + off, nb), bk(k + off, nb), bv(v + off, nb), bdo(dO + off, nb),
      bo(o_swa + off, nb), blse(lse + (size_t)bh * T_len, (u32)((size_t)T_len * 4));
  const float sl2 = scale * kLog2e;
  const int fb0 = swz64(r16, 8 * g), fb1 = swz64(r16, 32 + 8 * g);
  auto frag = [&](const bf16* tile, int blk, int p) {
    return ld8<bf16>(tile + 1024 * blk + (p ? fb1 : fb0));
  };

  // meta slots (zero past M)
  if (M > 0) {
    for (int e = tid; e < 16 * kD; e += kStreamThreads) {
      const int m = e / kD, c = e % kD;
      const bf16 kk = m < M ? mk[((size_t)h * M + m) * kD + c] : (bf16)0.f;
      const bf16 vv = m < M ? mv[((size_t)h * M + m) * kD + c] : (bf16)0.f;
      sm.mkr[swz64(m, c)] = kk;
      sm.mvr[swz64(m, c)] = vv;
      sm.mkT[c * 16 + m] = kk;
    }
  }

  // query tile j: rows, transposes, lse and D.  Thread p takes the 16-byte
  // piece of token (p & 1) | 2 (p >> 4), granule (p >> 1) & 7, so neighbouring
  // lanes hold neighbouring tokens of one granule.
  const int pt = (tid & 1) | ((tid >> 4) << 1), po = (tid >> 1) & 7;
  struct QIn {
    u32x4 q, d, o;
    u32 lse;
  };
  auto qload = [&](QIn& x, int j) {
    const u32 e = ((u32)(j * kT + pt) * kD + 8 * po) * 2;
    x.q = bq.ld128(e);
    x.d = bdo.ld128(e);
    x.o = bo.ld128(e);
    x.lse = blse.ld32((u32)(j * kT + (tid & 63)) * 4);
  };
  auto transpose_store = [&](bf16* dstT, const u32x4& x) {
    const u32 w0 = x[0], w1 = x[1], w2 = x[2], w3 = x[3];
    const u32 r0 = dpp_swap1(odd ? w0 : w2), r1 = dpp_swap1(odd ? w1 : w3);
    const u32 f0 = odd ? r0 : w0, f1 = odd ? r1 : w1;  // words of the even token
    const u32 s0 = odd ? w2 : r0, s1 = odd ? w3 : r1;  // words of the odd token
    const int j0 = 8 * po + 4 * odd, tc = split_pos(pt & ~1);
    *reinterpret_cast<u32*>(&dstT[swz64(j0 + 0, tc)]) = lo2(f0, s0);
    *reinterpret_cast<u32*>(&dstT[swz64(j0 + 1, tc)]) = hi2(f0, s0);
    *reinterpret_cast<u32*>(&dstT[swz64(j0 + 2, tc)]) = lo2(f1, s1);
    *reinterpret_cast<u32*>(&dstT[swz64(j0 + 3, tc)]) = hi2(f1, s1);
  };
  auto qstore = [&](const QIn& x, int slot) {
    *reinterpret_cast<u32x4*>(&sm.qr[slot][swz64(pt, 8 * po)]) = x.q;
    *reinterpret_cast<u32x4*>(&sm.dor[slot][swz64(pt, 8 * po)]) = x.d;
    transpose_store(sm.qT[slot], x.q);
    transpose_store(sm.doT[slot], x.d);
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) dot = dot2_bf16(x.d[e], x.o[e], dot);
    // the 8 lanes of one token differ in lane bits 1..3
    dot += __shfl_xor(dot, 2);
    dot += __shfl_xor(dot, 4);
    dot += __shfl_xor(dot, 8);
    if (po == 0) sm.Dt[slot][pt] = mix * dot;
    if (tid < kT) sm.lse2[slot][tid] = as_f(x.lse) * kLog2e;
  };
  // key tile i: lane (r16, g) of wave w holds key 16(w & 3) + r16, channels 32p + 8g..
  struct KIn {
    u32x4 k[2], v[2];
  };
  auto kload = [&](KIn& x, int i) {
    const u32 e = (u32)(i * kT + 16 * wl + r16) * kD;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      x.k[p] = bk.ld128((e + 32 * p + 8 * g) * 2);
      x.v[p] = bv.ld128((e + 32 * p + 8 * g) * 2);
    }
  };
  const int se = 16 * wl + (r16 & ~1);  // even key of this lane's pair
  auto kstore = [&](const KIn& x) {     // K^T [c][s] from key pairs in neighbouring lanes
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const u32 w0 = x.k[p][0], w1 = x.k[p][1], w2 = x.k[p][2], w3 = x.k[p][3];
      const u32 r0 = dpp_swap1(odd ? w0 : w2), r1 = dpp_swap1(odd ? w1 : w3);
      const u32 f0 = odd ? r0 : w0, f1 = odd ? r1 : w1;
      const u32 s0 = odd ? w2 : r0, s1 = odd ? w3 : r1;
      const int j0 = 32 * p + 8 * g + 4 * odd;
      *reinterpret_cast<u32*>(&sm.kT[swz64(j0 + 0, se)]) = lo2(f0, s0);
      *reinterpret_cast<u32*>(&sm.kT[swz64(j0 + 1, se)]) = hi2(f0, s0);
      *reinterpret_cast<u32*>(&sm.kT[swz64(j0 + 2, se)]) = lo2(f1, s1);
      *reinterpret_cast<u32*>(&sm.kT[swz64(j0 + 3, se)]) = hi2(f1, s1);
    }
  };
  // dS of this wave's two 16-row tiles ([t = 16(2grp + u) + 4g + r][s = 16wl +
  // r16]) into a [t][s] tile: neighbouring lanes (keys s, s+1) write (s, s+1)
  // pairs, the even lane rows 4g, 4g+1 and the odd lane rows 4g+2, 4g+3
  auto ds_store = [&](bf16* dst, const f32x4 (&x)[2]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const u32 a01 = pack_bf2(x[u][0], x[u][1]), a23 = pack_bf2(x[u][2], x[u][3]);
      const u32 R = dpp_swap1(odd ? a01 : a23);
      const u32 fst = odd ? R : a01, snd = odd ? a23 : R;
      const int row = 16 * (2 * grp + u) + 4 * g + 2 * odd;
      *reinterpret_cast<u32*>(&dst[swz64(row, se)]) = lo2(fst, snd);
      *reinterpret_cast<u32*>(&dst[swz64(row + 1, se)]) = hi2(fst, snd);
    }
  };

  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 dqc[4];   // block-B part of dq for query rows 16wl.. of this group's next tile
  f32x4 macc[8];  // meta-gradient partials (dk part 0..3, dv part 4..7), quad per lane
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) dqc[ct] = zero;
#pragma unroll
  for (int j = 0; j < 8; ++j) macc[j] = zero;
  const int start = i0 > 0 ? i0 - 1 : i0;
  QIn qx;
  KIn kx;
  bf16x8 kf[2], vf[2];
  qload(qx, start);
  kload(kx, start);
  qstore(qx, start & 1);
  qload(qx, start + 1);
  qstore(qx, (start + 1) & 1);
  if (grp == 0) kstore(kx);
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    kf[p] = as_bf8(kx.k[p]);
    vf[p] = as_bf8(kx.v[p]);
  }
  lds_barrier();

  for (int i = start; i < i1; ++i) {
    const bool pre = i < i0;  // carry-only step for the segment's first query tile
    const int a = i & 1, b = a ^ 1;
    const bool pq = i + 2 <= i1, pk = i + 1 < i1;
    if (pq) qload(qx, i + 2);
    if (pk) kload(kx, i + 1);
    const int s_lo = i * kT + 16 * wl, sg = s_lo + r16;  // this lane's key
    // ---- blocks A (queries of tile i, slot a) and B (tile i+1, slot b), query
    // rows 32grp..32grp+31: scores with the key per lane, dS to LDS for dq, and
    // this wave's part of dk, dv of key tile i
    f32x4 dkT[4], dvT[4];  // [c or j = 16ct + 4g + r][key]
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) dkT[ct] = dvT[ct] = zero;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      if (blk == 0 && pre) continue;
      const int sl = blk == 0 ? a : b;
      f32x4 P[2], dS[2];
      bool act[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int qb = 2 * grp + u;
        P[u] = dS[u] = zero;
        const int t_lo = (i + blk) * kT + 16 * qb;
        act[u] = (blk == 1 || t_lo + 15 >= s_lo) && t_lo - (s_lo + 15) < W && t_lo < T_len &&
                 s_lo < T_len;
        const bool full = (blk == 1 || t_lo > s_lo + 15) && t_lo + 15 - s_lo < W &&
                          t_lo + 15 < T_len && s_lo + 15 < T_len;
        if (act[u]) {
          f32x4 sc = zero, dp = zero;
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            mma(sc, frag(sm.qr[sl], qb, p), kf[p]);
            mma(dp, frag(sm.dor[sl], qb, p), vf[p]);
          }
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sm.lse2[sl][16 * qb + 4 * g]);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sm.Dt[sl][16 * qb + 4 * g]);
          if (full) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float pr = exp2_fast(sc[r] * sl2 - l4[r]);
              P[u][r] = pr;
              dS[u][r] = pr * (mix * dp[r] - d4[r]);
            }
          } else if (t_lo + 15 < T_len && s_lo + 15 < T_len) {
            // query t sees key s when 0 <= t - s < W (one unsigned compare)
            const int dt = t_lo + 4 * g - sg;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const bool ok = (u32)(dt + r) < (u32)W;
              const float pr = ok ? exp2_fast(sc[r] * sl2 - l4[r]) : 0.f;
              P[u][r] = pr;
              dS[u][r] = pr * (mix * dp[r] - d4[r]);
            }
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int t = t_lo + 4 * g + r;
              const bool ok = sg <= t && t - sg < W && t < T_len && sg < T_len;
              const float pr = ok ? exp2_fast(sc[r] * sl2 - l4[r]) : 0.f;
              P[u][r] = pr;
              dS[u][r] = pr * (mix * dp[r] - d4[r]);
            }
          }
        }
      }
      ds_store(blk == 0 ? sm.dsA : sm.dsB, dS);
      if (!pre && (act[0] || act[1])) {
        const bf16x8 bs = pack_acc<bf16>(dS[0], dS[1]);
        const bf16x8 bp = pack_acc<bf16>(P[0], P[1]);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          mma(dkT[ct], frag(sm.qT[sl], ct, grp), bs);
          mma(dvT[ct], frag(sm.doT[sl], ct, grp), bp);
        }
      }
    }
    // the first query half hands over its dv part, the second its dk part
    if (!pre) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) sm.u.x[grp == 0 ? 1 : 0][wl][ct][lane] = grp == 0 ? dvT[ct] : dkT[ct];
    }
    lds_barrier();
    // ---- dk (first query half) or dv (second) of key tile i complete
    if (!pre && sg < T_len) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        if (grp == 0)
          st4<bf16>(dk + off + (size_t)sg * kD + 16 * ct + 4 * g, (dkT[ct] + sm.u.x[0][wl][ct][lane]) * scale);
        else
          st4<bf16>(dv + off + (size_t)sg * kD + 16 * ct + 4 * g, (dvT[ct] + sm.u.x[1][wl][ct][lane]) * mix);
      }
    }
    // ---- dq: group a takes query rows 16wl.. of tile i (block A), the other
    // group those of tile i+1 (block B)
    const bool dqA = grp == a;
    if (!(dqA && pre)) {
      f32x4 dqx[4];  // [c = 16ct + 4g + r][query]
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) dqx[ct] = zero;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const bf16x8 fd = frag(dqA ? sm.dsA : sm.dsB, wl, p);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) mma(dqx[ct], frag(sm.kT, ct, p), fd);
      }
      if (!dqA) {
        // block B: the part of dq that tile i+1 gets from key tile i
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) dqc[ct] = dqx[ct];
      } else {
        const int tl = 16 * wl + r16, tg = i * kT + tl;
        if (M > 0) {
          // meta slots, query per lane: dq term
          bf16x8 qf[2], df[2];
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            qf[p] = frag(sm.qr[a], wl, p);
            df[p] = frag(sm.dor[a], wl, p);
          }
          f32x4 sc = zero, dp = zero;  // [slot 4g + r][query]
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            mma(sc, frag(sm.mkr, 0, p), qf[p]);
            mma(dp, frag(sm.mvr, 0, p), df[p]);
          }
          const float l2 = sm.lse2[a][tl], Dq = sm.Dt[a][tl];
          f32x4 ds;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool ok = 4 * g + r < M && tg < T_len;
            const float pr = ok ? exp2_fast(sc[r] * sl2 - l2) : 0.f;
            ds[r] = pr * (mix * dp[r] - Dq);
          }
          const bf16x8 bds = pack_acc<bf16>(ds, zero);
          const bf16 z = (bf16)0.f;
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) {
            const bf16x4 m4 = *reinterpret_cast<const bf16x4*>(&sm.mkT[(16 * ct + r16) * 16 + 4 * g]);
            mma(dqx[ct], bf16x8{m4[0], m4[1], m4[2], m4[3], z, z, z, z}, bds);
          }
          // slot per lane: this wave's 16 queries' share of the meta gradients
          f32x4 s2 = zero, dp2 = zero;  // [query 16wl + 4g + r][slot r16]
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            mma(s2, qf[p], frag(sm.mkr, 0, p));
            mma(dp2, df[p], frag(sm.mvr, 0, p));
          }
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sm.lse2[a][16 * wl + 4 * g]);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sm.Dt[a][16 * wl + 4 * g]);
          f32x4 p2, ds2;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool ok = r16 < M && i * kT + 16 * wl + 4 * g + r < T_len;
            p2[r] = ok ? exp2_fast(s2[r] * sl2 - l4[r]) : 0.f;
            ds2[r] = p2[r] * (mix * dp2[r] - d4[r]);
          }
          const bf16x8 b2 = pack_acc<bf16>(ds2, zero), bp2 = pack_acc<bf16>(p2, zero);
          // queries 16wl + 4g + e sit at split position 32(wl >> 1) + 8g + 4(wl & 1) + e
          const int fm = swz64(r16, 32 * (wl >> 1) + 8 * g + 4 * (wl & 1));
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) {
            const bf16x4 aq = *reinterpret_cast<const bf16x4*>(&sm.qT[a][1024 * ct + fm]);
            const bf16x4 ao = *reinterpret_cast<const bf16x4*>(&sm.doT[a][1024 * ct + fm]);
            mma(macc[ct], bf16x8{aq[0], aq[1], aq[2], aq[3], z, z, z, z}, b2);
            mma(macc[4 + ct], bf16x8{ao[0], ao[1], ao[2], ao[3], z, z, z, z}, bp2);
          }
        }
        if (tg < T_len) {
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
            st4<bf16>(dq + off + (size_t)tg * kD + 16 * ct + 4 * g, (dqc[ct] + dqx[ct]) * scale);
        }
      }
    }
    lds_barrier();
    // ---- the prefetched tiles into the freed slots
    if (pq) qstore(qx, a);  // query tile i + 2
    if (pk) {
      if (grp == 0) kstore(kx);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        kf[p] = as_bf8(kx.k[p]);
        vf[p] = as_bf8(kx.v[p]);
      }
    }
    lds_barrier();
  }

  // ---- meta partials of this (sequence, segment), waves added in a fixed order
  if (M > 0) {
    for (int wv = 0; wv < 8; ++wv) {
      if (w == wv) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int cc = 16 * ct + 4 * g + r;
            const float x0 = scale * macc[ct][r], x1 = mix * macc[4 + ct][r];
            sm.u.red[cc][r16] = (wv == 0 ? 0.f : sm.u.red[cc][r16]) + x0;
            sm.u.red[kD + cc][r16] = (wv == 0 ? 0.f : sm.u.red[kD + cc][r16]) + x1;
          }
      }
      __syncthreads();
    }
    float* mp = metap + ((size_t)bh * nseg + seg) * (size_t)M * 2 * kD;
    for (int e = tid; e < M * 2 * kD; e += kStreamThreads) {
      const int which = e / (M * kD), rem = e % (M * kD), m = rem / kD, cc = rem % kD;
      mp[e] = sm.u.red[which * kD + cc][m];
    }
  }
}

// ----------------------------------------------------------- 3. meta reduce
// Meta gradients: one block per (head, 64-entry strip), 16 thread groups
// (meta_reduce_strip).
constexpr int kMetaGroups = 16;
__global__ __launch_bounds__(64 * kMetaGroups) void swa_meta_reduce(MetaReduceArgs a) {
  __shared__ float part[kMetaGroups][64];
  meta_reduce_strip<kMetaGroups>(a, blockIdx.x, blockIdx.y, part);
}

// Segments per head of the window backward's work-groups (whole 64-query
// tiles): enough work-groups to fill the chip, at most one per tile.  The
// workspace is sized for the bound that holds for any T.
int swa_bwd_segments(int BH, int nqt) { return std::max(1, std::min(nqt, (256 + BH - 1) / BH)); }

template <typename T, int D>
hipError_t launch_swa_bwd_typed(const Shape& s, const void* q, const void* k, const void* v,
                                const void* mk, const void* mv, const void* o_swa,
                                const float* lse, const void* dO, void* dq, void* dk, void* dv,
                                float* dmk, float* dmv, float* Dws, float* metap,
                                MetaReduceArgs* defer, hipStream_t st) {
  const int BH = s.B * s.H;
  const int nqt = (s.T + kT - 1) / kT;
  int G = swa_bwd_segments(BH, nqt);
  const int per = (nqt + G - 1) / G;
  G = (nqt + per - 1) / per;
  const MetaReduceArgs meta{metap, dmk, dmv, s.B, s.H, G, s.n_meta * D};
  const dim3 mgrid(s.H, (2 * s.n_meta * D + 63) / 64);
  if constexpr (sizeof(T) == 2 && D == 64) {
    if (s.window <= 65 && s.hlen == 0 && s.tlen == 0) {
      // streaming form: B*H*G work-groups, G segments of whole tiles per sequence
      hipLaunchKernelGGL(swa_bwd_stream, dim3(G, BH), dim3(kStreamThreads), 0, st, (const T*)q,
                         (const T*)k, (const T*)v, (const T*)mk, (const T*)mv, (const T*)o_swa,
                         lse, (const T*)dO, (T*)dq, (T*)dk, (T*)dv, metap, s.T, s.H, s.window,
                         s.n_meta, s.scale, s.mix, per);
      // the reduction is left to the caller when it asks (it then runs inside
      // a later launch, beside that launch's own work)
      if (s.n_meta > 0) {
        if (defer)
          *defer = meta;
        else
          hipLaunchKernelGGL(swa_meta_reduce, mgrid, dim3(64 * kMetaGroups), 0, st, meta);
      }
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((swa_bwd_dq<T, D>), dim3(G, BH), dim3(kThreads), 0, st, (const T*)q,
                     (const T*)k, (const T*)v, (const T*)mk, (const T*)mv, (const T*)o_swa, lse,
                     (const T*)dO, (T*)dq, Dws, metap, s.T, s.H, s.window, s.n_meta, s.scale,
                     s.mix, per, (const T*)s.hk, (const T*)s.hv, s.hlen);
  hipLaunchKernelGGL((swa_bwd_dkdv<T, D>), dim3(nqt, BH), dim3(kThreads), 0, st, (const T*)q,
                     (const T*)k, (const T*)v, lse, (const T*)dO, Dws, (T*)dk, (T*)dv, s.T,
                     s.window, s.scale, s.mix, s.T, 0, s.tdk, s.tdv, s.tlen);
  if (s.hlen > 0 && s.dhk)
    hipLaunchKernelGGL((swa_bwd_dkdv<T, D, float>), dim3((s.hlen + kT - 1) / kT, BH),
                       dim3(kThreads), 0, st, (const T*)q, (const T*)s.hk, (const T*)s.hv, lse,
                       (const T*)dO, Dws, s.dhk, s.dhv, s.T, s.window, s.scale, s.mix, s.hlen,
                       -s.hlen, (const float*)nullptr, (const float*)nullptr, 0);
  if (s.n_meta > 0)
    hipLaunchKernelGGL(swa_meta_reduce, mgrid, dim3(64 * kMetaGroups), 0, st, meta);
  return hipGetLastError();
}

}  // namespace

// Meta-gradient partials per (sequence, head, segment); the segment count is
// at most ceil(256 / (B*H)) whatever T is.
size_t swa_bwd_workspace_bytes(const Shape& s) {
  const size_t bh = (size_t)s.B * s.H;
  if (bh == 0) return 0;
  const size_t gmax = (size_t)std::max<size_t>(1, (256 + bh - 1) / bh);
  return bh * gmax * s.n_meta * 2 * s.dk * sizeof(float);
}

// Dws: B*H*T floats of scratch for D_t = mix * dO_t . o_swa,t (the caller passes
// memory it overwrites later, so the workspace does not grow with T).
hipError_t launch_swa_bwd(const Shape& s, const void* q, const void* k, const void* v,
                          const void* mk, const void* mv, const void* o_swa, const float* lse,
                          const void* dO, void* dq, void* dk, void* dv, float* dmk, float* dmv,
                          float* Dws, void* ws, MetaReduceArgs* defer, hipStream_t st) {
  const int BH = s.B * s.H;
  const int nqt = (s.T + kT - 1) / kT;
  if (nqt == 0 || BH == 0) return hipSuccess;
  float* metap = (float*)ws;
  if (s.dtype == 1) {
    if (s.dk == 128)
      return launch_swa_bwd_typed<bf16, 128>(s, q, k, v, mk, mv, o_swa, lse, dO, dq, dk, dv, dmk,
                                             dmv, Dws, metap, defer, st);
    return launch_swa_bwd_typed<bf16, 64>(s, q, k, v, mk, mv, o_swa, lse, dO, dq, dk, dv, dmk,
                                          dmv, Dws, metap, defer, st);
  }
  if (s.dk == 128)
    return launch_swa_bwd_typed<float, 128>(s, q, k, v, mk, mv, o_swa, lse, dO, dq, dk, dv, dmk,
                                            dmv, Dws, metap, defer, st);
  return launch_swa_bwd_typed<float, 64>(s, q, k, v, mk, mv, o_swa, lse, dO, dq, dk, dv, dmk, dmv,
                                         Dws, metap, defer, st);
}

}  // namespace lz
