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
//   0. w <= 65: one streaming pass per (head, segment) for dq, dk, dv and the
//      segment's meta-gradient partial sums
//   otherwise
//   1. dq   per (head, 64-query tile): D_t, dq, and the tile's meta-gradient
//           partial sums
//   2. dkdv per (head, 64-key tile):   dk, dv
// This branch runs first and writes dq, dk, dv; the GLA branch adds to them.
//   3. meta reduction per head over (batch, tile) in a fixed order
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

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

// --------------------------------------------- 0. streaming form (w <= 65)
// With w <= 65 the keys of query tile i lie in key tiles i-1 and i, so one
// work-group can walk the key tiles of a segment in order and meet every
// (query, key) pair of the band exactly once.  Step i takes key tile i against
// query tiles i (block A, on and below the diagonal) and i+1 (block B, above
// it): dk_i and dv_i are then complete; dq_i is complete once block A is added
// to what block B of step i-1 left; block B's dq part carries to step i+1.  A
// segment starting at tile i0 > 0 first runs key tile i0-1 for that carry only.
// Query tiles sit in a two-slot LDS ring (tile j in slot j & 1), loaded one
// step ahead; the key tile's rows stay in registers (one key per lane) and its
// transpose goes to LDS.  dS of both blocks passes through LDS for dq.
constexpr int kTE = kT * kD;  // elements of one 64 x 64 tile

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
  f32x4 macc[4][8][64];  // per wave: meta-gradient partials, quad j of lane l at [j][l]
  float red[2 * kD][17];
};

__global__ __launch_bounds__(kThreads) void swa_bwd_stream(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ mk, const bf16* __restrict__ mv, const bf16* __restrict__ o_swa,
    const float* __restrict__ lse, const bf16* __restrict__ dO, bf16* __restrict__ dq,
    bf16* __restrict__ dk, bf16* __restrict__ dv, float* __restrict__ metap, int T_len, int H,
    int W, int M, float scale, float mix, int per) {
  __shared__ __attribute__((aligned(16))) StreamSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
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
    for (int e = tid; e < 16 * kD; e += kThreads) {
      const int m = e / kD, c = e % kD;
      const bf16 kk = m < M ? mk[((size_t)h * M + m) * kD + c] : (bf16)0.f;
      const bf16 vv = m < M ? mv[((size_t)h * M + m) * kD + c] : (bf16)0.f;
      sm.mkr[swz64(m, c)] = kk;
      sm.mvr[swz64(m, c)] = vv;
      sm.mkT[c * 16 + m] = kk;
    }
  }

  // query tile j: rows, transposes, lse and D.  Piece p of the 512 16-byte
  // pieces is token (p & 1) | 2 (p >> 4), granule (p >> 1) & 7, so neighbouring
  // lanes hold neighbouring tokens of one granule.
  int pt[2], po[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int p = tid + kThreads * hh;
    pt[hh] = (p & 1) | ((p >> 4) << 1);
    po[hh] = (p >> 1) & 7;
  }
  struct QIn {
    u32x4 q[2], d[2], o[2];
    u32 lse;
  };
  auto qload = [&](QIn& x, int j) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const u32 e = ((u32)(j * kT + pt[hh]) * kD + 8 * po[hh]) * 2;
      x.q[hh] = bq.ld128(e);
      x.d[hh] = bdo.ld128(e);
      x.o[hh] = bo.ld128(e);
    }
    x.lse = blse.ld32((u32)(j * kT + (tid & 63)) * 4);
  };
  auto transpose_store = [&](bf16* dstT, const u32x4& x, int hh) {
    const u32 w0 = x[0], w1 = x[1], w2 = x[2], w3 = x[3];
    const u32 r0 = dpp_swap1(odd ? w0 : w2), r1 = dpp_swap1(odd ? w1 : w3);
    const u32 f0 = odd ? r0 : w0, f1 = odd ? r1 : w1;  // words of the even token
    const u32 s0 = odd ? w2 : r0, s1 = odd ? w3 : r1;  // words of the odd token
    const int j0 = 8 * po[hh] + 4 * odd, tc = split_pos(pt[hh] & ~1);
    *reinterpret_cast<u32*>(&dstT[swz64(j0 + 0, tc)]) = lo2(f0, s0);
    *reinterpret_cast<u32*>(&dstT[swz64(j0 + 1, tc)]) = hi2(f0, s0);
    *reinterpret_cast<u32*>(&dstT[swz64(j0 + 2, tc)]) = lo2(f1, s1);
    *reinterpret_cast<u32*>(&dstT[swz64(j0 + 3, tc)]) = hi2(f1, s1);
  };
  auto qstore = [&](const QIn& x, int slot) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      *reinterpret_cast<u32x4*>(&sm.qr[slot][swz64(pt[hh], 8 * po[hh])]) = x.q[hh];
      *reinterpret_cast<u32x4*>(&sm.dor[slot][swz64(pt[hh], 8 * po[hh])]) = x.d[hh];
      transpose_store(sm.qT[slot], x.q[hh], hh);
      transpose_store(sm.doT[slot], x.d[hh], hh);
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dot += bf_at(x.d[hh], e) * bf_at(x.o[hh], e);
      // the 8 lanes of one token differ in lane bits 1..3
      dot += __shfl_xor(dot, 2);
      dot += __shfl_xor(dot, 4);
      dot += __shfl_xor(dot, 8);
      if (po[hh] == 0) sm.Dt[slot][pt[hh]] = mix * dot;
    }
    if (tid < kT) sm.lse2[slot][tid] = as_f(x.lse) * kLog2e;
  };
  // key tile i: lane (r16, g) of wave w holds key 16w + r16, channels 32p + 8g..
  struct KIn {
    u32x4 k[2], v[2];
  };
  auto kload = [&](KIn& x, int i) {
    const u32 e = (u32)(i * kT + 16 * w + r16) * kD;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      x.k[p] = bk.ld128((e + 32 * p + 8 * g) * 2);
      x.v[p] = bv.ld128((e + 32 * p + 8 * g) * 2);
    }
  };
  const int se = 16 * w + (r16 & ~1);  // even key of this lane's pair
  auto kstore = [&](const KIn& x) {    // K^T [c][s] from key pairs in neighbouring lanes
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
  // dS of four 16-row tiles ([t = 16qb + 4g + r][s = 16w + r16]) into a [t][s]
  // tile: neighbouring lanes (keys s, s+1) write (s, s+1) pairs, the even lane
  // rows 4g, 4g+1 and the odd lane rows 4g+2, 4g+3
  auto ds_store = [&](bf16* dst, const f32x4 (&x)[4]) {
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const u32 a01 = pack_bf2(x[qb][0], x[qb][1]), a23 = pack_bf2(x[qb][2], x[qb][3]);
      const u32 R = dpp_swap1(odd ? a01 : a23);
      const u32 fst = odd ? R : a01, snd = odd ? a23 : R;
      const int row = 16 * qb + 4 * g + 2 * odd;
      *reinterpret_cast<u32*>(&dst[swz64(row, se)]) = lo2(fst, snd);
      *reinterpret_cast<u32*>(&dst[swz64(row + 1, se)]) = hi2(fst, snd);
    }
  };

  f32x4 dqc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) dqc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 8; ++j) sm.macc[w][j][lane] = f32x4{0.f, 0.f, 0.f, 0.f};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  const int start = i0 > 0 ? i0 - 1 : i0;
  QIn qx;
  KIn kx;
  bf16x8 kf[2], vf[2];
  qload(qx, start);
  kload(kx, start);
  qstore(qx, start & 1);
  qload(qx, start + 1);
  qstore(qx, (start + 1) & 1);
  kstore(kx);
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
    const int s_lo = i * kT + 16 * w, sg = s_lo + r16;  // this lane's key
    // ---- block A (queries of tile i, slot a), then block B (tile i+1, slot b):
    // scores with the key per lane, dS to LDS for dq, and dk, dv of key tile i
    f32x4 dkT[4], dvT[4];  // [c or j = 16ct + 4g + r][key]
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) dkT[ct] = dvT[ct] = zero;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      if (blk == 0 && pre) continue;
      const int sl = blk == 0 ? a : b;
      f32x4 P[4], dS[4];
      bool act[4];
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        P[qb] = dS[qb] = zero;
        const int t_lo = (i + blk) * kT + 16 * qb;
        act[qb] = (blk == 1 || t_lo + 15 >= s_lo) && t_lo - (s_lo + 15) < W && t_lo < T_len &&
                  s_lo < T_len;
        const bool full = (blk == 1 || t_lo > s_lo + 15) && t_lo + 15 - s_lo < W &&
                          t_lo + 15 < T_len && s_lo + 15 < T_len;
        if (act[qb]) {
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
              P[qb][r] = pr;
              dS[qb][r] = pr * (mix * dp[r] - d4[r]);
            }
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int t = t_lo + 4 * g + r;
              const bool ok = sg <= t && t - sg < W && t < T_len && sg < T_len;
              const float pr = ok ? exp2_fast(sc[r] * sl2 - l4[r]) : 0.f;
              P[qb][r] = pr;
              dS[qb][r] = pr * (mix * dp[r] - d4[r]);
            }
          }
        }
      }
      ds_store(blk == 0 ? sm.dsA : sm.dsB, dS);
      if (!pre) {
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          if (act[2 * pp] || act[2 * pp + 1]) {
            const bf16x8 bs = pack_acc<bf16>(dS[2 * pp], dS[2 * pp + 1]);
            const bf16x8 bp = pack_acc<bf16>(P[2 * pp], P[2 * pp + 1]);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
              mma(dkT[ct], frag(sm.qT[sl], ct, pp), bs);
              mma(dvT[ct], frag(sm.doT[sl], ct, pp), bp);
            }
          }
        }
      }
    }
    if (!pre && sg < T_len) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        st4<bf16>(dk + off + (size_t)sg * kD + 16 * ct + 4 * g, dkT[ct] * scale);
        st4<bf16>(dv + off + (size_t)sg * kD + 16 * ct + 4 * g, dvT[ct] * mix);
      }
    }
    lds_barrier();
    // ---- dq: wave w takes queries 16w + r16 of tiles i (block A) and i+1 (block B)
    {
      f32x4 dqi[4], dqn[4];  // [c = 16ct + 4g + r][query]
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) dqi[ct] = dqn[ct] = zero;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const bf16x8 fa = frag(sm.dsA, w, p), fbb = frag(sm.dsB, w, p);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const bf16x8 kt = frag(sm.kT, ct, p);
          if (!pre) mma(dqi[ct], kt, fa);
          mma(dqn[ct], kt, fbb);
        }
      }
      if (!pre) {
        const int tl = 16 * w + r16, tg = i * kT + tl;
        if (M > 0) {
          // meta slots, query per lane: dq term
          bf16x8 qf[2], df[2];
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            qf[p] = frag(sm.qr[a], w, p);
            df[p] = frag(sm.dor[a], w, p);
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
            mma(dqi[ct], bf16x8{m4[0], m4[1], m4[2], m4[3], z, z, z, z}, bds);
          }
          // slot per lane: this wave's 16 queries' share of the meta gradients
          f32x4 s2 = zero, dp2 = zero;  // [query 16w + 4g + r][slot r16]
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            mma(s2, qf[p], frag(sm.mkr, 0, p));
            mma(dp2, df[p], frag(sm.mvr, 0, p));
          }
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sm.lse2[a][16 * w + 4 * g]);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sm.Dt[a][16 * w + 4 * g]);
          f32x4 p2, ds2;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool ok = r16 < M && i * kT + 16 * w + 4 * g + r < T_len;
            p2[r] = ok ? exp2_fast(s2[r] * sl2 - l4[r]) : 0.f;
            ds2[r] = p2[r] * (mix * dp2[r] - d4[r]);
          }
          const bf16x8 b2 = pack_acc<bf16>(ds2, zero), bp2 = pack_acc<bf16>(p2, zero);
          // queries 16w + 4g + e sit at split position 32(w >> 1) + 8g + 4(w & 1) + e
          const int fm = swz64(r16, 32 * (w >> 1) + 8 * g + 4 * (w & 1));
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) {
            const bf16x4 aq = *reinterpret_cast<const bf16x4*>(&sm.qT[a][1024 * ct + fm]);
            const bf16x4 ao = *reinterpret_cast<const bf16x4*>(&sm.doT[a][1024 * ct + fm]);
            f32x4 ak = sm.macc[w][ct][lane], av = sm.macc[w][4 + ct][lane];
            mma(ak, bf16x8{aq[0], aq[1], aq[2], aq[3], z, z, z, z}, b2);
            mma(av, bf16x8{ao[0], ao[1], ao[2], ao[3], z, z, z, z}, bp2);
            sm.macc[w][ct][lane] = ak;
            sm.macc[w][4 + ct][lane] = av;
          }
        }
        if (tg < T_len) {
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
            st4<bf16>(dq + off + (size_t)tg * kD + 16 * ct + 4 * g, (dqc[ct] + dqi[ct]) * scale);
        }
      }
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) dqc[ct] = dqn[ct];
    }
    lds_barrier();
    // ---- the prefetched tiles into the freed slots
    if (pq) qstore(qx, a);  // query tile i + 2
    if (pk) {
      kstore(kx);
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
    for (int wv = 0; wv < 4; ++wv) {
      if (w == wv) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int cc = 16 * ct + 4 * g + r;
            const float x0 = scale * sm.macc[w][ct][lane][r], x1 = mix * sm.macc[w][4 + ct][lane][r];
            sm.red[cc][r16] = (wv == 0 ? 0.f : sm.red[cc][r16]) + x0;
            sm.red[kD + cc][r16] = (wv == 0 ? 0.f : sm.red[kD + cc][r16]) + x1;
          }
      }
      __syncthreads();
    }
    float* mp = metap + ((size_t)bh * nseg + seg) * (size_t)M * 2 * kD;
    for (int e = tid; e < M * 2 * kD; e += kThreads) {
      const int which = e / (M * kD), rem = e % (M * kD), m = rem / kD, cc = rem % kD;
      mp[e] = sm.red[which * kD + cc][m];
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
  if (nqt > 0 && BH > 0 && s.window <= 65) {
    // streaming form: B*H*G work-groups, G segments of whole tiles per sequence
    int G = std::max(1, std::min(nqt, (256 + BH - 1) / BH));
    const int per = (nqt + G - 1) / G;
    G = (nqt + per - 1) / per;
    hipLaunchKernelGGL(swa_bwd_stream, dim3(G, BH), dim3(kThreads), 0, st, (const T*)q,
                       (const T*)k, (const T*)v, (const T*)mk, (const T*)mv, (const T*)o_swa, lse,
                       (const T*)dO, (T*)dq, (T*)dk, (T*)dv, metap, s.T, s.H, s.window, s.n_meta,
                       s.scale, s.mix, per);
    if (s.n_meta > 0 && s.H > 0)
      hipLaunchKernelGGL(swa_meta_reduce, dim3(s.H, (2 * s.n_meta * kD + 63) / 64),
                         dim3(64 * kMetaGroups), 0, st, metap, dmk, dmv, s.B, s.H, G, s.n_meta);
    return hipGetLastError();
  }
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
