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
// Kernels (bf16, d = 64), run per block of chunks c0..c1-1 (the caller walks a
// sequence block by block, last block first, so the chunk states of one block
// at a time are held):
//   1. scans (one launch): per head, the state scan forward writes S_c for every
//      chunk of the block from the state entering it, and the reverse scan
//      writes dS_{c+1} from the gradient leaving it
//   2. per chunk: dq, dk, dv and dlog_alpha from the chunk's inputs and the two
//      states of its boundaries
// Intra-chunk factors use 16-token sub-block midpoints R_i as references.
#include "common.hpp"
#include "kernels.hpp"

namespace lz {
namespace {

constexpr int kC = 64;
constexpr int kD = 64;          // head size supported by the backward
constexpr int kThreads = 256;
constexpr float kFastLog2 = 64.f;  // single-reference bound on the chunk decay (log2)

__host__ __device__ constexpr int pair_of(int i, int j) { return i * (i - 1) / 2 + j; }

constexpr int kTile = kC * kD;
// element offset of (row, col) in a swizzled 64 x 64 bf16 tile
__device__ __forceinline__ int at(int row, int col) { return swz_at<8>(row, col); }


// Fragment-major layout of the per-chunk states in the workspace: the 16-byte
// fragment (rows 16a + r, columns 32p + 8g..8g+7) of lane 16g + r sits at
// element ((2a + p) * 64 + 16g + r) * 8, so a wave reads one as 1 KiB in a row.
__device__ __forceinline__ int frag_major(int row, int col) {
  return (((row >> 4) * 2 + (col >> 5)) * 64 + ((col >> 3) & 3) * 16 + (row & 15)) * 8 + (col & 7);
}

// -------------------------------------------------------------- 1-2. scans
// Work-groups 0..BH-1 run the state scan of one head forward (writing S_c, the
// state entering chunk c); work-groups BH..2BH-1 run the reverse scan (writing
// dS_{c+1}, the state gradient leaving chunk c):
//   S_{c+1} = D_c S_c + K^_c^T V_c,   dS_c = D_c dS_{c+1} + Q^_c^T dO_c,
// D_c = diag(2^{b_last}), K^_s = k_s 2^{b_last - b_s}, Q^_t = q_t 2^{b_t}.
// Eight waves.  Gating: lane c is channel c and wave w holds tokens 8w..8w+7 of
// the chunk, so the cumsum is serial over the wave's eight tokens plus the
// totals of the waves before it, exchanged through LDS; the totals of chunk
// n+1 are made in step n, before that step's barrier, so a step has one
// barrier.  Each lane stores its eight gated tokens as one 16-byte granule of
// the [c][t] tiles.  Update: wave w owns the 16x16 state tiles of channels
// 16(w >> 1).. and value columns 32(w & 1)..  The next chunk's inputs are
// loaded two steps ahead into alternating register sets.
constexpr int kScanThreads = 512;
struct ScanSmem {
  bf16 xT[2][kTile];    // gated k (or q) transposed [c][t]
  bf16 yT[2][kTile];    // v (or dO) transposed [j][t]
  float tot[2][8][kD];  // per-wave log2-gate totals of a chunk
  float dec[2][kD];     // 2^{b_last} per channel
};

// Chunks c0..c1-1 only: the forward scan starts from fstart (per-head stride
// fstride floats; null = zero), the reverse scan from rstart (null = zero) and
// leaves the gradient entering chunk c0 in rend (null = not stored); chunk c's
// states go to slot c - c0 of the L per head.  Blocks past the 2 BH of the
// scans, when the launch has them, sum the window branch's meta-gradient
// partials (meta): a latency-bound step that runs here beside the scans
// instead of as a launch of its own.
template <typename GT>
__global__ __launch_bounds__(kScanThreads) void gla_bwd_scans(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const GT* __restrict__ la, const bf16* __restrict__ dO, const float* __restrict__ fstart,
    size_t fstride, const float* __restrict__ rstart, float* __restrict__ rend,
    bf16* __restrict__ S_all, bf16* __restrict__ dS_all, int BH, int T_len, int c0, int c1,
    int L, MetaReduceArgs meta) {
  __shared__ __attribute__((aligned(16))) ScanSmem sm;
  static_assert(sizeof(ScanSmem) >= sizeof(float) * (kScanThreads / 64) * 64, "meta strip LDS");
  if ((int)blockIdx.x >= 2 * BH) {  // uniform over the block
    const int r = blockIdx.x - 2 * BH;
    meta_reduce_strip<kScanThreads / 64>(meta, r % meta.H, r / meta.H,
                                         reinterpret_cast<float(*)[64]>(&sm));
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int r16 = lane & 15, g = lane >> 4;
  const bool rev = (int)blockIdx.x >= BH;
  const int bh = rev ? blockIdx.x - BH : blockIdx.x;
  const size_t off = (size_t)bh * T_len * kD;
  const u32 nb = (u32)((size_t)T_len * kD * sizeof(bf16));
  const Buf bx((rev ? q : k) + off, nb), by((rev ? dO : v) + off, nb),
      bla(la + off, nb / 2 * (u32)sizeof(GT));
  const int nc = c1 - c0;                   // chunks of this block
  const int cb = w >> 1, jh = 2 * (w & 1);  // state tiles: channels 16cb.., value blocks jh, jh+1
  const int fb0 = swz64(r16, 8 * g), fb1 = swz64(r16, 32 + 8 * g);

  // a1[u]: [j = 16(jh + u) + 4g + r][c = 16cb + r16] (the state, transposed)
  f32x4 a1[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) a1[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the forward scan starts from fstart (h0 or the block's entry state), the
  // reverse scan from rstart (dhT, the gradient of the final state, or the
  // gradient leaving the block), all [c][j] row-major; absent ones are zero
  const float* start = rev ? rstart : fstart;
  if (start) {
    const float* hp = start + (size_t)bh * (rev ? (size_t)kD * kD : fstride) +
                      (size_t)(16 * cb + r16) * kD + 4 * g;
#pragma unroll
    for (int u = 0; u < 2; ++u) a1[u] = *reinterpret_cast<const f32x4*>(hp + 16 * (jh + u));
  }
  // channel `lane` of tokens 8w..8w+7: gate (as its raw bits), x and y (bf16)
  struct In {
    u32 la[8], x[8], y[8];
  };
  auto load = [&](In& d, int ch) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32 e = (u32)(ch * kC + 8 * w + i) * kD + lane;
      if constexpr (sizeof(GT) == 4)
        d.la[i] = bla.ld32(e * 4);
      else
        d.la[i] = __builtin_amdgcn_raw_buffer_load_b16(bla.r, e * 2, 0, 0);
      d.x[i] = __builtin_amdgcn_raw_buffer_load_b16(bx.r, e * 2, 0, 0);
      d.y[i] = __builtin_amdgcn_raw_buffer_load_b16(by.r, e * 2, 0, 0);
    }
  };
  auto gate_of = [&](u32 bits) {
    if constexpr (sizeof(GT) == 4)
      return gate_log2(as_f(bits), GT());
    else
      return gate_log2(as_f(bits << 16), GT());
  };
  // in-wave inclusive cumsum of chunk ch's gates over this wave's tokens
  auto local_cumsum = [&](const In& d, int ch, float (&bloc)[8]) {
    float run = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      run += gate_row<GT>(gate_of(d.la[i]), ch * kC + 8 * w + i < T_len);
      bloc[i] = run;
    }
  };
  auto chunk_at = [&](int n) { return rev ? c1 - 1 - n : c0 + n; };
  float bloc[8];
  auto step = [&](In& d, In& dn, int n) {
    const int ch = chunk_at(n), buf = n & 1;
    // chunk-wide cumsum: the totals of the waves before this one, and b_last
    float pre = 0.f, blast = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float tj = sm.tot[buf][j][lane];
      pre += j < w ? tj : 0.f;
      blast += tj;
    }
    if (w == 0) sm.dec[buf][lane] = exp2_fast(blast);
    u32 X[4], Y[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float b0 = bloc[2 * m] + pre, b1 = bloc[2 * m + 1] + pre;
      const float f0 = exp2_fast(rev ? b0 : blast - b0);
      const float f1 = exp2_fast(rev ? b1 : blast - b1);
      X[m] = pack_bf2(bf_lo(d.x[2 * m]) * f0, bf_lo(d.x[2 * m + 1]) * f1);
      Y[m] = (d.y[2 * m] & 0xffffu) | (d.y[2 * m + 1] << 16);
    }
    *reinterpret_cast<u32x4*>(&sm.xT[buf][swz64(lane, 8 * w)]) = u32x4{X[0], X[1], X[2], X[3]};
    *reinterpret_cast<u32x4*>(&sm.yT[buf][swz64(lane, 8 * w)]) = u32x4{Y[0], Y[1], Y[2], Y[3]};
    // the next chunk's in-wave cumsum and total (its inputs are already loaded)
    local_cumsum(dn, chunk_at(min(n + 1, nc - 1)), bloc);
    sm.tot[buf ^ 1][w][lane] = bloc[7];
    // unconditional (clamped at the last chunk) so that the wait counts stay exact
    load(d, chunk_at(min(n + 2, nc - 1)));
    // the state at the chunk boundary, before this chunk's update
    // (all words packed before the first store, so no store's data register is
    // rewritten while earlier stores are in flight)
    {
      const size_t so = ((size_t)bh * L + (ch - c0)) * kTile;
      bf16* dst = (rev ? dS_all : S_all) + so;
      u32x2 w1[2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
        w1[u] = u32x2{pack_bf2(a1[u][0], a1[u][1]), pack_bf2(a1[u][2], a1[u][3])};
#pragma unroll
      for (int u = 0; u < 2; ++u)
        *reinterpret_cast<u32x2*>(dst + frag_major(16 * cb + r16, 16 * (jh + u) + 4 * g)) = w1[u];
    }
    lds_barrier();
    // decay, then add this chunk's outer products
    const float d1 = sm.dec[buf][16 * cb + r16];
    const bf16* xb = sm.xT[buf] + 1024 * cb;
    const bf16x8 xf0 = ld8<bf16>(xb + fb0), xf1 = ld8<bf16>(xb + fb1);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      a1[u] *= d1;
      const bf16* yb = sm.yT[buf] + 1024 * (jh + u);
      const bf16x8 y0 = ld8<bf16>(yb + fb0), y1 = ld8<bf16>(yb + fb1);
      mma(a1[u], y0, xf0);
      mma(a1[u], y1, xf1);
    }
  };
  In A, B;
  load(A, chunk_at(0));
  __builtin_amdgcn_sched_barrier(0);  // keep set A's loads ahead of set B's
  load(B, chunk_at(min(1, nc - 1)));
  __builtin_amdgcn_sched_barrier(0);
  local_cumsum(A, chunk_at(0), bloc);
  sm.tot[0][w][lane] = bloc[7];
  lds_barrier();
  for (int n = 0; n < nc; n += 2) {
    step(A, B, n);
    if (n + 1 < nc) step(B, A, n + 1);
  }
  // after chunk c0 the reverse scan holds dS_{c0}, the gradient entering the block
  if (rev && rend) {
    float* hp = rend + (size_t)bh * kD * kD + (size_t)(16 * cb + r16) * kD + 4 * g;
#pragma unroll
    for (int u = 0; u < 2; ++u) *reinterpret_cast<f32x4*>(hp + 16 * (jh + u)) = a1[u];
  }
}

// ------------------------------------------------------- 2. per-chunk grads
struct BwdSmem {
  bf16 qg[kTile];   // q~ rows [t][c] = q_t 2^{b_t - R_i}, i = block of t
  bf16 kg[kTile];   // k~ rows [s][c] = k_s 2^{R_j - b_s}, j = block of s
  bf16 qgT[kTile];  // q~ transposed [c][split_pos(t)]
  bf16 kgT[kTile];  // k~ transposed [c][split_pos(s)]
  bf16 dor[kTile];  // dO rows [t][j]
  bf16 doT[kTile];  // dO transposed [j][split_pos(t)]
  bf16 vr[kTile];   // v rows [s][j]
  bf16 dST[kTile];  // dS_{c+1} transposed [j][c] (swz64 layout)
  float tot[4][kD];  // per-block gate totals
  float R[4][kD];    // sub-block midpoints b[16i + 7]
  float Ru[4][kD];   // references in use: the midpoints, or 0 on the single-reference path
  float bl[kD];      // chunk total b_last
  float eR[4][kD];   // 2^{R_i}
  float elR[4][kD];  // 2^{b_last - R_i}
  float vij[6][kD];  // 2^{R_i - R_j}, i > j, index pair_of(i, j)
  float sx[4][kD];   // per-block totals of the suffix items of dlog_alpha
  float sy[4][kD];   // per-block totals of the prefix items
  float st[kD];      // state term 2^{b_last} sum_j dS_{c+1}[c][j] S_c[c][j]
};

// factor 2^{R_i - R_j} for query block i, key block j (1 on the diagonal, 0 above)
__device__ __forceinline__ float pair_factor(const BwdSmem& sm, int i, int j, int c) {
  return i > j ? sm.vij[pair_of(i, j)][c] : (i == j ? 1.f : 0.f);
}

// One work-group per (chunk, head): dq, dk, dv (added to what dq, dk, dv hold;
// with kAddQK false dq and dk are written, not added to) and dlog_alpha of the GLA branch, from the chunk's inputs and the states S_c,
// dS_{c+1} written by the two scans (dS_{c+1} is transposed here, in LDS).  Wave w owns token block w in both roles (query for
// dq, key for dk and dv), so the work of the two halves balances.  Lane
// (r16, g) owns token t = 16w + r16 and channels 16ct + 4g + r (ct, r < 4):
// the accumulator layout of every output tile, in which the gate cumsum and
// the dlog_alpha scans are also kept.
template <bool kAddQK, typename GT>
__global__ __launch_bounds__(kThreads, 2) void gla_bwd_chunk(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const GT* __restrict__ la, const bf16* __restrict__ dO, const bf16* __restrict__ S_all,
    const bf16* __restrict__ dS_all, bf16* __restrict__ dq,
    bf16* __restrict__ dk, bf16* __restrict__ dv, float* __restrict__ dla, int T_len, int c0,
    int L) {
  __shared__ __attribute__((aligned(16))) BwdSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int ch = c0 + blockIdx.x, bh = blockIdx.y;
  const int t0 = ch * kC;
  const size_t off = (size_t)bh * T_len * kD;
  const u32 nb = (u32)((size_t)T_len * kD * sizeof(bf16));
  const Buf bq(q + off, nb), bk(k + off, nb), bv(v + off, nb), bdo(dO + off, nb);
  const Buf bla(la + off, nb / 2 * (u32)sizeof(GT));
  const size_t soff = ((size_t)bh * L + blockIdx.x) * kTile;
  const u32 sb = (u32)(kTile * sizeof(bf16));
  const Buf bS(S_all + soff, sb), bdS(dS_all + soff, sb);
  const int t = 16 * w + r16;
  const bool live = t0 + t < T_len;
  const u32 rowe = (u32)(t0 + t) * kD;  // element offset of this lane's token row

  // ---- 0. every global read of the work-group, issued up front
  Gate4<GT> la4[4];
  u32x2 q2[4], k2[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const u32 e = rowe + 16 * ct + 4 * g;
    la4[ct].load(bla, e);
    q2[ct] = ld64v(bq, e * 2);
    k2[ct] = ld64v(bk, e * 2);
  }
  // dO / v staging: piece p -> token (p & 1) | 2 (p >> 4), granule (p >> 1) & 7,
  // so neighbouring lanes hold neighbouring tokens of the same granule
  u32x4 dog[2], vg[2];
  int pt[2], po[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int p = tid + kThreads * h;
    pt[h] = (p & 1) | ((p >> 4) << 1);
    po[h] = (p >> 1) & 7;
    const u32 e = (u32)(t0 + pt[h]) * kD + 8 * po[h];
    dog[h] = bdo.ld128(e * 2);
    vg[h] = bv.ld128(e * 2);
  }
  // state fragments (fragment-major): rows 16ct + r16, columns 32p + 8g..
  auto frag_off = [&](int ct, int p) { return (u32)(((2 * ct + p) * 64 + lane) * 16); };
  u32x4 Sf[4][2], dSf[4][2];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int p = 0; p < 2; ++p) Sf[ct][p] = bS.ld128(frag_off(ct, p));
  // the window branch's gradients, to which this branch's are added (read
  // early so that their latency hides behind the gating)
  const Buf bgq(dq + off, nb), bgk(dk + off, nb), bgv(dv + off, nb);
  u32x2 dqw[4], dkw[4], dvw[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
    dqw[ct] = kAddQK ? ld64v(bgq, (rowe + 16 * ct + 4 * g) * 2) : u32x2{0u, 0u};

  // ---- 1. dO and v tiles; gate cumsum within each 16-token block
  {
    const int odd = tid & 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *reinterpret_cast<u32x4*>(&sm.dor[at(pt[h], 8 * po[h])]) = dog[h];
      *reinterpret_cast<u32x4*>(&sm.vr[at(pt[h], 8 * po[h])]) = vg[h];
      const u32 w0 = dog[h][0], w1 = dog[h][1], w2 = dog[h][2], w3 = dog[h][3];
      const u32 r0 = dpp_swap1(odd ? w0 : w2), r1 = dpp_swap1(odd ? w1 : w3);
      const u32 f0 = odd ? r0 : w0, f1 = odd ? r1 : w1;  // words of the even token
      const u32 s0 = odd ? w2 : r0, s1 = odd ? w3 : r1;  // words of the odd token
      const int j0 = 8 * po[h] + 4 * odd, tc = split_pos(pt[h] & ~1);
      *reinterpret_cast<u32*>(&sm.doT[at(j0 + 0, tc)]) = lo2(f0, s0);
      *reinterpret_cast<u32*>(&sm.doT[at(j0 + 1, tc)]) = hi2(f0, s0);
      *reinterpret_cast<u32*>(&sm.doT[at(j0 + 2, tc)]) = lo2(f1, s1);
      *reinterpret_cast<u32*>(&sm.doT[at(j0 + 3, tc)]) = hi2(f1, s1);
    }
  }
  float b[4][4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) b[ct][r] = gate_row<GT>(la4[ct].log2_at(r), live);
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) b[ct][r] += dpp_shr<1>(b[ct][r]);
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) b[ct][r] += dpp_shr<2>(b[ct][r]);
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) b[ct][r] += dpp_shr<4>(b[ct][r]);
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) b[ct][r] += dpp_shr<8>(b[ct][r]);
  if (r16 == 15)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
      *reinterpret_cast<f32x4*>(&sm.tot[w][16 * ct + 4 * g]) = f32x4{b[ct][0], b[ct][1], b[ct][2], b[ct][3]};
  lds_barrier();

  // ---- 2. chunk-wide cumsum, references
  float Rw[4][4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    f32x4 pre = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < w; ++j) pre += *reinterpret_cast<const f32x4*>(&sm.tot[j][16 * ct + 4 * g]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      b[ct][r] += pre[r];
      Rw[ct][r] = dpp_bcast<7>(b[ct][r]);
    }
    if (r16 == 7)
      *reinterpret_cast<f32x4*>(&sm.R[w][16 * ct + 4 * g]) = f32x4{b[ct][0], b[ct][1], b[ct][2], b[ct][3]};
    if (w == 3 && r16 == 15)
      *reinterpret_cast<f32x4*>(&sm.bl[16 * ct + 4 * g]) = f32x4{b[ct][0], b[ct][1], b[ct][2], b[ct][3]};
  }
  lds_barrier();

  // ---- 3. factor tables; gated q, k tiles (rows and transposes)
  // A chunk whose decay 2^{b_last} stays above 2^-kFastLog2 in every channel
  // uses one reference, the chunk start (R_i = 0): k~ grows by at most
  // 2^kFastLog2, far inside bf16 range, and no pair factors are needed.  Every
  // wave tests the same 64 values, so the choice is uniform over the group.
  const bool fast = !__any(sm.bl[lane] < -kFastLog2);
  if (fast) {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) Rw[ct][r] = 0.f;
  }
  {
    const int c = tid & 63, x = tid >> 6;
    const float Rx = fast ? 0.f : sm.R[x][c], blc = sm.bl[c];
    sm.Ru[x][c] = Rx;
    sm.eR[x][c] = exp2_fast(Rx);
    sm.elR[x][c] = exp2_fast(blc - Rx);
    // pairs (1,0) (2,0) (2,1) (3,0) (3,1) (3,2): thread group x makes pairs x and x + 4
    const int pi[6] = {1, 2, 2, 3, 3, 3}, pj[6] = {0, 0, 1, 0, 1, 2};
    sm.vij[x][c] = fast ? 1.f : exp2_fast(sm.R[pi[x]][c] - sm.R[pj[x]][c]);
    if (x < 2) sm.vij[x + 4][c] = fast ? 1.f : exp2_fast(sm.R[pi[x + 4]][c] - sm.R[pj[x + 4]][c]);
  }
  {
    const int odd = r16 & 1, te = split_pos(t & ~1);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int c0 = 16 * ct + 4 * g;
      const u32 qa = q2[ct][0], qb = q2[ct][1], ka = k2[ct][0], kb = k2[ct][1];
      float fq[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) fq[r] = b[ct][r] - Rw[ct][r];
      const u32 Q0 = pack_bf2(bf_lo(qa) * exp2_fast(fq[0]), bf_hi(qa) * exp2_fast(fq[1]));
      const u32 Q1 = pack_bf2(bf_lo(qb) * exp2_fast(fq[2]), bf_hi(qb) * exp2_fast(fq[3]));
      const u32 K0 = pack_bf2(bf_lo(ka) * exp2_fast(-fq[0]), bf_hi(ka) * exp2_fast(-fq[1]));
      const u32 K1 = pack_bf2(bf_lo(kb) * exp2_fast(-fq[2]), bf_hi(kb) * exp2_fast(-fq[3]));
      *reinterpret_cast<u32x2*>(&sm.qg[at(t, c0)]) = u32x2{Q0, Q1};
      *reinterpret_cast<u32x2*>(&sm.kg[at(t, c0)]) = u32x2{K0, K1};
      // neighbouring lanes hold tokens t, t+1: the even lane writes channels
      // c0, c0+1 and the odd lane c0+2, c0+3 as (token, token+1) pairs
      const u32 rq = dpp_swap1(odd ? Q0 : Q1), rk = dpp_swap1(odd ? K0 : K1);
      const u32 fQ = odd ? rq : Q0, sQ = odd ? Q1 : rq;
      const u32 fK = odd ? rk : K0, sK = odd ? K1 : rk;
      const int cp = c0 + 2 * odd;
      *reinterpret_cast<u32*>(&sm.qgT[at(cp, te)]) = lo2(fQ, sQ);
      *reinterpret_cast<u32*>(&sm.qgT[at(cp + 1, te)]) = hi2(fQ, sQ);
      *reinterpret_cast<u32*>(&sm.kgT[at(cp, te)]) = lo2(fK, sK);
      *reinterpret_cast<u32*>(&sm.kgT[at(cp + 1, te)]) = hi2(fK, sK);
    }
  }
  // the dS_{c+1} fragments are needed only from the dk part on
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      dSf[ct][p] = bdS.ld128(frag_off(ct, p));
    }
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    dkw[ct] = kAddQK ? ld64v(bgk, (rowe + 16 * ct + 4 * g) * 2) : u32x2{0u, 0u};
    dvw[ct] = ld64v(bgv, (rowe + 16 * ct + 4 * g) * 2);
  }
  lds_barrier();

  float X[4][4], Y[4][4];  // dlog_alpha items: suffix-summed X, prefix-summed Y
  // ---- 4. dq: wave w is query block w
  {
    bf16x8 dof[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) dof[p] = ld8<bf16>(&sm.dor[at(t, 32 * p + 8 * g)]);
    f32x4 dAT[4];  // dA^T[s = 16j + 4g + r][t], strictly s < t
    float dAtt = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dAT[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (j <= w) {
#pragma unroll
        for (int p = 0; p < 2; ++p) mma(dAT[j], ld8<bf16>(&sm.vr[at(16 * j + r16, 32 * p + 8 * g)]), dof[p]);
        if (j == w) {
          dAtt = __shfl(dAT[j][r16 & 3], 16 * (r16 >> 2) + r16);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (4 * g + r >= r16) dAT[j][r] = 0.f;
        }
      }
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      f32x4 inter = {0.f, 0.f, 0.f, 0.f}, intra = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < 2; ++p) mma(inter, as_bf8(Sf[ct][p]), dof[p]);
      const int cl = 16 * ct + r16;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        if (2 * pp <= w) {
          bf16x8 af = ld8<bf16>(&sm.kgT[at(cl, 32 * pp + 8 * g)]);
          if (!fast) {
            const float f0 = pair_factor(sm, w, 2 * pp, cl), f1 = pair_factor(sm, w, 2 * pp + 1, cl);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              af[e] = (bf16)((float)af[e] * f0);
              af[e + 4] = (bf16)((float)af[e + 4] * f1);
            }
          }
          mma(intra, af, pack_acc<bf16>(dAT[2 * pp], dAT[2 * pp + 1]));
        }
      }
      const int c0 = 16 * ct + 4 * g;
      const f32x4 eR4 = *reinterpret_cast<const f32x4*>(&sm.eR[w][c0]);
      const f32x4 R4 = *reinterpret_cast<const f32x4*>(&sm.Ru[w][c0]);
      const u32 qa = q2[ct][0], qb = q2[ct][1], ka = k2[ct][0], kb = k2[ct][1];
      const float qv[4] = {bf_lo(qa), bf_hi(qa), bf_lo(qb), bf_hi(qb)};
      const float kv[4] = {bf_lo(ka), bf_hi(ka), bf_lo(kb), bf_hi(kb)};
      float o[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float od = exp2_fast(b[ct][r] - R4[r]) * (eR4[r] * inter[r] + intra[r]);
        o[r] = od + dAtt * kv[r];
        X[ct][r] = qv[r] * od;
      }
      if (live) {
        const u32x2 prev = dqw[ct];
        const u32 pa = prev[0], pb = prev[1];
        *reinterpret_cast<u32x2*>(dq + off + rowe + c0) =
            u32x2{pack_bf2(o[0] + bf_lo(pa), o[1] + bf_hi(pa)), pack_bf2(o[2] + bf_lo(pb), o[3] + bf_hi(pb))};
      }
    }
  }
  // state term, rows 16w.. by wave w (S_c is not needed after this)
  {
    float pc = 0.f;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
      if (ct == w)  // uniform over the wave
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int e = 0; e < 4; ++e) pc = dot2_bf16(Sf[ct][p][e], dSf[ct][p][e], pc);
    pc += __shfl_xor(pc, 16);
    pc += __shfl_xor(pc, 32);
    if (g == 0) sm.st[16 * w + r16] = pc * exp2_fast(sm.bl[16 * w + r16]);
  }
  // dS_{c+1} transposed into LDS for the dv inter product: neighbouring lanes
  // hold rows c, c+1; the even lane writes (c, c+1) pairs of columns j0..j0+3,
  // the odd lane of j0+4..j0+7
  {
    const int odd = r16 & 1;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const u32 W0 = dSf[ct][p][0], W1 = dSf[ct][p][1], W2 = dSf[ct][p][2], W3 = dSf[ct][p][3];
        const int ce = 16 * ct + (r16 & ~1), j0 = 32 * p + 8 * g + 4 * odd;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const u32 lo = m ? W1 : W0, hi = m ? W3 : W2;
          const u32 R = dpp_swap1(odd ? lo : hi);
          const u32 fst = odd ? R : lo, snd = odd ? hi : R;
          *reinterpret_cast<u32*>(&sm.dST[swz64(j0 + 2 * m, ce)]) = lo2(fst, snd);
          *reinterpret_cast<u32*>(&sm.dST[swz64(j0 + 2 * m + 1, ce)]) = hi2(fst, snd);
        }
      }
  }
  lds_barrier();
  // ---- 5. dk, dv: wave w is key block w
  {
    bf16x8 vf[2], kf[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      vf[p] = ld8<bf16>(&sm.vr[at(t, 32 * p + 8 * g)]);
      kf[p] = ld8<bf16>(&sm.kg[at(t, 32 * p + 8 * g)]);
    }
    f32x4 dA[4], Ab[4];  // [t = 16i + 4g + r][s]; dA strictly t > s, A with t >= s
    float dAss = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dA[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      Ab[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (i >= w) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          mma(dA[i], ld8<bf16>(&sm.dor[at(16 * i + r16, 32 * p + 8 * g)]), vf[p]);
          bf16x8 af = ld8<bf16>(&sm.qg[at(16 * i + r16, 32 * p + 8 * g)]);
          if (i > w && !fast) {
            const float* f = &sm.vij[pair_of(i, w)][32 * p + 8 * g];
#pragma unroll
            for (int e = 0; e < 8; ++e) af[e] = (bf16)((float)af[e] * f[e]);
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
    for (int ct = 0; ct < 4; ++ct) {
      f32x4 intra = {0.f, 0.f, 0.f, 0.f}, inter = {0.f, 0.f, 0.f, 0.f};
      const int cl = 16 * ct + r16;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        if (2 * pp + 1 >= w) {
          bf16x8 af = ld8<bf16>(&sm.qgT[at(cl, 32 * pp + 8 * g)]);
          if (!fast) {
            const float f0 = pair_factor(sm, 2 * pp, w, cl), f1 = pair_factor(sm, 2 * pp + 1, w, cl);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              af[e] = (bf16)((float)af[e] * f0);
              af[e + 4] = (bf16)((float)af[e + 4] * f1);
            }
          }
          mma(intra, af, pack_acc<bf16>(dA[2 * pp], dA[2 * pp + 1]));
        }
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) mma(inter, as_bf8(dSf[ct][p]), vf[p]);
      const int c0 = 16 * ct + 4 * g;
      const f32x4 bl4 = *reinterpret_cast<const f32x4*>(&sm.bl[c0]);
      const f32x4 R4 = *reinterpret_cast<const f32x4*>(&sm.Ru[w][c0]);
      const u32 qa = q2[ct][0], qb = q2[ct][1], ka = k2[ct][0], kb = k2[ct][1];
      const float qv[4] = {bf_lo(qa), bf_hi(qa), bf_lo(qb), bf_hi(qb)};
      const float kv[4] = {bf_lo(ka), bf_hi(ka), bf_lo(kb), bf_hi(kb)};
      float o[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float di = exp2_fast(R4[r] - b[ct][r]) * intra[r];
        const float de = exp2_fast(bl4[r] - b[ct][r]) * inter[r];
        o[r] = di + de + dAss * qv[r];
        X[ct][r] -= kv[r] * di;
        Y[ct][r] = kv[r] * de;
      }
      if (live) {
        const u32x2 prev = dkw[ct];
        const u32 pa = prev[0], pb = prev[1];
        *reinterpret_cast<u32x2*>(dk + off + rowe + c0) =
            u32x2{pack_bf2(o[0] + bf_lo(pa), o[1] + bf_hi(pa)), pack_bf2(o[2] + bf_lo(pb), o[3] + bf_hi(pb))};
      }
    }
    // K^_s = k~_s 2^{b_last - R_w}
    bf16x8 kh[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const float* f = &sm.elR[w][32 * p + 8 * g];
#pragma unroll
      for (int e = 0; e < 8; ++e) kh[p][e] = (bf16)((float)kf[p][e] * f[e]);
    }
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const int jl = 16 * jt + r16;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
        if (2 * pp + 1 >= w)
          mma(acc, ld8<bf16>(&sm.doT[at(jl, 32 * pp + 8 * g)]), pack_acc<bf16>(Ab[2 * pp], Ab[2 * pp + 1]));
#pragma unroll
      for (int p = 0; p < 2; ++p)
        mma(acc, ld8<bf16>(&sm.dST[1024 * jt + swz64(r16, 32 * p + 8 * g)]), kh[p]);
      if (live) {
        const u32x2 prev = dvw[jt];
        const u32 pa = prev[0], pb = prev[1];
        *reinterpret_cast<u32x2*>(dv + off + rowe + 16 * jt + 4 * g) =
            u32x2{pack_bf2(acc[0] + bf_lo(pa), acc[1] + bf_hi(pa)),
                  pack_bf2(acc[2] + bf_lo(pb), acc[3] + bf_hi(pb))};
      }
    }
  }
  // ---- 6. dlog_alpha: suffix sums of X and exclusive prefix sums of Y over
  // the chunk, plus the state term
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
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
      if (r16 == 0) sm.sx[w][16 * ct + 4 * g + r] = xs;
      if (r16 == 15) sm.sy[w][16 * ct + 4 * g + r] = yi;
    }
  lds_barrier();
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const int c0 = 16 * ct + 4 * g;
    f32x4 add = *reinterpret_cast<const f32x4*>(&sm.st[c0]);
    for (int j = w + 1; j < 4; ++j) add += *reinterpret_cast<const f32x4*>(&sm.sx[j][c0]);
    for (int j = 0; j < w; ++j) add += *reinterpret_cast<const f32x4*>(&sm.sy[j][c0]);
    f32x4 o;
#pragma unroll
    // with logit gates, d logit = d log(alpha) * sigmoid(-logit)
    for (int r = 0; r < 4; ++r) o[r] = (X[ct][r] + Y[ct][r] + add[r]) * gate_dlog(la4[ct].raw_at(r), GT());
    if (live) *reinterpret_cast<f32x4*>(dla + off + rowe + c0) = o;
  }
}

}  // namespace

// Chunks c0..c1-1 of every head (bf16, d = 64): both scans, then the
// per-chunk gradients (see launch_gla_bwd_block_gen for the arguments); with
// meta.n > 0 the scans launch also sums the window branch's meta gradients.
hipError_t launch_gla_bwd_block(const Shape& s, const void* q, const void* k, const void* v,
                                const void* la, const void* dO, const float* fstart,
                                size_t fstride, const float* rstart, float* rend, void* dq,
                                void* dk, void* dv, float* dla, void* S_ws, void* dS_ws,
                                bool add_qk, int c0, int c1, int L, const MetaReduceArgs& meta,
                                hipStream_t st) {
  typedef bf16 T;
  const int BH = s.B * s.H;
  // meta.n > 0: H strips of 64 entries per 2 n more blocks for the meta reduction
  const int nmeta = meta.n > 0 ? meta.H * ((2 * meta.n + 63) / 64) : 0;
  auto go = [&](auto gate_type) {
    typedef decltype(gate_type) GT;
    hipLaunchKernelGGL(gla_bwd_scans<GT>, dim3(2 * BH + nmeta), dim3(kScanThreads), 0, st,
                       (const T*)q, (const T*)k, (const T*)v, (const GT*)la, (const T*)dO, fstart,
                       fstride, rstart, rend, (T*)S_ws, (T*)dS_ws, BH, s.T, c0, c1, L, meta);
    auto kern = add_qk ? gla_bwd_chunk<true, GT> : gla_bwd_chunk<false, GT>;
    hipLaunchKernelGGL(kern, dim3(c1 - c0, BH), dim3(kThreads), 0, st, (const T*)q, (const T*)k,
                       (const T*)v, (const GT*)la, (const T*)dO, (const T*)S_ws,
                       (const T*)dS_ws, (T*)dq, (T*)dk, (T*)dv, dla, s.T, c0, L);
  };
  if (s.gate == 1)
    go(bf16());
  else
    go(float());
  return hipGetLastError();
}

}  // namespace lz
