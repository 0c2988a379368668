// Chunked gated linear attention forward for gfx950.
//
// Computes, per head, o_t = q_t S_t with S_t = diag(alpha_t) S_{t-1} + k_t^T v_t
// (state update of "Lizard: An Efficient Linearization Framework for Large
// Language Models", gist.science summary, section 2(a)).  Following the idea of
// that page's section 2(c), the cumulative gate is folded into q and k in log
// space so that every chunk's work is a matrix-core product; the page's kernel
// targets other hardware, so the blocking below is this library's own.
//
// Work split.  Each head's sequence is cut into G segments of whole 64-token
// chunks so that B*H*G work-groups fill the chip (G depends on B*H, not on T):
//   1. state pass   (segments 0..G-2, parallel): the segment's own end state
//                   from zero and its total log2 decay;
//   2. output pass  (all segments, parallel): S_in(g) from h0 and the earlier
//                   segments, S_in(j+1) = 2^{Gamma_j} S_in(j) + S_loc(j), then
//                   the chunk recurrence below started from S_in(g).
// The state is associative over (decay, state) pairs, so this is the same
// recurrence evaluated in another order.
//
// Output pass, one work-group of DK/16 waves per (head, segment); wave w owns
// value columns 16w..16w+15 and keeps its DK x 16 fp32 state slice in registers.
// Per chunk with tokens t0..t0+63 and b_t = log2-gate cumsum inside the chunk:
//   inter  O += (q_t * 2^{b_t}) S_c                     (state entering the chunk)
//   intra  O += A V,  A_ts = sum_ch q_t k_s 2^{b_t - b_s}  for s <= t in the chunk
//   state  S_{c+1} = diag(2^{b_last}) S_c + (k_s * 2^{b_last - b_s})^T V
// Intra scores use 16-token sub-blocks: for query block i the exponent is split
// at the block's midpoint R_i, 2^{b_t - R_i} * 2^{R_i - b_s}; off-diagonal blocks
// (j < i) take the extra per-channel factor 2^{R_i - R_j} <= 1 on the q operand.
// Every factor stays within 2^{8 max|log2 alpha|}, so extreme gates neither
// overflow nor lose the diagonal terms.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace lz {
namespace {

constexpr int kC = 64;       // chunk length
constexpr int kMaxSeg = 16;  // segments per head, at most

__host__ __device__ constexpr int blk_i(int b) { return b == 0 ? 0 : b < 3 ? 1 : b < 6 ? 2 : 3; }
__host__ __device__ constexpr int blk_j(int b) { return b - blk_i(b) * (blk_i(b) + 1) / 2; }
// index of the off-diagonal pair (i, j), j < i, in 0..5
__host__ __device__ constexpr int pair_of(int i, int j) { return i * (i - 1) / 2 + j; }
__host__ __device__ constexpr int pair_i(int p) { return p == 0 ? 1 : p < 3 ? 2 : 3; }
__host__ __device__ constexpr int pair_j(int p) { return p - pair_i(p) * (pair_i(p) - 1) / 2; }

struct Plan {
  int nc;   // chunks
  int cps;  // chunks per segment
  int G;    // segments
};

Plan make_plan(const Shape& s) {
  Plan p;
  p.nc = (s.T + kC - 1) / kC;
  const long long bh = (long long)s.B * s.H;
  int g = (int)((256 + bh - 1) / (bh > 0 ? bh : 1));
  g = g < 1 ? 1 : (g > kMaxSeg ? kMaxSeg : g);
  if (g > p.nc) g = p.nc > 0 ? p.nc : 1;
  p.cps = p.nc > 0 ? (p.nc + g - 1) / g : 1;
  p.G = p.nc > 0 ? (p.nc + p.cps - 1) / p.cps : 1;
  return p;
}

template <typename T, int DK>
struct OutSmem {
  // fp32 at DK = 128 keeps its tiles within the 160 KiB of LDS with less row
  // padding (some fragment reads of khT / vT then share banks)
  static constexpr bool kTight = sizeof(T) == 4 && DK == 128;
  static constexpr int DKP = DK + (kTight ? 4 : 8);
  static constexpr int CP = kC + (kTight ? 0 : 8);
  static constexpr int AP = kC + (kTight ? 4 : 8);
  T qg[kC][DKP];     // single reference: q_t 2^{b_t}; sub-blocks: q_t 2^{b_t - R_i}
  T kg[kC][DKP];     // k_s 2^{R_j - b_s} (R = 0 with a single reference)
  T khT[DK][CP];     // (k_s 2^{b_last - b_s})^T
  T vT[DK][CP];      // v^T
  T a[kC][AP];       // masked intra scores A[t][s]
  float tot[8][DK];  // per-8-row-group sums of log2 gates
  float vij[6][DK];  // 2^{R_i - R_j} for the off-diagonal pairs
  alignas(16) float eR[4][DK];  // 2^{R_i} (sub-block references; unused with a single one)
  alignas(16) float decay[DK];  // 2^{b_last}
};

// Double-buffered by chunk parity: the state pass gates chunk c into one set
// while the matrix cores still read the other.
template <typename T, int DK>
struct StateSmem {
  static constexpr int CP = kC + 8;
  T khT[2][DK][CP];
  T vT[2][DK][CP];
  float tot[2][8][DK];
  float decay[2][DK];
};

// Per-thread gating slice: 8 rows (8*rg ..) x 2 channels (2*cp, 2*cp+1); GT is
// the gate input type (float log alpha or bf16 logit).
template <typename T, int DK, typename GT = float>
struct Slice {
  static constexpr int ES = sizeof(T);
  typename Pair<T>::type q[8], k[8], v[8];
  typename Pair<GT>::type la[8];
  __device__ __forceinline__ void load(const Buf& bq, const Buf& bk, const Buf& bv,
                                       const Buf& bla, int t0, int rg, int cp, bool need_q) {
    const u32 row0 = (u32)(t0 + 8 * rg);
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const u32 e = (row0 + rr) * DK + 2 * cp;
      if (need_q) q[rr] = ld_pair<T>(bq, e * ES);
      k[rr] = ld_pair<T>(bk, e * ES);
      v[rr] = ld_pair<T>(bv, e * ES);
      la[rr] = ld_pair<GT>(bla, e * (u32)sizeof(GT));
    }
  }
};

// Local (row-group) log2 cumsum of the slice's gates; returns the group total.
// Summed first without the gate floor, and again with it only in a thread
// whose 8-row total falls below the floor (no row can lie below it otherwise).
template <typename T, int DK, typename GT>
// vrows: rows of the slice before the sequence end
__device__ __forceinline__ f32x2 local_cumsum(const Slice<T, DK, GT>& sl, f32x2* b, int vrows) {
  f32x2 run;
  auto sum = [&](auto floored) {
    run = f32x2{0.f, 0.f};
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const f32x2 la = unpack2(sl.la[rr], GT());
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const float g = decltype(floored)::value ? gate_log2(la[x], GT()) : gate_log2_nofloor(la[x], GT());
        run[x] += gate_row<GT>(g, rr < vrows);
      }
      b[rr] = run;
    }
  };
  sum(std::false_type());
  if (fminf(run[0], run[1]) < kMinLog2Gate) sum(std::true_type());
  return run;
}

template <typename T>
__device__ __forceinline__ void store8(T* dst, const float* x) {
  typename Frag<T>::type f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = to_t<T>(x[e]);
  *reinterpret_cast<typename Frag<T>::type*>(dst) = f;
}

// Scale a fragment by 8 per-channel factors (fp32, in LDS).
__device__ __forceinline__ bf16x8 scale8(const bf16x8& x, const float* f) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(f);
  const f32x4 b = *reinterpret_cast<const f32x4*>(f + 4);
  return bf16x8{(bf16)((float)x[0] * a[0]), (bf16)((float)x[1] * a[1]), (bf16)((float)x[2] * a[2]),
                (bf16)((float)x[3] * a[3]), (bf16)((float)x[4] * b[0]), (bf16)((float)x[5] * b[1]),
                (bf16)((float)x[6] * b[2]), (bf16)((float)x[7] * b[3])};
}
__device__ __forceinline__ f32x8 scale8(const f32x8& x, const float* f) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(f);
  const f32x4 b = *reinterpret_cast<const f32x4*>(f + 4);
  return f32x8{x[0] * a[0], x[1] * a[1], x[2] * a[2], x[3] * a[3],
               x[4] * b[0], x[5] * b[1], x[6] * b[2], x[7] * b[3]};
}

// ------------------------------------------------------------------ pass 1
template <typename T, int DK, typename GT>
__global__ __launch_bounds__(4 * DK, 1) void gla_state_pass(
    const T* __restrict__ k, const T* __restrict__ v, const GT* __restrict__ la,
    float* __restrict__ ws_state, float* __restrict__ ws_gamma, int T_arg, int cps, int G,
    const int* __restrict__ cu, int N, int H, int region_rows = 0) {
  constexpr int NCB = DK / 16;
  typedef typename Frag<T>::type F;
  __shared__ StateSmem<T, DK> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int cp = tid % (DK / 2), rg = tid / (DK / 2);
  const int seg = blockIdx.x, bh = blockIdx.y;
  const SeqRows sr = seq_rows(cu, N, T_arg, H, bh);
  const int T_len = sr.len;
  const size_t off = sr.row0 * DK;
  // a packed sequence has its own segment count; only segments before its
  // last one need a local end state
  const int nc_seq = (T_len + kC - 1) / kC;
  if (cu && seg >= max(1, (nc_seq + cps - 1) / cps) - 1) return;
  const Buf bk(k + off, (u32)((size_t)T_len * DK * sizeof(T)));
  const Buf bv(v + off, (u32)((size_t)T_len * DK * sizeof(T)));
  const Buf bla(la + off, (u32)((size_t)T_len * DK * sizeof(GT)));
  const int nc = (T_len + kC - 1) / kC;
  const int c_begin = seg * cps, c_end = min(nc, c_begin + cps);

  f32x4 S[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) S[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x2 gsum = {0.f, 0.f};

  // Chunk c_begin + n is gated in step n from register set n & 1; its row-group
  // totals were exchanged in step n-1 (or the prologue), so each step has one
  // barrier, before the matrix-core update.  Inputs are loaded two chunks ahead.
  Slice<T, DK, GT> A, B;
  f32x2 b[8];  // in-thread log2 cumsum of the chunk to gate next
  A.load(bk, bk, bv, bla, c_begin * kC, rg, cp, false);
  B.load(bk, bk, bv, bla, min(c_begin + 1, c_end - 1) * kC, rg, cp, false);
  {
    const f32x2 t0 = local_cumsum(A, b, T_len - c_begin * kC - 8 * rg);
    sm.tot[0][rg][2 * cp] = t0[0];
    sm.tot[0][rg][2 * cp + 1] = t0[1];
  }
  lds_barrier();
  auto step = [&](Slice<T, DK, GT>& d, const Slice<T, DK, GT>& dn, int n) {
    const int ch = c_begin + n, buf = n & 1;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int c = 2 * cp + x;
      float pre = 0.f, blast = 0.f;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float tr = sm.tot[buf][r][c];
        pre += (r < rg) ? tr : 0.f;
        blast += tr;
      }
      float kh[8], vc[8];
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        kh[rr] = unpack2(d.k[rr], T())[x] * exp2_fast(blast - (b[rr][x] + pre));
        vc[rr] = unpack2(d.v[rr], T())[x];
      }
      store8<T>(&sm.khT[buf][c][8 * rg], kh);
      store8<T>(&sm.vT[buf][c][8 * rg], vc);
      if (rg == 0) sm.decay[buf][c] = exp2_fast(blast);
      gsum[x] += blast;
    }
    // the next chunk's in-thread cumsum and row-group totals (past the last
    // chunk this repeats it; those totals are never read)
    const f32x2 tn = local_cumsum(dn, b, T_len - (ch + 1) * kC - 8 * rg);
    sm.tot[buf ^ 1][rg][2 * cp] = tn[0];
    sm.tot[buf ^ 1][rg][2 * cp + 1] = tn[1];
    // unconditional (clamped at the last chunk) so that the wait counts stay exact
    d.load(bk, bk, bv, bla, min(ch + 2, c_end - 1) * kC, rg, cp, false);
    lds_barrier();
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) S[cb][r] *= sm.decay[buf][16 * cb + 4 * g + r];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        F af = ld8<T>(&sm.khT[buf][16 * cb + r16][32 * p + 8 * g]);
        F bf = ld8<T>(&sm.vT[buf][16 * wave + r16][32 * p + 8 * g]);
        mma(S[cb], af, bf);
      }
    }
  };
  const int nch = c_end - c_begin;
  for (int n = 0; n < nch; n += 2) {
    step(A, B, n);
    if (n + 1 < nch) step(B, A, n + 1);
  }
  // stored column-major ([value column][key row]) so that the output pass reads
  // four consecutive rows of one column as one 16-byte load.  With region_rows
  // > 0 (checkpoints of the backward) segment seg's state and decay go to the
  // start of its own token rows of ws_state instead ([B*H, T, DK] floats; the
  // segment's region_rows rows hold DK*DK + DK floats).
  float* dst = region_rows > 0
                   ? ws_state + ((size_t)bh * T_len + (size_t)seg * region_rows) * DK
                   : ws_state + ((size_t)bh * (G - 1) + seg) * DK * DK;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
    *reinterpret_cast<f32x4*>(&dst[(16 * wave + r16) * DK + 16 * cb + 4 * g]) = S[cb];
  if (rg == 0) {
    float* gd = region_rows > 0 ? dst + DK * DK : ws_gamma + ((size_t)bh * (G - 1) + seg) * DK;
    gd[2 * cp] = gsum[0];
    gd[2 * cp + 1] = gsum[1];
  }
}

// ------------------------------------------------------------------ pass 2
// A chunk whose per-channel decay 2^{b_last} stays above 2^-kFastLog2 in every
// channel takes one reference for all its intra scores, the chunk start:
// q_t 2^{b_t} (<= |q_t|) against k_s 2^{-b_s} (<= 2^kFastLog2 |k_s|), both far
// inside the bf16/fp32 range.  Other chunks take the 16-token sub-block
// references.  The choice is made per chunk from the same shared totals by
// every wave, so it is uniform over the work-group.
constexpr float kFastLog2 = 64.f;

template <typename T, int DK>
__global__ __launch_bounds__(4 * DK, 1) void gla_output_pass(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ la, const float* __restrict__ h0, const float* __restrict__ ws_state,
    const float* __restrict__ ws_gamma, T* __restrict__ o, float* __restrict__ hT, int T_arg,
    int cps, int G, const int* __restrict__ cu, int N, int H) {
  constexpr int NCB = DK / 16;
  constexpr int KS = DK / 32;
  constexpr int NW = DK / 16;
  constexpr int NB = (10 + NW - 1) / NW;  // score blocks per wave, at most
  typedef typename Frag<T>::type F;
  __shared__ OutSmem<T, DK> sm;
  constexpr int DKP = OutSmem<T, DK>::DKP;

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int cp = tid % (DK / 2), rg = tid / (DK / 2);
  const int i_sub = rg >> 1;  // 16-row sub-block of this thread's rows
  const int seg = blockIdx.x, bh = blockIdx.y;
  const SeqRows sr = seq_rows(cu, N, T_arg, H, bh);
  const int T_len = sr.len;
  const size_t off = sr.row0 * DK;
  const u32 nbytes = (u32)((size_t)T_len * DK * sizeof(T));
  const Buf bq(q + off, nbytes), bk(k + off, nbytes), bv(v + off, nbytes);
  const Buf bla(la + off, (u32)((size_t)T_len * DK * 4));
  const int nc = (T_len + kC - 1) / kC;
  const int c_begin = seg * cps, c_end = min(nc, c_begin + cps);
  const int ncol = 16 * wave;
  const size_t s_base = (size_t)bh * DK * DK;
  // a packed sequence covers the first Gs of the plan's segments
  const int Gs = cu ? max(1, (nc + cps - 1) / cps) : G;
  if (seg >= Gs) return;
  if (nc == 0) {  // an empty packed sequence: the state passes through unchanged
    if (hT)
      for (int e = tid; e < DK * DK; e += 4 * DK) hT[s_base + e] = h0 ? h0[s_base + e] : 0.f;
    return;
  }

  // state slice S[16cb + 4g + r][ncol + r16] entering the segment: h0 carried
  // through the earlier segments' local end states and decays
  f32x4 S[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int r = 0; r < 4; ++r) S[cb][r] = h0 ? h0[s_base + (16 * cb + 4 * g + r) * DK + ncol + r16] : 0.f;
  for (int sg = 0; sg < seg; ++sg) {  // local states are column-major
    const float* loc = ws_state + ((size_t)bh * (G - 1) + sg) * DK * DK;
    const float* gm = ws_gamma + ((size_t)bh * (G - 1) + sg) * DK;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&loc[(ncol + r16) * DK + 16 * cb + 4 * g]);
      const f32x4 g4 = *reinterpret_cast<const f32x4*>(&gm[16 * cb + 4 * g]);
#pragma unroll
      for (int r = 0; r < 4; ++r) S[cb][r] = exp2_fast(g4[r]) * S[cb][r] + l4[r];
    }
  }

  // score blocks (0,1) and (2,3) lie above the diagonal; they are read by the
  // paired contraction steps and must stay zero
  for (int e = tid; e < 512; e += 4 * DK) {
    const int z = e >> 8, t = (e >> 4) & 15, s = e & 15;
    sm.a[32 * z + t][32 * z + 16 + s] = to_t<T>(0.f);
  }

  Slice<T, DK> cur;
  cur.load(bq, bk, bv, bla, c_begin * kC, rg, cp, true);
  for (int ch = c_begin; ch < c_end; ++ch) {
    const int t0 = ch * kC;
    f32x2 b[8];
    const f32x2 tot = local_cumsum(cur, b, T_len - ch * kC - 8 * rg);
    typename Pair<T>::type qq[8], kk[8], vv[8];
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) { qq[rr] = cur.q[rr]; kk[rr] = cur.k[rr]; vv[rr] = cur.v[rr]; }
    cur.load(bq, bk, bv, bla, min(ch + 1, c_end - 1) * kC, rg, cp, true);
    sm.tot[rg][2 * cp] = tot[0];
    sm.tot[rg][2 * cp + 1] = tot[1];
    lds_barrier();  // (A) group totals visible; previous chunk's LDS reads are done

    // prefix sums over row groups with selects only (run-time indices into a
    // register array would put it in scratch memory)
    const int pi = rg < 6 ? pair_i(rg) : 0, pj = rg < 6 ? pair_j(rg) : 0;
    float pre[2], blast[2], Ri[2], Rpi[2], Rpj[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int c = 2 * cp + x;
      pre[x] = blast[x] = Ri[x] = Rpi[x] = Rpj[x] = 0.f;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float tr = sm.tot[r][c];
        blast[x] += tr;
        pre[x] += (r < rg) ? tr : 0.f;
        Ri[x] += (r <= 2 * i_sub) ? tr : 0.f;  // b at row 16 i + 7
        Rpi[x] += (r <= 2 * pi) ? tr : 0.f;
        Rpj[x] += (r <= 2 * pj) ? tr : 0.f;
      }
    }
    // every wave's lanes cover all DK channels, so each wave reaches the same answer
    const bool fast = !__any(fminf(blast[0], blast[1]) < -kFastLog2);

    // ---- gated operands for rows 8rg..8rg+7, channels 2cp, 2cp+1
    if (fast) {
      float qhv[8][2], kiv[8][2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int c = 2 * cp + x;
        const float eB = exp2_fast(blast[x]);
        float kh[8], vc[8];
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          const float bt = b[rr][x] + pre[x];
          qhv[rr][x] = unpack2(qq[rr], T())[x] * exp2_fast(bt);
          kiv[rr][x] = unpack2(kk[rr], T())[x] * exp2_fast(-bt);
          kh[rr] = kiv[rr][x] * eB;
          vc[rr] = unpack2(vv[rr], T())[x];
        }
        store8<T>(&sm.khT[c][8 * rg], kh);
        store8<T>(&sm.vT[c][8 * rg], vc);
        if (rg == 7) sm.decay[c] = eB;
      }
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const int t = 8 * rg + rr;
        st_pair<T>(&sm.qg[t][2 * cp], qhv[rr][0], qhv[rr][1]);
        st_pair<T>(&sm.kg[t][2 * cp], kiv[rr][0], kiv[rr][1]);
      }
    } else {
      float qgv[8][2], kgv[8][2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int c = 2 * cp + x;
        const float eRi = exp2_fast(Ri[x]);
        const float eKh = exp2_fast(blast[x] - Ri[x]);
        float kh[8], vc[8];
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          const float d = b[rr][x] + pre[x] - Ri[x];
          qgv[rr][x] = unpack2(qq[rr], T())[x] * exp2_fast(d);
          kgv[rr][x] = unpack2(kk[rr], T())[x] * exp2_fast(-d);
          kh[rr] = kgv[rr][x] * eKh;
          vc[rr] = unpack2(vv[rr], T())[x];
        }
        store8<T>(&sm.khT[c][8 * rg], kh);
        store8<T>(&sm.vT[c][8 * rg], vc);
        if (rg < 6) {
          sm.vij[rg][c] = exp2_fast(Rpi[x] - Rpj[x]);
        } else if (rg == 7) {
          sm.decay[c] = exp2_fast(blast[x]);
        }
        if ((rg & 1) == 0) sm.eR[i_sub][c] = eRi;
      }
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const int t = 8 * rg + rr;
        st_pair<T>(&sm.qg[t][2 * cp], qgv[rr][0], qgv[rr][1]);
        st_pair<T>(&sm.kg[t][2 * cp], kgv[rr][0], kgv[rr][1]);
      }
    }
    lds_barrier();  // (B) operands ready

    // ---- intra scores: transposed blocks A^T[s][t], masked, stored as A[t][s].
    // All fragments of a phase are read before its first product so that the
    // LDS latency is paid once per phase, not once per product.
    {
      const T* qsrc = &sm.qg[0][0];
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const int blk = wave + n * NW;
        if (blk < 10) {
          const int i = blk_i(blk), j = blk_j(blk);
          F af[KS], bf[KS];
#pragma unroll
          for (int p = 0; p < KS; ++p) {
            af[p] = ld8<T>(&sm.kg[16 * j + r16][32 * p + 8 * g]);
            bf[p] = ld8<T>(qsrc + (16 * i + r16) * DKP + 32 * p + 8 * g);
          }
          if (!fast && j < i) {
#pragma unroll
            for (int p = 0; p < KS; ++p)
              bf[p] = scale8(bf[p], &sm.vij[pair_of(i, j)][32 * p + 8 * g]);
          }
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int p = 0; p < KS; ++p) mma(acc, af[p], bf[p]);
          if (i == j) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (4 * g + r > r16) acc[r] = 0.f;
          }
          st4<T>(&sm.a[16 * i + r16][16 * j + 4 * g], acc);
        }
      }
    }

    // phases are kept apart so that each one's fragments are not live at once
    __builtin_amdgcn_sched_barrier(0);

    // ---- inter: O^T[n][t] = sum_c S[c][n] 2^{R_i}[c] qg[t][c] (query block i of t;
    // 2^{R_i} = 1 with a single reference), with the state entering the chunk
    f32x4 O[4];
    {
      F sf[KS];
#pragma unroll
      for (int p = 0; p < KS; ++p) sf[p] = pack_acc<T>(S[2 * p], S[2 * p + 1]);
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        F qf[KS], sfs[KS];
#pragma unroll
        for (int p = 0; p < KS; ++p) {
          qf[p] = ld4x2<T>(&sm.qg[16 * qb + r16][32 * p + 4 * g]);
          sfs[p] = sf[p];
          if (!fast) {
            // fragment element e holds channel 32p + 4g + e (e < 4) or 32p + 12 + 4g + e
            const f32x4 lo = *reinterpret_cast<const f32x4*>(&sm.eR[qb][32 * p + 4 * g]);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(&sm.eR[qb][32 * p + 16 + 4 * g]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              sfs[p][e] = to_t<T>(to_f(sf[p][e]) * lo[e]);
              sfs[p][e + 4] = to_t<T>(to_f(sf[p][e + 4]) * hi[e]);
            }
          }
        }
        O[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < KS; ++p) mma(O[qb], sfs[p], qf[p]);
      }
    }

    __builtin_amdgcn_sched_barrier(0);

    // ---- state update: S = diag(2^{b_last}) S + khT V
    F vf[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) vf[p] = ld8<T>(&sm.vT[ncol + r16][32 * p + 8 * g]);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const f32x4 dec = *reinterpret_cast<const f32x4*>(&sm.decay[16 * cb + 4 * g]);
      F kf[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) kf[p] = ld8<T>(&sm.khT[16 * cb + r16][32 * p + 8 * g]);
      S[cb] *= dec;
#pragma unroll
      for (int p = 0; p < 2; ++p) mma(S[cb], kf[p], vf[p]);
    }
    lds_barrier();  // (C) scores ready

    // ---- intra: O^T[n][t] += sum_s vT[n][s] A[t][s]
    {
      F af[4][2];
#pragma unroll
      for (int qb = 0; qb < 4; ++qb)
#pragma unroll
        for (int p = 0; p <= qb / 2; ++p) af[qb][p] = ld8<T>(&sm.a[16 * qb + r16][32 * p + 8 * g]);
#pragma unroll
      for (int qb = 0; qb < 4; ++qb)
#pragma unroll
        for (int p = 0; p <= qb / 2; ++p) mma(O[qb], vf[p], af[qb][p]);
    }

    // ---- store O[t][ncol + 4g .. +3]
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const int t = t0 + 16 * qb + r16;
      if (t < T_len) st4<T>(o + off + (size_t)t * DK + ncol + 4 * g, O[qb]);
    }
  }

  if (hT && seg == Gs - 1) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) hT[s_base + (16 * cb + 4 * g + r) * DK + ncol + r16] = S[cb][r];
  }
}

// ------------------------------------------------------------------ pass 3, bf16
// Wave-specialised form of the output pass.  One chunk's work splits into a
// vector-ALU half (loads, cumulative sums, exponentials, the gated operand
// tiles) and a matrix half (scores and products reading those tiles).  The
// work-group holds two kinds of waves:
//   producers (DK/32 waves) load and gate chunk c+1 into one half of a double
//     buffer while
//   consumers (DK/32 waves, 32 value columns each, holding the state) run the
//     products of chunk c from the other half.
// Per chunk c, two barriers:
//   phase 1  consumers: load v(c+1); scores(c) -> a, inter(c), state update(c)
//            producers: load q, k, log-gates(c+2); gate(c+1) -> x[(c+1)&1]
//   ---- barrier A
//   phase 2  consumers: intra(c) from a, store O(c), v(c+1)^T -> x[(c+1)&1]
//            producers: take the loads of c+2
//   ---- barrier B
// (v needs no gating, so each consumer moves its own value columns.)
// A producer wave owns 32 channels of all 64 rows; a lane takes rows
// 4rq..4rq+3 and 8 channels, with 16-byte loads, and the 16 lanes of one
// 16-lane row hold the 16 row quads of the same channels.  The chunk's
// cumulative sums are then a scan inside the wave (in-thread over 4 rows,
// across the row quads by in-row lane shifts), so gating needs no exchange
// between waves.  Each
// producer wave picks the single-reference or the sub-block form for its own
// channels; the sub-block tables hold 1 for single-reference channels, so the
// two forms mix freely within a chunk.  Tiles whose contraction runs over
// tokens ([channel][token]) are unpadded with their 16-byte granules permuted
// by row (see swz), which keeps the row-strided fragment reads free of bank
// conflicts.

template <int DK>
struct PipeBuf {
  static constexpr int DKP = DK + 8;
  bf16 qs[kC][DKP];             // fast: q_t 2^{b_t}; sub-block: q_t 2^{b_t - R_i}
  bf16 ks[kC][DKP];             // fast: k_s 2^{-b_s}; sub-block: k_s 2^{R_j - b_s}
  bf16 khT[DK * kC];            // (k_s 2^{b_last - b_s})^T, swizzled
  bf16 vT[DK * kC];             // v^T, swizzled
  alignas(16) float decay[DK];  // 2^{b_last}
  alignas(16) float eR[4][DK];  // sub-block chunks only: 2^{R_i}
  alignas(16) float vij[6][DK]; // sub-block chunks only: 2^{R_i - R_j}
  int fastw[4];                 // per producer wave: 1 if its channels take one reference
};
template <int DK>
struct PipeSmem {
  PipeBuf<DK> x[2];
  bf16 a[kC][kC + 8];            // masked intra scores A[t][s]
};

// Cross-lane moves inside 16-lane rows (DPP): shift down by N lanes with zero
// fill, and broadcast of row lane N to the whole row.
template <int N>
__device__ __forceinline__ float row_shr(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + N, 0xf, 0xf, true));
}
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + N, 0xf, 0xf, false));
}

// element offset of (row, col) in a [rows][64] tile: granule col/8 permuted by row
__device__ __forceinline__ int swz(int row, int col) {
  return row * kC + ((((col >> 3) ^ row ^ (row >> 3)) & 7) << 3) + (col & 7);
}

template <int DK, typename GT>
__global__ __launch_bounds__(4 * DK, 1) void gla_output_ws(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const GT* __restrict__ la, const float* __restrict__ h0, const float* __restrict__ ws_state,
    const float* __restrict__ ws_gamma, bf16* __restrict__ o, float* __restrict__ hT, int T_arg,
    int cps, int G, const int* __restrict__ cu, int N, int H) {
  constexpr int NCB = DK / 16;             // 16-row blocks of the state
  constexpr int KS = DK / 32;              // contraction steps over channels
  constexpr int NWC = DK / 32;             // consumer waves (= producer waves)
  constexpr int NB = (10 + NWC - 1) / NWC; // score blocks per consumer wave, at most
  constexpr int OCT = DK / 8;              // 8-channel octets per row
  typedef bf16x8 F;
  __shared__ PipeSmem<DK> sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int r16 = lane & 15, g = lane >> 4;
  const bool consumer = wave < NWC;
  const int seg = blockIdx.x, bh = blockIdx.y;
  const SeqRows sr = seq_rows(cu, N, T_arg, H, bh);
  const int T_len = sr.len;
  const size_t off = sr.row0 * DK;
  const int nc = (T_len + kC - 1) / kC;
  const int c_begin = seg * cps, c_end = min(nc, c_begin + cps);
  const size_t s_base = (size_t)bh * DK * DK;
  // a packed sequence covers the first Gs of the plan's segments
  const int Gs = cu ? max(1, (nc + cps - 1) / cps) : G;
  if (seg >= Gs) return;
  if (nc == 0) {  // an empty packed sequence: the state passes through unchanged
    if (hT)
      for (int e = tid; e < DK * DK; e += 4 * DK) hT[s_base + e] = h0 ? h0[s_base + e] : 0.f;
    return;
  }

  for (int e = tid; e < 512; e += 4 * DK) {
    const int z = e >> 8, t = (e >> 4) & 15, s = e & 15;
    sm.a[32 * z + t][32 * z + 16 + s] = to_t<bf16>(0.f);
  }

  if (consumer) {
    // ---------------------------------------------------------- consumer
    const int cw = wave;  // value columns 32cw .. 32cw+31, as two 16-column blocks
    // state entering the segment: h0 carried through the earlier segments'
    // local end states and decays
    f32x4 S[2][NCB];  // S[nt][cb]: rows 16cb + 4g + r, column 32cw + 16nt + r16
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S[nt][cb][r] = h0 ? h0[s_base + (16 * cb + 4 * g + r) * DK + 32 * cw + 16 * nt + r16] : 0.f;
    for (int sg = 0; sg < seg; ++sg) {  // local states are column-major
      const float* loc = ws_state + ((size_t)bh * (G - 1) + sg) * DK * DK;
      const float* gm = ws_gamma + ((size_t)bh * (G - 1) + sg) * DK;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const f32x4 g4 = *reinterpret_cast<const f32x4*>(&gm[16 * cb + 4 * g]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&loc[(32 * cw + 16 * nt + r16) * DK + 16 * cb + 4 * g]);
#pragma unroll
          for (int r = 0; r < 4; ++r) S[nt][cb][r] = exp2_fast(g4[r]) * S[nt][cb][r] + l4[r];
        }
      }
    }

    // v of a chunk: lane takes rows 4vr..4vr+3, columns 32cw + 8vo .. +7
    const int vo = lane & 3, vr = lane >> 2;
    const u32 vv2 = (u32)((4 * vr * DK + 32 * cw + 8 * vo) * 2);
    u32x4 vl[4];
    auto load_v = [&](int ch) {
      const size_t e0 = off + (size_t)ch * kC * DK;
      const Buf cv(v + e0, (u32)(T_len - ch * kC) * DK * 2);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) vl[rr] = cv.ld128(vv2 + rr * DK * 2);
    };
    auto store_vT = [&](PipeBuf<DK>& X) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        u32 e[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const u32 w = vl[rr][c >> 1];
          e[rr] = (c & 1) ? (w >> 16) : (w & 0xffffu);
        }
        *reinterpret_cast<U2*>(&X.vT[swz(32 * cw + 8 * vo + c, 4 * vr)]) =
            U2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
      }
    };

    // alongside the producers' prologue (chunk c_begin gated, c_begin+1 taken)
    load_v(c_begin);
    store_vT(sm.x[c_begin & 1]);
    lds_barrier();
    for (int ch = c_begin; ch < c_end; ++ch) {
      PipeBuf<DK>& X = sm.x[ch & 1];
      const bool has_next = ch + 1 < c_end;
      if (has_next) load_v(ch + 1);
      int fw = 1;
#pragma unroll
      for (int w = 0; w < NWC; ++w) fw &= X.fastw[w];
      const bool fast = __builtin_amdgcn_readfirstlane(fw) != 0;
      // ---- phase 1: scores -> a
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const int blk = cw + n * NWC;
        if (blk < 10) {
          const int i = blk_i(blk), j = blk_j(blk);
          F af[KS], bf[KS];
#pragma unroll
          for (int p = 0; p < KS; ++p) {
            af[p] = ld8<bf16>(&X.ks[16 * j + r16][32 * p + 8 * g]);
            bf[p] = ld8<bf16>(&X.qs[16 * i + r16][32 * p + 8 * g]);
          }
          if (!fast && j < i) {
#pragma unroll
            for (int p = 0; p < KS; ++p) bf[p] = scale8(bf[p], &X.vij[pair_of(i, j)][32 * p + 8 * g]);
          }
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int p = 0; p < KS; ++p) mma(acc, af[p], bf[p]);
          if (i == j) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (4 * g + r > r16) acc[r] = 0.f;
          }
          st4<bf16>(&sm.a[16 * i + r16][16 * j + 4 * g], acc);
        }
      }
      // ---- phase 1: inter, O^T[n][t] = sum_c S[c][n] qs[t][c] (state entering the chunk)
      f32x4 O[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        F qf[2][KS];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int p = 0; p < KS; ++p)
            qf[u][p] = ld4x2<bf16>(&X.qs[16 * (2 * h + u) + r16][32 * p + 4 * g]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int qb = 2 * h + u;
            O[nt][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (fast) {
#pragma unroll
              for (int p = 0; p < KS; ++p)
                mma(O[nt][qb], pack_acc<bf16>(S[nt][2 * p], S[nt][2 * p + 1]), qf[u][p]);
            } else {
              // sub-block form: query block i sees the state rows scaled by 2^{R_i}
#pragma unroll
              for (int p = 0; p < KS; ++p) {
                const f32x4 e0 = *reinterpret_cast<const f32x4*>(&X.eR[qb][32 * p + 4 * g]);
                const f32x4 e1 = *reinterpret_cast<const f32x4*>(&X.eR[qb][32 * p + 16 + 4 * g]);
                mma(O[nt][qb], pack_acc<bf16>(S[nt][2 * p] * e0, S[nt][2 * p + 1] * e1), qf[u][p]);
              }
            }
          }
      }
      // ---- phase 1: state update, S = diag(2^{b_last}) S + khT V
      F vf[2][2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int p = 0; p < 2; ++p)
          vf[nt][p] = ld8<bf16>(&X.vT[swz(32 * cw + 16 * nt + r16, 32 * p + 8 * g)]);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        F kf[NCB / 2][2];
#pragma unroll
        for (int u = 0; u < NCB / 2; ++u)
#pragma unroll
          for (int p = 0; p < 2; ++p)
            kf[u][p] = ld8<bf16>(&X.khT[swz(16 * (h * NCB / 2 + u) + r16, 32 * p + 8 * g)]);
#pragma unroll
        for (int u = 0; u < NCB / 2; ++u) {
          const int cb = h * NCB / 2 + u;
          const f32x4 dec = *reinterpret_cast<const f32x4*>(&X.decay[16 * cb + 4 * g]);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            S[nt][cb] *= dec;
#pragma unroll
            for (int p = 0; p < 2; ++p) mma(S[nt][cb], kf[u][p], vf[nt][p]);
          }
        }
      }
      lds_barrier();  // (A) scores visible
      // ---- phase 2: intra, O^T[n][t] += sum_s vT[n][s] A[t][s]
      {
        F af[4][2];
#pragma unroll
        for (int qb = 0; qb < 4; ++qb)
#pragma unroll
          for (int p = 0; p <= qb / 2; ++p) af[qb][p] = ld8<bf16>(&sm.a[16 * qb + r16][32 * p + 8 * g]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int qb = 0; qb < 4; ++qb)
#pragma unroll
            for (int p = 0; p <= qb / 2; ++p) mma(O[nt][qb], vf[nt][p], af[qb][p]);
      }
      bf16* oc_ = o + off + (size_t)ch * kC * DK;  // chunk base (uniform)
      const int rows = T_len - ch * kC;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int qb = 0; qb < 4; ++qb)
          if (16 * qb + r16 < rows)
            st4<bf16>(oc_ + (u32)((16 * qb + r16) * DK + 32 * cw + 16 * nt + 4 * g), O[nt][qb]);
      if (has_next) store_vT(sm.x[(ch + 1) & 1]);
      lds_barrier();  // (B) chunk done
    }
    if (hT && seg == Gs - 1) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            hT[s_base + (16 * cb + 4 * g + r) * DK + 32 * cw + 16 * nt + r16] = S[nt][cb][r];
    }
  } else {
    // ---------------------------------------------------------- producer
    const int pw = wave - NWC;                // channels 32pw .. 32pw+31
    const int ol = lane >> 4, rq = lane & 15;  // channels ch0 .. ch0+7, rows 4rq .. 4rq+3
    const int ch0 = 32 * pw + 8 * ol;
    const int i_sub = rq >> 2;                // 16-row sub-block of the rows
    // per-thread byte offsets inside a chunk, fixed for the whole kernel: the
    // chunk moves the (scalar) buffer base instead, so no address register is
    // rewritten while a load that reads it may still be queued
    const u32 vo2 = (u32)((4 * rq * DK + ch0) * 2), ve = (u32)(4 * rq * DK + ch0);

    u32x4 nq[4], nk[4];  // loads in flight
    u32x4 hq[4], hk[4];  // chunk held for gating
    Gate8<GT> nla[4], hla[4];
    // loads of one chunk, one row of the quad at a time (issued spread over the
    // gating work, so a wave never blocks on a full memory queue for long)
    struct Src { Buf q, k, la; };
    auto src_of = [&](int ch) {
      const size_t e0 = off + (size_t)ch * kC * DK;
      const u32 rem = (u32)(T_len - ch * kC) * DK;  // elements from the chunk start to the end
      return Src{Buf(q + e0, rem * 2), Buf(k + e0, rem * 2), Buf(la + e0, rem * (u32)sizeof(GT))};
    };
    auto issue_row = [&](const Src& sr, int rr) {
      nq[rr] = sr.q.ld128(vo2 + rr * DK * 2);
      nk[rr] = sr.k.ld128(vo2 + rr * DK * 2);
      nla[rr].load(sr.la, ve + rr * DK);
    };
    auto issue = [&](int ch) {
      const Src sr = src_of(ch);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) issue_row(sr, rr);
    };
    auto take = [&]() {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        hq[rr] = nq[rr];
        hk[rr] = nk[rr];
        hla[rr] = nla[rr];
      }
    };
    auto gate = [&](PipeBuf<DK>& X, const Src& sr, int gch) {  // gch: the chunk gated
      issue_row(sr, 0);
      // b: inclusive log2 cumsum from the chunk start (in-thread over 4 rows,
      // then a scan over the 16 row quads inside the 16-lane row)
      // (summed without the gate floor, and again with it only in a thread
      // where some channel's 4-row total falls below the floor)
      float b[4][8], inc[8], blast[8];
      auto sum = [&](auto floored) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          float run = 0.f;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const float g = decltype(floored)::value ? hla[rr].log2_at(c) : hla[rr].log2_nofloor_at(c);
            run += gate_row<GT>(g, 4 * rq + rr < T_len - gch * kC);
            b[rr][c] = run;
          }
          inc[c] = run;
        }
      };
      sum(std::false_type());
      {
        float m = inc[0];
#pragma unroll
        for (int c = 1; c < 8; ++c) m = fminf(m, inc[c]);
        if (m < kMinLog2Gate) sum(std::true_type());
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) inc[c] += row_shr<1>(inc[c]);
#pragma unroll
      for (int c = 0; c < 8; ++c) inc[c] += row_shr<2>(inc[c]);
      issue_row(sr, 1);
#pragma unroll
      for (int c = 0; c < 8; ++c) inc[c] += row_shr<4>(inc[c]);
#pragma unroll
      for (int c = 0; c < 8; ++c) inc[c] += row_shr<8>(inc[c]);
      float bmin = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float ex = inc[c] - b[3][c];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) b[rr][c] += ex;
        blast[c] = row_bcast<15>(inc[c]);  // the last row quad holds the chunk total
        bmin = c ? fminf(bmin, blast[c]) : blast[c];
      }
      const bool fast = !__any(bmin < -kFastLog2);  // uniform over the wave
      if (lane == 0) X.fastw[pw] = fast ? 1 : 0;
      if (rq == 0) {
        *reinterpret_cast<f32x4*>(&X.decay[ch0]) =
            f32x4{exp2_fast(blast[0]), exp2_fast(blast[1]), exp2_fast(blast[2]), exp2_fast(blast[3])};
        *reinterpret_cast<f32x4*>(&X.decay[ch0 + 4]) =
            f32x4{exp2_fast(blast[4]), exp2_fast(blast[5]), exp2_fast(blast[6]), exp2_fast(blast[7])};
      }
      // references: none (fast) or b at row 16i+7 for sub-block i
      float Ri[8];
      if (fast) {
#pragma unroll
        for (int c = 0; c < 8; ++c) Ri[c] = 0.f;
        // the sub-block tables read 1 for these channels
        if (rq < 10) {
          float* dst = rq < 4 ? &X.eR[rq][ch0] : &X.vij[rq - 4][ch0];
          *reinterpret_cast<f32x4*>(dst) = f32x4{1.f, 1.f, 1.f, 1.f};
          *reinterpret_cast<f32x4*>(dst + 4) = f32x4{1.f, 1.f, 1.f, 1.f};
        }
      } else {
        float R[4][8];  // row 16i+7 is the last row of row quad 4i+1
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          R[0][c] = row_bcast<1>(b[3][c]);
          R[1][c] = row_bcast<5>(b[3][c]);
          R[2][c] = row_bcast<9>(b[3][c]);
          R[3][c] = row_bcast<13>(b[3][c]);
        }
#pragma unroll
        for (int c = 0; c < 8; ++c)
          Ri[c] = i_sub == 0 ? R[0][c] : i_sub == 1 ? R[1][c] : i_sub == 2 ? R[2][c] : R[3][c];
        if (rq < 4) {
          const int i = rq;
          float e[8];
#pragma unroll
          for (int c = 0; c < 8; ++c)
            e[c] = exp2_fast(i == 0 ? R[0][c] : i == 1 ? R[1][c] : i == 2 ? R[2][c] : R[3][c]);
          *reinterpret_cast<f32x4*>(&X.eR[i][ch0]) = f32x4{e[0], e[1], e[2], e[3]};
          *reinterpret_cast<f32x4*>(&X.eR[i][ch0 + 4]) = f32x4{e[4], e[5], e[6], e[7]};
        } else if (rq < 10) {
          const int pr = rq - 4, pi = pair_i(pr), pj = pair_j(pr);
          float e[8];
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const float a0 = pi == 1 ? R[1][c] : pi == 2 ? R[2][c] : R[3][c];
            const float a1 = pj == 0 ? R[0][c] : pj == 1 ? R[1][c] : R[2][c];
            e[c] = exp2_fast(a0 - a1);
          }
          *reinterpret_cast<f32x4*>(&X.vij[pr][ch0]) = f32x4{e[0], e[1], e[2], e[3]};
          *reinterpret_cast<f32x4*>(&X.vij[pr][ch0 + 4]) = f32x4{e[4], e[5], e[6], e[7]};
        }
      }
      issue_row(sr, 2);
      // gated tiles, two rows at a time, rounded to bf16 pairs as they are made
#pragma unroll
      for (int hp = 0; hp < 2; ++hp) {
        if (hp == 1) issue_row(sr, 3);
        u32 qw[2][4], kw[2][4];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float eKh = exp2_fast(blast[c] - Ri[c]);
          float qx[2], kx[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int rr = 2 * hp + u;
            const float d = b[rr][c] - Ri[c];
            qx[u] = bf_at(hq[rr], c) * exp2_fast(d);
            kx[u] = bf_at(hk[rr], c) * exp2_fast(-d);
            if (c & 1) {
              qw[u][c >> 1] |= pack_bf2(0.f, qx[u]) & 0xffff0000u;
              kw[u][c >> 1] |= pack_bf2(0.f, kx[u]) & 0xffff0000u;
            } else {
              qw[u][c >> 1] = pack_bf2(qx[u], 0.f) & 0xffffu;
              kw[u][c >> 1] = pack_bf2(kx[u], 0.f) & 0xffffu;
            }
          }
          *reinterpret_cast<u32*>(&X.khT[swz(ch0 + c, 4 * rq + 2 * hp)]) =
              pack_bf2(kx[0] * eKh, kx[1] * eKh);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int row = 4 * rq + 2 * hp + u;
          *reinterpret_cast<u32x4*>(&X.qs[row][ch0]) = u32x4{qw[u][0], qw[u][1], qw[u][2], qw[u][3]};
          *reinterpret_cast<u32x4*>(&X.ks[row][ch0]) = u32x4{kw[u][0], kw[u][1], kw[u][2], kw[u][3]};
        }
      }
    };

    // ---- prologue: chunk c_begin gated, c_begin+1 taken
    issue(c_begin);
    take();
    gate(sm.x[c_begin & 1], src_of(min(c_begin + 1, c_end - 1)), c_begin);
    take();
    lds_barrier();
    // Loads are issued at the top of an iteration and taken at its end, so no
    // load is in flight across the loop edge (a register copy there would have
    // to wait for it).  Past the end, the last chunk is loaded again, unused.
    for (int ch = c_begin; ch < c_end; ++ch) {
      const Src nx = src_of(min(ch + 2, c_end - 1));
      if (ch + 1 < c_end) {
        gate(sm.x[(ch + 1) & 1], nx, ch + 1);
      } else {
        issue(min(ch + 2, c_end - 1));
      }
      lds_barrier();  // (A)
      take();
      lds_barrier();  // (B)
    }
  }
}

// Backward checkpoints: the state entering each block b >= 1 of a head,
//   S_in(b) = diag(2^{Gamma(b-1)}) S_in(b-1) + S_loc(b-1),  S_in(0) = h0 or 0,
// from the local end states and log2 decays that the state pass left at the
// start of each block's rows; S_in(b) is written row-major ([c][j]) right after
// them (rows of block b-1, offset DK*DK + DK).
template <int DK>
__global__ __launch_bounds__(256) void gla_checkpoint_compose(const float* __restrict__ h0,
                                                              float* __restrict__ region,
                                                              int T_len, int nb, int rows) {
  constexpr int PER = DK * DK / 256;
  const int bh = blockIdx.x, tid = threadIdx.x;
  float* base = region + (size_t)bh * T_len * DK;
  float S[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) S[i] = h0 ? h0[(size_t)bh * DK * DK + tid + 256 * i] : 0.f;
  for (int b = 1; b < nb; ++b) {
    float* prev = base + (size_t)(b - 1) * rows * DK;
    const float* gam = prev + DK * DK;
    float* out = prev + DK * DK + DK;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + 256 * i, c = e / DK, j = e % DK;
      S[i] = exp2_fast(gam[c]) * S[i] + prev[j * DK + c];
      out[e] = S[i];
    }
  }
}

__global__ void state_copy_kernel(const float* __restrict__ h0, float* __restrict__ hT, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) hT[i] = h0 ? h0[i] : 0.f;
}

template <typename T, int DK, typename GT>
hipError_t launch_typed(const Shape& s, const Plan& pl, const void* q, const void* k,
                        const void* v, const void* la_, const float* h0, void* o, float* hT,
                        void* ws, hipStream_t st) {
  const GT* la = (const GT*)la_;
  const int BH = s.B * s.H;
  float* ws_state = (float*)ws;
  float* ws_gamma = ws_state + (size_t)BH * (pl.G - 1) * DK * DK;
  if (pl.G > 1) {
    hipLaunchKernelGGL((gla_state_pass<T, DK, GT>), dim3(pl.G - 1, BH), dim3(4 * DK), 0, st,
                       (const T*)k, (const T*)v, la, ws_state, ws_gamma, s.T, pl.cps, pl.G,
                       s.cu, s.n_tokens, s.H);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if constexpr (sizeof(T) == 2) {
    hipLaunchKernelGGL((gla_output_ws<DK, GT>), dim3(pl.G, BH), dim3(4 * DK), 0, st, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, la, h0, ws_state, ws_gamma, (bf16*)o, hT, s.T, pl.cps,
                       pl.G, s.cu, s.n_tokens, s.H);
  } else {
    static_assert(sizeof(GT) == 4, "fp32 problems take float log gates");
    hipLaunchKernelGGL((gla_output_pass<T, DK>), dim3(pl.G, BH), dim3(4 * DK), 0, st, (const T*)q,
                       (const T*)k, (const T*)v, la, h0, ws_state, ws_gamma, (T*)o, hT, s.T, pl.cps, pl.G,
                       s.cu, s.n_tokens, s.H);
  }
  return hipGetLastError();
}

}  // namespace

namespace {
template <typename T, int DK, typename GT>
void launch_checkpoints_typed(const Shape& s, const void* k, const void* v, const void* la,
                              const float* h0, float* region, int cps, int nb, hipStream_t st) {
  const int BH = s.B * s.H;
  hipLaunchKernelGGL((gla_state_pass<T, DK, GT>), dim3(nb - 1, BH), dim3(4 * DK), 0, st,
                     (const T*)k, (const T*)v, (const GT*)la, region, region, s.T, cps, nb,
                     (const int*)nullptr, 0, s.H, cps * kC);
  hipLaunchKernelGGL(gla_checkpoint_compose<DK>, dim3(BH), dim3(256), 0, st, h0, region, s.T, nb,
                     cps * kC);
}
}  // namespace

// States entering blocks 1..nb-1 of cps chunks (see gla_checkpoint_compose):
// region is [B*H, T, dk] floats, block b >= 1's entry state at rows
// (b-1)*cps*64 + offset dk*dk + dk, row-major.
hipError_t launch_gla_checkpoints(const Shape& s, const void* k, const void* v, const void* la,
                                  const float* h0, float* region, int cps, int nb,
                                  hipStream_t st) {
  if (nb < 2 || s.B * s.H == 0) return hipSuccess;
  if (s.dtype == 1) {
    if (s.gate == 1) {
      if (s.dk == 128) launch_checkpoints_typed<bf16, 128, bf16>(s, k, v, la, h0, region, cps, nb, st);
      else launch_checkpoints_typed<bf16, 64, bf16>(s, k, v, la, h0, region, cps, nb, st);
    } else {
      if (s.dk == 128) launch_checkpoints_typed<bf16, 128, float>(s, k, v, la, h0, region, cps, nb, st);
      else launch_checkpoints_typed<bf16, 64, float>(s, k, v, la, h0, region, cps, nb, st);
    }
  } else {
    if (s.dk == 128) launch_checkpoints_typed<float, 128, float>(s, k, v, la, h0, region, cps, nb, st);
    else launch_checkpoints_typed<float, 64, float>(s, k, v, la, h0, region, cps, nb, st);
  }
  return hipGetLastError();
}

// Pieces per segment of the hybrid path's state pass: the largest divisor m of
// the chunks per segment with (G-1) m B H <= 256 work-groups, so that a head
// count too small to fill the chip with whole segments still does (packed
// batches keep whole segments).
int state_pieces(const Shape& s, const Plan& pl) {
  if (s.cu || pl.G < 2) return 1;
  const long long used = (long long)(pl.G - 1) * s.B * s.H;
  int m = 1;
  for (int c = 2; c <= pl.cps; ++c)
    if (pl.cps % c == 0 && used * c <= 256) m = c;
  return m;
}

size_t gla_fwd_workspace_bytes(const Shape& s) {
  const Plan pl = make_plan(s);
  return (size_t)s.B * s.H * (pl.G - 1) * state_pieces(s, pl) * ((size_t)s.dk * s.dv + s.dk) *
         sizeof(float);
}

hipError_t launch_state_copy(const Shape& s, const float* h0, float* hT, hipStream_t st) {
  size_t n = (size_t)s.B * s.H * s.dk * s.dv;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(state_copy_kernel, dim3((n + 255) / 256), dim3(256), 0, st, h0, hT, n);
  return hipGetLastError();
}

hipError_t launch_gla_state(const Shape& s, const void* k, const void* v, const void* la,
                            void* ws, int* G, int* cps, int* m, hipStream_t st) {
  const Plan pl = make_plan(s);
  *G = pl.G;
  *cps = pl.cps;
  *m = state_pieces(s, pl);
  if (s.T == 0 || pl.G < 2 || s.dtype != 1 || (s.dk != 128 && s.dk != 64)) return hipSuccess;
  const int BH = s.B * s.H;
  // (G-1) m pieces of cps / m chunks: the state pass sees them as the first
  // segments of a plan with (G-1) m + 1 segments
  const int P = (pl.G - 1) * *m;
  float* ws_state = (float*)ws;
  float* ws_gamma = ws_state + (size_t)BH * P * s.dk * s.dk;
  auto go = [&](auto kernel, auto gt) {
    typedef decltype(gt) GT;
    hipLaunchKernelGGL(kernel, dim3(P, BH), dim3(4 * s.dk), 0, st, (const bf16*)k,
                       (const bf16*)v, (const GT*)la, ws_state, ws_gamma, s.T, pl.cps / *m, P + 1,
                       s.cu, s.n_tokens, s.H, 0);
  };
  if (s.dk == 128)
    s.gate == 1 ? go(gla_state_pass<bf16, 128, bf16>, bf16()) : go(gla_state_pass<bf16, 128, float>, 0.f);
  else
    s.gate == 1 ? go(gla_state_pass<bf16, 64, bf16>, bf16()) : go(gla_state_pass<bf16, 64, float>, 0.f);
  return hipGetLastError();
}

hipError_t launch_gla_fwd(const Shape& s, const void* q, const void* k, const void* v,
                          const void* la, const float* h0, void* o, float* hT, void* ws,
                          hipStream_t st) {
  if (s.T == 0) return hT ? launch_state_copy(s, h0, hT, st) : hipSuccess;
  const Plan pl = make_plan(s);
  if (s.dtype == 1) {
    if (s.gate == 1) {
      if (s.dk == 128) return launch_typed<bf16, 128, bf16>(s, pl, q, k, v, la, h0, o, hT, ws, st);
      return launch_typed<bf16, 64, bf16>(s, pl, q, k, v, la, h0, o, hT, ws, st);
    }
    if (s.dk == 128) return launch_typed<bf16, 128, float>(s, pl, q, k, v, la, h0, o, hT, ws, st);
    return launch_typed<bf16, 64, float>(s, pl, q, k, v, la, h0, o, hT, ws, st);
  }
  if (s.dk == 128) return launch_typed<float, 128, float>(s, pl, q, k, v, la, h0, o, hT, ws, st);
  return launch_typed<float, 64, float>(s, pl, q, k, v, la, h0, o, hT, ws, st);
}

}  // namespace lz
