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
//   2. carry pass   (per head): S_in(g+1) = 2^{Gamma_g} S_in(g) + S_loc(g);
//   3. output pass  (all segments, parallel): the chunk recurrence below,
//                   started from S_in(g).
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
#include "common.hpp"
#include "kernels.hpp"

namespace lz {
namespace {

constexpr int kC = 64;  // chunk length

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
  g = g < 1 ? 1 : (g > 16 ? 16 : g);
  if (g > p.nc) g = p.nc > 0 ? p.nc : 1;
  p.cps = p.nc > 0 ? (p.nc + g - 1) / g : 1;
  p.G = p.nc > 0 ? (p.nc + p.cps - 1) / p.cps : 1;
  return p;
}

template <typename T, int DK>
struct OutSmem {
  static constexpr int DKP = DK + 8;
  static constexpr int CP = kC + 8;
  T qg[kC][DKP];     // q_t 2^{b_t - R_i}
  T kg[kC][DKP];     // k_s 2^{R_j - b_s}
  T qh[kC][DKP];     // q_t 2^{b_t}
  T khT[DK][CP];     // (k_s 2^{b_last - b_s})^T
  T vT[DK][CP];      // v^T
  T a[kC][CP];       // masked intra scores A[t][s]
  float tot[8][DK];  // per-8-row-group sums of log2 gates
  float vij[6][DK];  // 2^{R_i - R_j} for the off-diagonal pairs
  float decay[DK];   // 2^{b_last}
};

template <typename T, int DK>
struct StateSmem {
  static constexpr int CP = kC + 8;
  T khT[DK][CP];
  T vT[DK][CP];
  float tot[8][DK];
  float decay[DK];
};

// Per-thread gating slice: 8 rows (8*rg ..) x 2 channels (2*cp, 2*cp+1).
template <typename T, int DK>
struct Slice {
  static constexpr int ES = sizeof(T);
  typename Pair<T>::type q[8], k[8], v[8];
  U2 la[8];
  __device__ __forceinline__ void load(const Buf& bq, const Buf& bk, const Buf& bv,
                                       const Buf& bla, int t0, int rg, int cp, bool need_q) {
    const u32 row0 = (u32)(t0 + 8 * rg);
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const u32 e = (row0 + rr) * DK + 2 * cp;
      if (need_q) q[rr] = ld_pair<T>(bq, e * ES);
      k[rr] = ld_pair<T>(bk, e * ES);
      v[rr] = ld_pair<T>(bv, e * ES);
      la[rr] = bla.ld64(e * 4);
    }
  }
};

// Local (row-group) log2 cumsum of the slice's gates; returns the group total.
template <typename T, int DK>
__device__ __forceinline__ f32x2 local_cumsum(const Slice<T, DK>& sl, f32x2* b) {
  f32x2 run = {0.f, 0.f};
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    const f32x2 la = unpack2(sl.la[rr], 0.f);
    run[0] += la[0] * kLog2e;
    run[1] += la[1] * kLog2e;
    b[rr] = run;
  }
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
template <typename T, int DK>
__global__ __launch_bounds__(4 * DK, 1) void gla_state_pass(
    const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ la,
    float* __restrict__ ws_state, float* __restrict__ ws_gamma, int T_len, int cps, int G) {
  constexpr int NCB = DK / 16;
  typedef typename Frag<T>::type F;
  __shared__ StateSmem<T, DK> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int cp = tid % (DK / 2), rg = tid / (DK / 2);
  const int seg = blockIdx.x, bh = blockIdx.y;
  const size_t off = (size_t)bh * T_len * DK;
  const Buf bk(k + off, (u32)((size_t)T_len * DK * sizeof(T)));
  const Buf bv(v + off, (u32)((size_t)T_len * DK * sizeof(T)));
  const Buf bla(la + off, (u32)((size_t)T_len * DK * 4));
  const int nc = (T_len + kC - 1) / kC;
  const int c_begin = seg * cps, c_end = min(nc, c_begin + cps);

  f32x4 S[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) S[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x2 gsum = {0.f, 0.f};

  Slice<T, DK> cur;
  cur.load(bk, bk, bv, bla, c_begin * kC, rg, cp, false);
  for (int ch = c_begin; ch < c_end; ++ch) {
    f32x2 b[8];
    const f32x2 tot = local_cumsum(cur, b);
    typename Pair<T>::type kk[8], vv[8];
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) { kk[rr] = cur.k[rr]; vv[rr] = cur.v[rr]; }
    cur.load(bk, bk, bv, bla, min(ch + 1, c_end - 1) * kC, rg, cp, false);
    sm.tot[rg][2 * cp] = tot[0];
    sm.tot[rg][2 * cp + 1] = tot[1];
    lds_barrier();
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int c = 2 * cp + x;
      float pre = 0.f, blast = 0.f;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float tr = sm.tot[r][c];
        pre += (r < rg) ? tr : 0.f;
        blast += tr;
      }
      float kh[8], vc[8];
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        kh[rr] = unpack2(kk[rr], T())[x] * exp2_fast(blast - (b[rr][x] + pre));
        vc[rr] = unpack2(vv[rr], T())[x];
      }
      store8<T>(&sm.khT[c][8 * rg], kh);
      store8<T>(&sm.vT[c][8 * rg], vc);
      if (rg == 0) sm.decay[c] = exp2_fast(blast);
      gsum[x] += blast;
    }
    lds_barrier();
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) S[cb][r] *= sm.decay[16 * cb + 4 * g + r];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        F af = ld8<T>(&sm.khT[16 * cb + r16][32 * p + 8 * g]);
        F bf = ld8<T>(&sm.vT[16 * wave + r16][32 * p + 8 * g]);
        mma(S[cb], af, bf);
      }
    }
  }
  float* dst = ws_state + ((size_t)bh * (G - 1) + seg) * DK * DK;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[(16 * cb + 4 * g + r) * DK + 16 * wave + r16] = S[cb][r];
  if (rg == 0) {
    float* gd = ws_gamma + ((size_t)bh * (G - 1) + seg) * DK;
    gd[2 * cp] = gsum[0];
    gd[2 * cp + 1] = gsum[1];
  }
}

// ------------------------------------------------------------------ pass 2
// S_in(g+1) = 2^{Gamma_g} S_in(g) + S_loc(g), written over S_loc(g).
__global__ __launch_bounds__(256) void gla_carry_pass(const float* __restrict__ h0,
                                                     float* __restrict__ ws_state,
                                                     const float* __restrict__ ws_gamma, int DK,
                                                     int G) {
  const int bh = blockIdx.x;
  const size_t n = (size_t)DK * DK;
  for (size_t e = threadIdx.x + (size_t)blockIdx.y * 256; e < n; e += 256 * gridDim.y) {
    const int c = (int)(e / DK);
    float S = h0 ? h0[(size_t)bh * n + e] : 0.f;
    for (int s = 0; s < G - 1; ++s) {
      float* slot = ws_state + ((size_t)bh * (G - 1) + s) * n;
      S = exp2_fast(ws_gamma[((size_t)bh * (G - 1) + s) * DK + c]) * S + slot[e];
      slot[e] = S;
    }
  }
}

// ------------------------------------------------------------------ pass 3
template <typename T, int DK>
__global__ __launch_bounds__(4 * DK, 1) void gla_output_pass(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ la, const float* __restrict__ h0, const float* __restrict__ ws_state,
    T* __restrict__ o, float* __restrict__ hT, int T_len, int cps, int G) {
  constexpr int NCB = DK / 16;
  constexpr int KS = DK / 32;
  constexpr int NW = DK / 16;
  typedef typename Frag<T>::type F;
  __shared__ OutSmem<T, DK> sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int cp = tid % (DK / 2), rg = tid / (DK / 2);
  const int i_sub = rg >> 1;  // 16-row sub-block of this thread's rows (uniform per wave)
  const int seg = blockIdx.x, bh = blockIdx.y;
  const size_t off = (size_t)bh * T_len * DK;
  const u32 nbytes = (u32)((size_t)T_len * DK * sizeof(T));
  const Buf bq(q + off, nbytes), bk(k + off, nbytes), bv(v + off, nbytes);
  const Buf bla(la + off, (u32)((size_t)T_len * DK * 4));
  const int nc = (T_len + kC - 1) / kC;
  const int c_begin = seg * cps, c_end = min(nc, c_begin + cps);
  const int ncol = 16 * wave;
  const size_t s_base = (size_t)bh * DK * DK;

  // state slice S[16cb + 4g + r][ncol + r16]
  const float* s0 = seg == 0 ? (h0 ? h0 + s_base : nullptr)
                             : ws_state + ((size_t)bh * (G - 1) + seg - 1) * DK * DK;
  f32x4 S[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int r = 0; r < 4; ++r) S[cb][r] = s0 ? s0[(16 * cb + 4 * g + r) * DK + ncol + r16] : 0.f;

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
    const f32x2 tot = local_cumsum(cur, b);
    typename Pair<T>::type qq[8], kk[8], vv[8];
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) { qq[rr] = cur.q[rr]; kk[rr] = cur.k[rr]; vv[rr] = cur.v[rr]; }
    cur.load(bq, bk, bv, bla, min(ch + 1, c_end - 1) * kC, rg, cp, true);
    sm.tot[rg][2 * cp] = tot[0];
    sm.tot[rg][2 * cp + 1] = tot[1];
    lds_barrier();  // (A) group totals visible; previous chunk's LDS reads are done

    // ---- gated operands for rows 8rg..8rg+7, channels 2cp, 2cp+1
    float qgv[8][2], kgv[8][2], qhv[8][2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int c = 2 * cp + x;
      // prefix sums over row groups with selects only (run-time indices into a
      // register array would put it in scratch memory)
      const int pi = rg < 6 ? pair_i(rg) : 0, pj = rg < 6 ? pair_j(rg) : 0;
      float pre = 0.f, blast = 0.f, Ri = 0.f, Rpi = 0.f, Rpj = 0.f;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float tr = sm.tot[r][c];
        blast += tr;
        pre += (r < rg) ? tr : 0.f;
        Ri += (r <= 2 * i_sub) ? tr : 0.f;  // b at row 16 i + 7
        Rpi += (r <= 2 * pi) ? tr : 0.f;
        Rpj += (r <= 2 * pj) ? tr : 0.f;
      }
      const float eRi = exp2_fast(Ri);
      const float eKh = exp2_fast(blast - Ri);
      float kh[8], vc[8];
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const float d = b[rr][x] + pre - Ri;
        const float qv = unpack2(qq[rr], T())[x];
        const float kv = unpack2(kk[rr], T())[x];
        qgv[rr][x] = qv * exp2_fast(d);
        kgv[rr][x] = kv * exp2_fast(-d);
        qhv[rr][x] = qgv[rr][x] * eRi;
        kh[rr] = kgv[rr][x] * eKh;
        vc[rr] = unpack2(vv[rr], T())[x];
      }
      store8<T>(&sm.khT[c][8 * rg], kh);
      store8<T>(&sm.vT[c][8 * rg], vc);
      if (rg < 6) {
        sm.vij[rg][c] = exp2_fast(Rpi - Rpj);
      } else if (rg == 7) {
        sm.decay[c] = exp2_fast(blast);
      }
    }
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const int t = 8 * rg + rr;
      st_pair<T>(&sm.qg[t][2 * cp], qgv[rr][0], qgv[rr][1]);
      st_pair<T>(&sm.kg[t][2 * cp], kgv[rr][0], kgv[rr][1]);
      st_pair<T>(&sm.qh[t][2 * cp], qhv[rr][0], qhv[rr][1]);
    }
    lds_barrier();  // (B) operands ready

    // ---- intra scores: transposed blocks A^T[s][t], masked, stored as A[t][s]
    for (int blk = wave; blk < 10; blk += NW) {
      const int i = blk_i(blk), j = blk_j(blk);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < KS; ++p) {
        F af = ld8<T>(&sm.kg[16 * j + r16][32 * p + 8 * g]);
        F bf = ld8<T>(&sm.qg[16 * i + r16][32 * p + 8 * g]);
        if (j < i) bf = scale8(bf, &sm.vij[pair_of(i, j)][32 * p + 8 * g]);
        mma(acc, af, bf);
      }
      if (i == j) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * g + r > r16) acc[r] = 0.f;
      }
      st4<T>(&sm.a[16 * i + r16][16 * j + 4 * g], acc);
    }

    // ---- inter: O^T[n][t] = sum_c S[c][n] qh[t][c], with the state entering the chunk
    f32x4 O[4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      O[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < KS; ++p) {
        F af = pack_acc<T>(S[2 * p], S[2 * p + 1]);
        F bf = ld4x2<T>(&sm.qh[16 * qb + r16][32 * p + 4 * g]);
        mma(O[qb], af, bf);
      }
    }

    // ---- state update: S = diag(2^{b_last}) S + khT V
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) S[cb][r] *= sm.decay[16 * cb + 4 * g + r];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        F af = ld8<T>(&sm.khT[16 * cb + r16][32 * p + 8 * g]);
        F bf = ld8<T>(&sm.vT[ncol + r16][32 * p + 8 * g]);
        mma(S[cb], af, bf);
      }
    }
    lds_barrier();  // (C) scores ready

    // ---- intra: O^T[n][t] += sum_s vT[n][s] A[t][s]
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
#pragma unroll
      for (int p = 0; p <= qb / 2; ++p) {
        F af = ld8<T>(&sm.vT[ncol + r16][32 * p + 8 * g]);
        F bf = ld8<T>(&sm.a[16 * qb + r16][32 * p + 8 * g]);
        mma(O[qb], af, bf);
      }
    }

    // ---- store O[t][ncol + 4g .. +3]
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const int t = t0 + 16 * qb + r16;
      if (t < T_len) st4<T>(o + off + (size_t)t * DK + ncol + 4 * g, O[qb]);
    }
  }

  if (hT && seg == G - 1) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) hT[s_base + (16 * cb + 4 * g + r) * DK + ncol + r16] = S[cb][r];
  }
}

__global__ void state_copy_kernel(const float* __restrict__ h0, float* __restrict__ hT, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) hT[i] = h0 ? h0[i] : 0.f;
}

template <typename T, int DK>
hipError_t launch_typed(const Shape& s, const Plan& pl, const void* q, const void* k,
                        const void* v, const float* la, const float* h0, void* o, float* hT,
                        void* ws, hipStream_t st) {
  const int BH = s.B * s.H;
  float* ws_state = (float*)ws;
  float* ws_gamma = ws_state + (size_t)BH * (pl.G - 1) * DK * DK;
  if (pl.G > 1) {
    hipLaunchKernelGGL((gla_state_pass<T, DK>), dim3(pl.G - 1, BH), dim3(4 * DK), 0, st,
                       (const T*)k, (const T*)v, la, ws_state, ws_gamma, s.T, pl.cps, pl.G);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gla_carry_pass, dim3(BH, 4), dim3(256), 0, st, h0, ws_state, ws_gamma,
                       DK, pl.G);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((gla_output_pass<T, DK>), dim3(pl.G, BH), dim3(4 * DK), 0, st, (const T*)q,
                     (const T*)k, (const T*)v, la, h0, ws_state, (T*)o, hT, s.T, pl.cps, pl.G);
  return hipGetLastError();
}

}  // namespace

size_t gla_fwd_workspace_bytes(const Shape& s) {
  const Plan pl = make_plan(s);
  return (size_t)s.B * s.H * (pl.G - 1) * ((size_t)s.dk * s.dv + s.dk) * sizeof(float);
}

hipError_t launch_state_copy(const Shape& s, const float* h0, float* hT, hipStream_t st) {
  size_t n = (size_t)s.B * s.H * s.dk * s.dv;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(state_copy_kernel, dim3((n + 255) / 256), dim3(256), 0, st, h0, hT, n);
  return hipGetLastError();
}

hipError_t launch_gla_fwd(const Shape& s, const void* q, const void* k, const void* v,
                          const float* la, const float* h0, void* o, float* hT, void* ws,
                          hipStream_t st) {
  if (s.T == 0) return hT ? launch_state_copy(s, h0, hT, st) : hipSuccess;
  const Plan pl = make_plan(s);
  if (s.dtype == 1) {
    if (s.dk == 128) return launch_typed<bf16, 128>(s, pl, q, k, v, la, h0, o, hT, ws, st);
    return launch_typed<bf16, 64>(s, pl, q, k, v, la, h0, o, hT, ws, st);
  }
  return launch_typed<float, 64>(s, pl, q, k, v, la, h0, o, hT, ws, st);
}

}  // namespace lz
