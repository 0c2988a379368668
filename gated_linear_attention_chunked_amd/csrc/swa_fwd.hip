// Sliding-window softmax attention with always-visible meta-memory slots, gfx950.
//
// Query t sees the keys j in [t-w+1, t] plus the M meta slots, all in one
// softmax ("Lizard: An Efficient Linearization Framework for Large Language
// Models", gist.science summary, section 2(a): the anchor window whose learnable
// meta tokens sit in the softmax denominator).  Meta values take part in the
// weighted sum as well; meta_v = 0 gives the pure-sink behaviour.
//
// One work-group = 64 queries (one 16-query block per wave).  The meta slots and
// then every 64-key tile overlapping the window are staged in LDS (K row-major,
// V transposed); each wave computes transposed logit blocks S^T = K Q^T, keeps a
// running max/sum in fp32 (base-2 domain) and accumulates O^T = V^T P^T, feeding
// the probabilities straight from the logit accumulators into the next product.
#include "common.hpp"
#include "kernels.hpp"

namespace lz {
namespace {

constexpr int kQT = 64;   // queries per work-group
constexpr int kKT = 64;   // keys per staged tile
constexpr float kNegBig = -1e30f;

template <typename T, int DK, int DV>
struct SwaSmem {
  static constexpr int DKP = DK + 8;
  T kt[kKT][DKP];
  T vT[DV][kKT + 8];
  T mk[16][DKP];
  T mvT[DV][32 + 8];
};

template <typename T, int DK, int DV>
__global__ __launch_bounds__(256, 2) void swa_fwd_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ mk, const T* __restrict__ mv, T* __restrict__ o,
    T* __restrict__ o_swa, float* __restrict__ lse, int T_len, int H, int W, int M,
    float scale_log2, float out_scale, int accumulate) {
  constexpr int KS = DK / 32;
  constexpr int NT = DV / 16;
  typedef typename Frag<T>::type F;
  __shared__ SwaSmem<T, DK, DV> sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int nqt = gridDim.x;
  const int logical = xcd_remap(blockIdx.y * nqt + blockIdx.x, nqt * gridDim.y);
  const int bh = logical / nqt, h = bh % H;
  const int t0 = (logical % nqt) * kQT;
  const int tq0 = t0 + 16 * wave;     // first query of this wave
  const int tq = tq0 + r16;           // this lane's query (column of the logit tiles)
  const size_t qk_base = (size_t)bh * T_len * DK;
  const size_t v_base = (size_t)bh * T_len * DV;
  const Buf bk(k + qk_base, (u32)((size_t)T_len * DK * sizeof(T)));
  const Buf bv(v + v_base, (u32)((size_t)T_len * DV * sizeof(T)));

  // q fragments (B operand, contiguous channel map)
  // (rows past the end load the last row; their outputs are never stored)
  F qf[KS];
  const int tq_ld = min(tq, T_len - 1);
#pragma unroll
  for (int p = 0; p < KS; ++p) qf[p] = ld8<T>(q + qk_base + (size_t)tq_ld * DK + 32 * p + 8 * g);

  f32x4 O[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) O[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegBig, l_run = 0.f;

  // Tile loaders.  Rows past the end of the buffer read as zero (buffer bounds),
  // so there are no branches around the loads.
  // row-major [rows x D] tile from rows row0.. of `src` into dst (leading dim ld_dst)
  auto stage_rows = [&](T* dst, int ld_dst, const Buf& src, int row0, int D, int rows) {
    const int per_row = D / 8;
    for (int e = tid; e < rows * per_row; e += 256) {
      const int r = e / per_row, c8 = (e % per_row) * 8;
      const u32 off = (u32)(((row0 + r) * D + c8) * sizeof(T));
      if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<u32x4*>(dst + r * ld_dst + c8) = src.ld128(off);
      } else {
        *reinterpret_cast<u32x4*>(dst + r * ld_dst + c8) = src.ld128(off);
        *reinterpret_cast<u32x4*>(dst + r * ld_dst + c8 + 4) = src.ld128(off + 16);
      }
    }
  };
  // transposed: dst[c][r] = src[row0 + r][c]
  auto stage_cols = [&](T* dst, int ld_dst, const Buf& src, int row0, int D, int rows) {
    for (int e = tid; e < (rows / 8) * (D / 2); e += 256) {
      const int cp = e % (D / 2), rg = e / (D / 2);
      float c0v[8], c1v[8];
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const u32 off = (u32)(((row0 + 8 * rg + rr) * D + 2 * cp) * sizeof(T));
        const f32x2 x = unpack2(ld_pair<T>(src, off), T());
        c0v[rr] = x[0];
        c1v[rr] = x[1];
      }
      typename Frag<T>::type f0, f1;
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) { f0[rr] = to_t<T>(c0v[rr]); f1[rr] = to_t<T>(c1v[rr]); }
      *reinterpret_cast<typename Frag<T>::type*>(dst + (2 * cp) * ld_dst + 8 * rg) = f0;
      *reinterpret_cast<typename Frag<T>::type*>(dst + (2 * cp + 1) * ld_dst + 8 * rg) = f1;
    }
  };

  // processes up to 4 key blocks of 16 whose logit tiles are in P[] (already
  // masked, base-2 scaled); updates the running softmax and O.
  auto softmax_pv = [&](f32x4* P, const bool* act, int nblk, const T* vT, int ldv) {
    float mt = kNegBig;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if (b < nblk && act[b])
#pragma unroll
        for (int r = 0; r < 4; ++r) mt = fmaxf(mt, P[b][r]);
    mt = wave_max16(mt);
    const float m_new = fmaxf(m_run, mt);
    const float corr = exp2_fast(m_run - m_new);
    m_run = m_new;
    l_run *= corr;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) O[nt] *= corr;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (b < nblk && act[b]) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pr = exp2_fast(P[b][r] - m_new);
          P[b][r] = pr;
          l_run += pr;
        }
      } else {
        P[b] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      if (2 * pp < nblk && (act[2 * pp] || (2 * pp + 1 < nblk && act[2 * pp + 1]))) {
        F bf = pack_acc<T>(P[2 * pp], P[2 * pp + 1]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          F af = ld4x2<T>(vT + (16 * nt + r16) * ldv + 32 * pp + 4 * g);
          mma(O[nt], af, bf);
        }
      }
    }
  };

  // ---- meta slots (always visible)
  if (M > 0) {
    const Buf bmk(mk + (size_t)h * M * DK, (u32)(M * DK * sizeof(T)));
    const Buf bmv(mv + (size_t)h * M * DV, (u32)(M * DV * sizeof(T)));
    stage_rows(&sm.mk[0][0], SwaSmem<T, DK, DV>::DKP, bmk, 0, DK, 16);
    stage_cols(&sm.mvT[0][0], 32 + 8, bmv, 0, DV, 32);
    __syncthreads();
    f32x4 P[4];
    bool act[4] = {true, false, false, false};
    P[0] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < KS; ++p) {
      F af = ld8<T>(&sm.mk[r16][32 * p + 8 * g]);
      mma(P[0], af, qf[p]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      P[0][r] = (4 * g + r < M) ? P[0][r] * scale_log2 : -INFINITY;
    softmax_pv(P, act, 2, &sm.mvT[0][0], 32 + 8);
  }

  // ---- key tiles overlapping [t0 - W + 1, t0 + 63]
  const int first_key = max(0, t0 - W + 1);
  const int last_key = min(T_len - 1, t0 + kQT - 1);
  for (int kt0 = (first_key / kKT) * kKT; kt0 <= last_key; kt0 += kKT) {
    __syncthreads();  // previous tile's readers are done
    stage_rows(&sm.kt[0][0], SwaSmem<T, DK, DV>::DKP, bk, kt0, DK, kKT);
    stage_cols(&sm.vT[0][0], kKT + 8, bv, kt0, DV, kKT);
    __syncthreads();

    f32x4 P[4];
    bool act[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int s_lo = kt0 + 16 * b;
      act[b] = (s_lo + 15 >= tq0 - W + 1) && (s_lo <= tq0 + 15) && (s_lo < T_len);
      P[b] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (act[b]) {
#pragma unroll
        for (int p = 0; p < KS; ++p) {
          F af = ld8<T>(&sm.kt[16 * b + r16][32 * p + 8 * g]);
          mma(P[b], af, qf[p]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = s_lo + 4 * g + r;
          const bool ok = (s <= tq) && (s > tq - W);
          P[b][r] = ok ? P[b][r] * scale_log2 : -INFINITY;
        }
      }
    }
    softmax_pv(P, act, 4, &sm.vT[0][0], kKT + 8);
  }

  // ---- normalise and store
  const float l_tot = wave_sum16(l_run);
  const float inv = 1.f / l_tot;
  if (tq < T_len) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const size_t off = v_base + (size_t)tq * DV + 16 * nt + 4 * g;
      f32x4 val = O[nt] * inv;
      if (o_swa) st4<T>(o_swa + off, val);
      f32x4 out = val * out_scale;
      if (accumulate) out += ld4f<T>(o + off);
      st4<T>(o + off, out);
    }
    if (lse && g == 0) lse[(size_t)bh * T_len + tq] = (m_run + log2_fast(l_tot)) * kLn2;
  }
}

template <typename T, int D>
hipError_t launch_typed(const Shape& s, const void* q, const void* k, const void* v,
                        const void* mk, const void* mv, void* o, float out_scale, int acc,
                        void* o_swa, float* lse, hipStream_t st) {
  dim3 grid((s.T + kQT - 1) / kQT, s.B * s.H);
  hipLaunchKernelGGL((swa_fwd_kernel<T, D, D>), grid, dim3(256), 0, st, (const T*)q, (const T*)k,
                     (const T*)v, (const T*)mk, (const T*)mv, (T*)o, (T*)o_swa, lse, s.T, s.H,
                     s.window, s.n_meta, s.scale * kLog2e, out_scale, acc);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_swa_fwd(const Shape& s, const void* q, const void* k, const void* v,
                          const void* mk, const void* mv, void* o, float out_scale,
                          int accumulate, void* o_swa, float* lse, hipStream_t st) {
  if (s.T == 0 || s.B * s.H == 0) return hipSuccess;
  if (s.dtype == 1) {
    if (s.dk == 128) return launch_typed<bf16, 128>(s, q, k, v, mk, mv, o, out_scale, accumulate, o_swa, lse, st);
    return launch_typed<bf16, 64>(s, q, k, v, mk, mv, o, out_scale, accumulate, o_swa, lse, st);
  }
  return launch_typed<float, 64>(s, q, k, v, mk, mv, o, out_scale, accumulate, o_swa, lse, st);
}

}  // namespace lz
