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
    T* __restrict__ o_swa, float* __restrict__ lse, int T_arg, int H, int W, int M,
    float scale_log2, float out_scale, int accumulate, const int* __restrict__ cu, int N,
    const T* __restrict__ hk, const T* __restrict__ hv, int hlen) {
  constexpr int KS = DK / 32;
  constexpr int NT = DV / 16;
  typedef typename Frag<T>::type F;
  __shared__ SwaSmem<T, DK, DV> sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int nqt = gridDim.x;
  const int logical = xcd_remap(blockIdx.y * nqt + blockIdx.x, nqt * gridDim.y);
  const int bh = logical / nqt, h = bh % H;
  const SeqRows sr = seq_rows(cu, N, T_arg, H, bh);
  const int T_len = sr.len;
  const int t0 = (logical % nqt) * kQT;
  if (t0 >= T_len) return;            // tiles past a packed sequence's end
  const int tq0 = t0 + 16 * wave;     // first query of this wave
  const int tq = tq0 + r16;           // this lane's query (column of the logit tiles)
  const size_t qk_base = sr.row0 * DK;
  const size_t v_base = sr.row0 * DV;
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

  // ---- halo: the hlen keys before the segment, row r at position r - hlen,
  // visible to query tq when r - hlen > tq - W
  if (hlen > 0 && t0 < W - 1) {
    const Buf bhk(hk + (size_t)bh * hlen * DK, (u32)((size_t)hlen * DK * sizeof(T)));
    const Buf bhv(hv + (size_t)bh * hlen * DV, (u32)((size_t)hlen * DV * sizeof(T)));
    const int first = max(0, t0 - W + 1 + hlen);
    for (int kt0 = (first / kKT) * kKT; kt0 < hlen; kt0 += kKT) {
      __syncthreads();
      stage_rows(&sm.kt[0][0], SwaSmem<T, DK, DV>::DKP, bhk, kt0, DK, kKT);
      stage_cols(&sm.vT[0][0], kKT + 8, bhv, kt0, DV, kKT);
      __syncthreads();
      f32x4 P[4];
      bool act[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int s_lo = kt0 + 16 * b;
        act[b] = (s_lo < hlen) && (s_lo + 15 - hlen > tq0 - W);
        P[b] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (act[b]) {
#pragma unroll
          for (int p = 0; p < KS; ++p) {
            F af = ld8<T>(&sm.kt[16 * b + r16][32 * p + 8 * g]);
            mma(P[b], af, qf[p]);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = s_lo + 4 * g + r;
            const bool ok = (row < hlen) && (row - hlen > tq - W);
            P[b][r] = ok ? P[b][r] * scale_log2 : -INFINITY;
          }
        }
      }
      softmax_pv(P, act, 4, &sm.vT[0][0], kKT + 8);
    }
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

// ------------------------------------------------------------- streaming form
// When w <= 64*NPREV + 1, every key a 64-query tile needs lies in the tile's own
// chunk or the NPREV chunks before it.  A work-group of 8 waves then walks a run
// of query tiles of one head in order, two tiles (128 queries, one 16-query
// block per wave) per step, and keeps the chunks those tiles need in an LDS ring
// of NS = NPREV + 2 slots (K row-major, V transposed), so each key/value row is
// staged once per work-group.  The next two chunks' K and V and the next
// queries are loaded into registers while the current step computes (loads
// issued at the top of an iteration and consumed at its end); two barriers per
// step.
// LDS: K rows and V^T rows in swizzled granule layouts; V^T tokens (and the
// meta V^T slots) in split order, so each P V operand is one granule read.
template <typename T, int D, int NS>
struct RingSmem {
  static constexpr int GK = D / 8;    // granules per K row
  static constexpr int VW = 4 * kKT;  // V^T row length (tokens), a power-of-two granule count
  T k[NS * kKT * D];
  T vT[D * VW];
  T mk[16 * D];
  T mvT[D * 32];
};

template <typename T, int D, int NS>
__global__ __launch_bounds__(512, 1) void swa_fwd_ring(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ mk, const T* __restrict__ mv, T* __restrict__ o,
    T* __restrict__ o_swa, float* __restrict__ lse, T* __restrict__ rk, T* __restrict__ rv,
    int T_arg, int H, int W, int M, float scale_log2, float out_scale, int accumulate, int cps,
    const int* __restrict__ cu, int N) {
  constexpr int KS = D / 32;
  constexpr int NT = D / 16;
  constexpr int NPREV = NS - 2;
  constexpr int GR = D * (int)sizeof(T) / 16;  // 16-byte granules per row
  constexpr int KPT = 2 * kKT * GR / 512;      // K granules per thread (two chunks)
  constexpr int RV = D / 32;                   // V rows per thread (8 channels each)
  constexpr int VG = (int)sizeof(T) / 2;       // 16-byte granules per 8 channels
  constexpr int GK = RingSmem<T, D, NS>::GK, VW = RingSmem<T, D, NS>::VW;
  static_assert(NS <= 4, "ring slots fit the V^T row");
  typedef typename Frag<T>::type F;
  __shared__ RingSmem<T, D, NS> sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int nseg = gridDim.x;
  const int logical = xcd_remap(blockIdx.y * nseg + blockIdx.x, nseg * gridDim.y);
  const int bh = logical / nseg, h = bh % H, seg = logical % nseg;
  const SeqRows sr = seq_rows(cu, N, T_arg, H, bh);
  const int T_len = sr.len;
  const int nc = (T_len + kKT - 1) / kKT;
  // a packed sequence covers the first Gs segments (an empty one: one segment
  // that only clears its window cache)
  const int Gs = cu ? max(1, (nc + cps - 1) / cps) : nseg;
  if (seg >= Gs) return;
  const int c_begin = seg * cps, c_end = min(nc, c_begin + cps);  // cps is even
  const int half = wave >> 2, wq = wave & 3;  // this wave's tile of the step, block in it
  const size_t base = sr.row0 * D;
  const u32 nbytes = (u32)((size_t)T_len * D * sizeof(T));
  const Buf bq(q + base, nbytes), bk(k + base, nbytes), bv(v + base, nbytes);

  // staging of the two chunks ch0, ch0+1 (threads 0..255 take ch0, the rest ch0+1):
  //   K granule e = (tid & 255) + 256 j -> row e / GR, granule e % GR;
  //   V rows RV*vr .. +RV-1, channels 8vo .. 8vo+7
  const int sc = tid >> 8, st = tid & 255;
  const int vo = st % (D / 8), vr = st / (D / 8);
  u32x4 pk[KPT], pv[RV][VG];
  auto load_kv = [&](int ch0) {
    const int ch = ch0 + sc;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int e = st + 256 * j;
      pk[j] = bk.ld128((u32)((ch * kKT + e / GR) * D * sizeof(T) + (e % GR) * 16));
    }
#pragma unroll
    for (int rr = 0; rr < RV; ++rr)
#pragma unroll
      for (int u = 0; u < VG; ++u)
        pv[rr][u] = bv.ld128((u32)(((ch * kKT + RV * vr + rr) * D + 8 * vo) * sizeof(T) + 16 * u));
  };
  auto store_kv = [&](int ch0) {
    const int ch = ch0 + sc;
    const int slot = ch % NS;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int e = st + 256 * j;
      const int row = e / GR, col = (e % GR) * (16 / (int)sizeof(T));
      *reinterpret_cast<u32x4*>(&sm.k[slot * kKT * D + swz_at<GK>(row, col)]) = pk[j];
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      T* dst = &sm.vT[swz_at<VW / 8>(8 * vo + c, slot * kKT + split_pos(RV * vr))];
      if constexpr (sizeof(T) == 2) {
        u32 e[RV];
#pragma unroll
        for (int rr = 0; rr < RV; ++rr) {
          const u32 w = pv[rr][0][c >> 1];
          e[rr] = (c & 1) ? (w >> 16) : (w & 0xffffu);
        }
        if constexpr (RV == 4) {
          *reinterpret_cast<U2*>(dst) = U2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
        } else {
          *reinterpret_cast<u32*>(dst) = e[0] | (e[1] << 16);
        }
      } else {
#pragma unroll
        for (int rr = 0; rr < RV; ++rr) {
          const u32 w = pv[rr][c >> 2][c & 3];
          reinterpret_cast<u32*>(dst)[rr] = w;
        }
      }
    }
  };
  // query fragments of the lane's query (B operand, contiguous channel map);
  // rows past the end read zero and are never stored
  F qf[KS], qn[KS];
  auto load_q = [&](int ch, F* dst) {
    const u32 row = (u32)(ch * kKT + 16 * wq + r16);
#pragma unroll
    for (int p = 0; p < KS; ++p) {
      if constexpr (sizeof(T) == 2) {
        const u32x4 x = bq.ld128((row * D + 32 * p + 8 * g) * 2);
        dst[p] = __builtin_bit_cast(bf16x8, x);
      } else {
        const u32x4 x0 = bq.ld128((row * D + 32 * p + 8 * g) * 4);
        const u32x4 x1 = bq.ld128((row * D + 32 * p + 8 * g) * 4 + 16);
        F f;
#pragma unroll
        for (int i = 0; i < 4; ++i) { f[i] = as_f(x0[i]); f[4 + i] = as_f(x1[i]); }
        dst[p] = f;
      }
    }
  };

  // ---- prologue: meta slots, the chunks before the first tile and its own chunk
  if (M > 0) {
    // meta K rows (slots >= M read zero) and meta V^T in split order
    const T* mkh = mk + (size_t)h * M * D;
    const T* mvh = mv + (size_t)h * M * D;
    for (int e = tid; e < 16 * D; e += 512) {
      const int r = e / D, c = e % D;
      sm.mk[swz_at<GK>(r, c)] = r < M ? mkh[r * D + c] : to_t<T>(0.f);
    }
    for (int e = tid; e < 32 * D; e += 512) {
      const int c = e / 32, t = e % 32;
      sm.mvT[swz_at<4>(c, split_pos(t))] = t < M ? mvh[t * D + c] : to_t<T>(0.f);
    }
  }
  // chunks c_begin-NPREV .. c_begin+1, two at a time (out-of-range rows read 0)
  for (int ch = c_begin - NPREV; ch <= c_begin + 1; ch += 2) {
    const bool mine = ch + sc >= 0 && ch + sc <= c_begin + 1;
    if (mine) load_kv(ch);
    if (mine) store_kv(ch);
  }
  load_q(c_begin + half, qf);
  lds_barrier();

  for (int cs = c_begin; cs < c_end; cs += 2) {
    const bool has_next = cs + 2 < c_end;
    if (has_next) {
      load_kv(cs + 2);
      load_q(cs + 2 + half, qn);
    }
    const int ch = cs + half;  // this wave's query tile
    const int t0 = ch * kKT;
    const int tq0 = t0 + 16 * wq, tq = tq0 + r16;
    const bool stores = ch < c_end && tq < T_len;
    // the branch output this step adds to, read now so the load overlaps the step
    typedef typename Pair<T>::type Raw2;
    Raw2 oacc[NT][2];
    if (accumulate && stores) {
      const T* src = o + base + (size_t)tq * D + 4 * g;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        oacc[nt][0] = *reinterpret_cast<const Raw2*>(src + 16 * nt);
        oacc[nt][1] = *reinterpret_cast<const Raw2*>(src + 16 * nt + 2);
      }
    }
    // The whole window of this wave's 16 queries is at most 4*(NPREV+1) key
    // blocks plus the meta block, so the softmax is taken exactly: every logit
    // tile first (independent product chains), one max, one exponential pass,
    // then every P V product -- no running rescale between key blocks.
    constexpr int NKB = 4 * (NPREV + 1);
    f32x4 Pm = {0.f, 0.f, 0.f, 0.f}, P[NKB];
    bool act[NKB];  // uniform over the wave
    if (M > 0) {
#pragma unroll
      for (int p = 0; p < KS; ++p) mma(Pm, ld8<T>(&sm.mk[swz_at<GK>(r16, 32 * p + 8 * g)]), qf[p]);
#pragma unroll
      for (int r = 0; r < 4; ++r) Pm[r] = (4 * g + r < M) ? Pm[r] * scale_log2 : -INFINITY;
    }
#pragma unroll
    for (int j = 0; j < NKB; ++j) {
      const int kc = ch - NPREV + (j >> 2);
      const int s_lo = kc * kKT + 16 * (j & 3);
      act[j] = kc >= 0 && (s_lo + 15 >= tq0 - W + 1) && (s_lo <= tq0 + 15) && (s_lo < T_len);
      P[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (act[j]) {
        const int slot = kc % NS;
#pragma unroll
        for (int p = 0; p < KS; ++p)
          mma(P[j], ld8<T>(&sm.k[slot * kKT * D + swz_at<GK>(16 * (j & 3) + r16, 32 * p + 8 * g)]),
              qf[p]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = s_lo + 4 * g + r;
          const bool ok = (s <= tq) && (s > tq - W);
          P[j][r] = ok ? P[j][r] * scale_log2 : -INFINITY;
        }
      }
    }
    float mt = kNegBig;
    if (M > 0)
#pragma unroll
      for (int r = 0; r < 4; ++r) mt = fmaxf(mt, Pm[r]);
#pragma unroll
    for (int j = 0; j < NKB; ++j)
      if (act[j])
#pragma unroll
        for (int r = 0; r < 4; ++r) mt = fmaxf(mt, P[j][r]);
    mt = wave_max16(mt);
    float l_run = 0.f;
    if (M > 0)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        Pm[r] = exp2_fast(Pm[r] - mt);
        l_run += Pm[r];
      }
#pragma unroll
    for (int j = 0; j < NKB; ++j)
      if (act[j])
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          P[j][r] = exp2_fast(P[j][r] - mt);
          l_run += P[j][r];
        }
    f32x4 O[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) O[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (M > 0) {
      const F bf = pack_acc<T>(Pm, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) mma(O[nt], ld8<T>(&sm.mvT[swz_at<4>(16 * nt + r16, 8 * g)]), bf);
    }
#pragma unroll
    for (int jp = 0; jp < NKB / 2; ++jp) {
      if (act[2 * jp] || act[2 * jp + 1]) {
        const int kc = ch - NPREV + (jp >> 1);
        const F bf = pack_acc<T>(P[2 * jp], P[2 * jp + 1]);
        const int pos = (kc % NS) * kKT + 32 * (jp & 1) + 8 * g;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) mma(O[nt], ld8<T>(&sm.vT[swz_at<VW / 8>(16 * nt + r16, pos)]), bf);
      }
    }
    const float m_run = mt;

    // ---- normalise and store
    const float l_tot = wave_sum16(l_run);
    const float inv = 1.f / l_tot;
    if (stores) {
      const size_t rowo = base + (size_t)tq * D;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const size_t off = rowo + 16 * nt + 4 * g;
        const f32x4 val = O[nt] * inv;
        if (o_swa) st4<T>(o_swa + off, val);
        f32x4 out = val * out_scale;
        if (accumulate) {
          const f32x2 a = unpack2(oacc[nt][0], T()), b = unpack2(oacc[nt][1], T());
          out += f32x4{a[0], a[1], b[0], b[1]};
        }
        st4<T>(o + off, out);
      }
      if (lse && g == 0) lse[(size_t)bh * T_len + tq] = (m_run + log2_fast(l_tot)) * kLn2;
    }

    lds_barrier();  // every read of the two oldest ring slots is done
    if (has_next) {
      store_kv(cs + 2);
#pragma unroll
      for (int p = 0; p < KS; ++p) qf[p] = qn[p];
    }
    lds_barrier();  // the next two chunks are in the ring
  }
  // window cache for decoding (rk, rv non-null): slot p mod W <- token p for the
  // last min(T, W) tokens, zero for slots without a token (T < W); the head's
  // segments share the slots, so no work-group's tail grows much
  if (rk) {
    constexpr int PER = 16 / (int)sizeof(T);  // elements per 16 bytes
    constexpr int RG = D / PER;               // 16-byte pieces per row
    const size_t rbase = (size_t)bh * W * D;
    const u32x4 z = {0u, 0u, 0u, 0u};
    const int s_lo = (int)((long long)W * seg / Gs), s_hi = (int)((long long)W * (seg + 1) / Gs);
    for (int e = s_lo * RG + tid; e < s_hi * RG; e += 512) {
      const int slot = e / RG, c = (e % RG) * PER;
      const int p = slot < T_len % W ? T_len - T_len % W + slot : T_len - T_len % W - W + slot;
      u32x4 xk = z, xv = z;
      if (p >= 0) {
        const u32 off = (u32)(((size_t)p * D + c) * sizeof(T));
        xk = bk.ld128(off);
        xv = bv.ld128(off);
      }
      *reinterpret_cast<u32x4*>(&rk[rbase + (size_t)slot * D + c]) = xk;
      *reinterpret_cast<u32x4*>(&rv[rbase + (size_t)slot * D + c]) = xv;
    }
  }
}

template <typename T, int D>
hipError_t launch_typed(const Shape& s, const void* q, const void* k, const void* v,
                        const void* mk, const void* mv, void* o, float out_scale, int acc,
                        void* o_swa, float* lse, void* rk, void* rv, hipStream_t st) {
  // the streaming ring holds up to four 64-key chunks of K and V^T: too large
  // for LDS in fp32 at D = 128, which takes the tiled kernel for every window
  constexpr bool kRing = !(sizeof(T) == 4 && D == 128);
  if constexpr (kRing) {
  if (s.window <= 2 * kKT + 1 && s.hlen == 0) {
    // streaming form: runs of query tiles, enough work-groups to fill the chip
    const int nc = (s.T + kKT - 1) / kKT;
    const long long bh = (long long)s.B * s.H;
    int g = (int)((256 + bh - 1) / bh);
    g = g < 1 ? 1 : (g > nc ? nc : g);
    int cps = (nc + g - 1) / g;
    cps += cps & 1;  // whole steps of two tiles
    const int G = (nc + cps - 1) / cps;
    const float sl = s.scale * kLog2e;
    if (s.window <= kKT + 1) {
      hipLaunchKernelGGL((swa_fwd_ring<T, D, 3>), dim3(G, s.B * s.H), dim3(512), 0, st, (const T*)q,
                         (const T*)k, (const T*)v, (const T*)mk, (const T*)mv, (T*)o, (T*)o_swa,
                         lse, (T*)rk, (T*)rv, s.T, s.H, s.window, s.n_meta, sl, out_scale, acc, cps,
                         s.cu, s.n_tokens);
    } else {
      hipLaunchKernelGGL((swa_fwd_ring<T, D, 4>), dim3(G, s.B * s.H), dim3(512), 0, st, (const T*)q,
                         (const T*)k, (const T*)v, (const T*)mk, (const T*)mv, (T*)o, (T*)o_swa,
                         lse, (T*)rk, (T*)rv, s.T, s.H, s.window, s.n_meta, sl, out_scale, acc, cps,
                         s.cu, s.n_tokens);
    }
    return hipGetLastError();
  }
  }
  dim3 grid((s.T + kQT - 1) / kQT, s.B * s.H);
  hipLaunchKernelGGL((swa_fwd_kernel<T, D, D>), grid, dim3(256), 0, st, (const T*)q, (const T*)k,
                     (const T*)v, (const T*)mk, (const T*)mv, (T*)o, (T*)o_swa, lse, s.T, s.H,
                     s.window, s.n_meta, s.scale * kLog2e, out_scale, acc, s.cu, s.n_tokens,
                     (const T*)s.hk, (const T*)s.hv, s.hlen);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && rk) e = launch_ring_fill(s, k, v, rk, rv, st);
  return e;
}

}  // namespace

hipError_t launch_swa_fwd(const Shape& s, const void* q, const void* k, const void* v,
                          const void* mk, const void* mv, void* o, float out_scale,
                          int accumulate, void* o_swa, float* lse, void* ring_k, void* ring_v,
                          hipStream_t st) {
  if (s.B * s.H == 0) return hipSuccess;
  if (s.T == 0) return ring_k ? launch_ring_fill(s, k, v, ring_k, ring_v, st) : hipSuccess;
  if (s.dtype == 1) {
    if (s.dk == 128)
      return launch_typed<bf16, 128>(s, q, k, v, mk, mv, o, out_scale, accumulate, o_swa, lse,
                                     ring_k, ring_v, st);
    return launch_typed<bf16, 64>(s, q, k, v, mk, mv, o, out_scale, accumulate, o_swa, lse,
                                  ring_k, ring_v, st);
  }
  if (s.dk == 128)
    return launch_typed<float, 128>(s, q, k, v, mk, mv, o, out_scale, accumulate, o_swa, lse,
                                    ring_k, ring_v, st);
  return launch_typed<float, 64>(s, q, k, v, mk, mv, o, out_scale, accumulate, o_swa, lse,
                                 ring_k, ring_v, st);
}

}  // namespace lz
