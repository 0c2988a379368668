// Hybrid forward as one output pass, gfx950, bf16, d_k = d_v = D in {64, 128},
// w <= 129.
//
// "Lizard: An Efficient Linearization Framework for Large Language Models"
// (gist.science summary, sections 2(a) and 2(b)) sums two branches computed from
// the same q, k, v: gated linear attention, o_gla,t = q_t S_t with
// S_t = diag(alpha_t) S_{t-1} + k_t^T v_t, and softmax attention over the keys
// s in (t - w, t] plus M meta slots that every query sees.  After the GLA state
// pass (segment end states, gla_fwd.hip) this pass reads q, k, v and the log
// gates once and writes o = o_gla + mix * o_swa once.  Run as two kernels, the
// window branch reads q, k, v a second time and reads and rewrites o; on an
// HBM-bound path those bytes are most of the difference.
//
// One work-group of 8 waves per (head, segment) walks the segment's 32-token
// chunks in order.  Chunk c (tokens t0..t0+31) in two phases:
//   phase 1  consumers (waves 0-3; value columns (D/4)w.. (D/4)w + D/4 - 1, their
//              fp32 state slice in registers): inter O = (q 2^b) S_c, the state update
//              S_{c+1} = diag(2^{b_last}) S_c + (k 2^{b_last - b})^T V, and
//              (waves 0-2, one 16x16 block each) the masked intra scores
//            producers (waves 4-7): window scores of query rows 16(p&1).. over
//              one half of the 16-key blocks they reach (the older blocks, or
//              the newer ones with the meta slots); exponentials from that
//              half's own row maxima; maxima, row sums and exponentials -> LDS
//   ---- barrier
//   phase 2  consumers: O += A V (intra) + the two halves' P V (V^T ring, meta
//              values), each scaled by f_h mix / (f_0 l_0 + f_1 l_1) with
//              f_h = 2^{(m_h - max(m_0, m_1)) scale}; store o; v of chunk c+1
//              into the V^T ring
//            producers (D/4 channels each): gate chunk c+1
//              (log2-gate cumsum, gated q and k tiles, k^T for the state
//              update), raw q and raw k of c+1 into LDS; issue the loads of c+3
//   ---- barrier
// The ring holds RING chunks, c-RING+1 .. c: 5 for w <= 129, 3 for w <= 65.
// With D = 64 the pass also writes the training outputs o_swa (the window
// branch alone) and lse (its natural-log softmax normaliser per query).
// 32-token chunks keep the GLA tiles and a ring of w + 32 window keys and
// values inside the 160 KB of LDS at once.  The GLA algebra is that of
// gla_fwd.hip: one reference (the chunk start) when every channel's chunk decay
// stays above 2^-64, otherwise 16-token sub-block references R_i with the pair
// factor 2^{R_1 - R_0} on the off-diagonal block.  The V^T ring is partitioned
// by value columns, so each consumer wave reads and writes only its own part
// and the ring needs no barrier of its own.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace lz {
namespace {

constexpr int kC = 32;             // tokens per chunk
constexpr float kFast = 64.f;      // single reference while every chunk decay >= 2^-64
// widest window a ring of RING chunks holds
__host__ __device__ constexpr int max_window(int ring) { return (ring - 1) * kC + 1; }
// Row of the transposed [channel][token] tiles (k-hat^T, the V^T ring, meta V^T):
// 32 tokens padded to 80 bytes.  Their staging stores write four rows 8 apart
// per instruction; at 64-byte rows those rows share one set of banks, at 80
// bytes they fall on two, and the 16-row fragment reads stay conflict-free.
constexpr int kTP = kC + 8;

template <int D, int RING>
struct Smem {
  static constexpr int kD = D, kRing = RING;
  bf16 qs[kC * D];               // gated q [t][ch]: q 2^{b_t} (or 2^{b_t - R_i})
  bf16 ks[kC * D];               // gated k [s][ch]: k 2^{-b_s} (or 2^{R_j - b_s})
  bf16 khT[D * kTP];             // [ch][s]: k 2^{b_last - b_s}
  bf16 a[kC * kC];               // masked intra scores [t][s]
  bf16 p[RING + 1][kC * kC];     // window probabilities [t][s] per ring chunk, meta last
  bf16 vT[RING][D * kTP];        // V^T ring [n][s]
  bf16 kr[RING][kC * D];         // raw K ring [s][ch]
  bf16 qr[kC * D];               // raw q [t][ch]
  bf16 mk[16 * D];               // meta keys (rows >= M zero)
  bf16 mvT[D * kTP];             // meta values transposed (slots >= M zero)
  alignas(16) float decay[D];    // 2^{b_last}
  alignas(16) float eR[2][D];    // 2^{R_i} (1 for single-reference channels)
  alignas(16) float vij[D];      // 2^{R_1 - R_0} (likewise)
  float pmax[2][kC];             // window: per key half, row maxima of the raw scores
  float psum[2][kC];             // per key half, row sums of exponentials taken from that maximum
  int fastw[4];                  // per producer wave: its channels take one reference
};

// [rows][D] and [rows][32] tiles, granules permuted by row
template <int D>
__device__ __forceinline__ int atd(int row, int col) { return swz_at<D / 8>(row, col); }
__device__ __forceinline__ int at4(int row, int col) { return swz_at<4>(row, col); }
// (row, col) of a padded transposed tile
__device__ __forceinline__ int atp(int row, int col) { return row * kTP + col; }

// Split-map fragment (elements col..col+3 and col+16..col+19) of a [rows][D] tile.
template <int D>
__device__ __forceinline__ bf16x8 ld_split(const bf16* t, int row, int col) {
  const bf16x4 x = *reinterpret_cast<const bf16x4*>(&t[atd<D>(row, col)]);
  const bf16x4 y = *reinterpret_cast<const bf16x4*>(&t[atd<D>(row, col + 16)]);
  return bf16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}

__device__ __forceinline__ bf16x8 scale8(const bf16x8& x, const float* f) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(f);
  const f32x4 b = *reinterpret_cast<const f32x4*>(f + 4);
  return bf16x8{(bf16)((float)x[0] * a[0]), (bf16)((float)x[1] * a[1]), (bf16)((float)x[2] * a[2]),
                (bf16)((float)x[3] * a[3]), (bf16)((float)x[4] * b[0]), (bf16)((float)x[5] * b[1]),
                (bf16)((float)x[6] * b[2]), (bf16)((float)x[7] * b[3])};
}

// Masked intra score block A[16i.., 16j..] (key block j <= i) into the a tile.
template <class SM>
__device__ __forceinline__ void intra_scores(SM& sm, int i, int j, bool fast, int r16, int g) {
  constexpr int D = SM::kD;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < D / 32; ++p) {
    const bf16x8 af = ld8<bf16>(&sm.ks[atd<D>(16 * j + r16, 32 * p + 8 * g)]);
    bf16x8 bf = ld8<bf16>(&sm.qs[atd<D>(16 * i + r16, 32 * p + 8 * g)]);
    if (!fast && j < i) bf = scale8(bf, &sm.vij[32 * p + 8 * g]);
    mma(acc, af, bf);
  }
  if (i == j) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * g + r > r16) acc[r] = 0.f;
  }
  st4<bf16>(&sm.a[at4(16 * i + r16, 16 * j + 4 * g)], acc);
}

// kSep: the window branch reads its own queries and keys qw, kw (otherwise qw,
// kw alias q, k and are not loaded a second time).  GT: gate input type (float
// log alpha or bf16 logit).  kSave: o_swa and lse (each nullable) receive the
// window branch alone and its log normaliser (always at D = 64; at D = 128 a
// separate instance, whose extra accumulators spill a few registers, so that
// the inference instance keeps none).
template <int D, int RING, bool kSep, typename GT, bool kSave = (D == 64)>
__global__ __launch_bounds__(512, 1) void hybrid_fwd_fused(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ qw,
    const bf16* __restrict__ kw, const bf16* __restrict__ v,
    const GT* __restrict__ la, const bf16* __restrict__ mk, const bf16* __restrict__ mv,
    const float* __restrict__ h0, const float* __restrict__ ws_state,
    const float* __restrict__ ws_gamma, bf16* __restrict__ o, float* __restrict__ hT,
    bf16* __restrict__ rk, bf16* __restrict__ rv, bf16* __restrict__ o_swa,
    float* __restrict__ lse, int T_arg, int H, int W, int M, float scale_log2, float mix, int cps,
    int G, int m, const int* __restrict__ cu, int N) {
  constexpr int kD = D, kRing = RING;
  constexpr int NT = D / 64;    // 16-column blocks of a consumer wave's state slice
  constexpr int CW = D / 4;     // value columns per consumer wave
  constexpr int NCB = D / 16;   // 16-row blocks of the state
  constexpr int KS = D / 32;    // contraction steps over channels
  // Every producer wave gates D/4 channels, CPL per lane: at D = 128 eight
  // (16-byte rows of q and k), at D = 64 four, so that all four producers
  // share the gating instead of two of them taking 32 channels each.
  constexpr int CPL = D / 16;   // channels per gating lane
  using RawV = typename std::conditional<CPL == 8, u32x4, u32x2>::type;  // CPL bf16
  using GateV = typename std::conditional<CPL == 8, Gate8<GT>, Gate4<GT>>::type;
  constexpr int NR0 = (RING + 1) / 2;  // ring chunks in the first key half
  static_assert(D == 64 || D == 128, "head size");
  static_assert(RING == 3 || RING == 5, "ring");
  __shared__ Smem<D, RING> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int seg = blockIdx.x, bh = blockIdx.y, h = bh % H;
  const SeqRows sr = seq_rows(cu, N, T_arg, H, bh);
  const int T_len = sr.len;
  const size_t off = sr.row0 * kD;
  const int nc = (T_len + kC - 1) / kC;
  // a packed sequence covers the first Gs of the plan's segments (at least
  // one, which for an empty sequence writes hT = h0 and an empty cache)
  const int Gs = cu ? max(1, (nc + 2 * cps - 1) / (2 * cps)) : G;
  if (seg >= Gs) return;
  // segments are whole 64-token chunks of the state pass
  const int c_begin = 2 * seg * cps, c_end = min(nc, c_begin + 2 * cps);
  const size_t s_base = (size_t)bh * kD * kD;

  // tiles that stay zero: the intra block above the diagonal, unused meta columns
  for (int e = tid; e < 16 * 16; e += 512) sm.a[at4(e >> 4, 16 + (e & 15))] = (bf16)0.f;
  for (int e = tid; e < kC * 16; e += 512) sm.p[kRing][at4(e >> 4, 16 + (e & 15))] = (bf16)0.f;
  // window blocks no query block reaches (see the producers' window scores):
  // rows 16..31 x keys 0..15 of the oldest ring chunk, rows 0..15 x keys
  // 16..31 of chunk c
  for (int e = tid; e < 2 * 16 * 16; e += 512) {
    const int x = (e >> 4) & 15, y = e & 15;
    if (e < 256)
      sm.p[0][at4(16 + x, y)] = (bf16)0.f;
    else
      sm.p[RING - 1][at4(x, 16 + y)] = (bf16)0.f;
  }
  {
    const bf16* mkh = mk + (size_t)h * M * kD;
    const bf16* mvh = mv + (size_t)h * M * kD;
    for (int e = tid; e < 16 * kD; e += 512) {
      const int r = e / kD, c = e % kD;
      sm.mk[atd<D>(r, c)] = r < M ? mkh[r * kD + c] : (bf16)0.f;
    }
    for (int e = tid; e < kD * kC; e += 512) {
      const int c = e / kC, t = e % kC;
      sm.mvT[atp(c, t)] = t < M ? mvh[t * kD + c] : (bf16)0.f;
    }
  }

  if (nc == 0) {
    // an empty packed sequence: the state passes through unchanged
    if (hT)
      for (int e = tid; e < kD * kD; e += 512) hT[s_base + e] = h0 ? h0[s_base + e] : 0.f;
  } else if (wave < 4) {
    // ------------------------------------------------------------ consumers
    const int cw = wave;
    // state entering the segment: h0 carried through the local end states
    // (column-major) and total log2 decays of the m pieces of each earlier
    // segment
    f32x4 S[NT][NCB];  // S[nt][cb]: rows 16cb + 4g + r, column CW cw + 16nt + r16
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S[nt][cb][r] = h0 ? h0[s_base + (16 * cb + 4 * g + r) * kD + CW * cw + 16 * nt + r16] : 0.f;
    const int P = (G - 1) * m;
    for (int sg = 0; sg < seg * m; ++sg) {
      const float* loc = ws_state + ((size_t)bh * P + sg) * kD * kD;
      const float* gm = ws_gamma + ((size_t)bh * P + sg) * kD;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const f32x4 g4 = *reinterpret_cast<const f32x4*>(&gm[16 * cb + 4 * g]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const f32x4 l4 =
              *reinterpret_cast<const f32x4*>(&loc[(CW * cw + 16 * nt + r16) * kD + 16 * cb + 4 * g]);
#pragma unroll
          for (int r = 0; r < 4; ++r) S[nt][cb][r] = exp2_fast(g4[r]) * S[nt][cb][r] + l4[r];
        }
      }
    }

    // v of a chunk: lane takes rows 2vr, 2vr+1 and columns CW cw + 8vo .. +7
    // (with D = 64 lanes 32..63 repeat lanes 0..31: same loads, same stores)
    constexpr int VO = CW / 8;
    const int vo = lane % VO, vr = (lane / VO) & 15;
    const u32 vb = (u32)((2 * vr * kD + CW * cw + 8 * vo) * 2);
    auto load_v = [&](int ch, u32x4* x) {
      const Buf cv(v + off + (size_t)ch * kC * kD, (u32)max(0, T_len - ch * kC) * kD * 2);
      x[0] = cv.ld128(vb);
      x[1] = cv.ld128(vb + kD * 2);
    };
    auto store_vT = [&](int slot, const u32x4* x) {
      bf16* dst = sm.vT[slot];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const u32 w0 = x[0][c >> 1], w1 = x[1][c >> 1];
        *reinterpret_cast<u32*>(&dst[atp(CW * cw + 8 * vo + c, 2 * vr)]) =
            (c & 1) ? hi2(w0, w1) : lo2(w0, w1);
      }
    };
    // slots that never receive a chunk (before the sequence start) hold zeros,
    // so the window product can run over every slot unconditionally
#pragma unroll
    for (int r = 0; r < kRing; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) *reinterpret_cast<u32*>(&sm.vT[r][atp(CW * cw + 8 * vo + c, 2 * vr)]) = 0u;
    {  // ring: chunks c_begin-RING+1 .. c_begin
      u32x4 pro[kRing][2];
#pragma unroll
      for (int r = 0; r < kRing; ++r)
        if (c_begin - (kRing - 1) + r >= 0) load_v(c_begin - (kRing - 1) + r, pro[r]);
#pragma unroll
      for (int r = 0; r < kRing; ++r)
        if (c_begin - (kRing - 1) + r >= 0) store_vT((c_begin - (kRing - 1) + r) % kRing, pro[r]);
    }
    // chunk c_begin + j is loaded into V[j & 1]; a set is refilled (chunk + 2)
    // right after its v^T store, so every load has two chunks of time
    u32x4 V0[2], V1[2];
    load_v(min(c_begin + 1, c_end - 1), V1);
    load_v(min(c_begin + 2, c_end - 1), V0);
    lds_barrier();

    auto step = [&](int c, u32x4* Vn) {
      const int slot = c % kRing;
      const int fw = sm.fastw[0] & sm.fastw[1] & sm.fastw[2] & sm.fastw[3];
      const bool fast = __builtin_amdgcn_readfirstlane(fw) != 0;
      // ---- phase 1: inter, O^T[n][t] = sum_ch S[ch][n] qs[t][ch]
      f32x4 O[NT][2];  // [nt][qb]: column (query) 16qb + r16, value columns CW cw + 16nt + 4g ..
      {
        bf16x8 qf[2][KS];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int p = 0; p < KS; ++p) qf[qb][p] = ld_split<D>(sm.qs, 16 * qb + r16, 32 * p + 4 * g);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) O[nt][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (fast) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int p = 0; p < KS; ++p) {
              const bf16x8 sf = pack_acc<bf16>(S[nt][2 * p], S[nt][2 * p + 1]);
#pragma unroll
              for (int qb = 0; qb < 2; ++qb) mma(O[nt][qb], sf, qf[qb][p]);
            }
        } else {
          // sub-block form: query block i sees the state rows scaled by 2^{R_i}
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int p = 0; p < KS; ++p) {
              const f32x4 e0 = *reinterpret_cast<const f32x4*>(&sm.eR[qb][32 * p + 4 * g]);
              const f32x4 e1 = *reinterpret_cast<const f32x4*>(&sm.eR[qb][32 * p + 16 + 4 * g]);
#pragma unroll
              for (int nt = 0; nt < NT; ++nt)
                mma(O[nt][qb], pack_acc<bf16>(S[nt][2 * p] * e0, S[nt][2 * p + 1] * e1), qf[qb][p]);
            }
        }
      }
      // ---- phase 1: state update, S = diag(2^{b_last}) S + khT V
      bf16x8 vf[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) vf[nt] = ld8<bf16>(&sm.vT[slot][atp(CW * cw + 16 * nt + r16, 8 * g)]);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const f32x4 dec = *reinterpret_cast<const f32x4*>(&sm.decay[16 * cb + 4 * g]);
        const bf16x8 kf = ld8<bf16>(&sm.khT[atp(16 * cb + r16, 8 * g)]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          S[nt][cb] *= dec;
          mma(S[nt][cb], kf, vf[nt]);
        }
      }
      // ---- phase 1: the masked intra scores, one block per wave 0..2
      if (cw < 3) intra_scores(sm, cw == 0 ? 0 : 1, cw == 2 ? 1 : 0, fast, r16, g);
      lds_barrier();  // (A) scores and probabilities visible
      // ---- phase 2: intra, O^T[n][t] += sum_s vT[n][s] A[t][s]
      {
        bf16x8 af[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) af[qb] = ld8<bf16>(&sm.a[at4(16 * qb + r16, 8 * g)]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) mma(O[nt][qb], vf[nt], af[qb]);
      }
      // ---- phase 2: window, O^T[n][t] += sum_s vT[n][s] P[t][s] over the ring.
      // Slot of chunk c-RING+1+r is (c+1+r) mod RING; meta slots >= M and P of
      // keys outside the window are zero.  The two key halves (ring chunks
      // r < NR0; the rest with the meta slots) carry exponentials from their own
      // row maxima m_h with sums l_h: with m = max(m_0, m_1),
      // f_h = 2^{(m_h - m) s}, half h's product is scaled by
      // f_h mix / (f_0 l_0 + f_1 l_1).  With the training outputs the window
      // branch is summed apart (without mix) and added once at the end.
      f32x4 Owin[kSave ? NT : 1][2];
      {
        float sc[2][2];  // [half][qb]
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const int row = 16 * qb + r16;
          const float m0 = sm.pmax[0][row], m1 = sm.pmax[1][row];
          const float mm = fmaxf(m0, m1);
          const float f0 = exp2_fast((m0 - mm) * scale_log2), f1 = exp2_fast((m1 - mm) * scale_log2);
          const float L = f0 * sm.psum[0][row] + f1 * sm.psum[1][row];
          const float inv = (kSave ? 1.f : mix) / L;
          sc[0][qb] = f0 * inv;
          sc[1][qb] = f1 * inv;
          if constexpr (kSave) {
            const int t = c * kC + row;
            if (lse && cw == 0 && g == 0 && t < T_len)
              lse[sr.row0 + t] = (mm * scale_log2 + log2_fast(L)) * kLn2;
          }
        }
        const int s0 = (c + 1) % kRing;
        // ring chunk NR0-1 belongs to half 0 for query rows 16..31; for rows
        // 0..15 its keys 0..15 (lanes g < 2 of a fragment) are in half 0 and
        // keys 16..31 in half 1
        const bool klo = g < 2;
        const bf16x8 z8 = {};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int r0 = h == 0 ? 0 : NR0 - 1, r1 = h == 0 ? NR0 - 1 : kRing;  // ring chunks (kRing: meta)
          bf16x8 wf[NR0 + 1][NT], pf[NR0 + 1][2];
#pragma unroll
          for (int r = r0; r <= r1; ++r) {
            const int sl = s0 + r < kRing ? s0 + r : s0 + r - kRing;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
              wf[r - r0][nt] = r == kRing - 1 ? vf[nt]
                             : r == kRing     ? ld8<bf16>(&sm.mvT[atp(CW * cw + 16 * nt + r16, 8 * g)])
                                              : ld8<bf16>(&sm.vT[sl][atp(CW * cw + 16 * nt + r16, 8 * g)]);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
              if (h == 1 && r == NR0 - 1 && qb == 1) continue;
              pf[r - r0][qb] = ld8<bf16>(&sm.p[r][at4(16 * qb + r16, 8 * g)]);
              if (r == NR0 - 1 && qb == 0) pf[r - r0][qb] = (klo == (h == 0)) ? pf[r - r0][qb] : z8;
            }
          }
          f32x4 Ow[NT][2];  // this half of the window branch, unnormalised
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) Ow[nt][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int r = r0; r <= r1; ++r)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
              for (int qb = 0; qb < 2; ++qb)
                if (!(h == 1 && r == NR0 - 1 && qb == 1)) mma(Ow[nt][qb], wf[r - r0][nt], pf[r - r0][qb]);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
              if constexpr (kSave)
                Owin[nt][qb] = h == 0 ? Ow[nt][qb] * sc[0][qb] : Owin[nt][qb] + Ow[nt][qb] * sc[1][qb];
              else
                O[nt][qb] += Ow[nt][qb] * sc[h][qb];
            }
        }
        if constexpr (kSave) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) O[nt][qb] += Owin[nt][qb] * mix;
        }
      }
      // v of chunk c+1 into the slot of chunk c-RING+1 (read above by this wave only);
      // past the segment end this stages an unused copy, so the loop body has no
      // branch around its loads and their waits stay exact
      store_vT((c + 1) % kRing, Vn);
      load_v(min(c + 3, c_end - 1), Vn);
      bf16* oc = o + off + (size_t)c * kC * kD;
      const int rows = T_len - c * kC;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          if (16 * qb + r16 < rows) {
            const u32 e = (u32)((16 * qb + r16) * kD + CW * cw + 16 * nt + 4 * g);
            st4<bf16>(oc + e, O[nt][qb]);
            if constexpr (kSave)
              if (o_swa) st4<bf16>(o_swa + off + (size_t)c * kC * kD + e, Owin[nt][qb]);
          }
      lds_barrier();  // (B) chunk c+1 staged
    };
    int c = c_begin;
    for (; c + 1 < c_end; c += 2) {
      step(c, V1);
      step(c + 1, V0);
    }
    if (c < c_end) step(c, V1);
    if (hT && seg == Gs - 1) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            hT[s_base + (16 * cb + 4 * g + r) * kD + CW * cw + 16 * nt + r16] = S[nt][cb][r];
    }
  } else {
    // ------------------------------------------------------------ producers
    // Issue priority over the consumer wave on the same SIMD: the window
    // scores are the longer path at either head size, and at d = 64 the gating
    // too (measured on B8 H16 T2048 with the training outputs: 76.4 against
    // 79.7 us); at d = 128 the gating of fp32 log alpha yields to the
    // consumers' outputs (on B2 H32 T4096: 0.1505 ms, against 0.154 with no
    // priority and 0.158 with the gating raised as well), while the gating of
    // bf16 logits, which adds a log-sigmoid per element, stays raised (0.152
    // against 0.156 ms lowered).
    __builtin_amdgcn_s_setprio(2);
    const int pw = wave - 4;                    // gates channels 4 CPL pw .. 4 CPL pw + 4 CPL - 1
    const int ol = lane >> 4, rq = lane & 15;   // channels ch0 .. ch0+CPL-1, rows 2rq, 2rq+1
    const int ch0 = 4 * CPL * pw + CPL * ol;
    const int isub = rq >> 3;                   // 16-row sub-block of the rows
    const u32 oe = (u32)(2 * rq * kD + ch0), o2 = oe * 2;
    struct In {
      RawV q[2], k[2];
      GateV la[2];
      RawV wq[2], wk[2];  // window queries and keys (kSep only)
    };
    auto ldv = [](const Buf& b, u32 o) -> RawV {
      if constexpr (CPL == 8)
        return b.ld128(o);
      else
        return ld64v(b, o);
    };
    auto packv = [](const u32 (&w)[CPL / 2]) -> RawV {
      if constexpr (CPL == 8)
        return u32x4{w[0], w[1], w[2], w[3]};
      else
        return u32x2{w[0], w[1]};
    };
    auto issue = [&](int ch, In& x) {
      const size_t e0 = off + (size_t)ch * kC * kD;
      const u32 rem = (u32)max(0, T_len - ch * kC) * kD;  // elements from the chunk start to the end
      const Buf bq(q + e0, rem * 2), bk(k + e0, rem * 2), bl(la + e0, rem * (u32)sizeof(GT));
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        x.q[rr] = ldv(bq, o2 + rr * kD * 2);
        x.k[rr] = ldv(bk, o2 + rr * kD * 2);
        x.la[rr].load(bl, oe + rr * kD);
      }
      if constexpr (kSep) {
        const Buf bwq(qw + e0, rem * 2), bwk(kw + e0, rem * 2);
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          x.wq[rr] = ldv(bwq, o2 + rr * kD * 2);
          x.wk[rr] = ldv(bwk, o2 + rr * kD * 2);
        }
      }
    };
    auto gate = [&](int ch, const In& x) {
      // b: inclusive log2 cumsum from the chunk start (in-thread over 2 rows,
      // then a scan over the 16 row pairs inside the 16-lane row)
      // The sums are first taken without the gate floor; only when some
      // channel's chunk total falls below the floor (then a token may lie
      // below it) are they taken again with it.
      float b[2][CPL], inc[CPL], blast[CPL], bmin = 0.f;
      auto scan = [&](auto floored) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          float run = 0.f;
#pragma unroll
          for (int rr = 0; rr < 2; ++rr) {
            const float g = decltype(floored)::value ? x.la[rr].log2_at(c) : x.la[rr].log2_nofloor_at(c);
            run += gate_row<GT>(g, 2 * rq + rr < T_len - ch * kC);
            b[rr][c] = run;
          }
          inc[c] = run;
        }
#pragma unroll
        for (int c = 0; c < CPL; ++c) inc[c] += dpp_shr<1>(inc[c]);
#pragma unroll
        for (int c = 0; c < CPL; ++c) inc[c] += dpp_shr<2>(inc[c]);
#pragma unroll
        for (int c = 0; c < CPL; ++c) inc[c] += dpp_shr<4>(inc[c]);
#pragma unroll
        for (int c = 0; c < CPL; ++c) inc[c] += dpp_shr<8>(inc[c]);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const float ex = inc[c] - b[1][c];
          b[0][c] += ex;
          b[1][c] += ex;
          blast[c] = dpp_bcast<15>(inc[c]);  // the last row pair holds the chunk total
          bmin = c ? fminf(bmin, blast[c]) : blast[c];
        }
      };
      scan(std::false_type());
      if (__any(bmin < kMinLog2Gate)) scan(std::true_type());  // uniform over the wave
      const bool fast = !__any(bmin < -kFast);  // uniform over the wave
      if (lane == 0) sm.fastw[pw] = fast ? 1 : 0;
      float dl[CPL];  // 2^{b_last}
#pragma unroll
      for (int c = 0; c < CPL; ++c) dl[c] = exp2_fast(blast[c]);
      if (rq == 0) {
#pragma unroll
        for (int c = 0; c < CPL; c += 4)
          *reinterpret_cast<f32x4*>(&sm.decay[ch0 + c]) = f32x4{dl[c], dl[c + 1], dl[c + 2], dl[c + 3]};
      }
      // references: none (fast) or b at row 16i+7 for sub-block i; eKh = 2^{b_last - R_i}
      float Ri[CPL], eKh[CPL];
      if (fast) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          Ri[c] = 0.f;
          eKh[c] = dl[c];
        }
        if (rq < 3) {  // the sub-block tables read 1 for these channels
          float* dst = rq < 2 ? &sm.eR[rq][ch0] : &sm.vij[ch0];
#pragma unroll
          for (int c = 0; c < CPL; c += 4) *reinterpret_cast<f32x4*>(dst + c) = f32x4{1.f, 1.f, 1.f, 1.f};
        }
      } else {
        float R0[CPL], R1[CPL];  // rows 7 and 23: the second row of row pairs 3 and 11
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          R0[c] = dpp_bcast<3>(b[1][c]);
          R1[c] = dpp_bcast<11>(b[1][c]);
          Ri[c] = isub ? R1[c] : R0[c];
          eKh[c] = exp2_fast(blast[c] - Ri[c]);
        }
        if (rq < 3) {
          float e[CPL];
#pragma unroll
          for (int c = 0; c < CPL; ++c) e[c] = exp2_fast(rq == 0 ? R0[c] : rq == 1 ? R1[c] : R1[c] - R0[c]);
          float* dst = rq < 2 ? &sm.eR[rq][ch0] : &sm.vij[ch0];
#pragma unroll
          for (int c = 0; c < CPL; c += 4)
            *reinterpret_cast<f32x4*>(dst + c) = f32x4{e[c], e[c + 1], e[c + 2], e[c + 3]};
        }
      }
      // gated tiles, rounded to bf16 pairs as they are made (the element loop
      // is specialised on the uniform form: the single reference is 0)
      u32 qw[2][CPL / 2], kw[2][CPL / 2];
      auto tiles = [&](auto single) {
        constexpr bool kSingle = decltype(single)::value;
#pragma unroll
        for (int c2 = 0; c2 < CPL / 2; ++c2) {
          float kx[2][2];
#pragma unroll
          for (int rr = 0; rr < 2; ++rr) {
            float qx[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int c = 2 * c2 + u;
              const float d = kSingle ? b[rr][c] : b[rr][c] - Ri[c];
              qx[u] = bf_at(x.q[rr], c) * exp2_fast(d);
              kx[rr][u] = bf_at(x.k[rr], c) * exp2_fast(-d);
            }
            qw[rr][c2] = pack_bf2(qx[0], qx[1]);
            kw[rr][c2] = pack_bf2(kx[rr][0], kx[rr][1]);
          }
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int c = 2 * c2 + u;
            const float e = kSingle ? dl[c] : eKh[c];
            *reinterpret_cast<u32*>(&sm.khT[atp(ch0 + c, 2 * rq)]) = pack_bf2(kx[0][u] * e, kx[1][u] * e);
          }
        }
      };
      if (fast)
        tiles(std::true_type());
      else
        tiles(std::false_type());
      bf16* kring = sm.kr[ch % kRing];
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int row = 2 * rq + rr;
        *reinterpret_cast<RawV*>(&sm.qs[atd<D>(row, ch0)]) = packv(qw[rr]);
        *reinterpret_cast<RawV*>(&sm.ks[atd<D>(row, ch0)]) = packv(kw[rr]);
        *reinterpret_cast<RawV*>(&sm.qr[atd<D>(row, ch0)]) = kSep ? x.wq[rr] : x.q[rr];
        *reinterpret_cast<RawV*>(&kring[atd<D>(row, ch0)]) = kSep ? x.wk[rr] : x.k[rr];
      }
    };
    // Window scores of query rows 16qb..16qb+15 of chunk c over one half of
    // their keys, one producer per (query block, half).  The 16-key blocks a
    // query block can reach, oldest first, are every (ring chunk r, key half
    // kb) but one that is outside every window the ring holds: (0, 0) for
    // qb = 1 (at least max_window(RING) tokens back) and (RING-1, 1) for
    // qb = 0 (after every query); with the meta block that is 2 RING blocks,
    // RING per half.  Half 0 takes the first RING, half 1 the rest and the
    // meta block, so for qb = 0 the halves meet inside ring chunk NR0-1 (its
    // first 16 keys in half 0) and the consumers separate them by key lanes.
    // Block j of half H is block id o + qb (id = 2 r + kb), o = j or RING + j.
    // Each half's exponentials are taken from its own row maximum; the row
    // maxima and sums go to LDS, and the consumers combine the two halves.
    // The probabilities of the unreached blocks are zero from the start.
    const int qbw = pw & 1;  // this producer's query block
    int kq[KS], kn[KS];      // raw-K tile offsets of key rows 16kb + r16: kb = qb, kb = 1 - qb
#pragma unroll
    for (int p = 0; p < KS; ++p) {
      kq[p] = atd<D>(16 * qbw + r16, 32 * p + 8 * g);
      kn[p] = atd<D>(16 * (1 - qbw) + r16, 32 * p + 8 * g);
    }
    const int prow = 16 * qbw + r16;
    const int pq = at4(prow, 16 * qbw + 4 * g), pn = at4(prow, 16 * (1 - qbw) + 4 * g);
    auto window = [&](int c, int qb, auto half) {
      constexpr int H = decltype(half)::value;
      constexpr int NB = kRing;  // blocks of this half (in half 1 the last is the meta block)
      bf16x8 qf[KS];
#pragma unroll
      for (int p = 0; p < KS; ++p) qf[p] = ld8<bf16>(&sm.qr[atd<D>(16 * qb + r16, 32 * p + 8 * g)]);
      const int t = c * kC + 16 * qb + r16;
      // every slot is multiplied (slots before the sequence start hold stale
      // data); the mask below selects -inf for every key outside the window
      const int s0 = (c + 1) % kRing;  // slot of chunk c-RING+1
      // ring chunk of block j (kb = qb for even o, 1 - qb for odd o)
      auto chunk_of = [&](int j) {
        const int o = H == 0 ? j : kRing + j;
        return (o >> 1) + ((o & 1) ? qb : 0);
      };
      f32x4 L[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) L[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const bool meta = H == 1 && j == NB - 1;
        const bool odd = ((H == 0 ? j : kRing + j) & 1) != 0;
        bf16x8 kf[KS];
        if (meta) {
#pragma unroll
          for (int p = 0; p < KS; ++p) kf[p] = ld8<bf16>(&sm.mk[atd<D>(r16, 32 * p + 8 * g)]);
        } else {
          const int r = chunk_of(j);
          const int sl = s0 + r < kRing ? s0 + r : s0 + r - kRing;
#pragma unroll
          for (int p = 0; p < KS; ++p) kf[p] = ld8<bf16>(&sm.kr[sl][odd ? kn[p] : kq[p]]);
        }
#pragma unroll
        for (int p = 0; p < KS; ++p) mma(L[j], kf[p], qf[p]);
      }
      // keys outside the window -> -inf; a 16-key block inside the window of
      // all 16 rows (uniform test) needs no per-key test
      const int tlo = c * kC + 16 * qb;
#pragma unroll
      for (int j = 0; j < NB - H; ++j) {
        const bool odd = ((H == 0 ? j : kRing + j) & 1) != 0;
        const int kb = odd ? 1 - qb : qb;
        const int slo = (c - (kRing - 1) + chunk_of(j)) * kC + 16 * kb;
        const bool full = slo >= 0 && slo + 15 <= tlo && slo > tlo + 15 - W;
        if (!full) {
          // key s inside the window of query t: 0 <= t - s < W (one unsigned
          // compare); keys before the sequence start only in its first chunks
          const int dt = t - slo - 4 * g;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool ok = (u32)(dt - i) < (u32)W && (slo >= 0 || slo + 4 * g + i >= 0);
            L[j][i] = ok ? L[j][i] : -INFINITY;
          }
        }
      }
      if (H == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) L[NB - 1][i] = (4 * g + i < M) ? L[NB - 1][i] : -INFINITY;
      }
      // exponentials from this half's own row maximum (scale > 0); a row with
      // no key in this half keeps m at a finite floor, so its terms are 0 and
      // the consumers' factor 2^{(m_h - m) s} underflows to 0
      float m = -INFINITY;
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, L[j][i]);
      m = fmaxf(swap_max16(m), -1e30f);
      const int row = 16 * qb + r16;
      if (g == 0) sm.pmax[H][row] = m;
      const float ms = -m * scale_log2;
      float l = 0.f;
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          L[j][i] = exp2_fast(fmaf(L[j][i], scale_log2, ms));
          l += L[j][i];
        }
      l = swap_sum16(l);
      if (g == 0) sm.psum[H][row] = l;
#pragma unroll
      for (int j = 0; j < NB - H; ++j) {
        const bool odd = ((H == 0 ? j : kRing + j) & 1) != 0;
        st4<bf16>(&sm.p[chunk_of(j)][odd ? pn : pq], L[j]);
      }
      if (H == 1) st4<bf16>(&sm.p[kRing][at4(row, 4 * g)], L[NB - 1]);
    };

    // ---- prologue: the raw-K ring before the segment, chunk c_begin gated,
    // c_begin+1 and c_begin+2 in flight
    In I0, I1;
    {
      issue(c_begin, I0);
      issue(min(c_begin + 1, c_end - 1), I1);
      RawV kp[kRing - 1][2];
#pragma unroll
      for (int r = 0; r < kRing - 1; ++r) {
        const int cr = c_begin - (kRing - 1) + r;
        if (cr >= 0) {
          const Buf bk(kw + off + (size_t)cr * kC * kD, (u32)(kC * kD * 2));
          kp[r][0] = ldv(bk, o2);
          kp[r][1] = ldv(bk, o2 + kD * 2);
        }
      }
#pragma unroll
      for (int r = 0; r < kRing - 1; ++r) {
        const int cr = c_begin - (kRing - 1) + r;
        if (cr >= 0) {
          *reinterpret_cast<RawV*>(&sm.kr[cr % kRing][atd<D>(2 * rq, ch0)]) = kp[r][0];
          *reinterpret_cast<RawV*>(&sm.kr[cr % kRing][atd<D>(2 * rq + 1, ch0)]) = kp[r][1];
        }
      }
      gate(c_begin, I0);
      issue(min(c_begin + 2, c_end - 1), I0);
    }
    lds_barrier();

    auto pstep = [&](int c, In& Xn) {
      if (pw < 2)
        window(c, pw & 1, std::integral_constant<int, 0>());
      else
        window(c, pw & 1, std::integral_constant<int, 1>());
      lds_barrier();  // (A) every read of the gated tiles, raw q and K(c-RING+1) done
      if constexpr (D == 128 && sizeof(GT) == 4) __builtin_amdgcn_s_setprio(0);
      // past the segment end this gates an unused copy of the last chunk (no
      // branch around the loads, so their waits stay exact)
      gate(c + 1, Xn);
      issue(min(c + 3, c_end - 1), Xn);
      lds_barrier();  // (B)
      if constexpr (D == 128) __builtin_amdgcn_s_setprio(2);
    };
    int c = c_begin;
    for (; c + 1 < c_end; c += 2) {
      pstep(c, I1);
      pstep(c + 1, I0);
    }
    if (c < c_end) pstep(c, I1);
  }

  // window cache for decoding (rk, rv non-null): slot p mod W <- token p for the
  // last min(T, W) tokens, zero for slots without a token; the head's segments
  // share the slots
  if (rk) {
    const Buf bk(kw + off, (u32)((size_t)T_len * kD * 2)), bv(v + off, (u32)((size_t)T_len * kD * 2));
    const size_t rbase = (size_t)bh * W * kD;
    const u32x4 z = {0u, 0u, 0u, 0u};
    constexpr int GR = kD / 8;  // 16-byte granules per row
    const int s_lo = (int)((long long)W * seg / Gs), s_hi = (int)((long long)W * (seg + 1) / Gs);
    for (int e = s_lo * GR + tid; e < s_hi * GR; e += 512) {
      const int slot = e / GR, c = (e % GR) * 8;
      const int p = slot < T_len % W ? T_len - T_len % W + slot : T_len - T_len % W - W + slot;
      u32x4 xk = z, xv = z;
      if (p >= 0) {
        const u32 bo = (u32)(((size_t)p * kD + c) * 2);
        xk = bk.ld128(bo);
        xv = bv.ld128(bo);
      }
      *reinterpret_cast<u32x4*>(&rk[rbase + (size_t)slot * kD + c]) = xk;
      *reinterpret_cast<u32x4*>(&rv[rbase + (size_t)slot * kD + c]) = xv;
    }
  }
}


template <int D, int RING, bool kSep, typename GT, bool kSave>
void launch_fused_kernel(const Shape& s, const void* q, const void* k, const void* qw,
                         const void* kw, const void* v, const void* la, const void* mk,
                         const void* mv, const float* h0, const float* ws_state,
                         const float* ws_gamma, void* o, float* hT, void* ring_k, void* ring_v,
                         void* o_swa, float* lse, int cps, int G_, int m, hipStream_t st) {
  hipLaunchKernelGGL((hybrid_fwd_fused<D, RING, kSep, GT, kSave>), dim3(G_, s.B * s.H), dim3(512), 0, st,
                     (const bf16*)q, (const bf16*)k, (const bf16*)qw, (const bf16*)kw,
                     (const bf16*)v, (const GT*)la, (const bf16*)mk, (const bf16*)mv, h0, ws_state,
                     ws_gamma, (bf16*)o, hT, (bf16*)ring_k, (bf16*)ring_v, (bf16*)o_swa, lse, s.T,
                     s.H, s.window, s.n_meta, s.scale * kLog2e, s.mix, cps, G_, m, s.cu, s.n_tokens);
}

template <int D, int RING, bool kSave = (D == 64)>
void launch_fused_ring(const Shape& s, bool sep, const void* q, const void* k, const void* qw,
                       const void* kw, const void* v, const void* la, const void* mk,
                       const void* mv, const float* h0, const float* ws_state,
                       const float* ws_gamma, void* o, float* hT, void* ring_k, void* ring_v,
                       void* o_swa, float* lse, int cps, int G, int m, hipStream_t st) {
  auto go = [&](auto kernel_launch) {
    kernel_launch(s, q, k, qw, kw, v, la, mk, mv, h0, ws_state, ws_gamma, o, hT, ring_k, ring_v,
                  o_swa, lse, cps, G, m, st);
  };
  if (s.gate == 1)
    sep ? go(launch_fused_kernel<D, RING, true, bf16, kSave>) : go(launch_fused_kernel<D, RING, false, bf16, kSave>);
  else
    sep ? go(launch_fused_kernel<D, RING, true, float, kSave>) : go(launch_fused_kernel<D, RING, false, float, kSave>);
}

}  // namespace
}  // namespace lz
