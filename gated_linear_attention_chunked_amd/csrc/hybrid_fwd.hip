// Hybrid forward as one output pass, gfx950, bf16, d_k = d_v = 128, w <= 129.
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
//   phase 1  consumers (waves 0-3; value columns 32w..32w+31, their fp32 state
//              slice in registers): inter O = (q 2^b) S_c, the state update
//              S_{c+1} = diag(2^{b_last}) S_c + (k 2^{b_last - b})^T V, and
//              (waves 0-2, one 16x16 block each) the masked intra scores
//            producers (waves 4-7): window scores of query rows 16(p&1).. over
//              one half of the keys (ring chunks c-4..c-2, or c-1, c and the
//              meta slots); exponentials from that half's own row maxima;
//              maxima, row sums and exponentials -> LDS
//   ---- barrier
//   phase 2  consumers: O += A V (intra) + the two halves' P V (V^T ring, meta
//              values), each scaled by f_h mix / (f_0 l_0 + f_1 l_1) with
//              f_h = 2^{(m_h - max(m_0, m_1)) scale}; store o; v of chunk c+1
//              into the V^T ring
//            producers: gate chunk c+1 (log2-gate cumsum, gated q and k tiles,
//              k^T for the state update), raw q and raw k of c+1 into LDS;
//              issue the loads of chunk c+3
//   ---- barrier
// 32-token chunks keep the GLA tiles and a ring of w + 32 window keys and
// values inside the 160 KB of LDS at once.  The GLA algebra is that of
// gla_fwd.hip: one reference (the chunk start) when every channel's chunk decay
// stays above 2^-64, otherwise 16-token sub-block references R_i with the pair
// factor 2^{R_1 - R_0} on the off-diagonal block.  The V^T ring is partitioned
// by value columns, so each consumer wave reads and writes only its own part
// and the ring needs no barrier of its own.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace lz {
namespace {

constexpr int kC = 32;             // tokens per chunk
constexpr int kD = 128;            // d_k = d_v
constexpr int kRing = 5;           // window ring slots: chunks c-4 .. c
constexpr int kMaxW = 4 * kC + 1;  // widest window the ring holds
constexpr float kFast = 64.f;      // single reference while every chunk decay >= 2^-64
// Row of the transposed [channel][token] tiles (k-hat^T, the V^T ring, meta V^T):
// 32 tokens padded to 80 bytes.  Their staging stores write four rows 8 apart
// per instruction; at 64-byte rows those rows share one set of banks, at 80
// bytes they fall on two, and the 16-row fragment reads stay conflict-free.
constexpr int kTP = kC + 8;

struct Smem {
  bf16 qs[kC * kD];              // gated q [t][ch]: q 2^{b_t} (or 2^{b_t - R_i})
  bf16 ks[kC * kD];              // gated k [s][ch]: k 2^{-b_s} (or 2^{R_j - b_s})
  bf16 khT[kD * kTP];            // [ch][s]: k 2^{b_last - b_s}
  bf16 a[kC * kC];               // masked intra scores [t][s]
  bf16 p[kRing + 1][kC * kC];    // window probabilities [t][s] per ring chunk, meta last
  bf16 vT[kRing][kD * kTP];      // V^T ring [n][s]
  bf16 kr[kRing][kC * kD];       // raw K ring [s][ch]
  bf16 qr[kC * kD];              // raw q [t][ch]
  bf16 mk[16 * kD];              // meta keys (rows >= M zero)
  bf16 mvT[kD * kTP];            // meta values transposed (slots >= M zero)
  alignas(16) float decay[kD];   // 2^{b_last}
  alignas(16) float eR[2][kD];   // 2^{R_i} (1 for single-reference channels)
  alignas(16) float vij[kD];     // 2^{R_1 - R_0} (likewise)
  float pmax[2][kC];             // window: per key half, row maxima of the raw scores
  float psum[2][kC];             // per key half, row sums of exponentials taken from that maximum
  int fastw[4];                  // per producer wave: its channels take one reference
};

// [rows][128] and [rows][32] tiles, granules permuted by row
__device__ __forceinline__ int at16(int row, int col) { return swz_at<16>(row, col); }
__device__ __forceinline__ int at4(int row, int col) { return swz_at<4>(row, col); }
// (row, col) of a padded transposed tile
__device__ __forceinline__ int atp(int row, int col) { return row * kTP + col; }

// Split-map fragment (elements col..col+3 and col+16..col+19) of a [rows][128] tile.
__device__ __forceinline__ bf16x8 ld_split16(const bf16* t, int row, int col) {
  const bf16x4 x = *reinterpret_cast<const bf16x4*>(&t[at16(row, col)]);
  const bf16x4 y = *reinterpret_cast<const bf16x4*>(&t[at16(row, col + 16)]);
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
__device__ __forceinline__ void intra_scores(Smem& sm, int i, int j, bool fast, int r16, int g) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const bf16x8 af = ld8<bf16>(&sm.ks[at16(16 * j + r16, 32 * p + 8 * g)]);
    bf16x8 bf = ld8<bf16>(&sm.qs[at16(16 * i + r16, 32 * p + 8 * g)]);
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
// log alpha or bf16 logit).
template <bool kSep, typename GT>
__global__ __launch_bounds__(512, 1) void hybrid_fwd_fused(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ qw,
    const bf16* __restrict__ kw, const bf16* __restrict__ v,
    const GT* __restrict__ la, const bf16* __restrict__ mk, const bf16* __restrict__ mv,
    const float* __restrict__ h0, const float* __restrict__ ws_state,
    const float* __restrict__ ws_gamma, bf16* __restrict__ o, float* __restrict__ hT,
    bf16* __restrict__ rk, bf16* __restrict__ rv, int T_arg, int H, int W, int M,
    float scale_log2, float mix, int cps, int G, const int* __restrict__ cu, int N) {
  __shared__ Smem sm;
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
  {
    const bf16* mkh = mk + (size_t)h * M * kD;
    const bf16* mvh = mv + (size_t)h * M * kD;
    for (int e = tid; e < 16 * kD; e += 512) {
      const int r = e / kD, c = e % kD;
      sm.mk[at16(r, c)] = r < M ? mkh[r * kD + c] : (bf16)0.f;
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
    // state entering the segment: h0 carried through the earlier segments'
    // local end states (column-major) and total log2 decays
    f32x4 S[2][8];  // S[nt][cb]: rows 16cb + 4g + r, column 32cw + 16nt + r16
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int cb = 0; cb < 8; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S[nt][cb][r] = h0 ? h0[s_base + (16 * cb + 4 * g + r) * kD + 32 * cw + 16 * nt + r16] : 0.f;
    for (int sg = 0; sg < seg; ++sg) {
      const float* loc = ws_state + ((size_t)bh * (G - 1) + sg) * kD * kD;
      const float* gm = ws_gamma + ((size_t)bh * (G - 1) + sg) * kD;
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        const f32x4 g4 = *reinterpret_cast<const f32x4*>(&gm[16 * cb + 4 * g]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const f32x4 l4 =
              *reinterpret_cast<const f32x4*>(&loc[(32 * cw + 16 * nt + r16) * kD + 16 * cb + 4 * g]);
#pragma unroll
          for (int r = 0; r < 4; ++r) S[nt][cb][r] = exp2_fast(g4[r]) * S[nt][cb][r] + l4[r];
        }
      }
    }

    // v of a chunk: lane takes rows 2vr, 2vr+1 and columns 32cw + 8vo .. +7
    const int vo = lane & 3, vr = lane >> 2;
    const u32 vb = (u32)((2 * vr * kD + 32 * cw + 8 * vo) * 2);
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
        *reinterpret_cast<u32*>(&dst[atp(32 * cw + 8 * vo + c, 2 * vr)]) =
            (c & 1) ? hi2(w0, w1) : lo2(w0, w1);
      }
    };
    // slots that never receive a chunk (before the sequence start) hold zeros,
    // so the window product can run over every slot unconditionally
#pragma unroll
    for (int r = 0; r < kRing; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) *reinterpret_cast<u32*>(&sm.vT[r][atp(32 * cw + 8 * vo + c, 2 * vr)]) = 0u;
    {  // ring: chunks c_begin-4 .. c_begin
      u32x4 pro[kRing][2];
#pragma unroll
      for (int r = 0; r < kRing; ++r)
        if (c_begin - 4 + r >= 0) load_v(c_begin - 4 + r, pro[r]);
#pragma unroll
      for (int r = 0; r < kRing; ++r)
        if (c_begin - 4 + r >= 0) store_vT((c_begin - 4 + r) % kRing, pro[r]);
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
      f32x4 O[2][2];  // [nt][qb]: column (query) 16qb + r16, value columns 32cw + 16nt + 4g ..
      {
        bf16x8 qf[2][4];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int p = 0; p < 4; ++p) qf[qb][p] = ld_split16(sm.qs, 16 * qb + r16, 32 * p + 4 * g);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) O[nt][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (fast) {
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const bf16x8 sf = pack_acc<bf16>(S[nt][2 * p], S[nt][2 * p + 1]);
#pragma unroll
              for (int qb = 0; qb < 2; ++qb) mma(O[nt][qb], sf, qf[qb][p]);
            }
        } else {
          // sub-block form: query block i sees the state rows scaled by 2^{R_i}
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const f32x4 e0 = *reinterpret_cast<const f32x4*>(&sm.eR[qb][32 * p + 4 * g]);
              const f32x4 e1 = *reinterpret_cast<const f32x4*>(&sm.eR[qb][32 * p + 16 + 4 * g]);
#pragma unroll
              for (int nt = 0; nt < 2; ++nt)
                mma(O[nt][qb], pack_acc<bf16>(S[nt][2 * p] * e0, S[nt][2 * p + 1] * e1), qf[qb][p]);
            }
        }
      }
      // ---- phase 1: state update, S = diag(2^{b_last}) S + khT V
      bf16x8 vf[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) vf[nt] = ld8<bf16>(&sm.vT[slot][atp(32 * cw + 16 * nt + r16, 8 * g)]);
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        const f32x4 dec = *reinterpret_cast<const f32x4*>(&sm.decay[16 * cb + 4 * g]);
        const bf16x8 kf = ld8<bf16>(&sm.khT[atp(16 * cb + r16, 8 * g)]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
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
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) mma(O[nt][qb], vf[nt], af[qb]);
      }
      // ---- phase 2: window, O^T[n][t] += sum_s vT[n][s] P[t][s] over the ring.
      // Slot of chunk c-4+r is (c+1+r) mod 5; meta slots >= M and P of keys
      // outside the window are zero.  The two key halves (ring chunks c-4..c-2;
      // c-1, c and the meta slots) carry exponentials from their own row
      // maxima m_h with sums l_h: with m = max(m_0, m_1), f_h = 2^{(m_h - m) s},
      // half h's product is scaled by f_h mix / (f_0 l_0 + f_1 l_1).
      {
        float sc[2][2];  // [half][qb]
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const int row = 16 * qb + r16;
          const float m0 = sm.pmax[0][row], m1 = sm.pmax[1][row];
          const float mm = fmaxf(m0, m1);
          const float f0 = exp2_fast((m0 - mm) * scale_log2), f1 = exp2_fast((m1 - mm) * scale_log2);
          const float inv = mix / (f0 * sm.psum[0][row] + f1 * sm.psum[1][row]);
          sc[0][qb] = f0 * inv;
          sc[1][qb] = f1 * inv;
        }
        const int s0 = (c + 1) % kRing;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int r0 = h == 0 ? 0 : 3, r1 = h == 0 ? 2 : kRing;  // ring chunks (kRing: meta)
          bf16x8 wf[3][2], pf[3][2];
#pragma unroll
          for (int r = r0; r <= r1; ++r) {
            const int sl = s0 + r < kRing ? s0 + r : s0 + r - kRing;
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
              wf[r - r0][nt] = r == kRing - 1 ? vf[nt]
                             : r == kRing     ? ld8<bf16>(&sm.mvT[atp(32 * cw + 16 * nt + r16, 8 * g)])
                                              : ld8<bf16>(&sm.vT[sl][atp(32 * cw + 16 * nt + r16, 8 * g)]);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) pf[r - r0][qb] = ld8<bf16>(&sm.p[r][at4(16 * qb + r16, 8 * g)]);
          }
          f32x4 Ow[2][2];  // this half of the window branch, unnormalised
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) Ow[nt][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int r = r0; r <= r1; ++r)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
              for (int qb = 0; qb < 2; ++qb) mma(Ow[nt][qb], wf[r - r0][nt], pf[r - r0][qb]);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) O[nt][qb] += Ow[nt][qb] * sc[h][qb];
        }
      }
      // v of chunk c+1 into the slot of chunk c-4 (read above by this wave only);
      // past the segment end this stages an unused copy, so the loop body has no
      // branch around its loads and their waits stay exact
      store_vT((c + 1) % kRing, Vn);
      load_v(min(c + 3, c_end - 1), Vn);
      bf16* oc = o + off + (size_t)c * kC * kD;
      const int rows = T_len - c * kC;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          if (16 * qb + r16 < rows)
            st4<bf16>(oc + (u32)((16 * qb + r16) * kD + 32 * cw + 16 * nt + 4 * g), O[nt][qb]);
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
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            hT[s_base + (16 * cb + 4 * g + r) * kD + 32 * cw + 16 * nt + r16] = S[nt][cb][r];
    }
  } else {
    // ------------------------------------------------------------ producers
    const int pw = wave - 4;                    // gating: channels 32pw .. 32pw+31
    const int ol = lane >> 4, rq = lane & 15;   // channels ch0 .. ch0+7, rows 2rq, 2rq+1
    const int ch0 = 32 * pw + 8 * ol;
    const int isub = rq >> 3;                   // 16-row sub-block of the rows
    const u32 oe = (u32)(2 * rq * kD + ch0), o2 = oe * 2;
    struct In {
      u32x4 q[2], k[2];
      Gate8<GT> la[2];
      u32x4 wq[2], wk[2];  // window queries and keys (kSep only)
    };
    auto issue = [&](int ch, In& x) {
      const size_t e0 = off + (size_t)ch * kC * kD;
      const u32 rem = (u32)max(0, T_len - ch * kC) * kD;  // elements from the chunk start to the end
      const Buf bq(q + e0, rem * 2), bk(k + e0, rem * 2), bl(la + e0, rem * (u32)sizeof(GT));
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        x.q[rr] = bq.ld128(o2 + rr * kD * 2);
        x.k[rr] = bk.ld128(o2 + rr * kD * 2);
        x.la[rr].load(bl, oe + rr * kD);
      }
      if constexpr (kSep) {
        const Buf bwq(qw + e0, rem * 2), bwk(kw + e0, rem * 2);
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          x.wq[rr] = bwq.ld128(o2 + rr * kD * 2);
          x.wk[rr] = bwk.ld128(o2 + rr * kD * 2);
        }
      }
    };
    auto gate = [&](int ch, const In& x) {
      // b: inclusive log2 cumsum from the chunk start (in-thread over 2 rows,
      // then a scan over the 16 row pairs inside the 16-lane row)
      float b[2][8], inc[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float run = 0.f;
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          run += gate_row<GT>(x.la[rr].log2_at(c), 2 * rq + rr < T_len - ch * kC);
          b[rr][c] = run;
        }
        inc[c] = run;
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) inc[c] += dpp_shr<1>(inc[c]);
#pragma unroll
      for (int c = 0; c < 8; ++c) inc[c] += dpp_shr<2>(inc[c]);
#pragma unroll
      for (int c = 0; c < 8; ++c) inc[c] += dpp_shr<4>(inc[c]);
#pragma unroll
      for (int c = 0; c < 8; ++c) inc[c] += dpp_shr<8>(inc[c]);
      float blast[8], bmin = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float ex = inc[c] - b[1][c];
        b[0][c] += ex;
        b[1][c] += ex;
        blast[c] = dpp_bcast<15>(inc[c]);  // the last row pair holds the chunk total
        bmin = c ? fminf(bmin, blast[c]) : blast[c];
      }
      const bool fast = !__any(bmin < -kFast);  // uniform over the wave
      if (lane == 0) sm.fastw[pw] = fast ? 1 : 0;
      float dl[8];  // 2^{b_last}
#pragma unroll
      for (int c = 0; c < 8; ++c) dl[c] = exp2_fast(blast[c]);
      if (rq == 0) {
        *reinterpret_cast<f32x4*>(&sm.decay[ch0]) = f32x4{dl[0], dl[1], dl[2], dl[3]};
        *reinterpret_cast<f32x4*>(&sm.decay[ch0 + 4]) = f32x4{dl[4], dl[5], dl[6], dl[7]};
      }
      // references: none (fast) or b at row 16i+7 for sub-block i; eKh = 2^{b_last - R_i}
      float Ri[8], eKh[8];
      if (fast) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          Ri[c] = 0.f;
          eKh[c] = dl[c];
        }
        if (rq < 3) {  // the sub-block tables read 1 for these channels
          float* dst = rq < 2 ? &sm.eR[rq][ch0] : &sm.vij[ch0];
          *reinterpret_cast<f32x4*>(dst) = f32x4{1.f, 1.f, 1.f, 1.f};
          *reinterpret_cast<f32x4*>(dst + 4) = f32x4{1.f, 1.f, 1.f, 1.f};
        }
      } else {
        float R0[8], R1[8];  // rows 7 and 23: the second row of row pairs 3 and 11
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          R0[c] = dpp_bcast<3>(b[1][c]);
          R1[c] = dpp_bcast<11>(b[1][c]);
          Ri[c] = isub ? R1[c] : R0[c];
          eKh[c] = exp2_fast(blast[c] - Ri[c]);
        }
        if (rq < 3) {
          float e[8];
#pragma unroll
          for (int c = 0; c < 8; ++c) e[c] = exp2_fast(rq == 0 ? R0[c] : rq == 1 ? R1[c] : R1[c] - R0[c]);
          float* dst = rq < 2 ? &sm.eR[rq][ch0] : &sm.vij[ch0];
          *reinterpret_cast<f32x4*>(dst) = f32x4{e[0], e[1], e[2], e[3]};
          *reinterpret_cast<f32x4*>(dst + 4) = f32x4{e[4], e[5], e[6], e[7]};
        }
      }
      // gated tiles, rounded to bf16 pairs as they are made (the element loop
      // is specialised on the uniform form: the single reference is 0)
      u32 qw[2][4], kw[2][4];
      auto tiles = [&](auto single) {
        constexpr bool kSingle = decltype(single)::value;
#pragma unroll
        for (int c2 = 0; c2 < 4; ++c2) {
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
        *reinterpret_cast<u32x4*>(&sm.qs[at16(row, ch0)]) = u32x4{qw[rr][0], qw[rr][1], qw[rr][2], qw[rr][3]};
        *reinterpret_cast<u32x4*>(&sm.ks[at16(row, ch0)]) = u32x4{kw[rr][0], kw[rr][1], kw[rr][2], kw[rr][3]};
        *reinterpret_cast<u32x4*>(&sm.qr[at16(row, ch0)]) = kSep ? x.wq[rr] : x.q[rr];
        *reinterpret_cast<u32x4*>(&kring[at16(row, ch0)]) = kSep ? x.wk[rr] : x.k[rr];
      }
    };
    // Window scores of query rows 16qb..16qb+15 of chunk c over one half of
    // the keys: ring chunks c-4..c-2 (half 0) or c-1, c and the meta slots
    // (half 1), one producer per (query block, half).  Each half's
    // exponentials are taken from its own row maximum; the row maxima and sums
    // go to LDS, and the consumers combine the two halves.
    auto window = [&](int c, int qb, auto half) {
      constexpr int H = decltype(half)::value;
      constexpr int R0 = H == 0 ? 0 : 3, NR = H == 0 ? 3 : 2;  // ring chunks r = R0 .. R0+NR-1
      constexpr int NB = 2 * NR + H;                           // 16-key blocks (+ the meta block)
      bf16x8 qf[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) qf[p] = ld8<bf16>(&sm.qr[at16(16 * qb + r16, 32 * p + 8 * g)]);
      const int t = c * kC + 16 * qb + r16;
      // every slot is multiplied (slots before the sequence start hold stale
      // data); the mask below selects -inf for every key outside the window
      const int s0 = (c + 1) % kRing;  // slot of chunk c-4
      f32x4 L[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) L[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int x = 0; x < NR + H; ++x) {
        const bool meta = x == NR;
        const int r = R0 + x;
        const int sl = s0 + r < kRing ? s0 + r : s0 + r - kRing;
        bf16x8 kf[2][4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int p = 0; p < 4; ++p)
            if (!meta || kb == 0)
              kf[kb][p] = ld8<bf16>(meta ? &sm.mk[at16(r16, 32 * p + 8 * g)]
                                         : &sm.kr[sl][at16(16 * kb + r16, 32 * p + 8 * g)]);
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            if (!meta || kb == 0) mma(L[2 * x + kb], kf[kb][p], qf[p]);
      }
      // keys outside the window -> -inf; a 16-key block inside the window of
      // all 16 rows (uniform test) needs no per-key test
      const int tlo = c * kC + 16 * qb;
#pragma unroll
      for (int x = 0; x < NR; ++x)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int slo = (c - (kRing - 1) + R0 + x) * kC + 16 * kb;
          const bool full = slo >= 0 && slo + 15 <= tlo && slo > tlo + 15 - W;
          if (!full) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int sk = slo + 4 * g + i;
              const bool ok = sk >= 0 && sk <= t && sk > t - W;
              L[2 * x + kb][i] = ok ? L[2 * x + kb][i] : -INFINITY;
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
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, L[b][i]);
      m = fmaxf(swap_max16(m), -1e30f);
      const int row = 16 * qb + r16;
      if (g == 0) sm.pmax[H][row] = m;
      const float ms = -m * scale_log2;
      float l = 0.f;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          L[b][i] = exp2_fast(fmaf(L[b][i], scale_log2, ms));
          l += L[b][i];
        }
      l = swap_sum16(l);
      if (g == 0) sm.psum[H][row] = l;
#pragma unroll
      for (int x = 0; x < NR; ++x)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          st4<bf16>(&sm.p[R0 + x][at4(row, 16 * kb + 4 * g)], L[2 * x + kb]);
      if (H == 1) st4<bf16>(&sm.p[kRing][at4(row, 4 * g)], L[NB - 1]);
    };

    // ---- prologue: the raw-K ring before the segment, chunk c_begin gated,
    // c_begin+1 and c_begin+2 in flight
    In I0, I1;
    issue(c_begin, I0);
    issue(min(c_begin + 1, c_end - 1), I1);
    {
      u32x4 kp[kRing - 1][2];
#pragma unroll
      for (int r = 0; r < kRing - 1; ++r) {
        const int cr = c_begin - 4 + r;
        if (cr >= 0) {
          const Buf bk(kw + off + (size_t)cr * kC * kD, (u32)(kC * kD * 2));
          kp[r][0] = bk.ld128(o2);
          kp[r][1] = bk.ld128(o2 + kD * 2);
        }
      }
#pragma unroll
      for (int r = 0; r < kRing - 1; ++r) {
        const int cr = c_begin - 4 + r;
        if (cr >= 0) {
          *reinterpret_cast<u32x4*>(&sm.kr[cr % kRing][at16(2 * rq, ch0)]) = kp[r][0];
          *reinterpret_cast<u32x4*>(&sm.kr[cr % kRing][at16(2 * rq + 1, ch0)]) = kp[r][1];
        }
      }
    }
    gate(c_begin, I0);
    issue(min(c_begin + 2, c_end - 1), I0);
    lds_barrier();

    auto pstep = [&](int c, In& Xn) {
      if (pw < 2)
        window(c, pw & 1, std::integral_constant<int, 0>());
      else
        window(c, pw & 1, std::integral_constant<int, 1>());
      lds_barrier();  // (A) every read of the gated tiles, raw q and K(c-4) done
      // past the segment end this gates an unused copy of the last chunk (no
      // branch around the loads, so their waits stay exact)
      gate(c + 1, Xn);
      issue(min(c + 3, c_end - 1), Xn);
      lds_barrier();  // (B)
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
    const int s_lo = (int)((long long)W * seg / Gs), s_hi = (int)((long long)W * (seg + 1) / Gs);
    for (int e = s_lo * 16 + tid; e < s_hi * 16; e += 512) {
      const int slot = e >> 4, c = (e & 15) * 8;
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

}  // namespace

bool hybrid_fused_ok(const Shape& s) {
  return s.dtype == 1 && s.dk == kD && s.dv == kD && s.window >= 1 && s.window <= kMaxW &&
         s.n_meta <= 16 && s.T > 0;
}

template <bool kSep, typename GT>
void launch_fused_kernel(const Shape& s, const void* q, const void* k, const void* qw,
                         const void* kw, const void* v, const void* la, const void* mk,
                         const void* mv, const float* h0, const float* ws_state,
                         const float* ws_gamma, void* o, float* hT, void* ring_k, void* ring_v,
                         int cps, int G_, hipStream_t st) {
  hipLaunchKernelGGL((hybrid_fwd_fused<kSep, GT>), dim3(G_, s.B * s.H), dim3(512), 0, st,
                     (const bf16*)q, (const bf16*)k, (const bf16*)qw, (const bf16*)kw,
                     (const bf16*)v, (const GT*)la, (const bf16*)mk, (const bf16*)mv, h0, ws_state,
                     ws_gamma, (bf16*)o, hT, (bf16*)ring_k, (bf16*)ring_v, s.T, s.H, s.window,
                     s.n_meta, s.scale * kLog2e, s.mix, cps, G_, s.cu, s.n_tokens);
}

hipError_t launch_hybrid_fused(const Shape& s, const void* q, const void* k, const void* qw,
                               const void* kw, const void* v, const void* la, const void* mk,
                               const void* mv, const float* h0, void* o, float* hT, void* ring_k,
                               void* ring_v, void* ws, hipStream_t st) {
  if (s.B * s.H == 0) return hipSuccess;
  int G = 1, cps = 1;
  hipError_t e = launch_gla_state(s, k, v, la, ws, &G, &cps, st);
  if (e != hipSuccess) return e;
  const int BH = s.B * s.H;
  const float* ws_state = (const float*)ws;
  const float* ws_gamma = ws_state ? ws_state + (size_t)BH * (G - 1) * kD * kD : nullptr;
  const bool sep = qw != nullptr;
  const void* qw_ = sep ? qw : q;
  const void* kw_ = sep ? kw : k;
  auto go = [&](auto kernel_launch) {
    kernel_launch(s, q, k, qw_, kw_, v, la, mk, mv, h0, ws_state, ws_gamma, o, hT, ring_k,
                  ring_v, cps, G, st);
  };
  if (s.gate == 1)
    sep ? go(launch_fused_kernel<true, bf16>) : go(launch_fused_kernel<false, bf16>);
  else
    sep ? go(launch_fused_kernel<true, float>) : go(launch_fused_kernel<false, float>);
  return hipGetLastError();
}

}  // namespace lz
