// Chunked gated linear attention forward for gfx950.
//
// Computes, per head, o_t = q_t S_t with S_t = diag(alpha_t) S_{t-1} + k_t^T v_t
// (state update of "Lizard: An Efficient Linearization Framework for Large
// Language Models", gist.science summary, section 2(a)).  Following the idea of
// that page's section 2(c), the cumulative gate is folded into q and k in log
// space so that every chunk's work is a matrix-core product; the page's own
// kernel targets other hardware, so the blocking below is this library's own.
//
// One work-group owns one head and 64 value columns and walks the 64-token
// chunks in order, keeping its 128 x 64 fp32 state slice in registers.
// Per chunk c with tokens t0..t0+63 and b_t = log2-gate cumsum inside the chunk:
//   inter  O += (q_t * 2^{b_t}) S_c                     (state entering the chunk)
//   intra  O += A V,  A_ts = sum_ch q_t k_s 2^{b_t - b_s}  for s <= t in the chunk
//   state  S_{c+1} = diag(2^{b_last}) S_c + (k_s * 2^{b_last - b_s})^T V
// Intra scores use 16-token sub-blocks: for query block i the exponent is split
// at the block's midpoint R_i, 2^{b_t - R_i} * 2^{R_i - b_s}; off-diagonal blocks
// (j < i) carry the extra per-channel factor 2^{R_i - R_j} <= 1 on the q side.
// Every factor is then bounded by 2^{8 |log2 alpha|max} inside a 16-token block,
// so extreme gates neither overflow nor lose the diagonal terms.
#include "common.hpp"
#include "kernels.hpp"

namespace lz {
namespace {

constexpr int kC = 64;    // chunk
constexpr int kBV = 64;   // value columns per work-group (16 per wave)

__host__ __device__ constexpr int blk_i(int b) { return b == 0 ? 0 : b < 3 ? 1 : b < 6 ? 2 : 3; }
__host__ __device__ constexpr int blk_j(int b) { return b - blk_i(b) * (blk_i(b) + 1) / 2; }
__host__ __device__ constexpr int blk_of(int i, int j) { return i * (i + 1) / 2 + j; }

template <typename T, int DK>
struct FwdSmem {
  static constexpr int DKP = DK + 8;
  static constexpr int CP = kC + 8;
  T qgs[10][16][DKP];  // gated q for score block (i, j): q_t 2^{b_t-R_i} 2^{R_i-R_j}
  T kg[kC][DKP];       // k_s 2^{R_j - b_s}
  T qh[kC][DKP];       // q_t 2^{b_t}
  T khT[DK][CP];       // (k_s 2^{b_last - b_s})^T
  T vT[kBV][CP];       // v^T for this work-group's columns
  T a[kC][CP];         // masked intra scores A[t][s]
  float tot[4][DK];    // per-quarter sums of log2 gates
  float mid[4][DK];    // quarter-local cumsum at the quarter's row 7
  float decay[DK];     // 2^{b_last}
};

// CPT channels of one row as fp32.
template <typename T, int CPT> struct RowIn;
template <> struct RowIn<bf16, 2> {
  bf16x2 x;
  __device__ void load(const bf16* p) { x = *reinterpret_cast<const bf16x2*>(p); }
  __device__ void zero() { x = bf16x2{(bf16)0.f, (bf16)0.f}; }
  __device__ float operator[](int i) const { return (float)x[i]; }
};
template <> struct RowIn<bf16, 1> {
  bf16 x;
  __device__ void load(const bf16* p) { x = *p; }
  __device__ void zero() { x = (bf16)0.f; }
  __device__ float operator[](int) const { return (float)x; }
};
template <> struct RowIn<float, 1> {
  float x;
  __device__ void load(const float* p) { x = *p; }
  __device__ void zero() { x = 0.f; }
  __device__ float operator[](int) const { return x; }
};
template <int CPT> struct LaIn;
template <> struct LaIn<2> {
  f32x2 x;
  __device__ void load(const float* p) { x = *reinterpret_cast<const f32x2*>(p); }
  __device__ void zero() { x = f32x2{0.f, 0.f}; }
  __device__ float operator[](int i) const { return x[i]; }
};
template <> struct LaIn<1> {
  float x;
  __device__ void load(const float* p) { x = *p; }
  __device__ void zero() { x = 0.f; }
  __device__ float operator[](int) const { return x; }
};

template <typename T, int DK>
__global__ __launch_bounds__(256, 1) void gla_fwd_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ la, const float* __restrict__ h0, T* __restrict__ o,
    float* __restrict__ hT, int T_len, int DV, int accumulate) {
  constexpr int NCB = DK / 16;  // 16-row blocks of the state
  constexpr int CPT = DK / 64;  // gating channels per lane
  constexpr int KS = DK / 32;   // contraction steps over channels
  typedef typename Frag<T>::type F;
  __shared__ FwdSmem<T, DK> sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int bh = blockIdx.y;
  const int n0 = blockIdx.x * kBV;
  const int ncol = n0 + wave * 16;          // first global value column of this wave
  const size_t qk_base = (size_t)bh * T_len * DK;
  const size_t v_base = (size_t)bh * T_len * DV;
  const size_t s_base = (size_t)bh * DK * DV;

  // State slice S[16cb + 4g + r][ncol + r16] in accumulator layout.
  f32x4 S[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      S[cb][r] = h0 ? h0[s_base + (size_t)(16 * cb + 4 * g + r) * DV + ncol + r16] : 0.f;

  // Score blocks (0,1) and (2,3) lie above the diagonal; they are read by the
  // paired contraction steps and must stay zero.
  for (int e = tid; e < 2 * 16 * 16; e += 256) {
    int blkz = e >> 8, t = (e >> 4) & 15, s = e & 15;
    sm.a[32 * blkz + t][32 * blkz + 16 + s] = to_t<T>(0.f);
  }

  const int quarter = wave;       // gating rows 16*quarter .. +15
  const int c0 = lane * CPT;      // gating channels c0 .. c0+CPT-1
  const int vcp = tid & 31, vrg = tid >> 5;  // v loader: columns 2*vcp, rows 8*vrg..

  RowIn<T, CPT> pq[16], pk[16];
  LaIn<CPT> pla[16];
  T pv[8][2];

  auto load_chunk = [&](int ch) {
    const int t0 = ch * kC;
    const int nv = min(kC, T_len - t0);
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int t = 16 * quarter + rr;
      if (t < nv) {
        const size_t off = qk_base + (size_t)(t0 + t) * DK + c0;
        pq[rr].load(q + off);
        pk[rr].load(k + off);
        pla[rr].load(la + off);
      } else {
        pq[rr].zero();
        pk[rr].zero();
        pla[rr].zero();
      }
    }
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const int t = 8 * vrg + rr;
      if (t < nv) {
        const T* p = v + v_base + (size_t)(t0 + t) * DV + n0 + 2 * vcp;
        pv[rr][0] = p[0];
        pv[rr][1] = p[1];
      } else {
        pv[rr][0] = to_t<T>(0.f);
        pv[rr][1] = to_t<T>(0.f);
      }
    }
  };

  const int nchunks = (T_len + kC - 1) / kC;
  if (nchunks > 0) load_chunk(0);

  for (int ch = 0; ch < nchunks; ++ch) {
    const int t0 = ch * kC;
    const int nv = min(kC, T_len - t0);

    // ---- take this chunk's inputs, start loading the next chunk
    float bq[16][CPT], qf[16][CPT], kf[16][CPT];
    float run[CPT];
#pragma unroll
    for (int x = 0; x < CPT; ++x) run[x] = 0.f;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr)
#pragma unroll
      for (int x = 0; x < CPT; ++x) {
        run[x] += pla[rr][x] * kLog2e;
        bq[rr][x] = run[x];
        qf[rr][x] = pq[rr][x];
        kf[rr][x] = pk[rr][x];
      }
    T cv[8][2];
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) { cv[rr][0] = pv[rr][0]; cv[rr][1] = pv[rr][1]; }
    if (ch + 1 < nchunks) load_chunk(ch + 1);

#pragma unroll
    for (int x = 0; x < CPT; ++x) {
      sm.tot[quarter][c0 + x] = run[x];
      sm.mid[quarter][c0 + x] = bq[7][x];
    }
    __syncthreads();  // (1) quarter totals visible; previous chunk's LDS reads done

    // ---- gated operands
#pragma unroll
    for (int x = 0; x < CPT; ++x) {
      const int c = c0 + x;
      float pre = 0.f, blast = 0.f, prej[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        prej[j] = blast;
        blast += sm.tot[j][c];
      }
      pre = prej[quarter];
      const float Ri = sm.mid[quarter][c] + pre;
      const float eRi = exp2_fast(Ri);
      const float eKh = exp2_fast(blast - Ri);
      float vij[3];
#pragma unroll
      for (int j = 0; j < 3; ++j)
        vij[j] = (j < quarter) ? exp2_fast(Ri - (sm.mid[j][c] + prej[j])) : 0.f;
      if (quarter == 0) sm.decay[c] = exp2_fast(blast);
      T khcol[16];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int t = 16 * quarter + rr;
        const float b = bq[rr][x] + pre;
        const float eq = exp2_fast(b - Ri);
        const float ek = exp2_fast(Ri - b);
        const float qg = qf[rr][x] * eq;
        const float kg = kf[rr][x] * ek;
        sm.qgs[blk_of(quarter, quarter)][rr][c] = to_t<T>(qg);
#pragma unroll
        for (int j = 0; j < 3; ++j)
          if (j < quarter) sm.qgs[blk_of(quarter, j)][rr][c] = to_t<T>(qg * vij[j]);
        sm.kg[t][c] = to_t<T>(kg);
        sm.qh[t][c] = to_t<T>(qg * eRi);
        khcol[rr] = to_t<T>(kg * eKh);
      }
      *reinterpret_cast<F*>(&sm.khT[c][16 * quarter]) = *reinterpret_cast<F*>(&khcol[0]);
      *reinterpret_cast<F*>(&sm.khT[c][16 * quarter + 8]) = *reinterpret_cast<F*>(&khcol[8]);
    }
    {
      T c0v[8], c1v[8];
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) { c0v[rr] = cv[rr][0]; c1v[rr] = cv[rr][1]; }
      *reinterpret_cast<F*>(&sm.vT[2 * vcp][8 * vrg]) = *reinterpret_cast<F*>(&c0v[0]);
      *reinterpret_cast<F*>(&sm.vT[2 * vcp + 1][8 * vrg]) = *reinterpret_cast<F*>(&c1v[0]);
    }
    __syncthreads();  // (2) operands ready

    // ---- intra scores (transposed blocks A^T[s][t]), masked, to LDS as A[t][s]
#pragma unroll
    for (int bi = 0; bi < 3; ++bi) {
      const int blk = wave + 4 * bi;
      if (blk < 10) {
        const int i = blk_i(blk), j = blk_j(blk);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < KS; ++p) {
          F af = ld8<T>(&sm.kg[16 * j + r16][32 * p + 8 * g]);
          F bf = ld8<T>(&sm.qgs[blk][r16][32 * p + 8 * g]);
          mma(acc, af, bf);
        }
        if (i == j) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (4 * g + r > r16) acc[r] = 0.f;
        }
        st4<T>(&sm.a[16 * i + r16][16 * j + 4 * g], acc);
      }
    }

    // ---- inter: O^T[n][t] = sum_c S[c][n] qh[t][c]  (state entering the chunk)
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
        F bf = ld8<T>(&sm.vT[16 * wave + r16][32 * p + 8 * g]);
        mma(S[cb], af, bf);
      }
    }
    __syncthreads();  // (3) scores ready

    // ---- intra: O^T[n][t] += sum_s vT[n][s] A[t][s]
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
#pragma unroll
      for (int p = 0; p <= qb / 2; ++p) {
        F af = ld8<T>(&sm.vT[16 * wave + r16][32 * p + 8 * g]);
        F bf = ld8<T>(&sm.a[16 * qb + r16][32 * p + 8 * g]);
        mma(O[qb], af, bf);
      }
    }

    // ---- store O[t][ncol + 4g .. +3]
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const int t = 16 * qb + r16;
      if (t < nv) {
        T* ptr = o + v_base + (size_t)(t0 + t) * DV + ncol + 4 * g;
        f32x4 val = O[qb];
        if (accumulate) val += ld4f<T>(ptr);
        st4<T>(ptr, val);
      }
    }
  }

  if (hT) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        hT[s_base + (size_t)(16 * cb + 4 * g + r) * DV + ncol + r16] = S[cb][r];
  }
}

template <typename T>
__global__ void state_copy_kernel(const float* __restrict__ h0, float* __restrict__ hT, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) hT[i] = h0 ? h0[i] : 0.f;
}

template <typename T, int DK>
hipError_t launch_typed(const Shape& s, const void* q, const void* k, const void* v,
                        const float* la, const float* h0, void* o, float* hT, int acc,
                        hipStream_t st) {
  dim3 grid(s.dv / kBV, s.B * s.H);
  hipLaunchKernelGGL((gla_fwd_kernel<T, DK>), grid, dim3(256), 0, st, (const T*)q, (const T*)k,
                     (const T*)v, la, h0, (T*)o, hT, s.T, s.dv, acc);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_state_copy(const Shape& s, const float* h0, float* hT, hipStream_t st) {
  size_t n = (size_t)s.B * s.H * s.dk * s.dv;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(state_copy_kernel<float>, dim3((n + 255) / 256), dim3(256), 0, st, h0, hT, n);
  return hipGetLastError();
}

hipError_t launch_gla_fwd(const Shape& s, const void* q, const void* k, const void* v,
                          const float* la, const float* h0, void* o, float* hT, int accumulate,
                          hipStream_t st) {
  if (s.T == 0) return hT ? launch_state_copy(s, h0, hT, st) : hipSuccess;
  if (s.dtype == 1) {
    if (s.dk == 128) return launch_typed<bf16, 128>(s, q, k, v, la, h0, o, hT, accumulate, st);
    return launch_typed<bf16, 64>(s, q, k, v, la, h0, o, hT, accumulate, st);
  }
  return launch_typed<float, 64>(s, q, k, v, la, h0, o, hT, accumulate, st);
}

}  // namespace lz
