// Device helpers shared by the gfx950 kernels: element types, 16x16 matrix-core
// tiles and their register layouts.
//
// Every matrix product here is a chain of 16x16 output tiles D += A * B with a
// contraction length of 32 per step:
//   bf16: one v_mfma_f32_16x16x32_bf16
//   fp32: eight v_mfma_f32_16x16x4_f32 (one per contraction sub-slice)
// Both use the same "fragment" layout, so kernels are written once:
//   lane l = 16*g + r (r = 0..15, g = 0..3)
//   A fragment: row r of A, eight contraction indices K(g, 0..7)
//   B fragment: column r of B, the same eight contraction indices K(g, 0..7)
//   accumulator: column r of D, rows 4*g + 0..3
// Any fixed map K(g, i) works as long as A and B use the same one; kernels use
// either K = 8g + i (contiguous) or the "split" map K = 4g + i for i < 4 and
// 16 + 4g + (i-4) otherwise, which is exactly what an accumulator tile pair
// holds and so lets a product's result feed the next product without moving.
#pragma once
#include <type_traits>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lz {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Hardware base-2 exponential (v_exp_f32).  Arguments are log2-domain values.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

template <typename T> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 type; };
template <> struct Frag<float> { typedef f32x8 type; };

__device__ __forceinline__ void mma(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], acc, 0, 0, 0);
}

template <typename T> __device__ __forceinline__ T to_t(float x);
template <> __device__ __forceinline__ bf16 to_t<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ float to_t<float>(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f(float x) { return x; }

// 8 contiguous elements (16 B for bf16, 32 B for fp32).
template <typename T>
__device__ __forceinline__ typename Frag<T>::type ld8(const T* p) {
  return *reinterpret_cast<const typename Frag<T>::type*>(p);
}

// Split-map fragment: elements p[0..3] then p[16..19].
template <typename T>
__device__ __forceinline__ typename Frag<T>::type ld4x2(const T* p);
template <> __device__ __forceinline__ bf16x8 ld4x2<bf16>(const bf16* p) {
  bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
  bf16x4 b = *reinterpret_cast<const bf16x4*>(p + 16);
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
template <> __device__ __forceinline__ f32x8 ld4x2<float>(const float* p) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 16);
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Fragment from an accumulator tile pair (rows 4g..4g+3 of tile a, then of tile b).
template <typename T>
__device__ __forceinline__ typename Frag<T>::type pack_acc(const f32x4& a, const f32x4& b);
template <> __device__ __forceinline__ bf16x8 pack_acc<bf16>(const f32x4& a, const f32x4& b) {
  return bf16x8{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3],
                (bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
}
template <> __device__ __forceinline__ f32x8 pack_acc<float>(const f32x4& a, const f32x4& b) {
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Store 4 values (one accumulator column slice) as 4 consecutive elements.
template <typename T> __device__ __forceinline__ void st4(T* p, const f32x4& x);
template <> __device__ __forceinline__ void st4<bf16>(bf16* p, const f32x4& x) {
  *reinterpret_cast<bf16x4*>(p) = bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
}
template <> __device__ __forceinline__ void st4<float>(float* p, const f32x4& x) {
  *reinterpret_cast<f32x4*>(p) = x;
}
template <typename T> __device__ __forceinline__ f32x4 ld4f(const T* p);
template <> __device__ __forceinline__ f32x4 ld4f<bf16>(const bf16* p) {
  bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
template <> __device__ __forceinline__ f32x4 ld4f<float>(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}

// Work-group barrier that waits only for this wave's LDS traffic.  The plain
// __syncthreads() also drains outstanding global loads, which would stall the
// next-chunk prefetch at every barrier.  Global data is never exchanged
// through these barriers, only LDS.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Raw buffer view of one tensor slice.  Reads at byte offsets >= `bytes` return
// zero, so ragged tails need neither clamping nor branches, and constant row
// offsets fold into the instruction's immediate field.
typedef unsigned int u32;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
struct U2 {
  u32 a, b;
};
struct Buf {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ Buf(const void* base, u32 bytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                            0x00020000)) {}
  __device__ __forceinline__ u32 ld32(u32 off) const {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  }
  // 8 bytes as two scalars.
  __device__ __forceinline__ U2 ld64(u32 off) const {
    return U2{__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0),
              __builtin_amdgcn_raw_buffer_load_b32(r, off + 4, 0, 0)};
  }
  // 16 bytes.  Elements are read out through as_f() / bf_at(), never by
  // __builtin_bit_cast on a vector element: hipcc for gfx950 lowers a bit_cast
  // whose operand is an ext-vector element to element 0 of that vector.
  __device__ __forceinline__ u32x4 ld128(u32 off) const {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  }
};
// Bit patterns to fp32, from a scalar (see the note on Buf::ld128).
__device__ __forceinline__ float as_f(u32 x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ float bf_lo(u32 x) { return as_f(x << 16); }
__device__ __forceinline__ float bf_hi(u32 x) { return as_f(x & 0xffff0000u); }
// acc + lo(x) lo(y) + hi(x) hi(y) for two packed bf16 pairs (one dot instruction)
__device__ __forceinline__ float dot2_bf16(u32 x, u32 y, float acc) {
  typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2v, x), __builtin_bit_cast(bf2v, y),
                                         acc, false);
}
// bf16 element c (0..7) of a 16-byte word as fp32
__device__ __forceinline__ float bf_at(const u32x4& v, int c) {
  const u32 w = v[c >> 1];
  return (c & 1) ? bf_hi(w) : bf_lo(w);
}
// bf16 element c (0..3) of an 8-byte word as fp32
__device__ __forceinline__ float bf_at(const u32x2& v, int c) {
  const u32 w = v[c >> 1];
  return (c & 1) ? bf_hi(w) : bf_lo(w);
}
// fp32 element c (0..3)
__device__ __forceinline__ float f_at(const u32x4& v, int c) {
  const u32 w = v[c];
  return as_f(w);
}
// two fp32 values rounded to a packed bf16 pair (a in the low half)
__device__ __forceinline__ u32 pack_bf2(float a, float b) {
  const bf16x2 p = {(bf16)a, (bf16)b};
  return __builtin_bit_cast(u32, p);
}

// Two consecutive elements as fp32.
__device__ __forceinline__ f32x2 unpack2(u32 x, bf16) {
  return f32x2{__builtin_bit_cast(float, x << 16), __builtin_bit_cast(float, x & 0xffff0000u)};
}
__device__ __forceinline__ f32x2 unpack2(U2 x, float) {
  return f32x2{__builtin_bit_cast(float, x.a), __builtin_bit_cast(float, x.b)};
}
template <typename T> struct Pair;                  // raw storage of two elements
template <> struct Pair<bf16> { typedef u32 type; };
template <> struct Pair<float> { typedef U2 type; };
template <typename T>
__device__ __forceinline__ typename Pair<T>::type ld_pair(const Buf& b, u32 off);
template <> __device__ __forceinline__ u32 ld_pair<bf16>(const Buf& b, u32 off) { return b.ld32(off); }
template <> __device__ __forceinline__ U2 ld_pair<float>(const Buf& b, u32 off) { return b.ld64(off); }

// Gate inputs.  A gate is given either as log alpha (float) or as a bf16 logit
// x of the sigmoid gate alpha = sigmoid(x) of "Lizard: An Efficient
// Linearization Framework for Large Language Models" (gist.science summary,
// section 2(a), the learnable gate).  The kernels work with log2 alpha:
//   log alpha:  log2 alpha = log_alpha * log2(e)
//   logit:      log2 sigmoid(x) = min(x, 0) log2(e) - log2(1 + 2^{-|x| log2(e)})
// (the second form never exponentiates a positive number).  Per token the log2
// gate is held at or above kMinLog2Gate: the 16-token sub-block references keep
// every gated operand within 2^{8 |log2 alpha|} of its token, which must stay
// inside the bf16/fp32 exponent range (2^127) with room for the operand itself.
// A gate below 2^-15 (alpha < 3.1e-5, a state all but reset at that token) is
// taken as 2^-15: the older state then enters with a weight of at most 2^-15
// instead of alpha, which moves an output by at most 2^-15 |q|_1 max|S|.
constexpr float kMinLog2Gate = -15.f;
// The same without the floor.  Every log2 gate is <= 0, so a run of tokens
// whose summed log2 gate stays at or above kMinLog2Gate holds no token below
// the floor: a kernel may sum these and take the floored form only for a run
// whose sum falls below it.
__device__ __forceinline__ float gate_log2_nofloor(float la, float) { return la * kLog2e; }
__device__ __forceinline__ float gate_log2_nofloor(float x, bf16) {
  const float t = x * kLog2e;
  return fminf(t, 0.f) - log2_fast(1.f + exp2_fast(-fabsf(t)));
}
// (a compare and select, not fmaxf: a NaN gate stays NaN and reaches the
// outputs, where fmaxf would return the floor)
template <typename GT>
__device__ __forceinline__ float gate_log2(float v, GT) {
  const float t = gate_log2_nofloor(v, GT());
  return t < kMinLog2Gate ? kMinLog2Gate : t;
}
// d log(alpha) / dx = sigmoid(-x) = 1 / (1 + 2^{x log2(e)}) for a logit x; 1 for
// log alpha itself.
__device__ __forceinline__ float gate_dlog(float, float) { return 1.f; }
__device__ __forceinline__ float gate_dlog(float x, bf16) {
  return __builtin_amdgcn_rcpf(1.f + exp2_fast(x * kLog2e));
}

// Token rows of one (sequence, head) pair.  Dense batches [B, H, T, d]: T rows
// from (b H + h) T.  Packed batches [H, N, d]: sequence b is rows cu[b] ..
// cu[b+1]-1 of head h's N rows (clamped into [0, N], and its length to T).
struct SeqRows {
  size_t row0;
  int len;
};
__device__ __forceinline__ SeqRows seq_rows(const int* cu, int N, int T, int H, int bh) {
  if (!cu) return SeqRows{(size_t)bh * T, T};
  const int b = bh / H, h = bh - b * H;
  const int s0 = min(max(cu[b], 0), N);
  const int s1 = min(max(cu[b + 1], s0), N);
  return SeqRows{(size_t)h * N + s0, min(s1 - s0, T)};
}

// Log2 gate of a token row: rows at or past the sequence end (loaded as zero
// bytes) must not decay.  A float log gate of 0 already means alpha = 1; a
// logit of 0 would mean alpha = 1/2, so logit rows there are masked to 0.
template <typename GT>
__device__ __forceinline__ float gate_row(float log2_gate, bool valid) {
  if constexpr (sizeof(GT) == 2)
    return valid ? log2_gate : 0.f;
  else
    return log2_gate;
}

// Eight consecutive gate inputs of one token: two 16-byte words of float log
// alpha, or one 16-byte word of bf16 logits.
template <typename G>
struct Gate8 {
  static constexpr int kWords = sizeof(G) / 2;
  u32x4 w[kWords];
  // elem: element offset from the buffer base
  __device__ __forceinline__ void load(const Buf& b, u32 elem) {
#pragma unroll
    for (int i = 0; i < kWords; ++i) w[i] = b.ld128(elem * (u32)sizeof(G) + 16u * i);
  }
  __device__ __forceinline__ float log2_at(int c) const {
    return gate_log2(raw_at(c), G());
  }
  __device__ __forceinline__ float log2_nofloor_at(int c) const {
    return gate_log2_nofloor(raw_at(c), G());
  }
  __device__ __forceinline__ float raw_at(int c) const {
    if constexpr (sizeof(G) == 4)
      return f_at(w[c >> 2], c & 3);
    else
      return bf_at(w[0], c);
  }
};

// Two fp32 values as a packed pair of T (one LDS store).
template <typename T> __device__ __forceinline__ void st_pair(T* p, float a, float b);
template <> __device__ __forceinline__ void st_pair<bf16>(bf16* p, float a, float b) {
  *reinterpret_cast<bf16x2*>(p) = bf16x2{(bf16)a, (bf16)b};
}
template <> __device__ __forceinline__ void st_pair<float>(float* p, float a, float b) {
  *reinterpret_cast<f32x2*>(p) = f32x2{a, b};
}

// Work-groups are handed to the 8 XCDs round-robin by linear id.  This maps
// linear id L to a logical index so that each XCD receives one contiguous run
// of logical indices: neighbouring tiles (which share K/V rows) then run on the
// same XCD and meet in its L2.  A bijection on [0, n).
__device__ __forceinline__ int xcd_remap(int L, int n) {
  constexpr int kXcd = 8;
  const int xcd = L % kXcd, idx = L / kXcd;
  const int base = n / kXcd, rem = n % kXcd;
  return xcd * base + min(xcd, rem) + idx;
}

// LDS tile layouts.  A "granule" is 8 consecutive elements (one matrix-core
// fragment: 16 bytes of bf16, 32 of fp32).  Tiles are stored unpadded with the
// granules of each row permuted by a row-dependent XOR, chosen so that the
// fragment reads (16 consecutive rows, one granule column) and the staging
// writes of every kernel hit distinct banks.
template <int GR>  // granules per row
__device__ __forceinline__ int swz_gran(int row, int gran) {
  if constexpr (GR == 4) {
    return gran ^ ((row ^ (row >> 2)) & 3);
  } else if constexpr (GR == 8) {
    return (gran ^ row ^ (row >> 3)) & 7;
  } else if constexpr (GR == 16) {
    return gran ^ ((row ^ (row >> 2)) & 15);
  } else {
    return gran ^ ((row ^ (row >> 3)) & 15);
  }
}
// element offset of (row, col) in a swizzled tile of GR granules per row
template <int GR>
__device__ __forceinline__ int swz_at(int row, int col) {
  return row * (8 * GR) + swz_gran<GR>(row, col >> 3) * 8 + (col & 7);
}
// Tile with 64-element rows whose granules are permuted by (row >> 1) & 7.  A
// fragment read (rows 16a..16a+15, one granule column) touches 16 distinct
// bank groups, and the permutation does not depend on a, so a lane's offset
// for rows 16a + r is 1024 a plus a per-lane base (an instruction immediate).
__device__ __forceinline__ int swz64(int row, int col) {
  return row * 64 + ((((col >> 3) ^ (row >> 1)) & 7) << 3) + (col & 7);
}
// Position of element c of a 32-element group in "split" order: quads
// 4g..4g+3 and 16+4g..16+4g+3 sit next to each other, so the granule at
// position 8g holds exactly lane group g's split-map fragment.
__host__ __device__ constexpr int split_pos(int c) {
  return (c & ~31) | (((c & 15) >> 2) << 3) | ((c & 16) >> 2) | (c & 3);
}

// ---- lane exchange and packing
// DPP moves within rows of 16 lanes (zero where the source leaves the row).
template <int N>
__device__ __forceinline__ float dpp_shr(float x) {  // lane i <- lane i - N
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + N, 0xf, 0xf, true));
}
template <int N>
__device__ __forceinline__ float dpp_shl(float x) {  // lane i <- lane i + N
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x100 + N, 0xf, 0xf, true));
}
template <int N>
__device__ __forceinline__ float dpp_bcast(float x) {  // every lane <- lane N of its row
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + N, 0xf, 0xf, false));
}
__device__ __forceinline__ u32 dpp_swap1(u32 x) {  // exchange with the neighbouring lane
  return (u32)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xf, 0xf, false);
}
// bf16 pairs: low halves of (a, b), high halves of (a, b)
__device__ __forceinline__ u32 lo2(u32 a, u32 b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ u32 hi2(u32 a, u32 b) { return (a >> 16) | (b & 0xffff0000u); }
__device__ __forceinline__ bf16x8 as_bf8(const u32x4& x) { return __builtin_bit_cast(bf16x8, x); }

// 8 bytes through a buffer view (elements read out as with Buf::ld128)
__device__ __forceinline__ u32x2 ld64v(const Buf& b, u32 off) {
  return __builtin_amdgcn_raw_buffer_load_b64(b.r, off, 0, 0);
}

// Four consecutive gate inputs of one token (float log alpha or bf16 logits).
template <typename G>
struct Gate4 {
  typename std::conditional<sizeof(G) == 4, u32x4, u32x2>::type w;
  __device__ __forceinline__ void load(const Buf& b, u32 elem) {
    if constexpr (sizeof(G) == 4)
      w = b.ld128(elem * 4);
    else
      w = ld64v(b, elem * 2);
  }
  __device__ __forceinline__ float raw_at(int r) const {
    if constexpr (sizeof(G) == 4)
      return as_f(w[r]);
    else
      return (r & 1) ? bf_hi(w[r >> 1]) : bf_lo(w[r >> 1]);
  }
  __device__ __forceinline__ float log2_at(int r) const { return gate_log2(raw_at(r), G()); }
  __device__ __forceinline__ float log2_nofloor_at(int r) const {
    return gate_log2_nofloor(raw_at(r), G());
  }
};

__device__ __forceinline__ int wave_id() {  // wave index as a scalar (uniform) value
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// Row-major [rows x D] tile, rows row0.. of `src`, into dst (leading dim ld).
// Out-of-range rows read as zero through the buffer bounds.
template <typename T>
__device__ __forceinline__ void stage_rows(T* dst, int ld, const Buf& src, int row0, int D,
                                           int rows, int tid, int nthr) {
  const int per_row = D / 8;
  for (int e = tid; e < rows * per_row; e += nthr) {
    const int r = e / per_row, c8 = (e % per_row) * 8;
    const u32 off = (u32)(((row0 + r) * D + c8) * sizeof(T));
    *reinterpret_cast<u32x4*>(dst + r * ld + c8) = src.ld128(off);
    if constexpr (sizeof(T) == 4)
      *reinterpret_cast<u32x4*>(dst + r * ld + c8 + 4) = src.ld128(off + 16);
  }
}

// Transposed tile: dst[c][r] = src[row0 + r][c] for r < rows (rows % 8 == 0).
template <typename T>
__device__ __forceinline__ void stage_cols(T* dst, int ld, const Buf& src, int row0, int D,
                                           int rows, int tid, int nthr) {
  for (int e = tid; e < (rows / 8) * (D / 2); e += nthr) {
    const int cp = e % (D / 2), rg = e / (D / 2);
    typename Frag<T>::type f0, f1;
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const u32 off = (u32)(((row0 + 8 * rg + rr) * D + 2 * cp) * sizeof(T));
      const f32x2 x = unpack2(ld_pair<T>(src, off), T());
      f0[rr] = to_t<T>(x[0]);
      f1[rr] = to_t<T>(x[1]);
    }
    *reinterpret_cast<typename Frag<T>::type*>(dst + (2 * cp) * ld + 8 * rg) = f0;
    *reinterpret_cast<typename Frag<T>::type*>(dst + (2 * cp + 1) * ld + 8 * rg) = f1;
  }
}

__device__ __forceinline__ float wave_max16(float x) {  // over lanes with equal (lane & 15)
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float wave_sum16(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}
// The same two reductions with VALU lane swaps instead of LDS permutes.
// v_permlane32_swap a, b exchanges the upper 32 lanes of a with the lower 32
// lanes of b; v_permlane16_swap does the same for the odd 16-lane rows of a and
// the even rows of b.  Started from a = b = x, lane l then holds
// x[l mod 32] and x[32 + l mod 32] (respectively rows 2k and 2k+1), and every
// lane ends with the identical value.  Written as asm with both registers
// read and written: this compiler's builtins for these instructions lose the
// second result when both results feed one expression.
__device__ __forceinline__ void lane_swap32(u32& a, u32& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void lane_swap16(u32& a, u32& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float swap_max16(float x) {
  u32 a = __builtin_bit_cast(u32, x), b = a;
  lane_swap32(a, b);
  const float m = fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
  a = __builtin_bit_cast(u32, m);
  b = a;
  lane_swap16(a, b);
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float swap_sum16(float x) {
  u32 a = __builtin_bit_cast(u32, x), b = a;
  lane_swap32(a, b);
  const float m = __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
  a = __builtin_bit_cast(u32, m);
  b = a;
  lane_swap16(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// Meta-memory gradients of the window branch: fixed-order sum (deterministic)
// of per-(sequence, query tile) partials.  metap holds, for partial p = b
// ntiles + tile of head h, 2 n floats at ((b H + h) ntiles + tile) 2 n:
// entries e < n belong to dmeta_k [H, n], the rest to dmeta_v (n = M d).
struct MetaReduceArgs {
  const float* metap = nullptr;
  float* dmk = nullptr;
  float* dmv = nullptr;
  int B = 0, H = 0, ntiles = 0, n = 0;  // n = 0: nothing to reduce
};

// One block sums the 64 entries of strip `strip` of head h: its NG groups of
// 64 threads sum interleaved NG-ths of the B ntiles partials (coalesced, up to
// 16 loads in flight per thread), then a fixed tree through `part` (NG x 64
// floats of LDS) adds the NG sums.  Every thread of the block calls it.
template <int NG>
__device__ __forceinline__ void meta_reduce_strip(const MetaReduceArgs& a, int h, int strip,
                                                  float (*part)[64]) {
  const int i = threadIdx.x & 63, grp = threadIdx.x >> 6;
  const int e = strip * 64 + i, n = a.n;
  const int np = a.B * a.ntiles;
  float s = 0.f;
  if (e < 2 * n) {
    auto at = [&](int p) {
      const int b = p / a.ntiles, tl = p - b * a.ntiles;
      return a.metap[(((size_t)(b * a.H + h)) * a.ntiles + tl) * 2 * n + e];
    };
    int p = grp;
    for (; p + 15 * NG < np; p += 16 * NG) {
      float x[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) x[u] = at(p + NG * u);
#pragma unroll
      for (int u = 0; u < 16; ++u) s += x[u];
    }
    for (; p < np; p += NG) s += at(p);
  }
  part[grp][i] = s;
  __syncthreads();
#pragma unroll
  for (int w = NG / 2; w >= 1; w >>= 1) {
    if (grp < w) part[grp][i] += part[grp + w][i];
    __syncthreads();
  }
  if (grp == 0 && e < 2 * n) {
    if (e < n) a.dmk[(size_t)h * n + e] = part[0][i];
    else a.dmv[(size_t)h * n + e - n] = part[0][i];
  }
}

}  // namespace lz
