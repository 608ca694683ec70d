// Shared device-side helpers for the gfx950 kernels: bf16 storage conversions,
// MFMA operand vector types, wave reductions. Host/device shared structs for the
// launchers live in launch.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // bf16 storage: the upper half of an fp32 bit pattern

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4_t;
// Native 16-byte vector (HIP's uint4 is a union class that defeats register promotion).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

#define LDS_PTR(T) __attribute__((address_space(3))) T*

__device__ __forceinline__ float bf2f(bf16_t v) {
  return __uint_as_float(((uint32_t)v) << 16);
}

// fp32 -> bf16, round to nearest even, NaN kept as a quiet NaN (gfx950's
// v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t f2bf(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}

// Two fp32 -> packed pair of bf16 (low half = a), one conversion instruction.
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Storage-type abstraction used by templated kernels.
template <typename T> struct Elt;
template <> struct Elt<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ float to_f(float v) { return v; }
  static __device__ __forceinline__ float from_f(float v) { return v; }
};
template <> struct Elt<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p) { return bf2f(*p); }
  static __device__ __forceinline__ float to_f(bf16_t v) { return bf2f(v); }
  static __device__ __forceinline__ bf16_t from_f(float v) { return f2bf(v); }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// silu(g) = g / (1 + e^-g) from the hardware exp2 and reciprocal (a few ulp; the
// limits g -> +inf, -inf give g and -0).
__device__ __forceinline__ float silu_f(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g));
}

// Value of lane (lane ^ 1) / (lane ^ 2) of the same quad (DPP quad permutes; every lane
// of the quad must be active).
__device__ __forceinline__ float quad_xor1(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
}

// Max / sum of x over the lane pair (l, l ^ 32) with gfx950's v_permlane32_swap (one
// VALU op, no LDS). Both lanes of a pair get bitwise the same result. The two results
// of the swap are copied to scalars before reinterpreting them: hipcc lowers
// __builtin_bit_cast applied directly to an element of the returned vector as element 0.
__device__ __forceinline__ void pair32_swap(float x, float& lo, float& hi) {
  const unsigned a = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(a, a, false, false);
  const unsigned r0 = r[0], r1 = r[1];
  lo = __builtin_bit_cast(float, r0);  // x of lane l & 31
  hi = __builtin_bit_cast(float, r1);  // x of lane (l & 31) + 32
}
__device__ __forceinline__ float pair32_max(float x) {
  float lo, hi;
  pair32_swap(x, lo, hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float pair32_sum(float x) {
  float lo, hi;
  pair32_swap(x, lo, hi);
  return lo + hi;
}

// 4 x 4 transpose inside each quad of lanes (q = lane & 3), in registers. On entry
// lane q holds rows 0..3 of column q (v[r] = X[r][q]); on exit it holds columns 0..3
// of row 2 (q & 1) + (q >> 1) (v[c] = X[row][c]). Used to turn MFMA result columns
// into row-contiguous 8- and 16-byte stores. All 64 lanes must be active.
__device__ __forceinline__ void quad_transpose(float (&v)[4], int lane) {
  const bool odd = lane & 1, hi = lane & 2;
  // Swap with lane ^ 1: even lanes keep rows 0, 1, odd lanes rows 2, 3; afterwards
  // (a0, a1) and (a2, a3) are two consecutive rows over the column pair (q & 2) + {0, 1}.
  const float r0 = quad_xor1(odd ? v[0] : v[2]);
  const float r1 = quad_xor1(odd ? v[1] : v[3]);
  const float a0 = odd ? r0 : v[0], a1 = odd ? v[2] : r0;
  const float a2 = odd ? r1 : v[1], a3 = odd ? v[3] : r1;
  // Swap with lane ^ 2: lanes q < 2 keep the first of the two rows, the others the second.
  const float p0 = quad_xor2(hi ? a0 : a2);
  const float p1 = quad_xor2(hi ? a1 : a3);
  v[0] = hi ? p0 : a0;
  v[1] = hi ? p1 : a1;
  v[2] = hi ? a2 : p0;
  v[3] = hi ? a3 : p1;
}

// The same transpose for values stored as bf16: each lane rounds its rows to bf16 in pairs
// first, so every exchange moves two values (10 VALU operations per 4 values instead of
// 18). On entry lane q holds rows 0..3 of column q; on exit the two dwords hold columns
// 0, 1 and 2, 3 (low half first) of row 2 (q & 1) + (q >> 1). All 64 lanes must be active.
__device__ __forceinline__ u32x2_t quad_transpose_bf16(const float (&v)[4], int lane) {
  const bool odd = lane & 1, hi = lane & 2;
  const uint32_t a = pack_bf2(v[0], v[1]);  // rows 0, 1 of column q
  const uint32_t b = pack_bf2(v[2], v[3]);  // rows 2, 3 of column q
  // Exchange with lane q ^ 1: even lanes keep rows 0, 1 and receive them for column q + 1,
  // odd lanes keep rows 2, 3 and receive them for column q - 1.
  const uint32_t own = odd ? b : a;
  const uint32_t rcv = (uint32_t)__builtin_amdgcn_mov_dpp((int)(odd ? a : b), 0xB1, 0xF, 0xF, false);
  // v_perm byte selects (bytes 0..3: own, 4..7: rcv): x = the lower row of the lane's pair
  // over the two columns (lower column first), y = the upper row.
  const uint32_t x = __builtin_amdgcn_perm(rcv, own, odd ? 0x01000504u : 0x05040100u);
  const uint32_t y = __builtin_amdgcn_perm(rcv, own, odd ? 0x03020706u : 0x07060302u);
  // Exchange with lane q ^ 2: lanes q < 2 keep the lower row and receive its other two
  // columns; lanes q >= 2 keep the upper row and receive its first two columns.
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)(hi ? x : y), 0x4E, 0xF, 0xF, false);
  u32x2_t o;
  o.x = hi ? r2 : x;
  o.y = hi ? y : r2;
  return o;
}

static constexpr float kLog2e = 1.4426950408889634f;
