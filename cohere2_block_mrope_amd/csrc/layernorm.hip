// Weight-only LayerNorm computed in fp32 ("Text decoder forward" of the mlxcel
// Compass issue: LayerNorm(h; layer_norm_eps), weight only, no bias, computed in
// f32): a = (x - mean) / sqrt(var + eps) * w with the biased variance.
//
// One 64-lane wave per row, four rows per workgroup. The row is read once into
// registers (16-byte loads), mean and variance are two passes over registers with
// wave reductions, and the normalized row is written in the input's dtype: bf16
// rows become the bf16 A operand of the projection GEMM.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace compass {
namespace {

constexpr int kRowsPerBlock = 4;

// VPL: values per lane held in registers (D <= 64 * VPL); bf16 loads are 8 wide.
// STATS: write only the row's (mean, rstd) to stats[row] (the fused projection GEMM then
// normalizes its A tiles itself, with the same values).
template <typename T, int VPL, bool STATS = false>
__global__ __launch_bounds__(256) void layernorm_kernel(const T* __restrict__ x,
                                                        const T* __restrict__ w, float eps,
                                                        T* __restrict__ a, int rows, int D, long long ldx,
                                                        float2* __restrict__ stats = nullptr) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const T* xr = x + (size_t)row * ldx;
  T* ar = a + (size_t)row * D;
  constexpr int V = (sizeof(T) == 2) ? 8 : 4;  // elements per 16-byte vector
  constexpr int NV = (VPL + V - 1) / V;        // vectors per lane
  float v[NV * V];
  // Small rows also fetch the weight up front, so its loads overlap the row's instead of
  // following the two reductions.
  using W16 = typename std::conditional<sizeof(T) == 2, u32x4_t, float4>::type;
  constexpr bool kEarlyW = NV <= 8 && !STATS;
  W16 wpre[kEarlyW ? NV : 1];
  if constexpr (kEarlyW) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = (i * 64 + lane) * V;
      if (e < D) wpre[i] = *reinterpret_cast<const W16*>(w + e);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = (i * 64 + lane) * V;
#pragma unroll
    for (int j = 0; j < V; ++j) v[i * V + j] = 0.f;
    if (e < D) {
      if constexpr (sizeof(T) == 2) {
        u32x4_t raw = *reinterpret_cast<const u32x4_t*>(xr + e);
        const uint32_t r4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[i * V + 2 * j] = __uint_as_float(r4[j] << 16);
          v[i * V + 2 * j + 1] = __uint_as_float(r4[j] & 0xffff0000u);
        }
      } else {
        float4 raw = *reinterpret_cast<const float4*>(xr + e);
        v[i * V + 0] = raw.x; v[i * V + 1] = raw.y; v[i * V + 2] = raw.z; v[i * V + 3] = raw.w;
      }
    }
#pragma unroll
    for (int j = 0; j < V; ++j) s += v[i * V + j];
  }
  const float mean = wave_sum(s) / (float)D;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = (i * 64 + lane) * V;
    if (e < D) {
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const float d = v[i * V + j] - mean;
        q += d * d;
      }
    }
  }
  const float var = wave_sum(q) / (float)D;
  const float rstd = 1.0f / sqrtf(var + eps);
  if constexpr (STATS) {
    if (lane == 0) stats[row] = make_float2(mean, rstd);
    return;
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = (i * 64 + lane) * V;
    if (e >= D) continue;
    W16 wr;
    if constexpr (kEarlyW) wr = wpre[i];
    else wr = *reinterpret_cast<const W16*>(w + e);
    if constexpr (sizeof(T) == 2) {
      const uint32_t w4[4] = {wr.x, wr.y, wr.z, wr.w};
      uint32_t o4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float w0 = __uint_as_float(w4[j] << 16), w1 = __uint_as_float(w4[j] & 0xffff0000u);
        o4[j] = pack_bf2((v[i * V + 2 * j] - mean) * rstd * w0,
                         (v[i * V + 2 * j + 1] - mean) * rstd * w1);
      }
      __builtin_nontemporal_store(u32x4_t{o4[0], o4[1], o4[2], o4[3]}, reinterpret_cast<u32x4_t*>(ar + e));
    } else {
      float4 o;
      o.x = (v[i * V + 0] - mean) * rstd * wr.x;
      o.y = (v[i * V + 1] - mean) * rstd * wr.y;
      o.z = (v[i * V + 2] - mean) * rstd * wr.z;
      o.w = (v[i * V + 3] - mean) * rstd * wr.w;
      *reinterpret_cast<float4*>(ar + e) = o;
    }
  }
}

template <typename T>
hipError_t launch_t(const void* x, long long ldx, const void* w, float eps, void* a, int rows, int D,
                    hipStream_t s) {
  const dim3 grid((rows + kRowsPerBlock - 1) / kRowsPerBlock);
  const T* xp = (const T*)x;
  const T* wp = (const T*)w;
  T* ap = (T*)a;
  // D is a multiple of 64 and at most 16384 (checked by the caller).
  if (D <= 64 * 8) layernorm_kernel<T, 8><<<grid, 256, 0, s>>>(xp, wp, eps, ap, rows, D, ldx);
  else if (D <= 64 * 32) layernorm_kernel<T, 32><<<grid, 256, 0, s>>>(xp, wp, eps, ap, rows, D, ldx);
  else if (D <= 64 * 64) layernorm_kernel<T, 64><<<grid, 256, 0, s>>>(xp, wp, eps, ap, rows, D, ldx);
  else layernorm_kernel<T, 256><<<grid, 256, 0, s>>>(xp, wp, eps, ap, rows, D, ldx);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ln_stats(const void* x, float eps, float2* stats, int rows, int D, hipStream_t s) {
  const dim3 grid((rows + kRowsPerBlock - 1) / kRowsPerBlock);
  const bf16_t* xp = (const bf16_t*)x;
  if (D <= 64 * 8) layernorm_kernel<bf16_t, 8, true><<<grid, 256, 0, s>>>(xp, nullptr, eps, nullptr, rows, D, D, stats);
  else if (D <= 64 * 32) layernorm_kernel<bf16_t, 32, true><<<grid, 256, 0, s>>>(xp, nullptr, eps, nullptr, rows, D, D, stats);
  else if (D <= 64 * 64) layernorm_kernel<bf16_t, 64, true><<<grid, 256, 0, s>>>(xp, nullptr, eps, nullptr, rows, D, D, stats);
  else layernorm_kernel<bf16_t, 256, true><<<grid, 256, 0, s>>>(xp, nullptr, eps, nullptr, rows, D, D, stats);
  return hipGetLastError();
}

hipError_t launch_layernorm(int dtype, const void* x, const void* w, float eps, void* a, int rows,
                            int D, hipStream_t s, long long ldx) {
  if (ldx <= 0) ldx = D;
  return dtype == 1 ? launch_t<bf16_t>(x, ldx, w, eps, a, rows, D, s)
                    : launch_t<float>(x, ldx, w, eps, a, rows, D, s);
}

}  // namespace compass
