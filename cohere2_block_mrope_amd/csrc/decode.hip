// Decode attention over a dense KV cache (one new token per row). The page's
// correction under "Acceptance criteria" of the mlxcel Compass issue keeps a dense
// cache and applies the sliding window as a mask: the query at index n = lens[b]
// sees keys n - window < j <= n on sliding layers and j <= n on full layers.
//
// The work is HBM-bound: every visible K and V row is read once. A workgroup owns one
// (row, kv head, chunk of keys) and serves all Hq / Hkv query heads of that kv head,
// so the cache is streamed once per kv head. Each key row is read by a group of
// hd / 8 lanes with 16-byte loads (a 256-byte bf16 row per 16 lanes, fully coalesced).
// Scores (prescaled by log2 e / sqrt(hd)) go through LDS for the chunk softmax; the
// chunk's unnormalized output, max and sum are written to a workspace and a second
// kernel merges the chunks of each (row, head).
#include "common.h"
#include "launch.h"

namespace compass {
namespace {

constexpr int CHUNK = 256;  // keys per workgroup (64 per wave)

template <typename T, int HD, int G>
__global__ __launch_bounds__(256) void decode_attn_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                          const T* __restrict__ v,
                                                          const int32_t* __restrict__ lens, int Hq,
                                                          int Hkv, int cap, int sliding, int window,
                                                          float scale_log2, int n_chunks,
                                                          float* __restrict__ part) {
  constexpr int VEC = 16 / sizeof(T);   // elements per 16-byte load
  constexpr int LPK = HD / VEC;         // lanes per key row
  constexpr int KPS = 64 / LPK;         // keys per wave step
  constexpr int STEPS = 64 / KPS;       // steps per wave (64 keys per wave)
  __shared__ float s_p[G][CHUNK];
  __shared__ float s_red[G][4];
  __shared__ float s_o[4][G][HD];

  const int chunk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane % LPK, kin = lane / LPK;
  const int n = lens[b];
  float* out = part + (((size_t)b * Hq + kvh * G) * n_chunks + chunk) * (HD + 2);
  const size_t head_stride = (size_t)n_chunks * (HD + 2);
  const bool row_ok = n >= 0 && n < cap;
  const int lo = sliding ? max(0, n - window + 1) : 0;
  const int kbeg = lo + chunk * CHUNK;
  const int kend = min(kbeg + CHUNK, n + 1);
  if (!row_ok || kbeg >= kend) {
    if (tid < G) {
      out[tid * head_stride + HD] = -INFINITY;
      out[tid * head_stride + HD + 1] = 0.f;
    }
    return;
  }

  // Query slices of the G heads: lane holds d in [VEC*sub, VEC*sub + VEC).
  float qv[G][VEC];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const T* qp = q + ((size_t)b * Hq + kvh * G + g) * HD + VEC * sub;
#pragma unroll
    for (int e = 0; e < VEC; ++e) qv[g][e] = Elt<T>::to_f(qp[e]);
  }

  const T* kb = k + ((size_t)b * Hkv + kvh) * cap * HD + VEC * sub;
  const T* vb = v + ((size_t)b * Hkv + kvh) * cap * HD + VEC * sub;
  u32x4_t kr[STEPS], vr[STEPS];
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int key = min(kbeg + 64 * wave + st * KPS + kin, kend - 1);
    kr[st] = *reinterpret_cast<const u32x4_t*>(kb + (size_t)key * HD);
  }
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int key = min(kbeg + 64 * wave + st * KPS + kin, kend - 1);
    vr[st] = *reinterpret_cast<const u32x4_t*>(vb + (size_t)key * HD);
  }

  auto unpack = [](const u32x4_t& r, float* f) {
    if constexpr (sizeof(T) == 2) {
      const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f[2 * j] = __uint_as_float(w[j] << 16);
        f[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
      }
    } else {
      f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y);
      f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
    }
  };

  // Scores.
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    float kf[VEC];
    unpack(kr[st], kf);
    float dot[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) d = fmaf(qv[g][e], kf[e], d);
#pragma unroll
      for (int o = 1; o < LPK; o <<= 1) d += __shfl_xor(d, o, 64);
      dot[g] = d;
    }
    const int kl = 64 * wave + st * KPS + kin;
    if (sub == 0) {
      const bool ok = kbeg + kl < kend;
#pragma unroll
      for (int g = 0; g < G; ++g) s_p[g][kl] = ok ? dot[g] * scale_log2 : -INFINITY;
    }
  }
  __syncthreads();
  // Chunk softmax: max and sum per head over the CHUNK scores (one per thread).
  float sv[G], mx[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    sv[g] = s_p[g][tid];
    const float wm = wave_max(sv[g]);
    if (lane == 0) s_red[g][wave] = wm;
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) mx[g] = fmaxf(fmaxf(s_red[g][0], s_red[g][1]), fmaxf(s_red[g][2], s_red[g][3]));
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float p = exp2f(sv[g] - mx[g]);
    s_p[g][tid] = p;
    const float ws = wave_sum(p);
    if (lane == 0) s_red[g][wave] = ws;
  }
  __syncthreads();

  // Weighted values.
  float acc[G][VEC];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[g][e] = 0.f;
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    float vf[VEC];
    unpack(vr[st], vf);
    const int kl = 64 * wave + st * KPS + kin;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float p = s_p[g][kl];
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[g][e] = fmaf(p, vf[e], acc[g][e]);
    }
  }
  // Reduce over the KPS key groups of the wave (lanes with equal `sub`).
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float a = acc[g][e];
#pragma unroll
      for (int o = LPK; o < 64; o <<= 1) a += __shfl_xor(a, o, 64);
      acc[g][e] = a;
    }
  if (kin == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < VEC; ++e) s_o[wave][g][VEC * sub + e] = acc[g][e];
  }
  __syncthreads();
  for (int i = tid; i < G * HD; i += 256) {
    const int g = i / HD, d = i % HD;
    out[g * head_stride + d] = s_o[0][g][d] + s_o[1][g][d] + s_o[2][g][d] + s_o[3][g][d];
  }
  if (tid < G) {
    out[tid * head_stride + HD] = mx[tid];
    out[tid * head_stride + HD + 1] = s_red[tid][0] + s_red[tid][1] + s_red[tid][2] + s_red[tid][3];
  }
}

template <typename T, int HD>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ part,
                                                            const int32_t* __restrict__ lens, int Hq,
                                                            int cap, int n_chunks, T* __restrict__ o,
                                                            int ldo) {
  const int bh = blockIdx.x, b = bh / Hq, h = bh % Hq, lane = threadIdx.x;
  const int n = lens[b];
  if (n < 0 || n >= cap) return;
  const float* p = part + (size_t)bh * n_chunks * (HD + 2);
  float M = -INFINITY;
  for (int c = 0; c < n_chunks; ++c) M = fmaxf(M, p[c * (HD + 2) + HD]);
  constexpr int DPL = (HD + 63) / 64;
  float acc[DPL] = {};
  float l = 0.f;
  for (int c = 0; c < n_chunks; ++c) {
    const float mc = p[c * (HD + 2) + HD];
    if (mc == -INFINITY) continue;
    const float w = exp2f(mc - M);
    l += w * p[c * (HD + 2) + HD + 1];
#pragma unroll
    for (int t = 0; t < DPL; ++t) {
      const int d = lane + 64 * t;
      if (d < HD) acc[t] += w * p[c * (HD + 2) + d];
    }
  }
  T* op = o + (size_t)b * ldo + (size_t)h * HD;
#pragma unroll
  for (int t = 0; t < DPL; ++t) {
    const int d = lane + 64 * t;
    if (d < HD) op[d] = Elt<T>::from_f(acc[t] / l);
  }
}

template <typename T, int HD>
hipError_t launch_attn_g(int G, const void* q, const void* k, const void* v, const int32_t* lens,
                         int B, int Hq, int Hkv, int cap, int sliding, int window, int n_chunks,
                         float* part, hipStream_t s) {
  const dim3 grid(n_chunks, Hkv, B);
  const float sl = kLog2e / sqrtf((float)HD);
#define COMPASS_DEC(GG)                                                                          \
  decode_attn_kernel<T, HD, GG><<<grid, 256, 0, s>>>((const T*)q, (const T*)k, (const T*)v, lens, \
                                                      Hq, Hkv, cap, sliding, window, sl,          \
                                                      n_chunks, part)
  switch (G) {
    case 1: COMPASS_DEC(1); break;
    case 2: COMPASS_DEC(2); break;
    case 4: COMPASS_DEC(4); break;
    case 8: COMPASS_DEC(8); break;
    default: return hipErrorInvalidValue;
  }
#undef COMPASS_DEC
  return hipGetLastError();
}

}  // namespace

int decode_chunk_keys(int /*dtype*/, int /*hd*/) { return CHUNK; }

hipError_t launch_decode_attention(int dtype, const void* q, const void* k, const void* v,
                                   const int32_t* lens, int B, int Hq, int Hkv, int cap, int hd,
                                   int sliding, int window, int n_chunks, float* part,
                                   hipStream_t s) {
  const int G = Hq / Hkv;
  if (dtype == 1) {
    return hd == 128 ? launch_attn_g<bf16_t, 128>(G, q, k, v, lens, B, Hq, Hkv, cap, sliding, window, n_chunks, part, s)
                     : launch_attn_g<bf16_t, 64>(G, q, k, v, lens, B, Hq, Hkv, cap, sliding, window, n_chunks, part, s);
  }
  return hd == 128 ? launch_attn_g<float, 128>(G, q, k, v, lens, B, Hq, Hkv, cap, sliding, window, n_chunks, part, s)
                   : launch_attn_g<float, 64>(G, q, k, v, lens, B, Hq, Hkv, cap, sliding, window, n_chunks, part, s);
}

hipError_t launch_decode_combine(int dtype, const float* part, const int32_t* lens, int B, int Hq,
                                 int cap, int hd, int n_chunks, void* o, int ldo, hipStream_t s) {
  const dim3 grid(B * Hq);
  if (dtype == 1) {
    if (hd == 128) decode_combine_kernel<bf16_t, 128><<<grid, 64, 0, s>>>(part, lens, Hq, cap, n_chunks, (bf16_t*)o, ldo);
    else decode_combine_kernel<bf16_t, 64><<<grid, 64, 0, s>>>(part, lens, Hq, cap, n_chunks, (bf16_t*)o, ldo);
  } else {
    if (hd == 128) decode_combine_kernel<float, 128><<<grid, 64, 0, s>>>(part, lens, Hq, cap, n_chunks, (float*)o, ldo);
    else decode_combine_kernel<float, 64><<<grid, 64, 0, s>>>(part, lens, Hq, cap, n_chunks, (float*)o, ldo);
  }
  return hipGetLastError();
}

}  // namespace compass
