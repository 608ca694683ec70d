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

// bf16 variant: the chunk's scores come from MFMA. For each 32-key block the wave computes
// S^T = K Q^T with v_mfma_f32_32x32x16_bf16: operand A is 32 key rows (lane l holds key
// l % 32, dims 8 (l / 32) + 16 ks .. + 8), operand B holds the G query heads in columns
// 0..G-1 (other columns zero). Lanes whose column is a real head then hold 16 keys'
// scores each, so no cross-lane reduction is needed for q . k.
// K and V rows are streamed with nontemporal 16-byte loads, hd / 8 lanes per row (whole
// rows per instruction: the nontemporal path only pays off for fully coalesced rows).
// Each wave's 64 K rows go through its own LDS tile, 16-byte chunks XOR-swizzled by row,
// from which the MFMA operand is read without bank conflicts. The PV product stays on
// the vector ALUs: each V row is read by hd / 8 lanes and the four key groups of a wave
// are summed once at the end.
template <int HD>
__device__ __forceinline__ int dk_swz(int row, int chunk) {  // 16-byte slot of (row, chunk)
  if constexpr (HD == 128) return row * 16 + (chunk ^ (row & 15));
  else return row * 8 + (chunk ^ ((row >> 1) & 7));
}

template <int HD, int G>
__global__ __launch_bounds__(256) void decode_attn_mfma_kernel(const bf16_t* __restrict__ q,
                                                               const bf16_t* __restrict__ k,
                                                               const bf16_t* __restrict__ v,
                                                               const int32_t* __restrict__ lens, int Hq,
                                                               int Hkv, int cap, int sliding, int window,
                                                               float scale_log2, int n_chunks,
                                                               float* __restrict__ part) {
  constexpr int KS = HD / 16;          // k-steps of 16 dims
  constexpr int LPK = HD / 8;          // lanes per K / V row (16-byte chunks per row)
  constexpr int KPS = 64 / LPK;        // rows per wave load instruction
  constexpr int STEPS = 64 / KPS;      // load instructions for the wave's 64 rows
  // Per-wave K tiles of 32 keys (the wave's 64 keys are staged in two rounds, which keeps
  // the workgroup at about 36 KB of LDS: three workgroups per CU stream at once); reused
  // for the per-wave output partials once every wave is done.
  __shared__ __align__(16) u32x4_t s_kbuf[4 * 32 * LPK];
  __shared__ float s_p[G][CHUNK];
  __shared__ float s_red[G][4];
  __shared__ __align__(16) u32x4_t s_q[G * LPK];
  static_assert(sizeof(float) * 4 * G * HD <= sizeof(u32x4_t) * 4 * 32 * LPK, "s_o must fit in the K tiles");
  float (*s_o)[G][HD] = reinterpret_cast<float (*)[G][HD]>(s_kbuf);

  const int chunk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  const bf16_t* kb = k + ((size_t)b * Hkv + kvh) * cap * HD;
  const bf16_t* vb = v + ((size_t)b * Hkv + kvh) * cap * HD;

  // K and V rows of this wave's 64 keys (clamped to the visible range), whole rows per
  // instruction: lane l reads chunk l % LPK of row KPS i + l / LPK.
  const int col = lane & 31, half = lane >> 5;
  const int sub = lane % LPK, kin = lane / LPK;
  u32x4_t kr[STEPS], vr[STEPS];
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int key = min(kbeg + 64 * wave + st * KPS + kin, kend - 1);
    kr[st] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kb + (size_t)key * HD + 8 * sub));
  }
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int key = min(kbeg + 64 * wave + st * KPS + kin, kend - 1);
    vr[st] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vb + (size_t)key * HD + 8 * sub));
  }
  // The G query rows (the Q^T operand, column `col` = head col, zero beyond G) go through
  // LDS, read per MFMA: holding them in registers for the whole kernel would cost the
  // occupancy that keeps three workgroups' loads in flight per CU.
  if (tid < G * LPK) s_q[tid] = *reinterpret_cast<const u32x4_t*>(q + ((size_t)b * Hq + kvh * G) * HD + 8 * tid);
  u32x4_t* kt = s_kbuf + 32 * LPK * wave;
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2) {
    // Stage keys 32 kb2 .. + 32 of this wave (load steps STEPS / 2 * kb2 ..). The previous
    // round's fragment reads were consumed by its MFMAs before this point.
#pragma unroll
    for (int st = 0; st < STEPS / 2; ++st)
      kt[dk_swz<HD>(st * KPS + kin, sub)] = kr[(STEPS / 2) * kb2 + st];
    __syncthreads();
    f32x16_t sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4_t kf = kt[dk_swz<HD>(col, 2 * ks + half)];
      const u32x4_t qw = col < G ? s_q[col * LPK + 2 * ks + half] : u32x4_t{0u, 0u, 0u, 0u};
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf),
                                                     __builtin_bit_cast(bf16x8_t, qw), sacc, 0, 0, 0);
    }
    if (col < G) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kl = 64 * wave + 32 * kb2 + 8 * (r >> 2) + 4 * half + (r & 3);
        s_p[col][kl] = (kbeg + kl < kend) ? sacc[r] * scale_log2 : -INFINITY;
      }
    }
  }
  __syncthreads();
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
  float acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const u32x4_t r = vr[st];
    const uint32_t w4[4] = {r.x, r.y, r.z, r.w};
    float vf[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      vf[2 * j] = __uint_as_float(w4[j] << 16);
      vf[2 * j + 1] = __uint_as_float(w4[j] & 0xffff0000u);
    }
    const int kl = 64 * wave + st * KPS + kin;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float p = s_p[g][kl];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(p, vf[e], acc[g][e]);
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float a2 = acc[g][e];
#pragma unroll
      for (int o = LPK; o < 64; o <<= 1) a2 += __shfl_xor(a2, o, 64);
      acc[g][e] = a2;
    }
  if (kin == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_o[wave][g][8 * sub + e] = acc[g][e];
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

// Merge the chunk partials of one (row, head): thread d owns output dimension d. Chunks
// are taken 16 at a time with every load of the group issued up front (chunk max, sum
// and the thread's output dimension), merged with an online maximum, so the merge costs
// about one memory round trip per 16 chunks. Weights are 2^(m_c - M); empty chunks
// (max -inf, only their statistics written) are skipped.
template <typename T, int HD>
__global__ __launch_bounds__(HD) void decode_combine_kernel(const float* __restrict__ part,
                                                            const int32_t* __restrict__ lens, int Hq,
                                                            int cap, int n_chunks, T* __restrict__ o,
                                                            int ldo) {
  constexpr int CG = 16;  // chunks per group
  const int bh = blockIdx.x, b = bh / Hq, h = bh % Hq, d = threadIdx.x;
  const int n = lens[b];
  if (n < 0 || n >= cap) return;
  const float* p = part + (size_t)bh * n_chunks * (HD + 2);
  float M = -INFINITY, l = 0.f, acc = 0.f;
  for (int c0 = 0; c0 < n_chunks; c0 += CG) {
    float mc[CG], lc[CG], oc[CG];
#pragma unroll
    for (int j = 0; j < CG; ++j) {
      const int c = min(c0 + j, n_chunks - 1);
      const float* pc = p + (size_t)c * (HD + 2);
      mc[j] = (c0 + j < n_chunks) ? pc[HD] : -INFINITY;
      lc[j] = pc[HD + 1];
      oc[j] = pc[d];
    }
    float mb = M;
#pragma unroll
    for (int j = 0; j < CG; ++j) mb = fmaxf(mb, mc[j]);
    if (mb == -INFINITY) continue;  // nothing visible yet
    const float r = (M == -INFINITY) ? 0.f : exp2f(M - mb);
    l *= r;
    acc *= r;
#pragma unroll
    for (int j = 0; j < CG; ++j) {
      // Skipped, not weighted by 0: an empty chunk's output slots are never written.
      if (mc[j] == -INFINITY) continue;
      const float w = exp2f(mc[j] - mb);
      l += w * lc[j];
      acc += w * oc[j];
    }
    M = mb;
  }
  o[(size_t)b * ldo + (size_t)h * HD + d] = Elt<T>::from_f(acc / l);
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
    const dim3 grid(n_chunks, Hkv, B);
    const float sl = kLog2e / sqrtf((float)hd);
#define COMPASS_DECM(HD, GG)                                                                    \
  decode_attn_mfma_kernel<HD, GG><<<grid, 256, 0, s>>>((const bf16_t*)q, (const bf16_t*)k,      \
                                                        (const bf16_t*)v, lens, Hq, Hkv, cap,    \
                                                        sliding, window, sl, n_chunks, part)
    if (hd == 128) {
      switch (G) { case 1: COMPASS_DECM(128, 1); break; case 2: COMPASS_DECM(128, 2); break;
                   case 4: COMPASS_DECM(128, 4); break; case 8: COMPASS_DECM(128, 8); break;
                   default: return hipErrorInvalidValue; }
    } else {
      switch (G) { case 1: COMPASS_DECM(64, 1); break; case 2: COMPASS_DECM(64, 2); break;
                   case 4: COMPASS_DECM(64, 4); break; case 8: COMPASS_DECM(64, 8); break;
                   default: return hipErrorInvalidValue; }
    }
#undef COMPASS_DECM
    return hipGetLastError();
  }
  return hd == 128 ? launch_attn_g<float, 128>(G, q, k, v, lens, B, Hq, Hkv, cap, sliding, window, n_chunks, part, s)
                   : launch_attn_g<float, 64>(G, q, k, v, lens, B, Hq, Hkv, cap, sliding, window, n_chunks, part, s);
}

hipError_t launch_decode_combine(int dtype, const float* part, const int32_t* lens, int B, int Hq,
                                 int cap, int hd, int n_chunks, void* o, int ldo, hipStream_t s) {
  const dim3 grid(B * Hq);
  if (dtype == 1) {
    if (hd == 128) decode_combine_kernel<bf16_t, 128><<<grid, 128, 0, s>>>(part, lens, Hq, cap, n_chunks, (bf16_t*)o, ldo);
    else decode_combine_kernel<bf16_t, 64><<<grid, 64, 0, s>>>(part, lens, Hq, cap, n_chunks, (bf16_t*)o, ldo);
  } else {
    if (hd == 128) decode_combine_kernel<float, 128><<<grid, 128, 0, s>>>(part, lens, Hq, cap, n_chunks, (float*)o, ldo);
    else decode_combine_kernel<float, 64><<<grid, 64, 0, s>>>(part, lens, Hq, cap, n_chunks, (float*)o, ldo);
  }
  return hipGetLastError();
}

}  // namespace compass
