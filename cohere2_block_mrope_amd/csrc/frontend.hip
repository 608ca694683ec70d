// Token-id front end and greedy head.
//
// Embedding ("Text decoder forward" of the mlxcel Compass issue: h = embed_tokens(tokens);
// the vision tower's final merger produces the embeddings that replace the image-pad
// tokens; FreeToken's "How it fits together" writes those rows with one index_copy):
// a row gather from the tied table, then the image rows overwritten.
// Decode positions ("Position ids": a generated token sits at offset + rope_delta on all
// three axes). Greedy head: the argmax over the vocabulary of the tied-embedding logits,
// smallest id on ties.
#include "common.h"
#include "launch.h"

namespace compass {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void embed_gather_kernel(const int32_t* __restrict__ tokens, int D, int V,
                                                           const T* __restrict__ E, T* __restrict__ h) {
  constexpr int VEC = 16 / sizeof(T);
  const int r = blockIdx.x;
  const int tok = tokens[r];
  const bool ok = tok >= 0 && tok < V;  // ids outside the table give a zero row (reported in status)
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(E + (size_t)(ok ? tok : 0) * D);
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(h + (size_t)r * D);
  for (int c = threadIdx.x; c < D / VEC; c += 256) dst[c] = ok ? src[c] : u32x4_t{0u, 0u, 0u, 0u};
}

// Blocks 0..n_img-1 copy image feature rows into h (rows outside [0, R) skipped); block
// n_img writes the status word: bit 0 set if a token id is outside [0, V), bit 1 if an
// image row is outside [0, R).
template <typename T>
__global__ __launch_bounds__(256) void embed_rows_kernel(const int32_t* __restrict__ rows,
                                                         const T* __restrict__ feats, int n_img, int R, int D,
                                                         const int32_t* __restrict__ tokens, int V,
                                                         T* __restrict__ h, int32_t* __restrict__ status) {
  constexpr int VEC = 16 / sizeof(T);
  if ((int)blockIdx.x < n_img) {
    const int row = rows[blockIdx.x];
    if (row < 0 || row >= R) return;
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(feats + (size_t)blockIdx.x * D);
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(h + (size_t)row * D);
    for (int c = threadIdx.x; c < D / VEC; c += 256) dst[c] = src[c];
    return;
  }
  if (!status) return;
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  int mine = 0;
  for (int r = threadIdx.x; r < R; r += 256) mine |= (tokens[r] < 0 || tokens[r] >= V) ? 1 : 0;
  for (int i = threadIdx.x; i < n_img; i += 256) mine |= (rows[i] < 0 || rows[i] >= R) ? 2 : 0;
  if (mine) atomicOr(&bad, mine);
  __syncthreads();
  if (threadIdx.x == 0) status[0] = bad;
}

__global__ __launch_bounds__(256) void decode_positions_kernel(int32_t* __restrict__ lens,
                                                               const int32_t* __restrict__ rope_delta, int B,
                                                               int32_t* __restrict__ pos, int advance) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= B) return;
  int n = lens[b];
  if (advance) lens[b] = n = n + advance;
  const int p = n + (rope_delta ? rope_delta[b] : 0);
  pos[b] = p;
  pos[B + b] = p;
  pos[2 * B + b] = p;
}

// Argmax in two passes. Pass 1: workgroup (c, r) scans columns [c * ARG_COLS, +ARG_COLS)
// of row r (16 coalesced loads in flight per thread) and writes its (value, id) winner;
// pass 2: one workgroup per row reduces the row's chunk winners. Larger value wins, equal
// values go to the smaller id; an all -inf (or NaN) row gives id 0.
constexpr int ARG_COLS = 4096;

__device__ __forceinline__ void arg_better(float& bv, int& bi, float ov, int oi) {
  if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
}

__device__ __forceinline__ void wave_argmax(float& bv, int& bi) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    arg_better(bv, bi, ov, oi);
  }
}

__global__ __launch_bounds__(256) void argmax_chunk_kernel(const float* __restrict__ raw, int V, long long ldr,
                                                           float scale, int nch, float* __restrict__ pv,
                                                           int* __restrict__ pi) {
  const int c = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  const float* row = raw + (size_t)r * ldr;
  const int c0 = c * ARG_COLS;
  float x[ARG_COLS / 256];
#pragma unroll
  for (int j = 0; j < ARG_COLS / 256; ++j) {
    const int v = c0 + j * 256 + tid;
    x[j] = v < V ? __builtin_nontemporal_load(row + v) : -INFINITY;
  }
  float bv = -INFINITY;
  int bi = 0x7fffffff;
#pragma unroll
  for (int j = 0; j < ARG_COLS / 256; ++j) {
    const int v = c0 + j * 256 + tid;
    if (v < V) arg_better(bv, bi, x[j] * scale, v);  // ids increase with j: first maximum kept
  }
  wave_argmax(bv, bi);
  __shared__ float s_v[4];
  __shared__ int s_i[4];
  if ((tid & 63) == 0) { s_v[tid >> 6] = bv; s_i[tid >> 6] = bi; }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w) arg_better(bv, bi, s_v[w], s_i[w]);
    pv[(size_t)r * nch + c] = bv;
    pi[(size_t)r * nch + c] = bi;
  }
}

__global__ __launch_bounds__(256) void argmax_final_kernel(const float* __restrict__ pv, const int* __restrict__ pi,
                                                           int nch, int32_t* __restrict__ token,
                                                           float* __restrict__ max_logit) {
  const int r = blockIdx.x, tid = threadIdx.x;
  const float* rv = pv + (size_t)r * nch;
  const int* ri = pi + (size_t)r * nch;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int c0 = 0; c0 < nch; c0 += 8 * 256) {
    float v[8];
    int id[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {  // all loads first, then the compares
      const int c = c0 + j * 256 + tid;
      v[j] = c < nch ? rv[c] : -INFINITY;
      id[j] = c < nch ? ri[c] : 0x7fffffff;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) arg_better(bv, bi, v[j], id[j]);
  }
  wave_argmax(bv, bi);
  __shared__ float s_v[4];
  __shared__ int s_i[4];
  if ((tid & 63) == 0) { s_v[tid >> 6] = bv; s_i[tid >> 6] = bi; }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w) arg_better(bv, bi, s_v[w], s_i[w]);
    token[r] = bi == 0x7fffffff ? 0 : bi;
    if (max_logit) max_logit[r] = bv;
  }
}

}  // namespace

hipError_t launch_embed(int dtype, const int32_t* tokens, int R, int D, int V, const void* E,
                        const int32_t* img_rows, const void* feats, int n_img, void* h, int32_t* status,
                        hipStream_t s) {
  if (dtype == 1) {
    embed_gather_kernel<bf16_t><<<R, 256, 0, s>>>(tokens, D, V, (const bf16_t*)E, (bf16_t*)h);
    embed_rows_kernel<bf16_t><<<n_img + 1, 256, 0, s>>>(img_rows, (const bf16_t*)feats, n_img, R, D, tokens, V,
                                                        (bf16_t*)h, status);
  } else {
    embed_gather_kernel<float><<<R, 256, 0, s>>>(tokens, D, V, (const float*)E, (float*)h);
    embed_rows_kernel<float><<<n_img + 1, 256, 0, s>>>(img_rows, (const float*)feats, n_img, R, D, tokens, V,
                                                       (float*)h, status);
  }
  return hipGetLastError();
}

hipError_t launch_decode_positions(int32_t* lens, const int32_t* rope_delta, int B, int32_t* pos, int advance,
                                   hipStream_t s) {
  decode_positions_kernel<<<(B + 255) / 256, 256, 0, s>>>(lens, rope_delta, B, pos, advance);
  return hipGetLastError();
}

int argmax_chunks(int V) { return (V + ARG_COLS - 1) / ARG_COLS; }

hipError_t launch_argmax(const float* raw, int R, int V, long long ldr, float scale, float* pv, int* pi,
                         int32_t* token, float* max_logit, hipStream_t s) {
  const int nch = argmax_chunks(V);
  argmax_chunk_kernel<<<dim3(nch, R), 256, 0, s>>>(raw, V, ldr, scale, nch, pv, pi);
  argmax_final_kernel<<<R, 256, 0, s>>>(pv, pi, nch, token, max_logit);
  return hipGetLastError();
}

hipError_t launch_argmax_partials(const float* pv, const int* pi, int R, int nparts, int32_t* token,
                                  float* max_logit, hipStream_t s) {
  argmax_final_kernel<<<R, 256, 0, s>>>(pv, pi, nparts, token, max_logit);
  return hipGetLastError();
}

}  // namespace compass
