// fp32 GEMM on the vector ALUs, C[m, n] = sum_k A[m, k] * B[n, k], for the fp32
// storage dtype (the small fp32 parity workload). 64 x 64 output tile per 256-thread
// workgroup, 4 x 4 outputs per thread, K in steps of 16 staged through LDS
// (transposed to k-major so the inner loop reads 4 consecutive rows/columns).
// Writes raw fp32 partial sums over K-slices: raw[z][m][n].
#include "common.h"
#include "launch.h"

namespace compass {
namespace {

constexpr int TM = 64, TN = 64, TK = 16;

__device__ __forceinline__ const float* f32_b_row(const BMap& bm, int n, int k0) {
  if (bm.kind == 2) {
    return k0 < bm.ksplit ? (const float*)bm.p[0] + (size_t)n * bm.ld0 + k0
                          : (const float*)bm.p[1] + (size_t)n * bm.ld1 + (k0 - bm.ksplit);
  }
  if (bm.kind == 1) {
    const int ch = n >> 6, r = n & 63;
    const int qe = bm.nq64, ke = qe + bm.nk64, ve = ke + bm.nk64;
    const float* base;
    int row;
    if (ch < qe) { base = (const float*)bm.p[0]; row = ch * 64 + r; }
    else if (ch < ke) { base = (const float*)bm.p[1]; row = (ch - qe) * 64 + r; }
    else if (ch < ve) { base = (const float*)bm.p[2]; row = (ch - ke) * 64 + r; }
    else {
      const int m = ch - ve;
      base = (m & 1) ? (const float*)bm.p[4] : (const float*)bm.p[3];
      row = (m >> 1) * 64 + r;
    }
    return base + (size_t)row * bm.ld0 + k0;
  }
  return (const float*)bm.p[0] + (size_t)n * bm.ld0 + k0;
}

__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, int lda, int M,
                                                       int K, BMap bm, int N, int kchunk,
                                                       float* __restrict__ raw, float scale) {
  __shared__ float As[TK][TM + 4];
  __shared__ float Bs[TK][TN + 4];
  const int tiles_m = (M + TM - 1) / TM;
  const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int m0 = tm * TM, n0 = tn * TN;
  const int kbeg = blockIdx.z * kchunk, kend = min(K, kbeg + kchunk);
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;  // outputs rows ty*4.., cols tx*4..
  float acc[4][4] = {};
  // Loader: 64 rows x 16 k = 1024 values per operand, 4 per thread (one float4).
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  const int am = min(m0 + lr, M - 1);
  const int bn = min(n0 + lr, N - 1);
  for (int k0 = kbeg; k0 < kend; k0 += TK) {
    const float4 av = *reinterpret_cast<const float4*>(A + (size_t)am * lda + k0 + lk);
    const float4 bv = *reinterpret_cast<const float4*>(f32_b_row(bm, bn, k0) + lk);
    __syncthreads();
    As[lk + 0][lr] = av.x; As[lk + 1][lr] = av.y; As[lk + 2][lr] = av.z; As[lk + 3][lr] = av.w;
    Bs[lk + 0][lr] = bv.x; Bs[lk + 1][lr] = bv.y; Bs[lk + 2][lr] = bv.z; Bs[lk + 3][lr] = bv.w;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = As[kk][ty * 4 + i]; b[i] = Bs[kk][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n < N) raw[((size_t)blockIdx.z * M + m) * N + n] = acc[i][j] * scale;
    }
  }
}

}  // namespace

hipError_t launch_gemm_f32_raw(const void* A, int lda, int M, int K, const BMap& bm, int N,
                               int splits, float* raw, float scale, hipStream_t s) {
  const int kc = ((K / splits + TK - 1) / TK) * TK;
  const int tiles = ((M + TM - 1) / TM) * ((N + TN - 1) / TN);
  gemm_f32_kernel<<<dim3(tiles, 1, splits), 256, 0, s>>>((const float*)A, lda, M, K, bm, N, kc, raw, scale);
  return hipGetLastError();
}

}  // namespace compass
