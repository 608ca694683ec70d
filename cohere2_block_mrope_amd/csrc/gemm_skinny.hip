// Skinny bf16 GEMM for the decode output projection (at most 64 rows): fp32 partial sums over
// K-slices,
//   raw[z][m][n] = sum_{k in slice z} A[m, k] * B[n, k],   B = [Wo | Wd] (BMap kind 2),
// the output GEMM of the parallel block in "Text decoder forward" (mlxcel Compass issue) at a
// decode batch. Every weight is read once per step, so the kernel's time is set by how many
// weight bytes it keeps in flight and how little each K step costs once its data is there.
//
// A workgroup (4 waves, 2 x 2 blocks of 32 x 32) owns 64 columns and one K-slice of NK steps of
// 64. Each step's A and B tiles (64 rows x 64 k, 8 KB each) are loaded into registers D steps
// ahead (coalesced 16-byte pieces, 8 lanes per 128-byte row segment), written to a
// double-buffered LDS stage one step ahead, and multiplied out of LDS. The K loop is unrolled
// completely (NK is a compile-time constant), so every register slot is static and the
// compiler's wait for a step's loads leaves the D - 2 younger steps in flight (a loop over
// runtime steps merges the waits of its entry and back edge and waits too early).
#include "gemm_common.h"

namespace compass {
namespace {

using namespace gemm;

constexpr int kSkinnyDepth = 4;

template <int NK, int D>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmParams P) {
  static_assert(D >= 2, "at least one step of lookahead");
  constexpr int STAGE = 2 * 64 * BK;  // elements: A [64][64], then B [64][64]
  __shared__ __align__(16) bf16_t smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * 64;
  const int kbeg = blockIdx.y * NK * BK;

  // This thread loads 16-byte chunk (lane & 7) of rows 16 w + 8 j + (lane >> 3), j = 0, 1, of
  // both tiles; rows beyond M or N are clamped to valid rows and never stored. B columns
  // k < ksplit come from p[0], the others from p[1] at k - ksplit (ksplit is a multiple of 64,
  // so a step never straddles it).
  const bf16_t* ap[2];
  const bf16_t* bp[2];
  const bf16_t* bq[2];
  int wo[2];  // LDS offset of the chunk (swizzled)
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 16 * wave + 8 * j + (lane >> 3);
    const int c = lane & 7;
    wo[j] = swz(r, c);
    ap[j] = P.A + (size_t)min(r, P.M - 1) * P.lda + c * 8;
    const int n = min(n0 + r, P.N - 1);
    bp[j] = (const bf16_t*)P.bm.p[0] + (size_t)n * P.bm.ld0 + c * 8;
    bq[j] = (const bf16_t*)P.bm.p[1] + (size_t)n * P.bm.ld1 + c * 8 - P.bm.ksplit;
  }

  u32x4_t ra[D][2], rb[D][2];
  auto load = [&](int kt) __attribute__((always_inline)) {
    const int k0 = kbeg + kt * BK;
    const int sl = kt % D;
    const bool second = k0 >= P.bm.ksplit;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      ra[sl][j] = *reinterpret_cast<const u32x4_t*>(ap[j] + k0);
      // Weights are read once: stream them past the caches.
      rb[sl][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>((second ? bq[j] : bp[j]) + k0));
    }
  };
  auto write = [&](int kt) __attribute__((always_inline)) {
    bf16_t* st = smem + (kt & 1) * STAGE;
    const int sl = kt % D;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      *reinterpret_cast<u32x4_t*>(st + wo[j]) = ra[sl][j];
      *reinterpret_cast<u32x4_t*>(st + 64 * 64 + wo[j]) = rb[sl][j];
    }
  };

  f32x16_t acc[1][1];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[0][0][r] = 0.f;

  int fa[BK / 16], fb[BK / 16];
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    const int c = 2 * ks + (lane >> 5);
    fa[ks] = swz(32 * wm + (lane & 31), c);
    fb[ks] = swz(32 * wn + (lane & 31), c);
  }

  // Stage s lives in register slot s % D from its load until it is written to LDS (at step
  // s - 1); the slot is then refilled with stage s + D.
#pragma unroll
  for (int s = 0; s < D && s < NK; ++s) load(s);
  write(0);
  if (D < NK) load(D);
  __syncthreads();
#pragma unroll
  for (int kt = 0; kt < NK; ++kt) {
    const bf16_t* a = smem + (kt & 1) * STAGE;
    const bf16_t* b = a + 64 * 64;
    bf16x8_t xa[BK / 16], xb[BK / 16];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      xa[ks] = *reinterpret_cast<const bf16x8_t*>(a + fa[ks]);
      xb[ks] = *reinterpret_cast<const bf16x8_t*>(b + fb[ks]);
    }
    if (kt + 1 < NK) write(kt + 1);
    if (kt + D + 1 < NK) load(kt + D + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks)
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[ks], xb[ks], acc[0][0], 0, 0, 0);
    __syncthreads();
  }
  gemm_epilogue<MODE_RAW, 1, 1>(P, acc, 32 * wm, n0 + 32 * wn, lane, blockIdx.y);
}

template <int NK>
hipError_t launch_skinny(const GemmParams& P, dim3 grid, hipStream_t s) {
  gemm_skinny_kernel<NK, kSkinnyDepth><<<grid, 256, 0, s>>>(P);
  return hipGetLastError();
}

// K steps per split that have an instantiation (the Compass decode output projection,
// K = 2048 + 8192 in 8 or 16 splits, and slices of 512 or 1024).
int skinny_steps(int K, int splits) {
  if (splits < 1 || K % (64 * splits) != 0) return 0;
  const int nk = K / (64 * splits);
  return (nk == 8 || nk == 10 || nk == 16 || nk == 20) ? nk : 0;
}

}  // namespace

bool gemm_skinny_fits(int M, int K, int N, int splits) {
  return M >= 1 && M <= 64 && N % 4 == 0 && skinny_steps(K, splits) > 0;
}

hipError_t launch_gemm_skinny_raw(const void* A, int lda, int M, int K, const BMap& bm, int N, int splits,
                                  float* raw, hipStream_t s) {
  if (bm.kind != 2 || bm.ksplit % 64 != 0 || !gemm_skinny_fits(M, K, N, splits)) return hipErrorInvalidValue;
  GemmParams P{};
  P.A = (const bf16_t*)A;
  P.lda = lda; P.M = M; P.K = K; P.N = N;
  P.bm = bm;
  P.raw = raw;
  P.kchunk = K / splits;
  const dim3 grid((N + 63) / 64, splits);
  switch (skinny_steps(K, splits)) {
    case 8: return launch_skinny<8>(P, grid, s);
    case 10: return launch_skinny<10>(P, grid, s);
    case 16: return launch_skinny<16>(P, grid, s);
    case 20: return launch_skinny<20>(P, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace compass
