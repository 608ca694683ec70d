// Split-K GEMM with 4-bit affine weights for the decode step:
//   raw[z][m][n] = sum over K-slice z of A[m, k] * W[n, k],
//   W[n, k] = scale[n, k / 64] * code[n, k] + bias[n, k / 64]
// (the checkpoint's quantization block in the config section of the mlxcel Compass issue:
// group size 64, 4 bits, affine mode). Codes are packed two per byte, column 2j in the low
// nibble of byte j.
//
// The weights are the HBM traffic of a decode step (0.5 byte per weight plus 4 bytes of
// scale and bias per 64 weights, against 2 bytes in bf16). One K step of 64 columns is one
// quantization group, so each weight row of a stage needs one (scale, bias) pair: the
// stage's codes are dequantized in registers (fp32 FMA, one rounding to bf16) on their way
// into the same swizzled LDS tile the bf16 GEMM uses, and the MFMA part is unchanged
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation). Tile 64 x 64, 4 waves of 32 x 32, two LDS
// stages fed from a register ring that keeps several K steps of loads in flight (the
// per-step MFMA work of a skinny tile is far shorter than the memory latency).
#include "gemm_common.h"

namespace compass {
namespace {

using namespace gemm;

// Stages in flight per workgroup (measured on MI355X at the decode widths: 2 beats 4 and 8,
// which cost registers without shortening the per-stage critical path).
constexpr int Q4_PD = 2;

struct Q4Params {
  const bf16_t* A;
  int lda, M, K, N;
  Q4Map bm;
  int kchunk, tiles_m, tiles_n;
  float* raw;
};

template <int BKIND, int PD>
__global__ __launch_bounds__(256, 2) void gemm_q4_raw_kernel(Q4Params P) {
  static_assert(PD % 2 == 0, "the LDS buffer of a stage is its ring slot's parity");
  constexpr int BM = 64, BN = 64;
  __shared__ __align__(16) bf16_t As[2][BM * BK];
  __shared__ __align__(16) bf16_t Bs[2][BN * BK];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int tm = blockIdx.x % P.tiles_m, tn = blockIdx.x / P.tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = blockIdx.z * P.kchunk;
  const int kend = min(P.K, kbeg + P.kchunk);

  // A staging: rows (tid >> 3) + 32 i of the tile, 16-byte chunk tid & 7 (rows beyond M
  // clamped; never stored).
  const int lchunk = tid & 7, arow = tid >> 3;
  uint32_t aoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) aoff[i] = (uint32_t)min(m0 + arow + 32 * i, P.M - 1) * (uint32_t)P.lda + lchunk * 8;

  // B staging: weight row brow of the tile, codes of columns 16 bq .. 16 bq + 15 of each
  // 64-column group (8 bytes), plus the row's scale and bias of that group.
  const int brow = tid >> 2, bq = tid & 3;
  const uint8_t* q0;
  const bf16_t* s0;
  const bf16_t* b0;
  const uint8_t* q1 = nullptr;
  const bf16_t* s1 = nullptr;
  const bf16_t* b1 = nullptr;
  if constexpr (BKIND == 1) {
    // Virtual projection layout in 64-row chunks (q | k | v | gate, up interleaved); a
    // 64-row tile is exactly one chunk.
    const int ch = n0 >> 6;
    const int qe = P.bm.nq64, ke = qe + P.bm.nk64, ve = ke + P.bm.nk64;
    int mat, first;
    if (ch < qe) { mat = 0; first = ch * 64; }
    else if (ch < ke) { mat = 1; first = (ch - qe) * 64; }
    else if (ch < ve) { mat = 2; first = (ch - ke) * 64; }
    else { mat = 3 + ((ch - ve) & 1); first = ((ch - ve) >> 1) * 64; }
    const size_t row = (size_t)(first + brow);
    q0 = (const uint8_t*)P.bm.q[mat] + row * (P.bm.cols0 / 2);
    s0 = (const bf16_t*)P.bm.s[mat] + row * (P.bm.cols0 / 64);
    b0 = (const bf16_t*)P.bm.b[mat] + row * (P.bm.cols0 / 64);
  } else {
    // Concatenation along K: columns k < ksplit from matrix 0, the rest from matrix 1.
    const size_t row = (size_t)min(n0 + brow, P.N - 1);
    q0 = (const uint8_t*)P.bm.q[0] + row * (P.bm.cols0 / 2);
    s0 = (const bf16_t*)P.bm.s[0] + row * (P.bm.cols0 / 64);
    b0 = (const bf16_t*)P.bm.b[0] + row * (P.bm.cols0 / 64);
    q1 = (const uint8_t*)P.bm.q[1] + row * (P.bm.cols1 / 2);
    s1 = (const bf16_t*)P.bm.s[1] + row * (P.bm.cols1 / 64);
    b1 = (const bf16_t*)P.bm.b[1] + row * (P.bm.cols1 / 64);
  }

  // Register ring of PD stages: the loads of stage kt + PD are issued right after stage
  // kt leaves its slot. The loop runs a multiple of PD stages without branches: stages past
  // the end re-read the last valid address and are dequantized as zero weights. Codes,
  // scales and biases use ordinary (cached) loads: a stage reads 32 of the 128 bytes of a
  // row's cache line and the next three stages read the rest, so streaming hints that
  // evict the line early cost a refetch (measured 30 vs 20 us on the projection).
  const int nk = max(0, (kend - kbeg) / BK);
  u32x4_t ra[PD][2];
  u32x2_t rq[PD];
  uint32_t rs[PD], rbias[PD];  // bf16 bits of the group's scale and bias
  auto load = [&](int slot, int kt) __attribute__((always_inline)) {
    const int k = kbeg + min(kt, nk - 1) * BK;
#pragma unroll
    for (int i = 0; i < 2; ++i) ra[slot][i] = *reinterpret_cast<const u32x4_t*>(P.A + aoff[i] + k);
    const uint8_t* q = q0;
    const bf16_t* sp = s0;
    const bf16_t* bp = b0;
    int kk = k;
    if constexpr (BKIND == 2) {
      const bool hi = k >= P.bm.ksplit;  // uniform over the workgroup
      q = hi ? q1 : q0;
      sp = hi ? s1 : s0;
      bp = hi ? b1 : b0;
      kk = hi ? k - P.bm.ksplit : k;
    }
    rq[slot] = *reinterpret_cast<const u32x2_t*>(q + kk / 2 + 8 * bq);
    rs[slot] = *reinterpret_cast<const uint16_t*>(sp + kk / 64);
    rbias[slot] = *reinterpret_cast<const uint16_t*>(bp + kk / 64);
  };
  auto store = [&](int buf, int slot, bool valid) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<u32x4_t*>(&As[buf][swz(arow + 32 * i, lchunk)]) = ra[slot][i];
    const float sc = valid ? __uint_as_float(rs[slot] << 16) : 0.f;
    const float bi = valid ? __uint_as_float(rbias[slot] << 16) : 0.f;
    const uint32_t w[2] = {rq[slot].x, rq[slot].y};
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // 8 codes per 32-bit word, column order from the low nibble
      u32x4_t o;
      uint32_t* op = reinterpret_cast<uint32_t*>(&o);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = __builtin_fmaf(sc, (float)((w[h] >> (8 * e)) & 15u), bi);
        const float hi = __builtin_fmaf(sc, (float)((w[h] >> (8 * e + 4)) & 15u), bi);
        op[e] = pack_bf2(lo, hi);
      }
      *reinterpret_cast<u32x4_t*>(&Bs[buf][swz(brow, 2 * bq + h)]) = o;
    }
  };

  f32x16_t acc[1][1];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[0][0][r] = 0.f;
  int fa_off[BK / 16], fb_off[BK / 16];
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    const int c = 2 * ks + (lane >> 5);
    fa_off[ks] = swz(wm * 32 + (lane & 31), c);
    fb_off[ks] = swz(wn * 32 + (lane & 31), c);
  }

  if (nk > 0) {
#pragma unroll
    for (int j = 0; j < PD; ++j) load(j, j);
    for (int kt0 = 0; kt0 < nk; kt0 += PD) {
#pragma unroll
      for (int j = 0; j < PD; ++j) {
        const int kt = kt0 + j;
        const int buf = j & 1;  // PD is even: the buffer of stage kt is kt & 1
        // Buffer `buf` was last read by the MFMAs of stage kt - 2, which every wave finished
        // before the barrier of stage kt - 1.
        store(buf, j, kt < nk);
        __syncthreads();
        load(j, kt + PD);
        bf16x8_t fa[BK / 16], fb[BK / 16];
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
          fa[ks] = *reinterpret_cast<const bf16x8_t*>(&As[buf][fa_off[ks]]);
          fb[ks] = *reinterpret_cast<const bf16x8_t*>(&Bs[buf][fb_off[ks]]);
        }
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks)
          acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks], fb[ks], acc[0][0], 0, 0, 0);
      }
    }
  }

  GemmParams G{};
  G.M = P.M;
  G.N = P.N;
  G.raw = P.raw;
  gemm_epilogue<MODE_RAW, 1, 1>(G, acc, m0 + wm * 32, n0 + wn * 32, lane, blockIdx.z);
}

}  // namespace

hipError_t launch_gemm_q4_raw(const void* A, int lda, int M, int K, const Q4Map& bm, int N, int splits, float* raw,
                              hipStream_t s) {
  Q4Params P{};
  P.A = (const bf16_t*)A;
  P.lda = lda;
  P.M = M;
  P.K = K;
  P.N = N;
  P.bm = bm;
  P.kchunk = ((K / splits + BK - 1) / BK) * BK;
  P.tiles_m = (M + 63) / 64;
  P.tiles_n = (N + 63) / 64;
  P.raw = raw;
  const dim3 grid(P.tiles_m * P.tiles_n, 1, splits);
  if (bm.kind == 1) gemm_q4_raw_kernel<1, Q4_PD><<<grid, 256, 0, s>>>(P);
  else gemm_q4_raw_kernel<2, Q4_PD><<<grid, 256, 0, s>>>(P);
  return hipGetLastError();
}

}  // namespace compass
