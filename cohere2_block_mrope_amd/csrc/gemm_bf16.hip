// bf16 GEMMs on gfx950 MFMA (v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//   C[m, n] = sum_k A[m, k] * B[n, k]    (A [M, K] and B [N, K] both K-contiguous)
//
// One kernel template serves the GEMMs of the layer and the head:
//   PROJ   the fused q/k/v/gate/up projection of "Text decoder forward" (mlxcel
//          Compass issue). Its epilogue applies interleaved MRoPE to q and k in
//          registers, scatters q to [B, Hq, L, hd], k/v to the cache [B, Hkv, cap, hd],
//          and writes act = silu(gate) * up (SwiGLU);
//   RESID  the output GEMM [o | act] . [Wo | Wd]^T plus the residual x (parallel
//          block: h + attn + mlp);
//   SCALED the tied-embedding logits times logit_scale, stored as fp32;
//   ARGMAX the same logits reduced in registers to per-row (max, id) partials (greedy
//          decoding without storing the logits);
//   RAW    fp32 partial sums over a K-slice (split-K for skinny decode GEMMs).
//
// Tiling: a 256-thread workgroup (4 waves, 2 x 2) computes a BM x BN tile; each wave
// owns a (BM/2) x (BN/2) sub-tile of 32 x 32 MFMA blocks. K advances in steps of 64
// through a double-buffered LDS stage (A and B tiles, 16-byte chunks XOR-swizzled by
// row so that the fragment reads of 8 consecutive rows hit distinct banks). Global
// loads run two K steps ahead through registers and are interleaved, one 16-byte piece
// at a time, with the MFMAs of the current step.
//
// MFMA lane layout (checked on gfx950): operand lane l holds row (l % 32) and
// k = 8 * (l / 32) .. + 8; result register r of lane l holds
// C[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32].
//
// The fused MRoPE epilogue needs the pair (x_j, x_{j + hd/2}) in one lane: with
// BN = 256 each wave owns 128 consecutive columns aligned to a head (hd = 128) or to
// two heads (hd = 64), so for hd = 128 block j and block j + 2 hold the two halves of
// the same rows in the same lane and register. Gate and up come in 64-column chunk
// pairs (see BMap kind 1), so silu(gate) * up is also a same-lane, same-register op.
#include "gemm_common.h"

namespace compass {
namespace {

using namespace gemm;

template <int BM, int BN, int MODE, int BKIND, bool LNA = false>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(GemmParams P) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int A_PER_T = BM / 32, B_PER_T = BN / 32;  // 16-byte chunks per thread per stage
  extern __shared__ __align__(16) bf16_t smem[];
  bf16_t* As = smem;                 // [2][BM * 64]
  bf16_t* Bs = smem + 2 * BM * BK;   // [2][BN * 64]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  int tm, tn;
  if (MODE == MODE_RAW) { tm = blockIdx.x % P.tiles_m; tn = blockIdx.x / P.tiles_m; }
  else tile_coords<MODE == MODE_PROJ ? 4 : 8>(P.tiles_m, P.tiles_n, tm, tn);  // row-tile groups: measured
  const int m0 = tm * BM, n0 = tn * BN;

  int kbeg = 0, kend = P.K;
  if (MODE == MODE_RAW) {
    kbeg = blockIdx.z * P.kchunk;
    kend = min(P.K, kbeg + P.kchunk);
  }

  // Operand loading: wave w stages rows w * (ROWS / 4) + (lane >> 3) + 8 i of each tile
  // (16-byte chunk lane & 7 of each row), so one wave's B rows always sit inside one
  // 64-row chunk of the virtual B operand: a wave-uniform base pointer plus 32-bit row
  // offsets. Rows beyond M / N are clamped to valid rows and never stored.
  const int lchunk = lane & 7, lsub = lane >> 3;
  const int arow0 = wave * (BM / 4) + lsub, brow0 = wave * (BN / 4) + lsub;
  uint32_t aoff[A_PER_T];
#pragma unroll
  for (int i = 0; i < A_PER_T; ++i)
    aoff[i] = (uint32_t)min(m0 + arow0 + 8 * i, P.M - 1) * (uint32_t)P.lda + lchunk * 8;
  const bf16_t* bbase0;
  const bf16_t* bbase1 = nullptr;
  uint32_t boff[B_PER_T];
  uint32_t boff1[BKIND == 2 ? B_PER_T : 1];
  if constexpr (BKIND == 1) {
    // Virtual projection layout: chunk -> (matrix, first row); all rows have stride ld0.
    const int nch = P.N >> 6;
    const int ch = min((n0 + wave * (BN / 4)) >> 6, nch - 1);
    const int qe = P.bm.nq64, ke = qe + P.bm.nk64, ve = ke + P.bm.nk64;
    const bf16_t* base;
    int first;
    if (ch < qe) { base = (const bf16_t*)P.bm.p[0]; first = ch * 64; }
    else if (ch < ke) { base = (const bf16_t*)P.bm.p[1]; first = (ch - qe) * 64; }
    else if (ch < ve) { base = (const bf16_t*)P.bm.p[2]; first = (ch - ke) * 64; }
    else {
      const int mm = ch - ve;
      base = (mm & 1) ? (const bf16_t*)P.bm.p[4] : (const bf16_t*)P.bm.p[3];
      first = (mm >> 1) * 64;
    }
    bbase0 = base;
    const int r0 = first + ((n0 + wave * (BN / 4)) & 63) + lsub;
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) boff[i] = (uint32_t)(r0 + 8 * i) * (uint32_t)P.bm.ld0 + lchunk * 8;
  } else {
    bbase0 = (const bf16_t*)P.bm.p[0];
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i)
      boff[i] = (uint32_t)min(n0 + brow0 + 8 * i, P.N - 1) * (uint32_t)P.bm.ld0 + lchunk * 8;
    if constexpr (BKIND == 2) {
      bbase1 = (const bf16_t*)P.bm.p[1] - P.bm.ksplit;
#pragma unroll
      for (int i = 0; i < B_PER_T; ++i)
        boff1[i] = (uint32_t)min(n0 + brow0 + 8 * i, P.N - 1) * (uint32_t)P.bm.ld1 + lchunk * 8;
    }
  }

  // Stage k + 1 sits in registers while stage k is multiplied out of LDS. Its 16-byte
  // pieces are written to the other LDS buffer one at a time between MFMAs, and each
  // register is refilled with stage k + 2 right after its write, so the memory
  // instructions spread over the MFMA stream instead of stalling it in one burst.
  constexpr int PIECES = A_PER_T + B_PER_T;
  constexpr int MFMAS = (BK / 16) * MB * NB;
  u32x4_t ra[A_PER_T], rb[B_PER_T];
  // LNA: the LayerNorm weight of the stage's 8 columns of this thread (loaded with the last
  // A piece, after the stage before has stored all its A pieces), and the tile rows'
  // (mean, rstd) in LDS.
  u32x4_t wv = {0u, 0u, 0u, 0u};
  float2* s_st = reinterpret_cast<float2*>(smem + 2 * (BM + BN) * BK);
  auto load_piece = [&](int k0, int p) __attribute__((always_inline)) {
    if (p < A_PER_T) {
      ra[p] = *reinterpret_cast<const u32x4_t*>(P.A + aoff[p] + k0);
      if constexpr (LNA) {
        if (p == A_PER_T - 1) wv = *reinterpret_cast<const u32x4_t*>(P.ln_w + k0 + lchunk * 8);
      }
    } else {
      const int i = p - A_PER_T;
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(
          (BKIND == 2 && k0 >= P.bm.ksplit) ? bbase1 + boff1[i] + k0 : bbase0 + boff[i] + k0);
      // Skinny GEMMs (split-K decode projections, logits of at most 128 rows: one row
      // tile) read each weight row once: stream it past the caches.
      if constexpr (MODE == MODE_RAW || ((MODE == MODE_SCALED || MODE == MODE_ARGMAX) && BM <= 128))
        rb[i] = __builtin_nontemporal_load(src);
      else rb[i] = *src;
    }
  };
  auto store_piece = [&](int buf, int p) __attribute__((always_inline)) {
    if (p < A_PER_T) {
      u32x4_t v = ra[p];
      if constexpr (LNA) {  // the same fp32 expression as the LayerNorm kernel, one bf16 rounding
        const float2 st = s_st[arow0 + 8 * p];
        const uint32_t xs[4] = {v.x, v.y, v.z, v.w}, ws[4] = {wv.x, wv.y, wv.z, wv.w};
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x0 = __uint_as_float(xs[j] << 16), x1 = __uint_as_float(xs[j] & 0xffff0000u);
          const float w0 = __uint_as_float(ws[j] << 16), w1 = __uint_as_float(ws[j] & 0xffff0000u);
          o[j] = pack_bf2((x0 - st.x) * st.y * w0, (x1 - st.x) * st.y * w1);
        }
        v = u32x4_t{o[0], o[1], o[2], o[3]};
      }
      *reinterpret_cast<u32x4_t*>(As + buf * BM * BK + swz(arow0 + 8 * p, lchunk)) = v;
    } else
      *reinterpret_cast<u32x4_t*>(Bs + buf * BN * BK + swz(brow0 + 8 * (p - A_PER_T), lchunk)) =
          rb[p - A_PER_T];
  };

  f32x16_t acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  int fa_off[BK / 16], fb_off[BK / 16];
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    const int c = 2 * ks + (lane >> 5);
    fa_off[ks] = swz(wm * WM + (lane & 31), c);
    fb_off[ks] = swz(wn * WN + (lane & 31), c);
  }

  // One K step: MFMAs over LDS buffer kt & 1; `wr` stores stage kt + 1 to the other
  // buffer, `ld` fetches stage kt + 2.
  auto step = [&](int kt, const bool wr, const bool ld) __attribute__((always_inline)) {
    const int cur = kt & 1;
    const bf16_t* a = As + cur * BM * BK;
    const bf16_t* b = Bs + cur * BN * BK;
    const int knext = kbeg + (kt + 2) * BK;
    bf16x8_t fa[2][MB], fb[2][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i) fa[0][i] = *reinterpret_cast<const bf16x8_t*>(a + fa_off[0] + 32 * i * BK);
#pragma unroll
    for (int j = 0; j < NB; ++j) fb[0][j] = *reinterpret_cast<const bf16x8_t*>(b + fb_off[0] + 32 * j * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int fs = ks & 1;
      if (ks + 1 < BK / 16) {
#pragma unroll
        for (int i = 0; i < MB; ++i)
          fa[fs ^ 1][i] = *reinterpret_cast<const bf16x8_t*>(a + fa_off[ks + 1] + 32 * i * BK);
#pragma unroll
        for (int j = 0; j < NB; ++j)
          fb[fs ^ 1][j] = *reinterpret_cast<const bf16x8_t*>(b + fb_off[ks + 1] + 32 * j * BK);
      }
#pragma unroll
      for (int t = 0; t < MB * NB; ++t) {
        acc[t / NB][t % NB] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[fs][t / NB], fb[fs][t % NB], acc[t / NB][t % NB], 0, 0, 0);
        const int f = ks * MB * NB + t;
#pragma unroll
        for (int p = 0; p < PIECES; ++p) {
          if ((p * MFMAS) / PIECES == f) {
            __builtin_amdgcn_sched_barrier(0);
            if (wr) store_piece(cur ^ 1, p);
            if (ld) load_piece(knext, p);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
    __syncthreads();
  };

  if constexpr (LNA) {
    for (int i = tid; i < BM; i += 256) s_st[i] = P.ln_stats[min(m0 + i, P.M - 1)];
    __syncthreads();
  }
  const int nk = (kend - kbeg) / BK;
  if (nk > 0) {
#pragma unroll
    for (int p = 0; p < PIECES; ++p) load_piece(kbeg, p);
#pragma unroll
    for (int p = 0; p < PIECES; ++p) store_piece(0, p);
    if (nk > 1) {
#pragma unroll
      for (int p = 0; p < PIECES; ++p) load_piece(kbeg + BK, p);
    }
    __syncthreads();
    int kt = 0;
    for (; kt + 2 < nk; ++kt) step(kt, true, true);
    if (kt + 1 < nk) {
      step(kt, true, false);
      ++kt;
    }
    step(kt, false, false);
  }

  if constexpr (MODE == MODE_ARGMAX) {
    argmax_epilogue<MB, NB>(P, acc, m0 + wm * WM, n0 + wn * WN, 2 * tn + wn, lane);
  } else if constexpr (MODE == MODE_PROJ) {
    // Tiles with q / k / v columns stage their rows' data in LDS (free after the main loop's
    // last barrier) for the q / k / v epilogue.
    ProjRow* s_row = reinterpret_cast<ProjRow*>(smem);
    if (n0 < (P.ep.nq64 + 2 * P.ep.nk64) * 64) {  // uniform over the workgroup
      stage_proj_rows<BM>(P, m0, s_row, tid);
      __syncthreads();
    }
    gemm_epilogue<MODE, MB, NB>(P, acc, m0 + wm * WM, n0 + wn * WN, lane, blockIdx.z, s_row + wm * WM);
  } else {
    gemm_epilogue<MODE, MB, NB>(P, acc, m0 + wm * WM, n0 + wn * WN, lane, blockIdx.z);
  }
}

template <int BM, int BN, int MODE, int BKIND, bool LNA = false>
hipError_t launch(const GemmParams& P, dim3 grid, hipStream_t s) {
  constexpr size_t lds = (size_t)2 * (BM + BN) * BK * sizeof(bf16_t) + (LNA ? BM * sizeof(float2) : 0);
  const hipError_t e = ensure_dynamic_lds((const void*)gemm_bf16_kernel<BM, BN, MODE, BKIND, LNA>, (int)lds);
  if (e != hipSuccess) return e;
  gemm_bf16_kernel<BM, BN, MODE, BKIND, LNA><<<grid, 256, lds, s>>>(P);
  return hipGetLastError();
}

GemmParams base_params(const void* A, int lda, int M, int K, const BMap& bm, int N) {
  GemmParams P{};
  P.A = (const bf16_t*)A;
  P.lda = lda; P.M = M; P.K = K; P.N = N;
  P.bm = bm;
  P.kchunk = K;
  return P;
}

}  // namespace

// Compute units of the current device (the tile-shape choices below count rounds of
// one workgroup per CU).
int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  }
  return cus;
}

hipError_t launch_gemm_bf16_proj(const void* A, int lda, int M, int K, const BMap& bm, int N,
                                 const ProjEpi& ep, const RopeTable& rt, hipStream_t s,
                                 const float2* ln_stats, const void* ln_w) {
  GemmParams P = base_params(A, lda, M, K, bm, N);
  P.ep = ep;
  P.rt = rt;
  P.ln_stats = ln_stats;
  P.ln_w = (const bf16_t*)ln_w;
  const bool lna = ln_stats != nullptr;
  P.tiles_n = (N + 255) / 256;
  // 128-row tiles when they need fewer rounds over the CUs, counting a 128 x 256 tile at
  // 0.6 of a 256 x 256 one (measured per-flop efficiency of the smaller tile).
  const long long cus = device_cus();
  const long long r256 = ((long long)((M + 255) / 256) * P.tiles_n + cus - 1) / cus;
  const long long r128 = ((long long)((M + 127) / 128) * P.tiles_n + cus - 1) / cus;
  if (3 * r128 < 5 * r256) {
    P.tiles_m = (M + 127) / 128;
    return lna ? launch<128, 256, MODE_PROJ, 1, true>(P, dim3(P.tiles_m * P.tiles_n), s)
               : launch<128, 256, MODE_PROJ, 1>(P, dim3(P.tiles_m * P.tiles_n), s);
  }
  P.tiles_m = (M + 255) / 256;
  return lna ? launch<256, 256, MODE_PROJ, 1, true>(P, dim3(P.tiles_m * P.tiles_n), s)
             : launch<256, 256, MODE_PROJ, 1>(P, dim3(P.tiles_m * P.tiles_n), s);
}

int gemm_bf16_resid_splits(int M, int N, int K) {
  const long long cus = device_cus();
  const long long t128 = (long long)((M + 127) / 128) * ((N + 255) / 256);
  if (t128 >= cus) return 1;
  const long long t256 = (long long)((M + 255) / 256) * ((N + 255) / 256);
  long long sp = (cus + t256 - 1) / t256;
  if (sp > K / 1024) sp = K / 1024;  // at least 16 K steps per split
  if (sp > 16) sp = 16;
  return sp < 2 ? 1 : (int)sp;
}

hipError_t launch_gemm_bf16_raw_wide(const void* A, int lda, int M, int K, const BMap& bm, int N,
                                     int splits, float* raw, hipStream_t s) {
  GemmParams P = base_params(A, lda, M, K, bm, N);
  P.raw = raw;
  P.kchunk = ((K / splits + BK - 1) / BK) * BK;
  P.tiles_m = (M + 255) / 256;
  P.tiles_n = (N + 255) / 256;
  const dim3 grid(P.tiles_m * P.tiles_n, 1, splits);
  return bm.kind == 2 ? launch<256, 256, MODE_RAW, 2>(P, grid, s) : launch<256, 256, MODE_RAW, 0>(P, grid, s);
}

hipError_t launch_gemm_bf16_resid(const void* A, int lda, int M, int K, const BMap& bm, int N,
                                  const void* x, void* out, int ldo, const RowStart& rs, hipStream_t s) {
  GemmParams P = base_params(A, lda, M, K, bm, N);
  P.rs = rs;
  if (P.rs.L < 1) P.rs.L = 1;
  P.x = (const bf16_t*)x;
  P.out = (bf16_t*)out;
  P.ldo = ldo;
  // 256 x 256 tiles when that gives at least one tile per CU, else 128 x 256 tiles
  // (twice as many workgroups).
  const long long t256 = (long long)((M + 255) / 256) * ((N + 255) / 256);
  if (t256 >= 256) {
    P.tiles_m = (M + 255) / 256; P.tiles_n = (N + 255) / 256;
    return bm.kind == 2 ? launch<256, 256, MODE_RESID, 2>(P, dim3(P.tiles_m * P.tiles_n), s)
                        : launch<256, 256, MODE_RESID, 0>(P, dim3(P.tiles_m * P.tiles_n), s);
  }
  P.tiles_m = (M + 127) / 128; P.tiles_n = (N + 255) / 256;
  return bm.kind == 2 ? launch<128, 256, MODE_RESID, 2>(P, dim3(P.tiles_m * P.tiles_n), s)
                      : launch<128, 256, MODE_RESID, 0>(P, dim3(P.tiles_m * P.tiles_n), s);
}

hipError_t launch_gemm_bf16_scaled_f32(const void* A, int lda, int M, int K, const BMap& bm, int N,
                                       float scale, float* out, long long ldo, hipStream_t s) {
  GemmParams P = base_params(A, lda, M, K, bm, N);
  P.outf = out;
  P.ldof = ldo;
  P.scale = scale;
  // Few rows (a decode batch): the table streams through once either way, so smaller
  // row tiles cut the padded MFMA work without adding table reads.
  if (M <= 64) {
    P.tiles_m = 1;
    P.tiles_n = (N + 255) / 256;
    return launch<64, 256, MODE_SCALED, 0>(P, dim3(P.tiles_n), s);
  }
  if (M <= 128) {
    P.tiles_m = 1;
    P.tiles_n = (N + 255) / 256;
    return launch<128, 256, MODE_SCALED, 0>(P, dim3(P.tiles_n), s);
  }
  P.tiles_m = (M + 255) / 256;
  P.tiles_n = (N + 255) / 256;
  return launch<256, 256, MODE_SCALED, 0>(P, dim3(P.tiles_m * P.tiles_n), s);
}

int gemm_bf16_argmax(const void* A, int lda, int M, int K, const BMap& bm, int N, float scale, float* pv,
                     int* pi, hipStream_t s, hipError_t* err) {
  GemmParams P = base_params(A, lda, M, K, bm, N);
  P.outf = pv;
  P.outi = pi;
  P.scale = scale;
  if (M <= 64) {
    P.tiles_m = 1;
    P.tiles_n = (N + 255) / 256;
    *err = launch<64, 256, MODE_ARGMAX, 0>(P, dim3(P.tiles_n), s);
  } else if (M <= 128) {
    P.tiles_m = 1;
    P.tiles_n = (N + 255) / 256;
    *err = launch<128, 256, MODE_ARGMAX, 0>(P, dim3(P.tiles_n), s);
  } else {
    P.tiles_m = (M + 255) / 256;
    P.tiles_n = (N + 255) / 256;
    *err = launch<256, 256, MODE_ARGMAX, 0>(P, dim3(P.tiles_m * P.tiles_n), s);
  }
  return 2 * P.tiles_n;
}

hipError_t launch_gemm_bf16_raw(const void* A, int lda, int M, int K, const BMap& bm, int N,
                                int splits, float* raw, hipStream_t s) {
  GemmParams P = base_params(A, lda, M, K, bm, N);
  P.raw = raw;
  const int kc = ((K / splits + BK - 1) / BK) * BK;
  P.kchunk = kc;
  P.tiles_m = (M + 63) / 64;
  P.tiles_n = (N + 63) / 64;
  const dim3 grid(P.tiles_m * P.tiles_n, 1, splits);
  switch (bm.kind) {
    case 1: return launch<64, 64, MODE_RAW, 1>(P, grid, s);
    case 2: return launch<64, 64, MODE_RAW, 2>(P, grid, s);
    default: return launch<64, 64, MODE_RAW, 0>(P, grid, s);
  }
}

}  // namespace compass
