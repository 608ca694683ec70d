// Shared definitions of the bf16 MFMA GEMM kernels: parameters, LDS swizzle, tile
// order and the epilogues (fused projection with interleaved MRoPE / q-k-v scatter /
// SwiGLU, residual add, scaled fp32 store, raw fp32 partial sums).
#pragma once
#include "common.h"
#include "launch.h"

namespace compass {
namespace gemm {

enum { MODE_PROJ = 0, MODE_RESID = 1, MODE_SCALED = 2, MODE_RAW = 3 };

struct GemmParams {
  const bf16_t* A;
  int lda, M, K, N;
  BMap bm;
  int kchunk;        // K elements per split (RAW)
  int tiles_m, tiles_n;
  float* raw;        // RAW
  const bf16_t* x;   // RESID
  bf16_t* out;
  int ldo;
  float* outf;       // SCALED
  long long ldof;
  float scale;
  ProjEpi ep;        // PROJ
  RopeTable rt;
};

constexpr int BK = 64;

// LDS offset (elements) of 16-byte chunk `chunk` of tile row `row` (rows of 64 bf16).
// The chunk is XOR-swizzled with (row & 7) ^ ((row >> 3) & 1): the fragment reads of
// 16 consecutive rows at one chunk then hit 16 distinct 16-byte bank slots of a
// 256-byte bank window (and 8 consecutive rows hit distinct slots of 128 bytes).
__device__ __forceinline__ int swz(int row, int chunk) {
  return (row << 6) + ((chunk ^ (row & 7) ^ ((row >> 3) & 1)) << 3);
}

// Workgroup id -> (tile_m, tile_n). Consecutive workgroup ids go round-robin over the
// 8 XCDs; ids are first regrouped so that each XCD gets a contiguous range of logical
// tiles, and logical tiles are ordered in column groups of GROUP_M row-tiles so that
// the tiles resident on one XCD at a time share A rows and B rows in its L2.
template <int GROUP_M>
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  const int nwg = tiles_m * tiles_n;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, local = bid >> 3;
  const int per = nwg >> 3, extra = nwg & 7;
  const int logical = xcd * per + min(xcd, extra) + local;
  const int group = logical / (GROUP_M * tiles_n);
  const int first_m = group * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int in_group = logical - group * GROUP_M * tiles_n;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

// Stores one wave's accumulators: MB x NB blocks of 32 x 32; the wave's block (i, j)
// covers rows mw0 + 32 i .. and columns nw0 + 32 j ... Result register r of lane l holds
// row 8 (r / 4) + 4 (l / 32) + r % 4 and column l % 32 of a block.
template <int MODE, int MB, int NB>
__device__ __forceinline__ void gemm_epilogue(const GemmParams& P, f32x16_t (&acc)[MB][NB], int mw0,
                                              int nw0, int lane, int z) {
  const int col_l = lane & 31;
  const int row_l = 4 * (lane >> 5);
  if constexpr (MODE == MODE_RAW || MODE == MODE_RESID || MODE == MODE_SCALED) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int n = nw0 + 32 * j + col_l;
        if (n >= P.N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = mw0 + 32 * i + 8 * (r >> 2) + row_l + (r & 3);
          if (m >= P.M) continue;
          const float v = acc[i][j][r];
          if constexpr (MODE == MODE_RAW) {
            P.raw[((size_t)z * P.M + m) * P.N + n] = v;
          } else if constexpr (MODE == MODE_RESID) {
            const size_t o = (size_t)m * P.ldo + n;
            P.out[o] = f2bf(bf2f(P.x[o]) + v);
          } else {
            P.outf[(size_t)m * P.ldof + n] = v * P.scale;
          }
        }
      }
  } else {
    // MODE_PROJ: requires WN == 128 (BN == 256); see the header comment.
    static_assert(MODE != MODE_PROJ || NB == 4, "fused projection epilogue needs 128-column waves");
    const ProjEpi& E = P.ep;
    if (nw0 >= P.N) return;
    const int ch0 = nw0 >> 6;
    const int qe = E.nq64, ke = qe + E.nk64, ve = ke + E.nk64;
    const int hd = E.hd;
    if (ch0 >= ve) {
      // SwiGLU: chunk ch0 is gate columns, ch0 + 1 the up columns of the same c.
      const int cbase = ((ch0 - ve) >> 1) * 64;
      bf16_t* act = (bf16_t*)E.act;
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = mw0 + 32 * i + 8 * (r >> 2) + row_l + (r & 3);
          if (m >= P.M) continue;
          bf16_t* dst = act + (size_t)m * E.ldact + E.act_col0 + cbase + col_l;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const float g = acc[i][j][r], u = acc[i][j + 2][r];
            dst[32 * j] = f2bf(silu_f(g) * u);
          }
        }
      return;
    }
    // q / k / v heads. For hd == 128 the wave holds one head: halves are blocks {0,1}
    // and {2,3}. For hd == 64 it holds two heads: blocks {0,1} and {2,3}.
    // This lane's frequencies: col_l (+ 32 for hd == 128).
    float invf[2];
    int axf[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int f = 32 * j + col_l;
      invf[j] = rope_inv_freq(P.rt, f, hd);
      axf[j] = rope_axis(P.rt, f);
    }
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      if (hd == 128 && hf == 1) break;
      const int ch = ch0 + hf;  // first chunk of this head
      int kind, head;
      if (ch < qe) { kind = 0; head = ch * 64 / hd; }
      else if (ch < ke) { kind = 1; head = (ch - qe) * 64 / hd; }
      else { kind = 2; head = (ch - ke) * 64 / hd; }
      const int half = hd >> 1;
      const bool rot = E.rope && kind < 2;
      // Blocks of this head: jlo .. jlo + hd/32 - 1; partner of block j is j + half/32.
      const int jlo = (hd == 128) ? 0 : 2 * hf;
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = mw0 + 32 * i + 8 * (r >> 2) + row_l + (r & 3);
          if (m >= P.M) continue;
          int b, l;
          if (E.decode) { b = m; l = E.lens[b]; } else { b = m / E.L; l = m - b * E.L; }
          bf16_t* dst;
          if (kind == 0) dst = (bf16_t*)E.q + (((size_t)b * E.Hq + head) * E.Lq + (E.decode ? 0 : l)) * hd;
          else dst = (bf16_t*)(kind == 1 ? E.kc : E.vc) + (((size_t)b * E.Hkv + head) * E.cap + l) * hd;
          if (hd == 128) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              float x1 = acc[i][j][r], x2 = acc[i][j + 2][r];
              const int f = 32 * j + col_l;
              if (rot) {
                const float p = (float)E.pos[(size_t)axf[j] * E.pos_stride + m];
                float sn, cs;
                sincosf(p * invf[j], &sn, &cs);
                const float y1 = x1 * cs - x2 * sn, y2 = x2 * cs + x1 * sn;
                x1 = y1; x2 = y2;
              }
              dst[f] = f2bf(x1);
              dst[f + half] = f2bf(x2);
            }
          } else {
            float x1 = acc[i][jlo][r], x2 = acc[i][jlo + 1][r];
            const int f = col_l;
            if (rot) {
              const float p = (float)E.pos[(size_t)axf[0] * E.pos_stride + m];
              float sn, cs;
              sincosf(p * invf[0], &sn, &cs);
              const float y1 = x1 * cs - x2 * sn, y2 = x2 * cs + x1 * sn;
              x1 = y1; x2 = y2;
            }
            dst[f] = f2bf(x1);
            dst[f + half] = f2bf(x2);
          }
        }
    }
  }
}

}  // namespace gemm
}  // namespace compass
