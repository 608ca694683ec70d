// Shared definitions of the bf16 MFMA GEMM kernels: parameters, LDS swizzle, tile
// order and the epilogues (fused projection with interleaved MRoPE / q-k-v scatter /
// SwiGLU, residual add, scaled fp32 store, raw fp32 partial sums).
#pragma once
#include "common.h"
#include "launch.h"

namespace compass {
namespace gemm {

enum { MODE_PROJ = 0, MODE_RESID = 1, MODE_SCALED = 2, MODE_RAW = 3, MODE_ARGMAX = 4 };

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
  float* outf;       // SCALED; ARGMAX: per-row partial maxima [M][2 * tiles_n]
  long long ldof;
  float scale;       // SCALED, ARGMAX
  int* outi;         // ARGMAX: the ids of those maxima
  RowStart rs;       // RESID: rows of batch rows that are not live are not stored
  ProjEpi ep;        // PROJ
  RopeTable rt;
  // PROJ with the LayerNorm fused: A is the layer input x, each A piece is normalized in
  // registers as (x - mean) * rstd * ln_w before it is staged in LDS.
  const float2* ln_stats;  // [M] (mean, rstd)
  const bf16_t* ln_w;      // [K]
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

// Epilogue layout. The wave's block (i, j) covers rows mw0 + 32 i .. and columns
// nw0 + 32 j ..; result register r of lane l holds row 8 (r / 4) + 4 (l / 32) + r % 4
// and column l % 32. Each group of 4 registers (rows 8 g + 4 (l / 32) + 0..3) is
// transposed inside lane quads (quad_transpose), after which the lane holds 4
// consecutive columns (l % 32) & ~3 .. + 3 of one row 8 g + 4 (l / 32) + rsel and
// stores them with one 8-byte (bf16) or 16-byte (fp32) access.
__device__ __forceinline__ int epi_row(int lane) {
  const int q = lane & 3;
  return 4 * (lane >> 5) + 2 * (q & 1) + (q >> 1);
}

template <int MB, int NB>
__device__ __forceinline__ void load_group(const f32x16_t (&acc)[MB][NB], int i, int j, int g, float (&v)[4]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) v[t] = acc[i][j][4 * g + t];
}

// dst is device (global) memory: the store is issued as a global store even where the
// compiler cannot trace dst back to a kernel argument (a flat store would also count as an
// LDS / scalar-memory operation in the waits that follow it).
__device__ __forceinline__ void store_bf16x4(bf16_t* dst, const float (&v)[4]) {
  u32x2_t o;
  o.x = pack_bf2(v[0], v[1]);
  o.y = pack_bf2(v[2], v[3]);
  *(__attribute__((address_space(1))) u32x2_t*)dst = o;
}
// The same with a streaming hint: for outputs no later kernel reads while they could still
// be in this XCD's L2, so they leave no dirty lines for the write-back at the kernel's end.
__device__ __forceinline__ void store_bf16x4_nt(bf16_t* dst, const float (&v)[4]) {
  u32x2_t o;
  o.x = pack_bf2(v[0], v[1]);
  o.y = pack_bf2(v[2], v[3]);
  __builtin_nontemporal_store(o, reinterpret_cast<u32x2_t*>(dst));
}

// Regroups two transposed 4-column pieces of each lane's row, p0 at columns col4.. and p1
// at 32 + col4.. of a 64-column span, across the half-waves (v_permlane32_swap): afterwards
// p0 belongs to row (rowq & 3) and p1 to row (rowq & 3) + 4 of the 8-row group, both at
// column (lane >= 32 ? 32 : 0) + col4, so that one store instruction writes 4 rows x 128
// contiguous bytes (whole cache lines) instead of 8 rows x 64 bytes.
__device__ __forceinline__ void line_swap(u32x2_t& p0, u32x2_t& p1) {
  const auto a = __builtin_amdgcn_permlane32_swap(p0.x, p1.x, false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(p0.y, p1.y, false, false);
  const unsigned a0 = a[0], a1 = a[1], b0 = b[0], b1 = b[1];
  p0 = u32x2_t{a0, b0};
  p1 = u32x2_t{a1, b1};
}

// Per-row data of the fused projection epilogue, staged in LDS by the workgroup (one row
// per thread) after the main loop, so that the loads it takes (positions, decode cache
// indices, chunk starts, varlen sequences) are issued once per row and together, and the
// waves' epilogues read them from LDS: an LDS read does not wait for earlier global stores,
// while a global load does (global loads and stores retire through one in-order counter).
struct ProjRow {
  int b, lq;    // q: batch row and query index
  int bkv, lc;  // k / v: cache row and cache index
  float pt, ph, pw;
  int kv;       // 1: the row's K / V are written
};

template <int BM>
__device__ __forceinline__ void stage_proj_rows(const GemmParams& P, int m0, ProjRow* s_row, int tid) {
  const ProjEpi& E = P.ep;
  for (int r = tid; r < BM; r += 256) {
    const int m = m0 + r;
    const int mm = min(m, P.M - 1);
    int pi[3] = {0, 0, 0};
    if (E.rope) {
#pragma unroll
      for (int a = 0; a < 3; ++a) pi[a] = E.pos[(size_t)a * E.pos_stride + mm];
    }
    int b, l;
    if (E.decode) { b = mm; l = E.lens[mm]; } else { b = mm / E.L; l = mm - b * E.L; }
    // Cache row and index of this row's K/V: chunked prefill continues after kv_start[b]
    // tokens (rows whose chunk does not fit are not written); a packed varlen row goes to
    // its sequence's cache row (or stays in the packed scratch).
    int bkv = b, lc = l;
    bool kv = m < P.M;
    if (!E.decode) {
      if (E.row_seq) {
        const int sq = E.row_seq[mm];
        kv = kv && sq >= 0;
        if (E.kv_by_seq && sq >= 0) {
          bkv = sq;
          lc = (E.kv_start ? E.kv_start[sq] : 0) + (mm - E.cu[sq]);
        }
      } else if (E.kv_start) {
        const int s0 = E.kv_start[b];
        kv = kv && s0 >= 0 && s0 <= E.cap - E.L;
        lc = l + (kv ? s0 : 0);
      }
    }
    ProjRow R;
    R.b = b;
    R.lq = E.decode ? 0 : l;
    R.bkv = bkv;
    R.lc = lc;
    R.pt = (float)pi[0];
    R.ph = (float)pi[1];
    R.pw = (float)pi[2];
    R.kv = kv ? 1 : 0;
    s_row[r] = R;
  }
}

// q / k / v part of the fused projection epilogue for head_dim HD. For HD = 128 the
// wave's 128 columns are one head (first half blocks 0, 1, second half 2, 3); for
// HD = 64 two heads (blocks {0, 1} and {2, 3}). Pairs (x_f, x_{f + HD/2}) sit in the
// same lane and register of blocks j and j + HD/64, so MRoPE is applied after the
// transpose, on whole rows. The rotation angle pos * inv_freq is evaluated in
// revolutions (inv_freq / 2 pi rounded once to fp32, reduced to [-1/2, 1/2]) for the
// hardware sin / cos.
template <int HD, int MB, int NB>
__device__ __forceinline__ void proj_qkv_epilogue(const GemmParams& P, const f32x16_t (&acc)[MB][NB], int mw0,
                                                  int ch0, int lane, const ProjRow* s_row) {
  constexpr int PB = HD / 64;          // 32-column blocks per half head
  constexpr int NHEAD = 128 / HD;      // heads per wave
  constexpr int HALF = HD / 2;
  const ProjEpi& E = P.ep;
  const int qe = E.nq64, ke = qe + E.nk64;
  const int col4 = (lane & 31) & ~3;
  const int rowq = epi_row(lane);

  // Inverse frequencies (in revolutions per position) and axes of this lane's columns:
  // frequency 32 jj + col4 + t of the first half.
  float invr[PB][4];
  int axis[PB][4];
  if (!P.rt.layout) {
    // Interleaved layout: consecutive pairs have consecutive frequency indices.
    const double th = (double)P.rt.theta;
    const double r1 = pow(th, -2.0 / HD), r32 = pow(th, -64.0 / HD);
    double f0 = pow(th, -2.0 * col4 / HD) * 0.15915494309189535;  // / (2 pi)
#pragma unroll
    for (int jj = 0; jj < PB; ++jj) {
      double f = f0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        invr[jj][t] = (float)f;
        axis[jj][t] = rope_axis(P.rt, 32 * jj + col4 + t);
        f *= r1;
      }
      f0 *= r32;
    }
  } else {
    const double l2t = log2((double)P.rt.theta);
#pragma unroll
    for (int jj = 0; jj < PB; ++jj)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int f = 32 * jj + col4 + t;
        invr[jj][t] = (float)(exp2(-2.0 * rope_freq_index(P.rt, f) / HD * l2t) * 0.15915494309189535);
        axis[jj][t] = rope_axis(P.rt, f);
      }
  }

#pragma unroll
  for (int hf = 0; hf < NHEAD; ++hf) {
    const int ch = ch0 + hf * PB;  // first 64-column chunk of this head
    int kind, head;
    if (ch < qe) { kind = 0; head = ch * 64 / HD; }
    else if (ch < ke) { kind = 1; head = (ch - qe) * 64 / HD; }
    else { kind = 2; head = (ch - ke) * 64 / HD; }
    const bool rot = E.rope && kind < 2;
    // Pointer chosen arithmetically: a select between fields of P would become a load
    // through a selected address and force P out of registers.
    const uint64_t sel_q = kind == 0, sel_k = kind == 1, sel_v = kind == 2;
    bf16_t* const base = (bf16_t*)(sel_q * (uint64_t)E.q + sel_k * (uint64_t)E.kc + sel_v * (uint64_t)E.vc);
    const int jlo = hf * 2 * PB;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int m = mw0 + 32 * i + 8 * g + rowq;
        const ProjRow R = s_row[32 * i + 8 * g + rowq];  // s_row starts at the wave's first row
        bool store = m < P.M;
        bf16_t* dst;
        if (kind == 0) {
          dst = base + (((size_t)R.b * E.Hq + head) * E.Lq + R.lq) * HD;
        } else {
          store = store && R.kv;
          dst = base + (((size_t)R.bkv * E.Hkv + head) * E.cap + R.lc) * HD;
        }
        const float pt = R.pt, ph = R.ph, pw = R.pw;
#pragma unroll
        for (int jj = 0; jj < PB; ++jj) {
          float x1[4], x2[4];
          load_group(acc, i, jlo + jj, g, x1);
          load_group(acc, i, jlo + jj + PB, g, x2);
          quad_transpose(x1, lane);
          quad_transpose(x2, lane);
          if (rot) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const float p = axis[jj][t] == 0 ? pt : axis[jj][t] == 1 ? ph : pw;
              float rev = p * invr[jj][t];
              rev -= rintf(rev);
              const float sn = __builtin_amdgcn_sinf(rev), cs = __builtin_amdgcn_cosf(rev);
              const float y1 = x1[t] * cs - x2[t] * sn, y2 = x2[t] * cs + x1[t] * sn;
              x1[t] = y1;
              x2[t] = y2;
            }
          }
          if (store) {
            store_bf16x4(dst + 32 * jj + col4, x1);
            store_bf16x4(dst + HALF + 32 * jj + col4, x2);
          }
        }
      }
  }
}

// ARGMAX: per row, the largest scale * C over the wave's 128 columns and its column
// (smallest column on ties; NaN never wins), written as partial 2 tn + wn of the row.
// Register r of lane l holds row 8 (r / 4) + 4 (l / 32) + r % 4 of each block, column
// l % 32: the scan runs over the blocks j in column order, then over the 32 lanes of
// each half-wave (the xor offsets below 32 stay inside a half).
template <int MB, int NB>
__device__ __forceinline__ void argmax_epilogue(const GemmParams& P, const f32x16_t (&acc)[MB][NB], int mw0,
                                                int nw0, int part, int lane) {
  const int c = lane & 31;
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int n = nw0 + 32 * j + c;
        const float x = acc[i][j][r] * P.scale;
        if (n < P.N && x > bv) { bv = x; bi = n; }
      }
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      const int m = mw0 + 32 * i + 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
      if (c == 0 && m < P.M) {
        const size_t o = (size_t)m * (2 * P.tiles_n) + part;
        P.outf[o] = bv;
        P.outi[o] = bi;
      }
    }
}

// Stores one wave's accumulators (MB x NB blocks of 32 x 32 at rows mw0.., columns nw0..).
// RAW, RESID and PROJ need N and the row strides to be multiples of 4 (checked by the
// launchers); SCALED falls back to element stores otherwise.
template <int MODE, int MB, int NB>
__device__ __forceinline__ void gemm_epilogue(const GemmParams& P, f32x16_t (&acc)[MB][NB], int mw0,
                                              int nw0, int lane, int z, const ProjRow* s_row = nullptr) {
  const int col4 = (lane & 31) & ~3;
  const int rowq = epi_row(lane);
  if constexpr (MODE == MODE_RESID) {
    // The residual values and row flags of two row blocks at a time are loaded before their
    // first store: global loads and stores retire through one in-order counter, so a load
    // issued after a store would also wait for that store (one memory round trip per row
    // group instead of one per two row blocks).
    constexpr int IC = MB < 2 ? MB : 2;
#pragma unroll
    for (int i0 = 0; i0 < MB; i0 += IC) {
      bool live[IC][4];
      u32x2_t xv[IC][NB][4];
#pragma unroll
      for (int ii = 0; ii < IC; ++ii)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int m = mw0 + 32 * (i0 + ii) + 8 * g + rowq;
          live[ii][g] = m < P.M && row_live_m(P.rs, m);
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const int n = nw0 + 32 * j + col4;
            if (live[ii][g] && n < P.N) xv[ii][j][g] = *reinterpret_cast<const u32x2_t*>(P.x + (size_t)m * P.ldo + n);
          }
        }
#pragma unroll
      for (int ii = 0; ii < IC; ++ii)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float v[4];
            load_group(acc, i0 + ii, j, g, v);
            quad_transpose(v, lane);
            const int m = mw0 + 32 * (i0 + ii) + 8 * g + rowq;
            const int n = nw0 + 32 * j + col4;
            if (!live[ii][g] || n >= P.N) continue;
            const u32x2_t x2 = xv[ii][j][g];
            v[0] += __uint_as_float(x2.x << 16);
            v[1] += __uint_as_float(x2.x & 0xffff0000u);
            v[2] += __uint_as_float(x2.y << 16);
            v[3] += __uint_as_float(x2.y & 0xffff0000u);
            store_bf16x4_nt(P.out + (size_t)m * P.ldo + n, v);
          }
    }
  } else if constexpr (MODE == MODE_RAW || MODE == MODE_SCALED) {
    const bool vec = MODE == MODE_RAW || ((P.N & 3) == 0 && (P.ldof & 3) == 0);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float v[4];
          load_group(acc, i, j, g, v);
          quad_transpose(v, lane);
          const int m = mw0 + 32 * i + 8 * g + rowq;
          const int n = nw0 + 32 * j + col4;
          if (m >= P.M || n >= P.N) continue;
          if constexpr (MODE == MODE_RAW) {
            *reinterpret_cast<f32x4_t*>(P.raw + ((size_t)z * P.M + m) * P.N + n) = f32x4_t{v[0], v[1], v[2], v[3]};
          } else {
            float* d = P.outf + (size_t)m * P.ldof + n;
            if (vec) {
              *reinterpret_cast<f32x4_t*>(d) = f32x4_t{v[0] * P.scale, v[1] * P.scale, v[2] * P.scale, v[3] * P.scale};
            } else {
#pragma unroll
              for (int t = 0; t < 4; ++t)
                if (n + t < P.N) d[t] = v[t] * P.scale;
            }
          }
        }
  } else {
    // MODE_PROJ: requires WN == 128 (BN == 256).
    static_assert(MODE != MODE_PROJ || NB == 4, "fused projection epilogue needs 128-column waves");
    const ProjEpi& E = P.ep;
    if (nw0 >= P.N) return;  // wave-uniform
    const int ch0 = nw0 >> 6;
    const int ve = E.nq64 + 2 * E.nk64;
    if (ch0 >= ve) {
      // SwiGLU: chunk ch0 holds gate columns, ch0 + 1 the up columns of the same c.
      // Every value of the wave is computed (and packed to bf16) before the first store: a
      // vector-memory operation that followed a store (a spill reload, say) would wait for
      // it, global loads and stores retiring through one in-order counter.
      bf16_t* act = (bf16_t*)E.act + E.act_col0 + ((ch0 - ve) >> 1) * 64 + (lane >= 32 ? 32 : 0) + col4;
      const int rlo = rowq & 3;
      u32x2_t o[MB][4][2];
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            float v[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] = silu_f(acc[i][j][4 * g + t]) * acc[i][j + 2][4 * g + t];
            o[i][g][j] = quad_transpose_bf16(v, lane);
          }
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          line_swap(o[i][g][0], o[i][g][1]);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int m = mw0 + 32 * i + 8 * g + 4 * h + rlo;
            if (m < P.M) __builtin_nontemporal_store(o[i][g][h], reinterpret_cast<u32x2_t*>(act + (size_t)m * E.ldact));
          }
        }
      return;
    }
    if (E.hd == 128) proj_qkv_epilogue<128>(P, acc, mw0, ch0, lane, s_row);
    else proj_qkv_epilogue<64>(P, acc, mw0, ch0, lane, s_row);
  }
}

}  // namespace gemm
}  // namespace compass
