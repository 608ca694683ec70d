// Elementwise kernels that finish a GEMM whose sums were written raw (fp32 partial
// sums over K-slices), used by the decode path and by the fp32 path:
//   * projection epilogue: interleaved MRoPE on q and k ("Interleaved MRoPE" of the
//     mlxcel Compass issue: x_j' = x_j cos - x_{j+hd/2} sin, x_{j+hd/2}' = x_{j+hd/2}
//     cos + x_j sin with angle pos[axis(j)] * inv_freq[j]), q/k/v scatter into the
//     attention layouts, and act = silu(gate) * up (SwiGLU);
//   * split-K reduction plus the residual (parallel block: out = x + attn + mlp);
//   * the deepstack row update h[rows] += ds ("after layers 0, 1, 2").
// Each thread handles one rotation pair (or one gate/up pair) so that both members
// of the pair are combined in registers.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace compass {
namespace {

// MAXS > 0: at most MAXS splits, every partial load issued before the first add (one memory
// round trip); MAXS = 0: any count, four splits' loads in flight at a time.
template <typename T, int MAXS>
__global__ __launch_bounds__(256) void proj_epilogue_kernel(const float* __restrict__ raw, int splits,
                                                            int M, int N, ProjEpi E, RopeTable rt) {
  const int hd = E.hd, half = hd >> 1;
  const int qkv_units = (E.Hq + 2 * E.Hkv) * half;
  const int units = qkv_units + E.I;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)M * units) return;
  const int m = (int)(idx / units);
  const int u = (int)(idx - (long long)m * units);
  const size_t slab = (size_t)M * N;
  // Sum of the split-K partials of column c: groups of four splits, then the rest, in order.
  auto sum = [&](int c) {
    const float* r = raw + (size_t)m * N + c;
    float s = 0.f;
    int z = 0;
    for (; z + 4 <= splits; z += 4)
      s += (r[z * slab] + r[(z + 1) * slab]) + (r[(z + 2) * slab] + r[(z + 3) * slab]);
    for (; z < splits; ++z) s += r[z * slab];
    return s;
  };
  // The same sum from partials already loaded (the same additions in the same order).
  auto sum_loaded = [&](const float* v) {
    float s = 0.f;
    int z = 0;
#pragma unroll
    for (; z + 4 <= MAXS; z += 4)
      if (z + 4 <= splits) s += (v[z] + v[z + 1]) + (v[z + 2] + v[z + 3]);
#pragma unroll
    for (int y = 0; y < MAXS; ++y)
      if (y >= (splits & ~3) && y < splits) s += v[y];
    return s;
  };
  const bool gu = u >= qkv_units;
  const int hh = u / half, f = u - hh * half;
  const int c1 = hh * hd + f;
  const int cg = u - qkv_units;                                             // gate/up column
  const int vg = (E.nq64 + 2 * E.nk64) * 64 + (cg >> 6) * 128 + (cg & 63);  // virtual gate col
  const int ca = gu ? vg : c1, cb = gu ? vg + 64 : c1 + half;
  // Every load of the thread (partials, cache index, position) is issued before its first use.
  float va[MAXS > 0 ? MAXS : 1], vb[MAXS > 0 ? MAXS : 1];
  if constexpr (MAXS > 0) {
    const float* ra = raw + (size_t)m * N + ca;
    const float* rb = raw + (size_t)m * N + cb;
#pragma unroll
    for (int z = 0; z < MAXS; ++z) {
      va[z] = z < splits ? ra[z * slab] : 0.f;
      vb[z] = z < splits ? rb[z * slab] : 0.f;
    }
  }
  const int lens_b = E.decode ? E.lens[m] : 0;
  const bool rot = E.rope && !gu && hh < E.Hq + E.Hkv;
  const float p = rot ? (float)E.pos[(size_t)rope_axis(rt, f) * E.pos_stride + m] : 0.f;
  float x1, x2;
  if constexpr (MAXS > 0) {
    x1 = sum_loaded(va);
    x2 = sum_loaded(vb);
  } else {
    x1 = sum(ca);
    x2 = sum(cb);
  }
  int b, l, lc;
  if (E.decode) {
    b = m; l = lens_b;
    if (l < 0 || l >= E.cap) return;
    lc = l;
  } else {
    b = m / E.L; l = m - b * E.L;
    lc = l;
    if (E.row_seq) {  // varlen: rows of sequences that are not processed are skipped
      const int sq = E.row_seq[m];
      if (sq < 0) return;
      if (E.kv_by_seq && !gu && u / half >= E.Hq) {  // K/V to the sequence's cache row
        b = sq;
        lc = (E.kv_start ? E.kv_start[sq] : 0) + (m - E.cu[sq]);
      }
    } else if (E.kv_start) {  // chunked prefill: rows whose chunk does not fit the cache are skipped
      const int s0 = E.kv_start[b];
      if (s0 < 0 || s0 > E.cap - E.L) return;
      lc = l + s0;
    }
  }
  if (gu) {
    T* act = (T*)E.act;
    act[(size_t)m * E.ldact + E.act_col0 + cg] = Elt<T>::from_f(silu_f(x1) * x2);
    return;
  }
  T* dst;
  if (hh < E.Hq) {
    dst = (T*)E.q + (((size_t)b * E.Hq + hh) * E.Lq + (E.decode ? 0 : l)) * hd;
  } else {
    const int kv = hh - E.Hq;
    const bool isk = kv < E.Hkv;
    const int head = isk ? kv : kv - E.Hkv;
    dst = (T*)(isk ? E.kc : E.vc) + (((size_t)b * E.Hkv + head) * E.cap + lc) * hd;
  }
  if (rot) {
    float sn, cs;
    sincosf(p * rope_inv_freq(rt, f, hd), &sn, &cs);
    const float y1 = x1 * cs - x2 * sn, y2 = x2 * cs + x1 * sn;
    x1 = y1; x2 = y2;
  }
  dst[f] = Elt<T>::from_f(x1);
  dst[f + half] = Elt<T>::from_f(x2);
}

// out = x + sum of the split-K partials; four consecutive columns per thread (16-byte
// partial loads). N % 4 == 0. SPL > 0: exactly SPL splits, every load issued before the first
// add (one memory round trip); SPL = 0: any count, four splits' loads in flight at a time. The
// additions run in the same order either way: groups of four, then the rest.
template <typename T, int SPL>
__global__ __launch_bounds__(256) void splitk_resid_kernel(const float* __restrict__ raw, int splits,
                                                           int M, int N, const T* x, T* out, RowStart rs) {
  const long long q = (long long)blockIdx.x * 256 + threadIdx.x;  // quad of columns
  if (q * 4 >= (long long)M * N) return;
  const long long idx = q * 4;
  const size_t slab = (size_t)M * N;
  const f32x4_t* r = reinterpret_cast<const f32x4_t*>(raw + idx);
  const size_t sq = slab / 4;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (SPL > 0) {
    f32x4_t v[SPL];
#pragma unroll
    for (int z = 0; z < SPL; ++z) v[z] = r[z * sq];
    int z = 0;
#pragma unroll
    for (; z + 4 <= SPL; z += 4) acc += (v[z] + v[z + 1]) + (v[z + 2] + v[z + 3]);
#pragma unroll
    for (; z < SPL; ++z) acc += v[z];
  } else {
    int z = 0;
    for (; z + 4 <= splits; z += 4)
      acc += (r[z * sq] + r[(z + 1) * sq]) + (r[(z + 2) * sq] + r[(z + 3) * sq]);
    for (; z < splits; ++z) acc += r[z * sq];
  }
  if (!row_live_m(rs, (int)(idx / N))) return;  // rows left untouched
#pragma unroll
  for (int e = 0; e < 4; ++e) out[idx + e] = Elt<T>::from_f(Elt<T>::to_f(x[idx + e]) + acc[e]);
}

// The bf16 split-K residual of a decode layer fused with the next layer's LayerNorm. One
// workgroup per row: each thread forms 8 columns of out = x + sum of the partials with the
// additions of splitk_resid_kernel and keeps the bf16 results (as floats) in LDS; wave 0
// takes the row's mean and biased variance in the LayerNorm kernel's own order (lane l sums
// columns 8 (64 i + l) .. + 8 for i = 0, 1, ..., then the xor-shuffle reduction); every
// thread then writes its 8 columns of (y - mean) * rstd * ln_w with the LayerNorm kernel's
// expression and rounding, so norm is what that kernel would write for out. Rows that are
// not live are left untouched.
template <int SPL>
__global__ __launch_bounds__(256) void splitk_resid_ln_kernel(const float* __restrict__ raw, int splits, int M,
                                                              int N, const bf16_t* x, bf16_t* out, RowStart rs,
                                                              const bf16_t* __restrict__ ln_w, float eps,
                                                              bf16_t* __restrict__ norm) {
  extern __shared__ float s_y[];  // [N], then (mean, rstd)
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  if (!row_live_m(rs, row)) return;
  // The weight of this thread's first 8 columns is loaded with the partials, not after the
  // statistics (one memory round trip fewer; N <= 2048 has no other columns).
  u32x4_t w_first = {0u, 0u, 0u, 0u};
  if (tid * 8 < N) w_first = *reinterpret_cast<const u32x4_t*>(ln_w + tid * 8);
  const size_t sq = (size_t)M * N / 4;
  for (int c = tid * 8; c < N; c += 256 * 8) {
    const size_t idx = (size_t)row * N + c;
    const f32x4_t* r = reinterpret_cast<const f32x4_t*>(raw + idx);
    const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(x + idx);
    const uint32_t x4[4] = {xv.x, xv.y, xv.z, xv.w};
    uint32_t o4[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // two quads of columns
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (SPL > 0) {
        f32x4_t v[SPL];
#pragma unroll
        for (int z = 0; z < SPL; ++z) v[z] = r[z * sq + h];
        int z = 0;
#pragma unroll
        for (; z + 4 <= SPL; z += 4) acc += (v[z] + v[z + 1]) + (v[z + 2] + v[z + 3]);
#pragma unroll
        for (; z < SPL; ++z) acc += v[z];
      } else {
        int z = 0;
        for (; z + 4 <= splits; z += 4)
          acc += (r[z * sq + h] + r[(z + 1) * sq + h]) + (r[(z + 2) * sq + h] + r[(z + 3) * sq + h]);
        for (; z < splits; ++z) acc += r[z * sq + h];
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t xw = x4[2 * h + j];
        const bf16_t y0 = f2bf(__uint_as_float(xw << 16) + acc[2 * j]);
        const bf16_t y1 = f2bf(__uint_as_float(xw & 0xffff0000u) + acc[2 * j + 1]);
        o4[2 * h + j] = (uint32_t)y0 | ((uint32_t)y1 << 16);
        s_y[c + 4 * h + 2 * j] = bf2f(y0);
        s_y[c + 4 * h + 2 * j + 1] = bf2f(y1);
      }
    }
    *reinterpret_cast<u32x4_t*>(out + idx) = u32x4_t{o4[0], o4[1], o4[2], o4[3]};
  }
  __syncthreads();
  if (tid < 64) {
    float sum = 0.f;
    for (int e = lane * 8; e < N; e += 512)
#pragma unroll
      for (int j = 0; j < 8; ++j) sum += s_y[e + j];
    const float mean = wave_sum(sum) / (float)N;
    float q = 0.f;
    for (int e = lane * 8; e < N; e += 512)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float d = s_y[e + j] - mean;
        q += d * d;
      }
    const float var = wave_sum(q) / (float)N;
    if (lane == 0) {
      s_y[N] = mean;
      s_y[N + 1] = 1.0f / sqrtf(var + eps);
    }
  }
  __syncthreads();
  const float mean = s_y[N], rstd = s_y[N + 1];
  for (int c = tid * 8; c < N; c += 256 * 8) {
    const u32x4_t wr = c == tid * 8 ? w_first : *reinterpret_cast<const u32x4_t*>(ln_w + c);
    const uint32_t w4[4] = {wr.x, wr.y, wr.z, wr.w};
    uint32_t o4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float w0 = __uint_as_float(w4[j] << 16), w1 = __uint_as_float(w4[j] & 0xffff0000u);
      o4[j] = pack_bf2((s_y[c + 2 * j] - mean) * rstd * w0, (s_y[c + 2 * j + 1] - mean) * rstd * w1);
    }
    *reinterpret_cast<u32x4_t*>(norm + (size_t)row * N + c) = u32x4_t{o4[0], o4[1], o4[2], o4[3]};
  }
}

template <typename T>
__global__ __launch_bounds__(256) void deepstack_kernel(const int32_t* __restrict__ rows,
                                                        const T* __restrict__ ds, int D, int n_rows,
                                                        RowStart rs, T* out) {
  const int r = blockIdx.x;
  const int row = rows[r];
  if (row < 0 || row >= n_rows || !row_live_m(rs, row)) return;
  for (int c = blockIdx.y * 256 + threadIdx.x; c < D; c += gridDim.y * 256) {
    T* o = out + (size_t)row * D + c;
    *o = Elt<T>::from_f(Elt<T>::to_f(*o) + Elt<T>::to_f(ds[(size_t)r * D + c]));
  }
}

// The same update with 16 bytes per thread (one workgroup per deepstack row at D = 2048 bf16):
// each thread loads its piece of the output row and of the deepstack row together.
template <typename T>
__global__ __launch_bounds__(256) void deepstack_vec_kernel(const int32_t* __restrict__ rows,
                                                            const T* __restrict__ ds, int D, int n_rows,
                                                            RowStart rs, T* out) {
  constexpr int VEC = 16 / sizeof(T);
  const int r = blockIdx.x;
  const int row = rows[r];
  if (row < 0 || row >= n_rows || !row_live_m(rs, row)) return;
  for (int c = (blockIdx.y * 256 + threadIdx.x) * VEC; c < D; c += gridDim.y * 256 * VEC) {
    u32x4_t* o = reinterpret_cast<u32x4_t*>(out + (size_t)row * D + c);
    const u32x4_t a = *o, b = *reinterpret_cast<const u32x4_t*>(ds + (size_t)r * D + c);
    const T* av = reinterpret_cast<const T*>(&a);
    const T* bv = reinterpret_cast<const T*>(&b);
    u32x4_t res;
    T* rv = reinterpret_cast<T*>(&res);
#pragma unroll
    for (int e = 0; e < VEC; ++e) rv[e] = Elt<T>::from_f(Elt<T>::to_f(av[e]) + Elt<T>::to_f(bv[e]));
    *o = res;
  }
}

}  // namespace

hipError_t launch_proj_epilogue(int dtype, const float* raw, int splits, int M, int N,
                                const ProjEpi& ep, const RopeTable& rt, hipStream_t s) {
  const long long units = (long long)M * ((ep.Hq + 2 * ep.Hkv) * (ep.hd / 2) + ep.I);
  const dim3 grid((unsigned)((units + 255) / 256));
  if (dtype == 1) {
    if (splits <= 4) proj_epilogue_kernel<bf16_t, 4><<<grid, 256, 0, s>>>(raw, splits, M, N, ep, rt);
    else proj_epilogue_kernel<bf16_t, 0><<<grid, 256, 0, s>>>(raw, splits, M, N, ep, rt);
  } else {
    if (splits <= 4) proj_epilogue_kernel<float, 4><<<grid, 256, 0, s>>>(raw, splits, M, N, ep, rt);
    else proj_epilogue_kernel<float, 0><<<grid, 256, 0, s>>>(raw, splits, M, N, ep, rt);
  }
  return hipGetLastError();
}

hipError_t launch_splitk_resid_ln(const float* raw, int splits, int M, int N, const void* x, void* out,
                                  const RowStart& rs_in, const void* ln_w, float eps, void* norm, hipStream_t s) {
  if (N % 8 != 0) return hipErrorInvalidValue;
  RowStart rs = rs_in;
  if (rs.L < 1) rs.L = 1;
  const size_t lds = (size_t)(N + 2) * sizeof(float);
  auto go = [&](auto spl) -> hipError_t {
    constexpr int SPL = decltype(spl)::value;
    const hipError_t e = ensure_dynamic_lds((const void*)splitk_resid_ln_kernel<SPL>, (int)lds);
    if (e != hipSuccess) return e;
    splitk_resid_ln_kernel<SPL><<<M, 256, lds, s>>>(raw, splits, M, N, (const bf16_t*)x, (bf16_t*)out, rs,
                                                   (const bf16_t*)ln_w, eps, (bf16_t*)norm);
    return hipGetLastError();
  };
  switch (splits) {
    case 1: return go(std::integral_constant<int, 1>{});
    case 2: return go(std::integral_constant<int, 2>{});
    case 4: return go(std::integral_constant<int, 4>{});
    case 8: return go(std::integral_constant<int, 8>{});
    case 16: return go(std::integral_constant<int, 16>{});
    default: return go(std::integral_constant<int, 0>{});
  }
}

hipError_t launch_splitk_resid(int dtype, const float* raw, int splits, int M, int N, const void* x,
                               void* out, const RowStart& rs_in, hipStream_t s) {
  const long long n = (long long)M * N / 4;  // column quads (N % 4 == 0)
  const dim3 grid((unsigned)((n + 255) / 256));
  RowStart rs = rs_in;
  if (rs.L < 1) rs.L = 1;
  auto go = [&](auto spl) {
    constexpr int SPL = decltype(spl)::value;
    if (dtype == 1)
      splitk_resid_kernel<bf16_t, SPL><<<grid, 256, 0, s>>>(raw, splits, M, N, (const bf16_t*)x, (bf16_t*)out, rs);
    else
      splitk_resid_kernel<float, SPL><<<grid, 256, 0, s>>>(raw, splits, M, N, (const float*)x, (float*)out, rs);
  };
  switch (splits) {
    case 1: go(std::integral_constant<int, 1>{}); break;
    case 2: go(std::integral_constant<int, 2>{}); break;
    case 4: go(std::integral_constant<int, 4>{}); break;
    case 8: go(std::integral_constant<int, 8>{}); break;
    case 16: go(std::integral_constant<int, 16>{}); break;
    default: go(std::integral_constant<int, 0>{});
  }
  return hipGetLastError();
}

hipError_t launch_deepstack(int dtype, const int32_t* rows, const void* ds, int n_ds, int D,
                            int n_rows, const RowStart& rs_in, void* out, hipStream_t s) {
  if (n_ds <= 0) return hipSuccess;
  RowStart rs = rs_in;
  if (rs.L < 1) rs.L = 1;
  const int esz = dtype == 1 ? 2 : 4;
  const int vec = 16 / esz;
  if (D % vec == 0 && ((uintptr_t)ds & 15) == 0 && ((uintptr_t)out & 15) == 0) {
    const int per_wg = 256 * vec;
    const dim3 grid(n_ds, (D + per_wg - 1) / per_wg);
    if (dtype == 1)
      deepstack_vec_kernel<bf16_t><<<grid, 256, 0, s>>>(rows, (const bf16_t*)ds, D, n_rows, rs, (bf16_t*)out);
    else
      deepstack_vec_kernel<float><<<grid, 256, 0, s>>>(rows, (const float*)ds, D, n_rows, rs, (float*)out);
    return hipGetLastError();
  }
  const dim3 grid(n_ds, (D + 255) / 256);
  if (dtype == 1)
    deepstack_kernel<bf16_t><<<grid, 256, 0, s>>>(rows, (const bf16_t*)ds, D, n_rows, rs, (bf16_t*)out);
  else
    deepstack_kernel<float><<<grid, 256, 0, s>>>(rows, (const float*)ds, D, n_rows, rs, (float*)out);
  return hipGetLastError();
}

}  // namespace compass
