// Plain fp32 C++ CPU reference of the Compass/Cohere2 parallel decoder layer.
//
// TEST INFRASTRUCTURE ONLY: only the tests (and the build step that compiles it) use this
// file; the HIP library shares no code with it. It is a second, independent oracle next
// to the fp64 numpy one: data are fp32 (float storage for every tensor and every
// intermediate), each dot product, mean or softmax sum is accumulated in double and
// rounded once. Straight loops in the order of the definitions, no blocking. Independent
// rows, queries and heads run in parallel (OpenMP); each result is computed by one thread
// in the same order as a serial run, so the output does not depend on the thread count.
//
// Definitions followed (mlxcel issue "feat(vlm): add Cohere Compass / North-Micro-Vision
// (cohere_compass) VLM"):
//  * "Text decoder forward": h = LayerNorm(x) (weight only); attention and SwiGLU MLP both
//    read h; out = x + o_proj(attn) + down(silu(gate) * up); sliding layers rotate q / k
//    with MRoPE and use a window, full layers use no positional encoding.
//  * "Interleaved MRoPE": inv_freq[j] = theta^(-2j / hd); frequency j uses axis h when
//    j % 3 == 1 and j < 3 s_h, axis w when j % 3 == 2 and j < 3 s_w, else axis t; split
//    halves rotate as (x1 cos - x2 sin, x2 cos + x1 sin).
//  * The correction under "Acceptance criteria": dense cache, window as a mask; the
//    rotary class's contiguous [H, W, T] sections (layout 1, read as: each section carries
//    the frequency indices the interleave gives its axis, in increasing order).
//  * "Position ids (get_rope_index)": text advances all three axes; an image of merged
//    grid (t, h / m, w / m) covers t * (h / m) * (w / m) pad tokens at start + (i, j, k);
//    the next text position is start + max(t, h / m, w / m).
//  * Tied logits: LayerNorm then the embedding as a linear map, times logit_scale.
#include <omp.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

struct Shape {
  int D, Hq, Hkv, hd, I;
  int sliding, window;
  int section[3];
  float theta, eps;
  int layout;
};

double dot(const float* a, const float* b, int n) {
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += (double)a[i] * (double)b[i];
  return s;
}

// y[r] = LayerNorm(x[r]) * w over rows of n (biased variance).
void layer_norm(const float* x, const float* w, float eps, int rows, int n, float* y) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r) {
    const float* xr = x + (size_t)r * n;
    double mu = 0.0;
    for (int i = 0; i < n; ++i) mu += xr[i];
    mu /= n;
    double var = 0.0;
    for (int i = 0; i < n; ++i) var += ((double)xr[i] - mu) * ((double)xr[i] - mu);
    var /= n;
    const double rstd = 1.0 / std::sqrt(var + (double)eps);
    for (int i = 0; i < n; ++i) y[(size_t)r * n + i] = (float)(((double)xr[i] - mu) * rstd * (double)w[i]);
  }
}

// y[r][o] = sum_i x[r][i] * W[o][i]  (W in nn.Linear [out, in] layout)
void linear(const float* x, const float* W, int rows, int in, int out, float* y) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int r = 0; r < rows; ++r)
    for (int o = 0; o < out; ++o) y[(size_t)r * out + o] = (float)dot(x + (size_t)r * in, W + (size_t)o * in, in);
}

// Axis and frequency index of rotation pair f.
void rope_pair(const Shape& s, int f, int* axis, int* j) {
  const int half = s.hd / 2;
  std::vector<int> ax(half);
  for (int k = 0; k < half; ++k)
    ax[k] = (k % 3 == 1 && k < 3 * s.section[1]) ? 1 : (k % 3 == 2 && k < 3 * s.section[2]) ? 2 : 0;
  if (!s.layout) {
    *axis = ax[f];
    *j = f;
    return;
  }
  int n = 0;
  const int order[3] = {1, 2, 0};
  for (int a : order)
    for (int k = 0; k < half; ++k)
      if (ax[k] == a) {
        if (n == f) {
          *axis = a;
          *j = k;
          return;
        }
        ++n;
      }
}

// Rotate one head vector v[hd] in place at position triple p[3].
void rope(const Shape& s, const int64_t p[3], float* v) {
  const int half = s.hd / 2;
  for (int f = 0; f < half; ++f) {
    int axis, j;
    rope_pair(s, f, &axis, &j);
    const double inv = std::pow((double)s.theta, -2.0 * j / s.hd);
    const double ang = (double)p[axis] * inv;
    const double c = std::cos(ang), sn = std::sin(ang);
    const double x1 = v[f], x2 = v[f + half];
    v[f] = (float)(x1 * c - x2 * sn);
    v[f + half] = (float)(x2 * c + x1 * sn);
  }
}

float silu(float g) { return (float)((double)g / (1.0 + std::exp(-(double)g))); }

}  // namespace

extern "C" {

// Threads the parallel loops use (OMP_NUM_THREADS, else the cores the runtime sees).
int cref_num_threads(void) { return omp_get_max_threads(); }

typedef struct {
  int32_t D, Hq, Hkv, hd, I;
  int32_t sliding;     // 1: MRoPE + window; 0: full layer (no positional encoding)
  int32_t window;
  int32_t section[3];  // s_t, s_h, s_w
  float theta, eps;
  int32_t layout;      // 0 interleaved, 1 sections
} cref_shape;

// Position ids. tok [B, L]; grid [n_img, 3] (patch units); img_off [B + 1]; pos out
// [3, B, L]; delta out [B]. Returns 0, or the code of the first failing row (1 span
// mismatch, 2 extra pads, 3 unused images, 4 bad grid), leaving that row unwritten.
int cref_mrope_positions(const int32_t* tok, int B, int L, int image_id, const int32_t* grid,
                         const int32_t* img_off, int merge, int32_t* pos, int32_t* delta) {
  for (int b = 0; b < B; ++b) {
    std::vector<int32_t> p(3 * (size_t)L);
    long long st = 0;
    int k = img_off[b];
    const int k_end = img_off[b + 1];
    int l = 0;
    while (l < L) {
      if (tok[(size_t)b * L + l] != image_id) {
        p[l] = p[L + l] = p[2 * L + l] = (int32_t)st;
        ++st;
        ++l;
        continue;
      }
      if (k >= k_end) return 2;
      const int t = grid[3 * k], h = grid[3 * k + 1], w = grid[3 * k + 2];
      if (t < 1 || h < 1 || w < 1 || h % merge || w % merge) return 4;
      const int gh = h / merge, gw = w / merge;
      const __int128 n_exact = (__int128)t * gh * gw;  // exact: no int64 wrap for any int32 grid
      if (l + n_exact > L) return 1;
      const long long n = (long long)n_exact;
      for (long long r = 0; r < n; ++r)
        if (tok[(size_t)b * L + l + r] != image_id) return 1;
      for (long long r = 0; r < n; ++r) {
        p[l + r] = (int32_t)(st + r / ((long long)gh * gw));
        p[L + l + r] = (int32_t)(st + (r / gw) % gh);
        p[2 * L + l + r] = (int32_t)(st + r % gw);
      }
      long long adv = t;
      if (gh > adv) adv = gh;
      if (gw > adv) adv = gw;
      st += adv;
      ++k;
      l += (int)n;
    }
    if (k != k_end) return 3;
    for (int a = 0; a < 3; ++a)
      for (int i = 0; i < L; ++i) pos[((size_t)a * B + b) * L + i] = p[(size_t)a * L + i];
    delta[b] = (int32_t)(st - L);
  }
  return 0;
}

// One layer over a [B, L] block of new tokens. Row b already holds start[b] cached tokens
// (start NULL: none; a prefill); token l sits at cache index start[b] + l. kc, vc: the
// cached keys / values [B, Hkv, cap, hd] (keys already rotated); read for indices below
// start[b]. pos [3, B, L]. w: ln_w, wq, wk, wv, wo, w_gate, w_up, w_down (nn.Linear
// layout). Deepstack: out[ds_rows[r]] += ds[r] (rows of the flattened [B * L]).
// Outputs: out [B, L, D]; k_new, v_new [B, Hkv, L, hd] (the block's keys after rotation).
void cref_layer_forward(const cref_shape* cs, const float* const* w, int B, int L, const float* x,
                        const int32_t* pos, const float* kc, const float* vc, int cap, const int32_t* start,
                        const int32_t* ds_rows, const float* ds, int n_ds, float* out, float* k_new,
                        float* v_new) {
  Shape s{cs->D, cs->Hq, cs->Hkv, cs->hd, cs->I, cs->sliding, cs->window,
          {cs->section[0], cs->section[1], cs->section[2]}, cs->theta, cs->eps, cs->layout};
  const int D = s.D, Hq = s.Hq, Hkv = s.Hkv, hd = s.hd, I = s.I, g = Hq / Hkv;
  const size_t T = (size_t)B * L;
  std::vector<float> a(T * D), q(T * Hq * hd), k(T * Hkv * hd), v(T * Hkv * hd);
  std::vector<float> gt(T * I), up(T * I), act(T * I), o(T * Hq * hd);
  layer_norm(x, w[0], s.eps, (int)T, D, a.data());
  linear(a.data(), w[1], (int)T, D, Hq * hd, q.data());
  linear(a.data(), w[2], (int)T, D, Hkv * hd, k.data());
  linear(a.data(), w[3], (int)T, D, Hkv * hd, v.data());
  linear(a.data(), w[5], (int)T, D, I, gt.data());
  linear(a.data(), w[6], (int)T, D, I, up.data());
#pragma omp parallel for schedule(static)
  for (size_t i = 0; i < T * I; ++i) act[i] = (float)((double)silu(gt[i]) * (double)up[i]);
  if (s.sliding) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b)
      for (int l = 0; l < L; ++l) {
        const int64_t p[3] = {pos[((size_t)0 * B + b) * L + l], pos[((size_t)1 * B + b) * L + l],
                              pos[((size_t)2 * B + b) * L + l]};
        const size_t r = (size_t)b * L + l;
        for (int h = 0; h < Hq; ++h) rope(s, p, &q[(r * Hq + h) * hd]);
        for (int h = 0; h < Hkv; ++h) rope(s, p, &k[(r * Hkv + h) * hd]);
      }
  }
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < Hkv; ++h)
      for (int l = 0; l < L; ++l)
        for (int d = 0; d < hd; ++d) {
          const size_t src = (((size_t)b * L + l) * Hkv + h) * hd + d;
          k_new[(((size_t)b * Hkv + h) * L + l) * hd + d] = k[src];
          v_new[(((size_t)b * Hkv + h) * L + l) * hd + d] = v[src];
        }
  // Attention: query l of row b at cache index n = s0 + l sees keys j <= n (and j > n - W
  // on sliding layers); key j < s0 comes from the cache, j >= s0 from this block.
  const double scale = 1.0 / std::sqrt((double)hd);
#pragma omp parallel for collapse(3) schedule(dynamic, 16)
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < Hq; ++h) {
      for (int l = 0; l < L; ++l) {
        const int s0 = start ? start[b] : 0;
        const int kvh = h / g;
        const int n = s0 + l;
        const int lo = s.sliding ? (n - s.window + 1 > 0 ? n - s.window + 1 : 0) : 0;
        const float* qv = &q[(((size_t)b * L + l) * Hq + h) * hd];
        std::vector<double> sc(n - lo + 1);
        double mx = -INFINITY;
        for (int j = lo; j <= n; ++j) {
          const float* kv = j < s0 ? &kc[(((size_t)b * Hkv + kvh) * cap + j) * hd]
                                   : &k[(((size_t)b * L + (j - s0)) * Hkv + kvh) * hd];
          sc[j - lo] = dot(qv, kv, hd) * scale;
          if (sc[j - lo] > mx) mx = sc[j - lo];
        }
        double z = 0.0;
        for (int j = lo; j <= n; ++j) z += std::exp(sc[j - lo] - mx);
        // p_j = exp(s_j - max) / z, each evaluated once.
        for (int j = lo; j <= n; ++j) sc[j - lo] = std::exp(sc[j - lo] - mx) / z;
        for (int d = 0; d < hd; ++d) {
          double acc = 0.0;
          for (int j = lo; j <= n; ++j) {
            const float* vv = j < s0 ? &vc[(((size_t)b * Hkv + kvh) * cap + j) * hd]
                                     : &v[(((size_t)b * L + (j - s0)) * Hkv + kvh) * hd];
            acc += sc[j - lo] * (double)vv[d];
          }
          o[(((size_t)b * L + l) * Hq + h) * hd + d] = (float)acc;
        }
      }
    }
  }
  // out = x + o Wo^T + act Wd^T (the two branches added to the residual).
#pragma omp parallel for collapse(2) schedule(static)
  for (size_t r = 0; r < T; ++r)
    for (int c = 0; c < D; ++c) {
      const double attn = dot(&o[r * Hq * hd], w[4] + (size_t)c * Hq * hd, Hq * hd);
      const double mlp = dot(&act[r * I], w[7] + (size_t)c * I, I);
      out[r * D + c] = (float)((double)x[r * D + c] + attn + mlp);
    }
  for (int i = 0; i < n_ds; ++i) {
    const int r = ds_rows[i];
    if (r < 0 || (size_t)r >= T) continue;
    for (int c = 0; c < D; ++c) out[(size_t)r * D + c] = (float)((double)out[(size_t)r * D + c] + ds[(size_t)i * D + c]);
  }
}

// logits[r][v] = fp32(LayerNorm(h[r]) . E[v]) * scale, the scale multiplied in fp32.
void cref_logits(int R, int D, int V, const float* h, const float* nw, float eps, const float* E, float scale,
                 float* logits) {
  std::vector<float> a((size_t)R * D);
  layer_norm(h, nw, eps, R, D, a.data());
#pragma omp parallel for collapse(2) schedule(static)
  for (int r = 0; r < R; ++r)
    for (int v = 0; v < V; ++v) {
      const float l = (float)dot(&a[(size_t)r * D], E + (size_t)v * D, D);
      logits[(size_t)r * V + v] = l * scale;  // the scale as the last fp32 operation
    }
}

}  // extern "C"
