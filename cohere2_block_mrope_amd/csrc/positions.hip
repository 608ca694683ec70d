// MRoPE position ids, following "Position ids (get_rope_index)" of the mlxcel
// Compass issue: text tokens advance (t, h, w) by one; the t*(h/m)*(w/m) pads of
// an image get start + (t_i, h_i, w_i) on the merged grid; the next text token
// starts at max position + 1; rope_delta = max position + 1 - L.
//
// One workgroup per row. The images of a row are walked in order by the whole
// workgroup: each step finds the next pad token with a cooperative scan, checks
// the image's span, and records (start, end, first position, offset after). The
// positions of all L tokens are then written in parallel from those records.
// Errors are detected in the order a left-to-right walk over the tokens meets them.
#include "common.h"
#include "launch.h"
#include "../../include/compass.h"

namespace compass {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxImg = COMPASS_MAX_IMAGES_PER_ROW;

__global__ __launch_bounds__(kThreads) void positions_kernel(
    const int32_t* __restrict__ tok, int L, int image_id, const int32_t* __restrict__ grid,
    const int32_t* __restrict__ img_off, int merge, int32_t* __restrict__ pos,
    int32_t* __restrict__ delta, int32_t* __restrict__ status, int B) {
  __shared__ int s_start[kMaxImg];
  __shared__ int s_end[kMaxImg];
  __shared__ int s_base[kMaxImg];   // position of the image's first pad (t, h, w all equal)
  __shared__ int s_after[kMaxImg];  // text offset (position - index) after the image
  __shared__ int s_gh[kMaxImg];
  __shared__ int s_gw[kMaxImg];
  __shared__ int s_found;
  __shared__ int s_bad;
  __shared__ int s_err;
  __shared__ int s_nimg;

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t* row = tok + (size_t)b * L;
  const int k0 = img_off[b];
  const int nimg = img_off[b + 1] - k0;

  if (tid == 0) { s_err = COMPASS_POS_OK; s_nimg = 0; }
  __syncthreads();
  if (nimg > kMaxImg || nimg < 0) {
    if (tid == 0) status[b] = COMPASS_POS_TOO_MANY_IMAGES;
    return;
  }

  int p = 0;        // next token index the walk has not consumed
  int offset = 0;   // position - index of text tokens at p
  for (int k = 0; k <= nimg; ++k) {
    // Next pad token at or after p (L if none).
    if (tid == 0) s_found = L;
    __syncthreads();
    for (int base = p; base < L; base += kThreads * 4) {
      int best = L;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        int idx = base + u * kThreads + tid;
        if (idx < L && row[idx] == image_id) best = min(best, idx);
      }
      if (best < L) atomicMin(&s_found, best);
      __syncthreads();
      int f = s_found;
      __syncthreads();
      if (f < L) break;
    }
    const int sidx = s_found;
    if (k == nimg) {  // all images consumed: any pad left over is an error
      if (tid == 0 && sidx < L) s_err = COMPASS_POS_EXTRA_PADS;
      __syncthreads();
      break;
    }
    if (sidx >= L) {
      if (tid == 0) s_err = COMPASS_POS_UNUSED_IMAGES;
      __syncthreads();
      break;
    }
    const int t = grid[(size_t)(k0 + k) * 3 + 0];
    const int h = grid[(size_t)(k0 + k) * 3 + 1];
    const int w = grid[(size_t)(k0 + k) * 3 + 2];
    if (t < 1 || h < 1 || w < 1 || h % merge || w % merge) {
      if (tid == 0) s_err = COMPASS_POS_BAD_GRID;
      __syncthreads();
      break;
    }
    const int gh = h / merge, gw = w / merge;
    const long long nll = (long long)t * gh * gw;
    if (nll > (long long)(L - sidx)) {
      if (tid == 0) s_err = COMPASS_POS_SPAN_MISMATCH;
      __syncthreads();
      break;
    }
    const int n = (int)nll;
    if (tid == 0) s_bad = 0;
    __syncthreads();
    int bad = 0;
    for (int idx = sidx + tid; idx < sidx + n; idx += kThreads) bad |= (row[idx] != image_id);
    if (bad) s_bad = 1;
    __syncthreads();
    if (s_bad) {
      if (tid == 0) s_err = COMPASS_POS_SPAN_MISMATCH;
      __syncthreads();
      break;
    }
    const int first = sidx + offset;          // position of the image's first pad
    const int adv = max(t, max(gh, gw));
    if (tid == 0) {
      s_start[k] = sidx;
      s_end[k] = sidx + n;
      s_base[k] = first;
      s_after[k] = first + adv - (sidx + n);
      s_gh[k] = gh;
      s_gw[k] = gw;
      s_nimg = k + 1;
    }
    offset = first + adv - (sidx + n);
    p = sidx + n;
    __syncthreads();
  }
  __syncthreads();
  const int err = s_err;
  if (tid == 0) status[b] = err;
  if (err != COMPASS_POS_OK) return;

  const int ni = s_nimg;
  const size_t plane = (size_t)B * L;
  int32_t* pt = pos + (size_t)b * L;
  for (int l = tid; l < L; l += kThreads) {
    // Last image whose span starts at or before l.
    int lo = 0, hi = ni - 1, kk = -1;
    while (lo <= hi) {
      int mid = (lo + hi) >> 1;
      if (s_start[mid] <= l) { kk = mid; lo = mid + 1; } else { hi = mid - 1; }
    }
    int pt_t, pt_h, pt_w;
    if (kk >= 0 && l < s_end[kk]) {
      const int r = l - s_start[kk];
      const int gh = s_gh[kk], gw = s_gw[kk];
      pt_t = s_base[kk] + r / (gh * gw);
      pt_h = s_base[kk] + (r / gw) % gh;
      pt_w = s_base[kk] + r % gw;
    } else {
      const int off = kk >= 0 ? s_after[kk] : 0;
      pt_t = pt_h = pt_w = l + off;
    }
    pt[l] = pt_t;
    pt[plane + l] = pt_h;
    pt[2 * plane + l] = pt_w;
  }
  if (tid == 0) delta[b] = (ni > 0 ? s_after[ni - 1] : 0);  // (L + offset) - L
}

}  // namespace

hipError_t launch_positions(const int32_t* tok, int B, int L, int image_id, const int32_t* grid,
                            const int32_t* img_off, int merge, int32_t* pos, int32_t* delta,
                            int32_t* status, hipStream_t s) {
  positions_kernel<<<B, kThreads, 0, s>>>(tok, L, image_id, grid, img_off, merge, pos, delta,
                                          status, B);
  return hipGetLastError();
}

}  // namespace compass
