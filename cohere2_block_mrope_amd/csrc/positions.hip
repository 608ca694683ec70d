// MRoPE position ids, following "Position ids (get_rope_index)" of the mlxcel
// Compass issue: text tokens advance (t, h, w) by one; the t*(h/m)*(w/m) pads of
// an image get start + (t_i, h_i, w_i) on the merged grid; the next text token
// starts at max position + 1; rope_delta = max position + 1 - L.
//
// One 1024-thread workgroup per row. The row's tokens are read once, coalesced, into an
// LDS bitmask of image-pad tokens (one ballot per wave and 64 tokens). The images of the
// row are then walked in order on that mask: each step finds the next pad with one
// parallel pass over the mask words, checks the image's span, and records (start, end,
// first position, offset after). The positions of all L tokens are then written in
// parallel from those records. Errors are detected in the order a left-to-right walk
// over the tokens meets them.
#include "common.h"
#include "launch.h"
#include "../../include/compass.h"

namespace compass {

namespace {

constexpr int kThreads = 1024;
constexpr int kMaxImg = COMPASS_MAX_IMAGES_PER_ROW;
constexpr int kRecInts = 9 * kMaxImg;  // per-image records and grids in dynamic LDS, then the mask
constexpr int kUnroll = 4;             // token loads in flight per lane while building the mask

__global__ __launch_bounds__(kThreads) void positions_kernel(
    const int32_t* __restrict__ tok, int L, int image_id, const int32_t* __restrict__ grid,
    const int32_t* __restrict__ img_off, int merge, int32_t* __restrict__ pos,
    int32_t* __restrict__ delta, int32_t* __restrict__ status, int B) {
  extern __shared__ __align__(16) int smem[];
  int* s_start = smem;                  // first pad of image k
  int* s_end = smem + kMaxImg;          // one past its last pad
  int* s_base = smem + 2 * kMaxImg;     // position of the image's first pad (t, h, w all equal)
  int* s_after = smem + 3 * kMaxImg;    // text offset (position - index) after the image
  int* s_gh = smem + 4 * kMaxImg;
  int* s_gw = smem + 5 * kMaxImg;
  int* s_grid = smem + 6 * kMaxImg;     // the row's image grids (t, h, w), prefetched
  uint32_t* s_mask = reinterpret_cast<uint32_t*>(smem + kRecInts);  // bit l: token l is a pad
  __shared__ int s_found;
  __shared__ int s_bad;
  __shared__ int s_err;
  __shared__ int s_nimg;

  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t* row = tok + (size_t)b * L;
  const int k0 = img_off[b];
  const int nimg = img_off[b + 1] - k0;
  const int nw = (L + 31) >> 5;

  if (tid == 0) { s_err = COMPASS_POS_OK; s_nimg = 0; }
  if (nimg > kMaxImg || nimg < 0) {
    if (tid == 0) status[b] = COMPASS_POS_TOO_MANY_IMAGES;
    return;
  }
  // The row's grids go to LDS while the tokens are read.
  for (int i = tid; i < 3 * nimg; i += kThreads) s_grid[i] = grid[(size_t)k0 * 3 + i];
  // Pad bitmask: wave w covers tokens 64 i .. 64 i + 63 for i = w, w + 16, ...; kUnroll
  // chunks of a lane are loaded before any is tested, so their latencies overlap.
  constexpr int kStride = 64 * (kThreads / 64);
  for (int base0 = 64 * wave; base0 < L; base0 += kUnroll * kStride) {
    int v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int idx = base0 + u * kStride + lane;
      v[u] = idx < L ? row[idx] : 0;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int base = base0 + u * kStride;
      const uint64_t bal = __ballot(base + lane < L && v[u] == image_id);
      if (lane == 0 && base < L) {
        s_mask[base >> 5] = (uint32_t)bal;
        if ((base >> 5) + 1 < nw) s_mask[(base >> 5) + 1] = (uint32_t)(bal >> 32);
      }
    }
  }
  __syncthreads();

  int p = 0;        // next token index the walk has not consumed
  int offset = 0;   // position - index of text tokens at p
  for (int k = 0; k <= nimg; ++k) {
    // Next pad token at or after p (L if none).
    if (tid == 0) s_found = L;
    __syncthreads();
    for (int w = (p >> 5) + tid; w < nw; w += kThreads) {
      uint32_t m = s_mask[w];
      if (w == (p >> 5)) m &= ~0u << (p & 31);
      if (m) atomicMin(&s_found, 32 * w + __ffs((int)m) - 1);
    }
    __syncthreads();
    const int sidx = s_found;
    if (k == nimg) {  // all images consumed: any pad left over is an error
      if (tid == 0 && sidx < L) s_err = COMPASS_POS_EXTRA_PADS;
      break;
    }
    if (sidx >= L) {
      if (tid == 0) s_err = COMPASS_POS_UNUSED_IMAGES;
      break;
    }
    const int t = s_grid[3 * k + 0];
    const int h = s_grid[3 * k + 1];
    const int w = s_grid[3 * k + 2];
    if (t < 1 || h < 1 || w < 1 || h % merge || w % merge) {
      if (tid == 0) s_err = COMPASS_POS_BAD_GRID;
      break;
    }
    const int gh = h / merge, gw = w / merge;
    // The span t * gh * gw must fit in the rest of the row. Each factor is at least one, so
    // a factor beyond the rest already fails; otherwise the product is below 2^57 (the row
    // holds at most 2^19 tokens) and cannot wrap.
    const long long rest = (long long)(L - sidx);
    const bool too_big = t > rest || gh > rest || gw > rest || (long long)t * gh * gw > rest;
    const long long nll = too_big ? rest + 1 : (long long)t * gh * gw;
    if (too_big) {
      if (tid == 0) s_err = COMPASS_POS_SPAN_MISMATCH;
      break;
    }
    const int n = (int)nll;
    // Every token of [sidx, sidx + n) must be a pad.
    if (tid == 0) s_bad = 0;
    __syncthreads();
    const int wlo = sidx >> 5, whi = (sidx + n - 1) >> 5;
    for (int wi = wlo + tid; wi <= whi; wi += kThreads) {
      uint32_t need = ~0u;
      if (wi == wlo) need &= ~0u << (sidx & 31);
      if (wi == whi) need &= ~0u >> (31 - ((sidx + n - 1) & 31));
      if ((s_mask[wi] & need) != need) s_bad = 1;
    }
    __syncthreads();
    if (s_bad) {
      if (tid == 0) s_err = COMPASS_POS_SPAN_MISMATCH;
      break;
    }
    const int first = sidx + offset;  // position of the image's first pad
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
      const int mid = (lo + hi) >> 1;
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
  const size_t lds = sizeof(int) * ((size_t)kRecInts + ((size_t)L + 31) / 32);
  const size_t max_lds = sizeof(int) * ((size_t)kRecInts + COMPASS_MAX_TOKENS_PER_ROW / 32);
  const hipError_t e = ensure_dynamic_lds((const void*)positions_kernel, (int)max_lds);
  if (e != hipSuccess) return e;
  positions_kernel<<<B, kThreads, lds, s>>>(tok, L, image_id, grid, img_off, merge, pos, delta, status, B);
  return hipGetLastError();
}

}  // namespace compass
