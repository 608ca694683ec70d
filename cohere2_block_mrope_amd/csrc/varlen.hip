// Plan of a varlen prefill: packed sequences of different lengths in one launch, each
// continuing its own cache (FreeToken PR "feat(mm): serve image input on the Qwen
// families", "How it fits together": prefill planned per request; mlxcel Compass issue,
// "Validation": prefill causal within a sequence).
//
// One 1024-thread workgroup validates the offsets, decides which sequences are processed
// (a chunk must fit its cache), writes the sequence of every packed row (-1 for rows not
// processed) and lists the attention's query tiles, latest query block first so that the
// longest tiles of causal attention start earliest. The position of a tile inside its
// level comes from an LDS atomic; the order inside a level does not change any result.
#include "common.h"
#include "launch.h"

namespace compass {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kMaxLevels = kVarlenMaxTokens / 128;  // query blocks of 128 rows per sequence

__global__ __launch_bounds__(kPlanThreads) void varlen_plan_kernel(VarlenPlan vp, int T, const int32_t* start,
                                                                   int cap, int tile_rows, int32_t* status) {
  __shared__ int s_cu[kVarlenMaxSeqs + 1];
  __shared__ int s_nt[kVarlenMaxSeqs];   // query tiles of each sequence (0 when not processed)
  __shared__ int s_lev[kMaxLevels];      // tiles per level, then each level's next free slot
  __shared__ int s_bad, s_skip, s_maxnt;
  const int tid = threadIdx.x;
  const int n = vp.n_seq;
  if (tid == 0) { s_bad = 0; s_skip = 0; s_maxnt = 0; }
  __syncthreads();
  for (int i = tid; i <= n; i += kPlanThreads) {
    const int c = vp.cu[i];
    s_cu[i] = c;
    if (c < 0 || c > T || (i == 0 && c != 0) || (i == n && c != T)) s_bad = 1;
  }
  __syncthreads();
  for (int i = tid; i < n; i += kPlanThreads)
    if (s_cu[i + 1] < s_cu[i]) s_bad = 1;
  __syncthreads();
  const bool bad = s_bad != 0;
  // Sequences processed, and their tiles.
  for (int i = tid; i < n; i += kPlanThreads) {
    const int len = bad ? 0 : s_cu[i + 1] - s_cu[i];
    bool live = !bad;
    if (live && start) {
      const int s0 = start[i];
      live = s0 >= 0 && s0 <= cap - len;
      if (!live) s_skip = 1;
    }
    const int nt = (live && tile_rows > 0) ? (len + tile_rows - 1) / tile_rows : (live ? 0 : -1);
    s_nt[i] = nt;
    if (nt > 0) atomicMax(&s_maxnt, nt);
  }
  __syncthreads();
  // Sequence of every packed row: the last sequence whose first row is at or before it
  // (empty sequences share their first row with the next one and are passed over).
  for (int m = tid; m < T; m += kPlanThreads) {
    int sq = -1;
    if (!bad) {
      int lo = 0, hi = n - 1;
      while (lo <= hi) {
        const int mid = (lo + hi) >> 1;
        if (s_cu[mid] <= m) { sq = mid; lo = mid + 1; } else { hi = mid - 1; }
      }
      if (sq >= 0 && s_nt[sq] < 0) sq = -1;
    }
    vp.row_seq[m] = sq;
  }
  if (tile_rows > 0) {
    const int levels = s_maxnt;
    for (int lv = tid; lv < levels; lv += kPlanThreads) s_lev[lv] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kPlanThreads)
      for (int lv = 0; lv < s_nt[i]; ++lv) atomicAdd(&s_lev[lv], 1);
    __syncthreads();
    // Level lv starts after every tile of the levels above it (one thread: levels are few).
    if (tid == 0) {
      int acc = 0;
      for (int lv = levels - 1; lv >= 0; --lv) {
        const int c = s_lev[lv];
        s_lev[lv] = acc;
        acc += c;
      }
      vp.n_tiles[0] = acc;
    }
    __syncthreads();
    for (int i = tid; i < n; i += kPlanThreads)
      for (int lv = 0; lv < s_nt[i]; ++lv) {
        const int t = atomicAdd(&s_lev[lv], 1);
        vp.tiles[2 * t] = i;
        vp.tiles[2 * t + 1] = lv;
      }
  } else if (tid == 0) {
    vp.n_tiles[0] = 0;
  }
  if (tid == 0 && status) status[0] = (bad ? 1 : 0) | (s_skip ? 2 : 0);
}

}  // namespace

hipError_t launch_varlen_plan(const VarlenPlan& vp, int T, const int32_t* start, int cap, int tile_rows,
                              int32_t* status, hipStream_t s) {
  varlen_plan_kernel<<<1, kPlanThreads, 0, s>>>(vp, T, start, cap, tile_rows, status);
  return hipGetLastError();
}

}  // namespace compass
