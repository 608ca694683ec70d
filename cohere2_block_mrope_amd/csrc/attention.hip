// Causal GQA attention for prefill: o = softmax(q k^T / sqrt(hd)) v over the keys the
// layer type allows ("Text decoder forward" of the mlxcel Compass issue: sliding
// layers see the last `window` keys, full layers everything up to the query).
// Query head h reads key/value head h / (Hq / Hkv).
//
// bf16 kernel (gfx950 MFMA). A 256-thread workgroup takes 128 queries of one head;
// each wave owns 32 queries. Scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_bf16: the result lane l then holds one query (l % 32) and 16 of
// the tile's keys per 32-key block, so the online-softmax max and sum are in-lane
// reductions plus one exchange with lane l ^ 32. The probabilities are already in
// the B-operand layout of O^T = V^T P^T (the key order inside a 16-key step is
// permuted identically on both operands), and the V^T operand is read from the
// row-major V tile with ds_read_b64_tr_b16, the gfx950 LDS transpose read.
// K/V tiles of 64 keys are double-buffered in LDS (rows padded against bank
// conflicts); tiles outside the causal/window range are skipped, and only tiles that
// straddle the diagonal or the window edge are masked.
// Online softmax in the log2 domain with a lazily moved reference: a row's running
// maximum m is only raised (rescaling O and l by 2^(m_old - m_new)) when a tile's
// maximum exceeds it by more than 8, so probabilities 2^(s - m) stay below 256 and
// most tiles skip the rescale. O / l is unchanged by the choice of m. Row sums are taken
// over the bf16-rounded probabilities the PV MFMA multiplies.
// Each wave runs a software pipeline over key tiles: the next tile's S^T MFMAs are issued
// among the current tile's exponentials (see the loop below).
//
// fp32 kernel: one wave per query, keys in 64-lane chunks with an online softmax.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace compass {
namespace {

struct AttnParams {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  int B, Hq, Hkv, L, cap;
  int sliding, window;
  const int32_t* start;  // chunked prefill: query l of row b sits at cache index start[b] + l
  bf16_t* o;
  int ldo;
  float scale_log2;  // log2(e) / sqrt(hd)
  int nqb;
  // Varlen prefill (tiles != NULL): workgroup x takes tile x of the plan; q is [Hq, T, hd]
  // and o row m holds packed row m; keys come from cache row s (kv_by_seq, first query at
  // start[s]) or from the packed scratch [Hkv, T, hd] (first query at index 0).
  const int32_t* tiles;
  const int32_t* n_tiles;
  const int32_t* cu;
  int T;
  int kv_by_seq;
  // XCD-aware order of the dense grid (1-D grid; xmode 0: grid (nqb, Hq, B) as is). The
  // workgroups that share one (row, kv head) K/V slice run on one XCD so that its L2 serves
  // their key tiles: workgroup id i runs on XCD i % 8. xmode 1 (B * Hkv a multiple of 8):
  // XCD x takes groups x, x + 8, ... one after the other; xmode 2 (B * Hkv divides 8):
  // 8 / (B * Hkv) XCDs share a group, dealing its work units round-robin. Inside a group the
  // units run latest query block first, the group's query heads next to each other.
  int xmode;
};

constexpr int QB = 128, KB = 64;
constexpr float kLazyMax = 8.0f;  // log2 headroom before the reference max is raised
// Fourth dword of a raw (unstrided) buffer resource: 32-bit data format, range-checked.
constexpr int kBufferDword3 = 0x00020000;

template <int HD>
__global__ __launch_bounds__(256, 2) void attn_prefill_bf16(AttnParams P) {
  constexpr int KS = HD + 8;    // K row stride (elements): 8 consecutive rows -> distinct banks
  // V row stride = 16 dwords mod 64 banks: the 32 lanes of a tr16 read (4 rows x 2 column
  // groups of 32 B) then hit 64 distinct banks.
  constexpr int VS = HD + 32;
  constexpr int DB = HD / 32;   // 32-wide d blocks of O^T
  constexpr int QK = HD / 16;   // 16-deep k-steps of S^T
  constexpr int CH = HD / 8;    // 16-byte chunks per key row
  constexpr int LD_PER_T = KB * CH / 256;
  __shared__ __align__(16) bf16_t Ks[2][KB * KS];
  __shared__ __align__(16) bf16_t Vs[2][KB * VS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
  const int g = P.Hq / P.Hkv;
  int h = blockIdx.y;
  int bx = blockIdx.x, bz = blockIdx.z;  // dense grid coordinates (x: heaviest first)
  if (P.xmode) {
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    const int groups = P.B * P.Hkv, per_group = P.nqb * g;
    int grp, j;
    if (P.xmode == 1) {
      grp = xcd + 8 * (local / per_group);
      j = local - (local / per_group) * per_group;
    } else {
      const int r = 8 / groups;
      grp = xcd % groups;
      j = local * r + xcd / groups;
      if (j >= per_group) return;  // uniform: past the group's units
    }
    bz = grp / P.Hkv;
    h = (grp - bz * P.Hkv) * g + j % g;
    bx = j / g;
  }
  const int kvh = h / g;
  // The workgroup's sequence b, query block qb, its L queries, the rows of its first query in
  // q (rows of HD) and in o, the start of its (row, kv head) K/V slice and the slice's rows.
  int b, qb, L, s0, slice_rows;
  size_t qrow0, orow0, kvrow0;
  if (P.tiles) {
    if ((int)blockIdx.x >= P.n_tiles[0]) return;  // past the plan's tiles (uniform)
    b = P.tiles[2 * blockIdx.x];
    qb = P.tiles[2 * blockIdx.x + 1];
    const int m0 = P.cu[b];
    L = P.cu[b + 1] - m0;
    qrow0 = (size_t)h * P.T + m0;
    orow0 = m0;
    if (P.kv_by_seq) {  // the plan lists live sequences only: 0 <= start[b] <= cap - L
      s0 = P.start ? P.start[b] : 0;
      kvrow0 = ((size_t)b * P.Hkv + kvh) * P.cap;
      slice_rows = P.cap;
    } else {
      s0 = 0;
      kvrow0 = (size_t)kvh * P.T + m0;
      slice_rows = L;
    }
  } else {
    qb = P.nqb - 1 - bx;  // heaviest (latest) query blocks first
    b = bz;
    L = P.L;
    qrow0 = ((size_t)b * P.Hq + h) * L;
    orow0 = (size_t)b * L;
    // Cache index of the chunk's first query (rows whose chunk does not fit are computed
    // as if it started at 0: in bounds, and their outputs are never stored by the layer).
    s0 = P.start ? P.start[b] : 0;
    if (s0 < 0 || s0 > P.cap - L) s0 = 0;
    kvrow0 = ((size_t)b * P.Hkv + kvh) * P.cap;
    slice_rows = P.cap;
  }
  const int q0 = qb * QB;
  const int qw = q0 + 32 * wave + (lane & 31);  // this lane's query (row of the chunk)
  const int a0 = s0 + q0;   // cache index of the workgroup's first query
  const int aw = s0 + qw;   // cache index of this lane's query
  const int half = lane >> 5;

  // Q fragments (B operand of S^T): lane holds query qw, d = 16 ks + 8 half .. + 8.
  bf16x8_t qf[QK];
  {
    const bf16_t* qp = P.q + (qrow0 + min(qw, L - 1)) * HD + 8 * half;
#pragma unroll
    for (int ks = 0; ks < QK; ++ks) qf[ks] = *reinterpret_cast<const bf16x8_t*>(qp + 16 * ks);
  }

  const int q_hi = s0 + min(q0 + QB - 1, L - 1);
  const int k_lo = P.sliding ? max(0, a0 - P.window + 1) : 0;
  const int kt0 = k_lo / KB, kt1 = q_hi / KB;

  const bf16_t* kbase = P.k + kvrow0 * HD;
  const bf16_t* vbase = P.v + kvrow0 * HD;
  // Software pipeline over key tiles: S^T of tile t + 1 is computed while the softmax of
  // tile t runs (independent MFMA and VALU work in one instruction stream). Tile t sits in
  // K buffer (t - kt0) & 1 and V buffer (t - kt0) & 1; K runs one tile ahead of V, so during
  // iteration t the registers hold K(t + 2) and V(t + 1) on their way to LDS.
  u32x4_t rk[LD_PER_T], rv[LD_PER_T];
  // Keys past the chunk's last row are clamped to it (valid data; those keys are masked).
  // K and V are read with buffer loads: the tile's start is a uniform byte offset in an
  // SGPR, so tiles that lie wholly before that row (all but the last) need no per-tile
  // address arithmetic, only this thread's fixed offsets.
  const int last_key = s0 + L - 1;
  const int slice_bytes = slice_rows * HD * 2;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, slice_bytes, kBufferDword3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, slice_bytes, kBufferDword3);
  int toff[LD_PER_T];
#pragma unroll
  for (int i = 0; i < LD_PER_T; ++i) {
    const int c = tid + 256 * i;
    toff[i] = ((c / CH) * HD + 8 * (c % CH)) * 2;
  }
  auto gload = [&](u32x4_t* r, __amdgpu_buffer_rsrc_t rs, int kt) __attribute__((always_inline)) {
    if (kt * KB + KB - 1 <= last_key) {
#pragma unroll
      for (int i = 0; i < LD_PER_T; ++i) r[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, toff[i], kt * KB * HD * 2, 0);
    } else {
#pragma unroll
      for (int i = 0; i < LD_PER_T; ++i) {
        const int c = tid + 256 * i;
        const int key = min(kt * KB + c / CH, last_key);
        r[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, (key * HD + 8 * (c % CH)) * 2, 0, 0);
      }
    }
  };
  auto sstore = [&](const u32x4_t* r, bf16_t* tile, int stride) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LD_PER_T; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<u32x4_t*>(&tile[(c / CH) * stride + 8 * (c % CH)]) = r[i];
    }
  };
  // S^T for 64 keys x 32 queries (two 32-key blocks) from the K tile in buffer kbuf.
  auto qk = [&](int kbuf, f32x16_t (&S)[2]) __attribute__((always_inline)) {  // kbuf: constant
    const bf16_t* ks_ = Ks[kbuf];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) S[kb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < QK; ++ks) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(
            ks_ + (32 * kb + (lane & 31)) * KS + 16 * ks + 8 * half);
        S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], S[kb], 0, 0, 0);
      }
    }
  };

  f32x16_t O[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[i][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // Tile kt, scores in S: mask, row maximum, lazy raise of the reference (rescaling O).
  // Returns -m_run (0 while a row has seen no visible key).
  auto softmax_max = [&](int kt, f32x16_t (&S)[2]) __attribute__((always_inline)) -> float {
    const int k0 = kt * KB;
    // Mask only tiles that are not entirely visible to every query of the workgroup.
    // The maximum is taken on raw scores (the scale is positive) and the scale folded
    // into the exponent's FMA.
    const bool full_vis = (k0 + KB - 1 <= a0) && (!P.sliding || k0 >= a0 + QB - P.window);
    float mx = -INFINITY;
    if (full_vis) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kb][r]);
    } else {
      // Key k0 + c is visible to the query at cache index aw iff 0 <= aw - k0 - c < window
      // (causal: window = 2^31 - 1), one unsigned compare.
      const unsigned wlim = P.sliding ? (unsigned)P.window : 0x7fffffffu;
      const int dq = aw - k0 - 4 * half;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float sc = ((unsigned)(dq - (32 * kb + 8 * (r >> 2) + (r & 3))) < wlim) ? S[kb][r] : -INFINITY;
          S[kb][r] = sc;
          mx = fmaxf(mx, sc);
        }
    }
    mx = pair32_max(mx) * P.scale_log2;
    // Raise the reference only when this tile's maximum is more than kLazyMax above it
    // (always on a row's first visible tile, where m_run = -inf). alpha = 2^(m_old - m_new)
    // is 1 when the reference stays and 0 on the first raise.
    const bool raise = mx > m_run + kLazyMax;
    const float alpha = __builtin_amdgcn_exp2f(raise ? m_run - mx : 0.f);
    m_run = raise ? mx : m_run;
    if (__builtin_amdgcn_ballot_w64(raise)) {
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[i][r] *= alpha;
    }
    l_run *= alpha;
    // Rows with no visible key yet keep m_run = -inf and get p = 0 (their scores are -inf).
    return (m_run == -INFINITY) ? 0.f : -m_run;
  };
  // Probabilities of tile kt, with S^T of the next tile (K buffer PAR ^ 1) issued in the
  // same straight-line block when NEXT, then O^T += V^T P^T from V buffer PAR.
  auto exp_pv = [&](auto par, f32x16_t (&S)[2], float neg_m, auto next, f32x16_t (&Sn)[2])
      __attribute__((always_inline)) {
    constexpr int PAR = decltype(par)::value;
    // The 32 exponentials are spread over NQ chunks, one MFMA of the next tile's S^T each
    // (K fragments read two chunks ahead); sched_barrier keeps the chunks in order so the
    // MFMAs run under the VALU work.
    constexpr bool NEXT = decltype(next)::value;
    constexpr int NQ = 2 * QK;
    constexpr int EPC = 32 / NQ;
    const bf16_t* kn = Ks[PAR ^ 1];
    auto kfrag = [&](int c) __attribute__((always_inline)) {
      return *reinterpret_cast<const bf16x8_t*>(kn + (32 * (c / QK) + (lane & 31)) * KS + 16 * (c % QK) + 8 * half);
    };
    // Row sum of the bf16-rounded probabilities (the values the PV MFMA multiplies), two
    // per dot2 against (1, 1).
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
    // Wave priority: the exponentials (with the next tile's S^T MFMAs among them) are the
    // longer dependent chain of an iteration, the PV MFMAs below need no VALU. Raising the
    // priority for the first part and dropping it for the second lets the other wave of the
    // SIMD (the other workgroup's) issue its exponentials while this one's PV MFMAs run.
    __builtin_amdgcn_s_setprio(1);
    float rs = 0.f;
    uint32_t pw[2][2][4];
    bf16x8_t kf[3];
    if constexpr (NEXT) {
      kf[0] = kfrag(0);
      kf[1] = kfrag(1);
    }
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      if constexpr (NEXT) {
        if (c + 2 < NQ) kf[(c + 2) % 3] = kfrag(c + 2);
        const int kb = c / QK, ks = c % QK;
        if (ks == 0) {
#pragma unroll
          for (int r = 0; r < 16; ++r) Sn[kb][r] = 0.f;
        }
        Sn[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[c % 3], qf[ks], Sn[kb], 0, 0, 0);
      }
#pragma unroll
      for (int e = c * EPC; e < (c + 1) * EPC; e += 2) {
        const int kb = e / 16, r = e % 16;
        float p0 = __builtin_amdgcn_exp2f(fmaf(S[kb][r], P.scale_log2, neg_m));
        float p1 = __builtin_amdgcn_exp2f(fmaf(S[kb][r + 1], P.scale_log2, neg_m));
        asm volatile("" : "+v"(p0), "+v"(p1));  // keeps the exponentials in their chunk
        const uint32_t w = pack_bf2(p0, p1);
        rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), ones, rs, false);
        pw[kb][r / 8][(r % 8) / 2] = w;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run += pair32_sum(rs);
    bf16x8_t pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const u32x4_t q4 = {pw[kb][st][0], pw[kb][st][1], pw[kb][st][2], pw[kb][st][3]};
        pf[kb][st] = __builtin_bit_cast(bf16x8_t, q4);
      }

    // O^T[d, q] += sum_key V[key, d] P[q, key]. The V^T operand comes from two
    // transpose reads: lane m of each 16-lane group addresses row key0 + m / 4,
    // columns d0 + 4 (m % 4) .. + 4, and receives V[key0 + j][d0 + lane % 16], j < 4.
    // MFMA c takes 16-key step c / DB and d block c % DB (consecutive MFMAs feed
    // different accumulators); its V^T fragment is read three MFMAs ahead.
    const bf16_t* vs_ = Vs[PAR];
    const int grp = lane >> 4, m16 = lane & 15;
    constexpr int NP = 4 * DB;
    auto vfrag = [&](int c) __attribute__((always_inline)) {
      const int kst = c / DB, db = c % DB;
      const int key0 = 16 * kst + 4 * half;
      const bf16_t* v0 = vs_ + (key0 + (m16 >> 2)) * VS + 32 * db + 16 * (grp & 1) + 4 * (m16 & 3);
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(s16x4_t))v0);
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(s16x4_t))(v0 + 8 * VS));
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    __builtin_amdgcn_s_setprio(0);
    bf16x8_t vf[4];
#pragma unroll
    for (int c = 0; c < 3; ++c) vf[c] = vfrag(c);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < NP; ++c) {
      if (c + 3 < NP) vf[(c + 3) % 4] = vfrag(c + 3);
      const int kst = c / DB, db = c % DB;
      O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[c % 4], pf[kst / 2][kst % 2], O[db], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Prologue: K(kt0), V(kt0), K(kt0 + 1) in LDS, S of tile kt0, then K(kt0 + 2) and
  // V(kt0 + 1) into registers.
  gload(rk, krs, kt0);
  gload(rv, vrs, kt0);
  sstore(rk, Ks[0], KS);
  sstore(rv, Vs[0], VS);
  if (kt0 < kt1) {
    gload(rk, krs, kt0 + 1);
    sstore(rk, Ks[1], KS);
  }
  __syncthreads();
  f32x16_t Sa[2], Sb[2];
  qk(0, Sa);
  if (kt0 + 2 <= kt1) gload(rk, krs, kt0 + 2);
  if (kt0 + 1 <= kt1) gload(rv, vrs, kt0 + 1);
  // The first iteration stores K(kt0 + 2) into K buffer 0, which every wave has just read.
  __syncthreads();
  // Iteration t (PAR = (t - kt0) & 1, a constant of the unrolled loop, so every LDS address
  // is a base plus an immediate): S of tile t + 1 from K buffer PAR ^ 1, softmax and PV of
  // tile t from V buffer PAR, then K(t + 2) into K buffer PAR (K(t) was last read in
  // iteration t - 1) and V(t + 1) into V buffer PAR ^ 1 (V(t - 1) was last read in
  // iteration t - 1), one barrier.
  auto iter = [&](int t, auto par, f32x16_t (&Sc)[2], f32x16_t (&Sn)[2], auto next)
      __attribute__((always_inline)) {
    constexpr int PAR = decltype(par)::value;
    const float neg_m = softmax_max(t, Sc);
    exp_pv(par, Sc, neg_m, next, Sn);
    if (t + 2 <= kt1) sstore(rk, Ks[PAR], KS);
    if (t + 1 <= kt1) sstore(rv, Vs[PAR ^ 1], VS);
    if (t + 3 <= kt1) gload(rk, krs, t + 3);
    if (t + 2 <= kt1) gload(rv, vrs, t + 2);
    __syncthreads();
  };
  using more = std::true_type;
  using last = std::false_type;
  using even = std::integral_constant<int, 0>;
  using odd = std::integral_constant<int, 1>;
  int t = kt0;
  for (; t + 2 <= kt1; t += 2) {
    iter(t, even{}, Sa, Sb, more{});
    iter(t + 1, odd{}, Sb, Sa, more{});
  }
  if (t < kt1) {
    iter(t, even{}, Sa, Sb, more{});
    iter(t + 1, odd{}, Sb, Sa, last{});
  } else {
    iter(t, even{}, Sa, Sb, last{});
  }

  if (qw >= L) return;
  const float inv = 1.0f / l_run;
  bf16_t* op = P.o + (orow0 + qw) * P.ldo + (size_t)h * HD;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = 32 * db + 8 * r4 + 4 * half;
      u32x2_t v;
      v.x = pack_bf2(O[db][4 * r4 + 0] * inv, O[db][4 * r4 + 1] * inv);
      v.y = pack_bf2(O[db][4 * r4 + 2] * inv, O[db][4 * r4 + 3] * inv);
      *reinterpret_cast<u32x2_t*>(op + d) = v;
    }
}

// ---------------------------------------------------------------- fp32
// Varlen (row_seq != NULL): workgroup x takes packed row x (skipped when not live); q is
// [Hq, T, hd], keys come from cache row s (kv_by_seq) or the packed scratch [Hkv, T, hd].
struct AttnVarlenF32 {
  const int32_t* row_seq;
  const int32_t* cu;
  int T;
  int kv_by_seq;
};

template <int HD>
__global__ __launch_bounds__(64) void attn_prefill_f32(const float* __restrict__ q,
                                                       const float* __restrict__ k,
                                                       const float* __restrict__ v, int Hq, int Hkv,
                                                       int L, int cap, int sliding, int window,
                                                       const int32_t* __restrict__ start,
                                                       float scale, float* __restrict__ o, int ldo,
                                                       AttnVarlenF32 vl) {
  constexpr int DPL = (HD + 63) / 64;  // d values per lane in the PV accumulation
  __shared__ float qs[HD];
  const int h = blockIdx.y, lane = threadIdx.x;
  const int kvh = h / (Hq / Hkv);
  int il, s0;
  const float *qp, *kb, *vb;
  float* op;
  if (vl.row_seq) {
    const int m = blockIdx.x;
    const int sq = vl.row_seq[m];
    if (sq < 0) return;  // row not processed (uniform)
    const int m0 = vl.cu[sq];
    il = m - m0;
    qp = q + ((size_t)h * vl.T + m) * HD;
    op = o + (size_t)m * ldo + (size_t)h * HD;
    if (vl.kv_by_seq) {
      s0 = start ? start[sq] : 0;
      kb = k + ((size_t)sq * Hkv + kvh) * cap * HD;
      vb = v + ((size_t)sq * Hkv + kvh) * cap * HD;
    } else {
      s0 = 0;
      kb = k + ((size_t)kvh * vl.T + m0) * HD;
      vb = v + ((size_t)kvh * vl.T + m0) * HD;
    }
  } else {
    il = blockIdx.x;
    const int b = blockIdx.z;
    s0 = start ? start[b] : 0;  // cache index of the chunk's first query
    if (s0 < 0 || s0 > cap - L) s0 = 0;
    qp = q + (((size_t)b * Hq + h) * L + il) * HD;
    op = o + ((size_t)b * L + il) * ldo + (size_t)h * HD;
    kb = k + ((size_t)b * Hkv + kvh) * cap * HD;
    vb = v + ((size_t)b * Hkv + kvh) * cap * HD;
  }
  const int i = s0 + il;          // cache index of this query
  for (int d = lane; d < HD; d += 64) qs[d] = qp[d];
  __syncthreads();
  const int lo = sliding ? max(0, i - window + 1) : 0;
  float m = -INFINITY, l = 0.f, acc[DPL];
#pragma unroll
  for (int t = 0; t < DPL; ++t) acc[t] = 0.f;
  for (int c0 = lo; c0 <= i; c0 += 64) {
    const int key = c0 + lane;
    float s = -INFINITY;
    if (key <= i) {
      const float* kp = kb + (size_t)key * HD;
      float dot = 0.f;
      for (int d = 0; d < HD; ++d) dot = fmaf(qs[d], kp[d], dot);
      s = dot * scale;
    }
    const float m_new = fmaxf(m, wave_max(s));
    const float alpha = expf(m - m_new);
    const float p = (key <= i) ? expf(s - m_new) : 0.f;
    l = l * alpha + wave_sum(p);
    m = m_new;
#pragma unroll
    for (int t = 0; t < DPL; ++t) acc[t] *= alpha;
    const int n = min(64, i - c0 + 1);
    for (int j = 0; j < n; ++j) {
      const float pj = __shfl(p, j, 64);
      const float* vp = vb + (size_t)(c0 + j) * HD;
#pragma unroll
      for (int t = 0; t < DPL; ++t) {
        const int d = lane + 64 * t;
        if (d < HD) acc[t] = fmaf(pj, vp[d], acc[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < DPL; ++t) {
    const int d = lane + 64 * t;
    if (d < HD) op[d] = acc[t] / l;
  }
}

}  // namespace

hipError_t launch_attention_prefill(int dtype, const void* q, const void* k, const void* v, int B,
                                    int Hq, int Hkv, int L, int cap, int hd, int sliding, int window,
                                    const int32_t* start, void* o, int ldo, hipStream_t s) {
  if (dtype == 1) {
    AttnParams P;
    P.q = (const bf16_t*)q; P.k = (const bf16_t*)k; P.v = (const bf16_t*)v;
    P.B = B; P.Hq = Hq; P.Hkv = Hkv; P.L = L; P.cap = cap;
    P.sliding = sliding; P.window = window;
    P.start = start;
    P.o = (bf16_t*)o; P.ldo = ldo;
    P.scale_log2 = kLog2e / sqrtf((float)hd);
    P.nqb = (L + QB - 1) / QB;
    P.tiles = nullptr; P.n_tiles = nullptr; P.cu = nullptr; P.T = 0; P.kv_by_seq = 0;
    const int groups = B * Hkv, per_group = P.nqb * (Hq / Hkv);
    dim3 grid(P.nqb, Hq, B);
    if (groups % 8 == 0) {
      P.xmode = 1;
      grid = dim3((unsigned)(groups * per_group), 1, 1);
    } else if (8 % groups == 0) {
      P.xmode = 2;
      const int r = 8 / groups;
      grid = dim3((unsigned)(8 * ((per_group + r - 1) / r)), 1, 1);
    } else {
      P.xmode = 0;
    }
    if (hd == 128) attn_prefill_bf16<128><<<grid, 256, 0, s>>>(P);
    else attn_prefill_bf16<64><<<grid, 256, 0, s>>>(P);
  } else {
    const dim3 grid(L, Hq, B);
    const float scale = 1.0f / sqrtf((float)hd);
    const AttnVarlenF32 vl{nullptr, nullptr, 0, 0};
    if (hd == 128)
      attn_prefill_f32<128><<<grid, 64, 0, s>>>((const float*)q, (const float*)k, (const float*)v, Hq,
                                                Hkv, L, cap, sliding, window, start, scale, (float*)o, ldo, vl);
    else
      attn_prefill_f32<64><<<grid, 64, 0, s>>>((const float*)q, (const float*)k, (const float*)v, Hq,
                                               Hkv, L, cap, sliding, window, start, scale, (float*)o, ldo, vl);
  }
  return hipGetLastError();
}

int varlen_tile_rows(int dtype) { return dtype == 1 ? QB : 0; }

hipError_t launch_attention_prefill_varlen(int dtype, const void* q, const void* k, const void* v, int T,
                                           int Hq, int Hkv, int cap, int hd, int sliding, int window,
                                           const int32_t* start, int kv_by_seq, const VarlenPlan& vp,
                                           void* o, int ldo, hipStream_t s) {
  if (dtype == 1) {
    AttnParams P;
    P.q = (const bf16_t*)q; P.k = (const bf16_t*)k; P.v = (const bf16_t*)v;
    P.B = 1; P.Hq = Hq; P.Hkv = Hkv; P.L = T; P.cap = cap;
    P.sliding = sliding; P.window = window;
    P.start = start;
    P.o = (bf16_t*)o; P.ldo = ldo;
    P.scale_log2 = kLog2e / sqrtf((float)hd);
    P.nqb = 0;
    P.tiles = vp.tiles; P.n_tiles = vp.n_tiles; P.cu = vp.cu; P.T = T; P.kv_by_seq = kv_by_seq;
    P.xmode = 0;
    const dim3 grid(vp.max_tiles, Hq, 1);
    if (hd == 128) attn_prefill_bf16<128><<<grid, 256, 0, s>>>(P);
    else attn_prefill_bf16<64><<<grid, 256, 0, s>>>(P);
  } else {
    const dim3 grid(T, Hq, 1);
    const float scale = 1.0f / sqrtf((float)hd);
    const AttnVarlenF32 vl{vp.row_seq, vp.cu, T, kv_by_seq};
    if (hd == 128)
      attn_prefill_f32<128><<<grid, 64, 0, s>>>((const float*)q, (const float*)k, (const float*)v, Hq,
                                                Hkv, T, cap, sliding, window, start, scale, (float*)o, ldo, vl);
    else
      attn_prefill_f32<64><<<grid, 64, 0, s>>>((const float*)q, (const float*)k, (const float*)v, Hq,
                                               Hkv, T, cap, sliding, window, start, scale, (float*)o, ldo, vl);
  }
  return hipGetLastError();
}

}  // namespace compass
