// Host-side launcher declarations and the small structs passed to kernels by value.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace compass {

// MRoPE parameters. Interleaved layout (layout 0): rotation pair f < head_dim / 2 uses
// frequency index j = f, inverse frequency theta^(-2j / head_dim) (evaluated in double,
// rounded once to fp32), and axis h when j % 3 == 1 and j < sh3 (= 3 * s_h), axis w when
// j % 3 == 2 and j < sw3 (= 3 * s_w), axis t otherwise. Sections layout (layout 1): pairs
// f < s_h use axis h, the next s_w axis w, the rest axis t, and each section carries, in
// increasing order, the frequency indices the interleaved layout gives its axis.
struct RopeTable {
  float theta;
  int sh3, sw3;
  int layout;
};

#ifdef __HIPCC__
__device__ __forceinline__ int rope_freq_index(const RopeTable& rt, int f) {
  if (!rt.layout) return f;
  const int sh = rt.sh3 / 3, sw = rt.sw3 / 3;
  if (f < sh) return 3 * f + 1;
  if (f < sh + sw) return 3 * (f - sh) + 2;
  // t section: below 3 min(s_h, s_w) the t indices are the multiples of 3; up to
  // 3 max(s_h, s_w) also the residue of the shorter axis; beyond that every index.
  const int k = f - sh - sw, a = min(sh, sw), bm = max(sh, sw);
  if (k < a) return 3 * k;
  const int mid = 2 * (bm - a);
  if (k < a + mid) {
    const int i = k - a;
    return 3 * (a + i / 2) + ((i & 1) ? (sh < sw ? 1 : 2) : 0);
  }
  return 3 * bm + (k - a - mid);
}
__device__ __forceinline__ float rope_inv_freq(const RopeTable& rt, int f, int hd) {
  return (float)pow((double)rt.theta, -2.0 * (double)rope_freq_index(rt, f) / (double)hd);
}
__device__ __forceinline__ int rope_axis(const RopeTable& rt, int f) {
  if (rt.layout) {
    const int sh = rt.sh3 / 3, sw = rt.sw3 / 3;
    return f < sh ? 1 : (f < sh + sw ? 2 : 0);
  }
  const int r = f % 3;
  return (r == 1 && f < rt.sh3) ? 1 : (r == 2 && f < rt.sw3) ? 2 : 0;
}
#endif

// Where row n of the virtual B operand ([N, K], K contiguous) lives.
//  kind 0: one matrix p[0] with row stride ld0.
//  kind 1: the fused projection. N is split in 64-row chunks: nq64 chunks of wq,
//          nk64 of wk, nk64 of wv, then 2*I/64 chunks alternating w_gate / w_up
//          (chunk 2c -> gate rows [64c, 64c+64), chunk 2c+1 -> up rows of the same c).
//          All five matrices have row stride ld0 (= D).
//  kind 2: concatenation along K: columns k < ksplit come from p[0] (stride ld0),
//          columns k >= ksplit from p[1] (stride ld1) at k - ksplit.
struct BMap {
  int kind;
  const void* p[5];
  int ld0, ld1;
  int ksplit;
  int nq64, nk64;
};

// 4-bit affine B operand (rows of codes packed two per byte, column 2j in the low nibble;
// bf16 scale and bias per 64 columns). kind 1: the projection's virtual N layout of BMap
// kind 1 (matrices 0..4 = q, k, v, gate, up; all cols0 columns wide). kind 2: concatenation
// along K (matrix 0, cols0 columns, for k < ksplit; matrix 1, cols1 columns, after).
struct Q4Map {
  int kind;
  const void* q[5];
  const void* s[5];
  const void* b[5];
  int cols0, cols1;
  int ksplit;
  int nq64, nk64;
};

// Destinations of the projection epilogue (q/k/v with MRoPE, KV write, SwiGLU).
struct ProjEpi {
  int decode;           // 0: row m is (b = m / L, l = m % L); 1: row m is b = m, l = lens[b]
  int L;
  const int32_t* pos;   // prefill [3, B, L]; decode [3, B]; NULL when rope == 0
  int pos_stride;       // distance between the t, h, w planes (B*L or B)
  int rope;             // 1: rotate q and k
  int Hq, Hkv, hd;
  void* q;              // [B, Hq, Lq, hd]
  int Lq;
  void* kc;             // [B, Hkv, cap, hd]
  void* vc;
  int cap;
  const int32_t* lens;  // decode: cache index of the new token, per row
  const int32_t* kv_start;  // chunked prefill: row b's K/V go to cache index kv_start[b] + l
                            // (rows with kv_start[b] outside [0, cap - L] write none); else NULL.
                            // Varlen: the cached tokens of each sequence (NULL: none).
  // Varlen prefill (packed sequences, B = 1 and L = T): row_seq[m] is the sequence of packed
  // row m, or -1 when the row is not processed (its K/V are not written); cu[s] is the first
  // packed row of sequence s. kv_by_seq: K/V of row m go to cache row s at kv_start[s] +
  // m - cu[s]; otherwise to the packed scratch [1, Hkv, T, hd] at row m. NULL when not varlen.
  const int32_t* row_seq;
  const int32_t* cu;
  int kv_by_seq;
  void* act;            // act[m * ldact + act_col0 + c] = silu(gate) * up
  int ldact;
  int act_col0;
  int nq64, nk64;
  int I;
};

// Chunked prefill rows: row b of a [B, L] chunk continues a cache holding start[b] tokens
// and is processed only when 0 <= start[b] <= cap - L; otherwise it is skipped (no K/V
// written, its output rows left as they were). start == NULL: every row is live.
// Varlen prefill: row_seq (when not NULL) decides instead, row m being live iff
// row_seq[m] >= 0.
struct RowStart {
  const int32_t* start;
  int L;
  int cap;
  const int32_t* row_seq;
};
#ifdef __HIPCC__
__device__ __forceinline__ bool row_live(const RowStart& r, int b) {
  if (!r.start) return true;
  const int s0 = r.start[b];
  return s0 >= 0 && s0 <= r.cap - r.L;
}
// Liveness of flattened row m (= b * L + l, or a packed varlen row).
__device__ __forceinline__ bool row_live_m(const RowStart& r, int m) {
  if (r.row_seq) return r.row_seq[m] >= 0;
  return row_live(r, m / r.L);
}
#endif

// Varlen prefill plan (device buffers carved from the workspace): the packed rows' sequences
// and the attention's query tiles. tiles[2 t], tiles[2 t + 1] = (sequence, query block) of
// tile t < *n_tiles, ordered by query block, latest first.
struct VarlenPlan {
  const int32_t* cu;  // [n_seq + 1], caller's offsets (validated on the device)
  int n_seq;
  int32_t* row_seq;   // [T]
  int32_t* tiles;     // [2 * max_tiles]
  int32_t* n_tiles;   // [1]
  int max_tiles;
};
constexpr int kVarlenMaxSeqs = 4096;
constexpr int kVarlenMaxTokens = 1 << 19;

// Raise `kernel`'s dynamic LDS limit to `bytes` on the current device, once per (device,
// kernel); thread-safe (defined in api.hip).
hipError_t ensure_dynamic_lds(const void* kernel, int bytes);

// ---------------------------------------------------------------- launchers
hipError_t launch_positions(const int32_t* tok, int B, int L, int image_id, const int32_t* grid,
                            const int32_t* img_off, int merge, int32_t* pos, int32_t* delta,
                            int32_t* status, hipStream_t s);

// a = LN(x) over rows [rows, D] (x rows ldx elements apart, default D; a contiguous);
// dtype 1 = bf16, 0 = f32 (a has the dtype of x).
hipError_t launch_layernorm(int dtype, const void* x, const void* w, float eps, void* a, int rows,
                            int D, hipStream_t s, long long ldx = 0);

// bf16 MFMA GEMMs, C[m, n] = sum_k A[m, k] * B[n, k], A [M, lda] bf16.
// Fused projection epilogue (MRoPE, q/k/v scatter, SwiGLU); N = virtual projection width.
// ln_stats != NULL: A is the layer input x and the LayerNorm is fused: each A piece is
// normalized in registers, (x - mean) * rstd * ln_w with the rows' (mean, rstd) from
// launch_ln_stats, before it is staged in LDS.
hipError_t launch_gemm_bf16_proj(const void* A, int lda, int M, int K, const BMap& bm, int N,
                                 const ProjEpi& ep, const RopeTable& rt, hipStream_t s,
                                 const float2* ln_stats = nullptr, const void* ln_w = nullptr);
// Per-row (mean, rstd) of bf16 rows [rows, D], the LayerNorm kernel's own values.
hipError_t launch_ln_stats(const void* x, float eps, float2* stats, int rows, int D, hipStream_t s);
// out[m, n] = x[m, n] + C (bf16; out may alias x); rows m of batch rows b = m / rs.L that
// are not live (RowStart) are not stored.
hipError_t launch_gemm_bf16_resid(const void* A, int lda, int M, int K, const BMap& bm, int N,
                                  const void* x, void* out, int ldo, const RowStart& rs, hipStream_t s);
// out[m, n] = C * scale (fp32).
hipError_t launch_gemm_bf16_scaled_f32(const void* A, int lda, int M, int K, const BMap& bm, int N,
                                       float scale, float* out, long long ldo, hipStream_t s);
// Greedy head without storing the logits: pv[m][p], pi[m][p] = the largest C * scale over
// the p-th 128-column span of row m and its column (smallest on ties). Returns the number
// of spans per row (2 * ceil(N / 256)); *err receives the launch status.
int gemm_bf16_argmax(const void* A, int lda, int M, int K, const BMap& bm, int N, float scale, float* pv,
                     int* pi, hipStream_t s, hipError_t* err);
// raw[z][m][n] = partial C over K-slice z (fp32), splits slices of K (64 x 64 tiles, for
// skinny decode GEMMs; the _wide variant uses 256 x 256 tiles).
hipError_t launch_gemm_bf16_raw(const void* A, int lda, int M, int K, const BMap& bm, int N,
                                int splits, float* raw, hipStream_t s);
// The same raw partial sums for at most 64 rows and a BMap of kind 2 (the decode output
// projection [Wo | Wd]; N a multiple of 4), with K / splits equal to 512, 640, 1024 or 1280: one 64-column
// tile per workgroup and K-slice, weights loaded several steps ahead.
bool gemm_skinny_fits(int M, int K, int N, int splits);
hipError_t launch_gemm_skinny_raw(const void* A, int lda, int M, int K, const BMap& bm, int N, int splits,
                                  float* raw, hipStream_t s);
hipError_t launch_gemm_bf16_raw_wide(const void* A, int lda, int M, int K, const BMap& bm, int N,
                                     int splits, float* raw, hipStream_t s);
// K splits for the residual output GEMM: 1 when 128 x 256 tiles fill the CUs, else enough
// 256 x 256 split-K workgroups to (the partials then go through launch_splitk_resid).
int gemm_bf16_resid_splits(int M, int N, int K);

// Same contract as launch_gemm_bf16_raw with the B operand in 4-bit affine form (64 x 64
// tiles; K, N, ksplit and the matrices' widths multiples of 64).
hipError_t launch_gemm_q4_raw(const void* A, int lda, int M, int K, const Q4Map& bm, int N, int splits, float* raw,
                              hipStream_t s);

// fp32 GEMM (VALU), same contract as launch_gemm_bf16_raw with fp32 operands; every
// stored sum is multiplied by `scale` (1 for raw partials).
hipError_t launch_gemm_f32_raw(const void* A, int lda, int M, int K, const BMap& bm, int N,
                               int splits, float* raw, float scale, hipStream_t s);

// Projection epilogue over raw fp32 partial sums [splits][M][N].
hipError_t launch_proj_epilogue(int dtype, const float* raw, int splits, int M, int N,
                                const ProjEpi& ep, const RopeTable& rt, hipStream_t s);
// out[m, n] = x[m, n] + sum_z raw[z][m][n]; rows m of batch rows b = m / rs.L that are not
// live (RowStart; decode passes lens with L = 1) are skipped.
// bf16 split-K residual (as launch_splitk_resid) that also writes the next layer's LayerNorm
// of each live output row, norm[m] = LayerNorm(out[m]; ln_w, eps) in bf16, with the values
// the LayerNorm kernel gives. N % 8 == 0.
hipError_t launch_splitk_resid_ln(const float* raw, int splits, int M, int N, const void* x, void* out,
                                  const RowStart& rs, const void* ln_w, float eps, void* norm, hipStream_t s);
hipError_t launch_splitk_resid(int dtype, const float* raw, int splits, int M, int N, const void* x,
                               void* out, const RowStart& rs, hipStream_t s);

// Prefill attention: q [B, Hq, L, hd]; k, v [B, Hkv, cap, hd]; o written to
// o[(b*L + l) * ldo + h*hd + d]. Query l of row b sits at cache index start[b] + l
// (start == NULL: l) and sees the cache keys up to it; rows that are not live are
// computed as if start[b] = 0 (memory-safe; their outputs are not used).
hipError_t launch_attention_prefill(int dtype, const void* q, const void* k, const void* v, int B,
                                    int Hq, int Hkv, int L, int cap, int hd, int sliding, int window,
                                    const int32_t* start, void* o, int ldo, hipStream_t s);
// Varlen prefill attention over T packed rows (q [Hq, T, hd]; o row m at o[m * ldo + h * hd]).
// kv_by_seq: keys of sequence s in cache row s of k, v [n_seq, Hkv, cap, hd], its first query
// at cache index start[s] (start NULL: 0); else keys in the packed scratch [Hkv, T, hd].
// Only the plan's tiles (bf16) or live rows (fp32) are computed.
hipError_t launch_attention_prefill_varlen(int dtype, const void* q, const void* k, const void* v, int T,
                                           int Hq, int Hkv, int cap, int hd, int sliding, int window,
                                           const int32_t* start, int kv_by_seq, const VarlenPlan& vp,
                                           void* o, int ldo, hipStream_t s);
// Builds the plan: validates cu (cu[0] = 0, non-decreasing, cu[n_seq] = T), marks each
// sequence live iff start == NULL or 0 <= start[s] <= cap - len_s, fills row_seq (-1 for
// rows not processed) and, when tile_rows > 0, the query tiles of tile_rows queries.
// status (may be NULL) gets bit 0 for invalid offsets (then nothing is live) and bit 1
// when a sequence was skipped.
hipError_t launch_varlen_plan(const VarlenPlan& vp, int T, const int32_t* start, int cap, int tile_rows,
                              int32_t* status, hipStream_t s);
int varlen_tile_rows(int dtype);

// Decode attention, split over key chunks, then combine.
int decode_chunk_keys(int dtype, int hd);
hipError_t launch_decode_attention(int dtype, const void* q, const void* k, const void* v,
                                   const int32_t* lens, int B, int Hq, int Hkv, int cap, int hd,
                                   int sliding, int window, int n_chunks, float* part,
                                   hipStream_t s);
hipError_t launch_decode_combine(int dtype, const float* part, const int32_t* lens, int B, int Hq,
                                 int cap, int hd, int n_chunks, void* o, int ldo, hipStream_t s);

// out[rows[r]] += ds[r], rows outside [0, n_rows) or in batch rows that are not live skipped.
hipError_t launch_deepstack(int dtype, const int32_t* rows, const void* ds, int n_ds, int D,
                            int n_rows, const RowStart& rs, void* out, hipStream_t s);

// Token-id front end: h[r] = E[tokens[r]] (zero row for ids outside [0, V)), then
// h[img_rows[i]] = feats[i] (rows outside [0, R) skipped); status[0] (may be NULL) gets
// bit 0 if an id was outside [0, V), bit 1 if an image row was outside [0, R).
hipError_t launch_embed(int dtype, const int32_t* tokens, int R, int D, int V, const void* E,
                        const int32_t* img_rows, const void* feats, int n_img, void* h, int32_t* status,
                        hipStream_t s);
// lens[b] += advance; pos[a][b] = lens[b] + rope_delta[b] on the three axes.
hipError_t launch_decode_positions(int32_t* lens, const int32_t* rope_delta, int B, int32_t* pos, int advance,
                                   hipStream_t s);
// token[r] = argmax_v scale * raw[r * ldr + v] (smallest v on ties); max_logit optional.
// pv / pi: per-row chunk winners, R * argmax_chunks(V) floats / ints of scratch.
int argmax_chunks(int V);
// token[r] / max_logit[r] from nparts (value, id) partials per row (smallest id on ties).
hipError_t launch_argmax_partials(const float* pv, const int* pi, int R, int nparts, int32_t* token,
                                  float* max_logit, hipStream_t s);
hipError_t launch_argmax(const float* raw, int R, int V, long long ldr, float scale, float* pv, int* pi,
                         int32_t* token, float* max_logit, hipStream_t s);

}  // namespace compass
