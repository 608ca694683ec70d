/*
 * compass.h — C ABI of the MI355X (gfx950) Compass/Cohere2 parallel decoder layer.
 *
 * The layer is the one the mlxcel issue "feat(vlm): add Cohere Compass /
 * North-Micro-Vision (cohere_compass) VLM" defines in its section "Text decoder
 * forward": one weight-only LayerNorm a = LN(h) feeds an attention branch and a
 * SwiGLU branch, and h + attn(a) + mlp(a) is the output (parallel block, no
 * post-attention norm). Sliding-window layers rotate q and k with interleaved
 * three-axis MRoPE (section "Interleaved MRoPE"); full-attention layers use no
 * positional encoding. The stack alternates them 3:1 and ends with a tied
 * embedding head times logit_scale.
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless stated otherwise; the caller owns every
 *     buffer (inputs, outputs, caches, workspace). Nothing here allocates, frees
 *     or synchronizes device memory (the profiling helpers at the end excepted).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Calls
 *     enqueue their kernels on it and return immediately.
 *   - Return value: COMPASS_OK (0) or a negative compass_status. Argument checks
 *     happen on the host before anything is enqueued: on an error nothing runs
 *     and compass_last_error() returns a message (thread-local, valid until the
 *     next call on that thread). No C++ exception crosses this interface.
 *   - Tensors are contiguous, row-major, and 16-byte aligned. Dtype is
 *     COMPASS_BF16 (bf16 storage, fp32 accumulation) or COMPASS_F32 throughout a
 *     call: x, out, weights, KV cache and deepstack rows share the dtype.
 *   - Supported widths: head_dim in {64, 128}; hidden, intermediate and
 *     n_q_heads*head_dim multiples of 64; (n_q_heads + 2*n_kv_heads)*head_dim a
 *     multiple of 128; n_q_heads a multiple of n_kv_heads. Others return
 *     COMPASS_E_UNSUPPORTED.
 */
#ifndef COMPASS_H
#define COMPASS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  COMPASS_OK = 0,
  COMPASS_E_INVALID = -1,      /* null pointer, non-positive size, inconsistent shape */
  COMPASS_E_UNSUPPORTED = -2,  /* valid but outside the widths/dtypes listed above */
  COMPASS_E_ALIGN = -3,        /* a tensor pointer is not 16-byte aligned */
  COMPASS_E_WORKSPACE = -4,    /* workspace missing or smaller than the size query says */
  COMPASS_E_DEVICE = -5        /* the HIP runtime reported an error at launch */
} compass_status;

typedef enum { COMPASS_F32 = 0, COMPASS_BF16 = 1 } compass_dtype;
typedef enum { COMPASS_SLIDING = 0, COMPASS_FULL = 1 } compass_kind;
typedef enum { COMPASS_ROPE_INTERLEAVED = 0, COMPASS_ROPE_SECTIONS = 1 } compass_rope_layout;

/* Status words written by compass_mrope_positions (device, one per call). */
enum {
  COMPASS_POS_OK = 0,
  COMPASS_POS_SPAN_MISMATCH = 1,  /* an image's pad span runs past L or meets a non-pad token */
  COMPASS_POS_EXTRA_PADS = 2,     /* pad tokens remain but the row has no image left */
  COMPASS_POS_UNUSED_IMAGES = 3,  /* the row ends with images not consumed */
  COMPASS_POS_BAD_GRID = 4,       /* a grid entry < 1, or h / w not divisible by the merge size */
  COMPASS_POS_TOO_MANY_IMAGES = 5 /* more than COMPASS_MAX_IMAGES_PER_ROW images in a row */
};
#define COMPASS_MAX_IMAGES_PER_ROW 2048
#define COMPASS_MAX_TOKENS_PER_ROW 524288 /* compass_mrope_positions: L above this is unsupported */

/* One decoder layer's shape (host struct).
 * kind: COMPASS_SLIDING applies MRoPE and the window; COMPASS_FULL uses no
 *   positional encoding and a plain causal mask ("Text decoder forward").
 * window: sliding layers only; key j is visible to query i iff i - window < j <= i
 *   (the last `window` keys, the query's own key included). Must be >= 1.
 * mrope_section: {s_t, s_h, s_w} frequency counts, sum == head_dim / 2. Frequency j
 *   uses axis h when j % 3 == 1 and j < 3*s_h, axis w when j % 3 == 2 and j < 3*s_w,
 *   axis t otherwise ("Interleaved MRoPE"; [24, 20, 20] on the real model).
 * rope_theta: MRoPE base (50000 on the real model); inv_freq[j] = theta^(-2j/head_dim).
 * ln_eps: LayerNorm epsilon (the value is not printed by the page; callers pass it).
 * rope_layout: COMPASS_ROPE_INTERLEAVED (0), the layout above; or COMPASS_ROPE_SECTIONS
 *   (1), the correction under the issue's "Acceptance criteria" (contiguous [H, W, T]
 *   sections over a permuted inv_freq). Its permutation is not printed; this library
 *   reads it as: rotation pairs f < s_h use axis h, the next s_w axis w, the rest axis t,
 *   and each section carries, in increasing order, the frequency indices j the
 *   interleaved layout gives its axis (unverified against the real rotary class). */
typedef struct {
  int32_t hidden;        /* D */
  int32_t n_q_heads;     /* Hq */
  int32_t n_kv_heads;    /* Hkv; query head h reads kv head h / (Hq / Hkv) */
  int32_t head_dim;      /* hd */
  int32_t intermediate;  /* I, SwiGLU width */
  int32_t kind;          /* compass_kind */
  int32_t window;
  int32_t mrope_section[3];
  float rope_theta;
  float ln_eps;
  int32_t dtype;         /* compass_dtype */
  int32_t rope_layout;   /* compass_rope_layout; 0 = interleaved */
  int32_t ln_fuse;       /* bf16 prefill only: 0 (default) = LayerNorm kernel writing the
                            normalized bf16 rows, then the projection GEMM; 1 = the LayerNorm
                            fused into the projection GEMM ("Text decoder forward": one shared
                            LayerNorm feeding both branches): a statistics pass writes each
                            row's (mean, rstd), and the GEMM normalizes every A tile in
                            registers, (x - mean) * rstd * ln_w, as it stages it into LDS.
                            The two give bitwise identical results. 0 is faster on MI355X:
                            each A row block is staged by every column tile (76 of them at
                            the Compass widths), so normalizing there costs more than the
                            LayerNorm kernel it saves. Decode and fp32 ignore the field. */
} compass_layer_desc;

/* Weights of one layer, nn.Linear layout [out, in], no biases (section "Weight keys":
 * input_layernorm.weight, self_attn.{q,k,v,o}_proj.weight, mlp.{gate,up,down}_proj.weight). */
typedef struct {
  const void *ln_w;    /* [D] */
  const void *wq;      /* [Hq*hd, D] */
  const void *wk;      /* [Hkv*hd, D] */
  const void *wv;      /* [Hkv*hd, D] */
  const void *wo;      /* [D, Hq*hd] */
  const void *w_gate;  /* [I, D] */
  const void *w_up;    /* [I, D] */
  const void *w_down;  /* [D, I] */
} compass_layer_weights;

/* Dense KV cache of one layer (the page's correction under "Acceptance criteria":
 * a dense cache with the window applied as a mask). Keys are stored AFTER MRoPE on
 * sliding layers. The library never advances `lens`; the caller does, once per
 * decode step, after all layers have run. */
typedef struct {
  void *k;              /* [B, Hkv, capacity, hd] */
  void *v;              /* [B, Hkv, capacity, hd] */
  int32_t capacity;     /* rows per (row, kv head) slice; prefill requires capacity * hd * element
                           size < 2^31 bytes (COMPASS_E_UNSUPPORTED otherwise) */
  const int32_t *lens;  /* device [B]: tokens already cached (decode only; prefill ignores it) */
} compass_kv;

/* Position ids, section "Position ids (get_rope_index)" of the mlxcel issue: text
 * tokens advance (t, h, w) by one; image k with patch grid (t, h, w) and merge m
 * takes the next t*(h/m)*(w/m) image-pad tokens, which get start + (t_i, h_i, w_i)
 * on the merged grid; the next text token starts at max(position) + 1;
 * rope_delta[b] = max position + 1 - L. Integer arithmetic, bit-exact.
 *   token_ids  [B, L] int32     grid_thw [n_img, 3] int32 (patch units, images in
 *   row order)    img_offset [B+1] int32: images of row b are [img_offset[b],
 *   img_offset[b+1])    pos out [3, B, L] int32    rope_delta out [B] int32
 *   status out [B] int32: COMPASS_POS_* per row, the first error a left-to-right walk
 *   over the row's tokens meets (read it after the stream has synchronized); for a
 *   failing row, pos and rope_delta of that row are left unwritten.
 * Decode positions are lens[b] + rope_delta[b] on all three axes (caller computes). */
int compass_mrope_positions(const int32_t *token_ids, int32_t B, int32_t L,
                            int32_t image_token_id, const int32_t *grid_thw,
                            const int32_t *img_offset, int32_t spatial_merge,
                            int32_t *pos, int32_t *rope_delta, int32_t *status,
                            void *stream);

/* Bytes of device workspace compass_layer_prefill (L > 1, or decode == 0) or
 * compass_layer_decode (decode != 0, L ignored) needs for this shape; `capacity`
 * is the KV capacity (decode) and is ignored for prefill. Returns 0 for an
 * invalid or unsupported descriptor. */
size_t compass_workspace_size(const compass_layer_desc *d, int32_t B, int32_t L,
                              int32_t capacity, int32_t decode);

/* Prefill of one layer over B rows of L tokens (the "Text decoder forward" loop body):
 *   out = x + o_proj(attn(MRoPE(q), MRoPE(k), v)) + down(silu(gate(a)) * up(a)),
 *   a = LN(x), then out[ds_rows[r]] += ds[r] (deepstack, "after layers 0, 1, 2").
 *   x    [B, L, D]           pos [3, B, L] int32 (sliding only; may be NULL for FULL)
 *   kv   optional (NULL = keep K/V in the workspace): K/V of rows [0, L) are written
 *        to kv->k / kv->v (capacity >= L)
 *   ds_rows [n_ds] int32 flattened row indices b*L + l, distinct; ds [n_ds, D];
 *        n_ds == 0 (pointers may be NULL) for no deepstack. Rows outside [0, B*L)
 *        are skipped.
 *   out  [B, L, D]; may alias x exactly (in-place residual update).
 *   workspace: compass_workspace_size(d, B, L, 0, 0) bytes, 256-byte aligned. */
int compass_layer_prefill(const compass_layer_desc *d, const compass_layer_weights *w,
                          int32_t B, int32_t L, const void *x, const int32_t *pos,
                          const compass_kv *kv, const int32_t *ds_rows, const void *ds,
                          int32_t n_ds, void *out, void *workspace, size_t ws_bytes,
                          void *stream);

/* Chunked prefill: the [B, L] chunk continues a dense cache ("Acceptance criteria"
 * correction of the mlxcel Compass issue: dense cache, window as a mask; chunk
 * boundaries as in FreeToken's "How it fits together"). Row b already holds
 * kv->lens[b] tokens; token l of the chunk sits at cache index lens[b] + l, its K/V
 * (after MRoPE on sliding layers) are written there, and it attends to cache keys
 * j <= lens[b] + l (and j > lens[b] + l - window on sliding layers). pos [3, B, L]
 * holds the chunk tokens' positions (they continue the row's positions). With L = 1 this
 * is the decode step; with lens = 0 it is compass_layer_prefill writing the cache.
 *   kv (required, lens required, capacity >= L). Rows with lens[b] < 0 or
 *   lens[b] + L > capacity are skipped: no K/V written, their out rows (deepstack
 *   included) left as they were. The library does not advance lens.
 *   Other arguments, the workspace (compass_workspace_size(d, B, L, 0, 0)) and the
 *   error behaviour are those of compass_layer_prefill. */
int compass_layer_prefill_chunk(const compass_layer_desc *d, const compass_layer_weights *w,
                                int32_t B, int32_t L, const void *x, const int32_t *pos,
                                const compass_kv *kv, const int32_t *ds_rows, const void *ds,
                                int32_t n_ds, void *out, void *workspace, size_t ws_bytes,
                                void *stream);

/* Varlen prefill: n_seq sequences of different lengths packed into T rows, one launch,
 * no padding (FreeToken PR "feat(mm): serve image input on the Qwen families", "How it
 * fits together": prefill planned per request, each with its own MRoPE positions and its
 * own prefix cache; mlxcel Compass issue, "Validation": prefill causal within a sequence,
 * and the "Acceptance criteria" correction: dense cache, window as a mask). Sequence s is
 * packed rows [cu_seqlens[s], cu_seqlens[s + 1]); its token i attends to the keys of that
 * sequence only.
 *   cu_seqlens: device int32 [n_seq + 1], cu[0] = 0, non-decreasing, cu[n_seq] = T
 *     (empty sequences allowed). 1 <= n_seq <= 4096, 1 <= T <= 524288.
 *   x [T, D]; pos [3, T] int32 (each sequence's own positions; sliding only); out [T, D]
 *     (may alias x); ds_rows index packed rows.
 *   kv (optional): caches [n_seq, Hkv, capacity, hd]; kv->lens (optional, device [n_seq]):
 *     tokens sequence s already holds (NULL: none). Token i of sequence s then sits at cache
 *     index lens[s] + i, its K/V (after MRoPE on sliding layers) are written there, and it
 *     sees cache keys j <= lens[s] + i (and > lens[s] + i - window on sliding layers). A
 *     sequence with lens[s] < 0 or lens[s] + len_s > capacity is skipped: no K/V written,
 *     its out rows left as they were. kv NULL: K/V stay in the workspace.
 *   status (optional, device int32 [1], read after the stream synchronizes): bit 0 = the
 *     offsets are invalid (then nothing is computed or written), bit 1 = a sequence was
 *     skipped.
 *   workspace: compass_varlen_workspace_size(d, n_seq, T) bytes, 256-byte aligned. Other
 *   errors as compass_layer_prefill (all checked on the host before any launch). */
size_t compass_varlen_workspace_size(const compass_layer_desc *d, int32_t n_seq, int32_t T);
int compass_layer_prefill_varlen(const compass_layer_desc *d, const compass_layer_weights *w,
                                 int32_t n_seq, int32_t T, const int32_t *cu_seqlens,
                                 const void *x, const int32_t *pos, const compass_kv *kv,
                                 const int32_t *ds_rows, const void *ds, int32_t n_ds,
                                 void *out, int32_t *status, void *workspace, size_t ws_bytes,
                                 void *stream);

/* One decode step of one layer: one new token per row. The mlxcel Compass issue defines
 * it: "Text decoder forward" gives the layer (one shared LayerNorm, the attention and
 * SwiGLU branches summed into the residual, MRoPE on sliding layers only); the correction
 * under "Acceptance criteria" keeps a dense cache with the window applied as a mask; and
 * "Position ids (get_rope_index)" places a generated token at its cache offset plus the
 * row's rope_delta on all three axes.
 *   x [B, D]; pos [3, B] int32 (lens[b] + rope_delta[b] on every axis; unread for FULL)
 *   kv (required): the new token's K/V are written at index lens[b]; keys
 *   max(0, lens[b] - window + 1) .. lens[b] (sliding) or 0 .. lens[b] (full) are
 *   attended. Requires 0 <= lens[b] < capacity (rows violating it are skipped
 *   and their output left unwritten).
 *   out [B, D]; may alias x.
 *   workspace: compass_workspace_size(d, B, 1, kv->capacity, 1) bytes. */
int compass_layer_decode(const compass_layer_desc *d, const compass_layer_weights *w,
                         int32_t B, const void *x, const int32_t *pos, const compass_kv *kv,
                         void *out, void *workspace, size_t ws_bytes, void *stream);

/* compass_layer_decode for a stack of layers called one after another, with each layer's
 * shared LayerNorm ("Text decoder forward" of the mlxcel Compass issue: LayerNorm of the
 * layer input, weight only, in fp32) computed by the layer before it: the call that
 * produces a layer's input also writes that input's LayerNorm, from its residual kernel,
 * and the next call reads it instead of running its own LayerNorm kernel.
 *   x_norm: NULL (the layer runs its LayerNorm kernel on x), or bf16 [B, D] holding
 *     LayerNorm(x) with this layer's ln_w and ln_eps, as written to out_norm by the call
 *     that produced x (given that call's next_ln_w = this layer's ln_w and next_ln_eps =
 *     its ln_eps). Any other values give a different layer.
 *   next_ln_w, next_ln_eps, out_norm: out_norm NULL, or bf16 [B, D] that receives
 *     LayerNorm(out) with the weight next_ln_w (bf16 [D]) and eps next_ln_eps, equal bit
 *     for bit to what the LayerNorm kernel computes from out; rows that are skipped (lens
 *     out of range) are not written. next_ln_w is required with out_norm.
 *   16-byte aligned device buffers; x_norm and out_norm may be the same buffer (x_norm is
 *   read before out_norm is written, in stream order). Other arguments, the workspace
 *   (compass_workspace_size(d, B, 1, kv->capacity, 1)), outputs and errors are those of
 *   compass_layer_decode; the results equal a chain of compass_layer_decode calls bit for
 *   bit. Needs d->dtype == COMPASS_BF16 when x_norm or out_norm is given (else
 *   COMPASS_E_UNSUPPORTED). */
int compass_layer_decode_chained(const compass_layer_desc *d, const compass_layer_weights *w,
                                 int32_t B, const void *x, const void *x_norm, const int32_t *pos,
                                 const compass_kv *kv, void *out, const void *next_ln_w,
                                 float next_ln_eps, void *out_norm, void *workspace, size_t ws_bytes,
                                 void *stream);

/* Decode without allocation, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. It is
 * compass_layer_decode (same arguments, kernels, outputs and errors) with the workspace
 * taken from a device array of COMPASS_NOALLOC_SCRATCH_BYTES that the library holds on
 * each GPU it runs on until the process ends; the call allocates and frees nothing.
 * The first call on a device looks up that device's array (make that first call outside
 * any graph capture). The decode step needs no workspace byte to start at zero.
 * A step whose workspace (compass_workspace_size(d, B, 1, kv->capacity, 1)) exceeds
 * COMPASS_NOALLOC_SCRATCH_BYTES returns COMPASS_E_WORKSPACE before any launch; at the
 * Compass widths (hidden 2048, 16/4 heads, head_dim 128, I 8192) and B = 64 that allows
 * a full-attention layer a capacity of about 22,000 keys. Every call on one GPU shares
 * that GPU's array and it keeps the last call's contents: calls that overlap on one GPU
 * (on different streams or threads) race and must be serialized by the caller. */
#define COMPASS_NOALLOC_SCRATCH_BYTES (64u << 20)
int compass_layer_decode_noalloc(const compass_layer_desc *d, const compass_layer_weights *w,
                                 int32_t B, const void *x, const int32_t *pos,
                                 const compass_kv *kv, void *out, void *stream);

/* 4-bit affine weights: the quantization block of the 4-bit checkpoint in the mlxcel
 * Compass issue's config section (group size 64, 4 bits, affine mode). For a matrix of
 * [rows, cols] (cols a multiple of 64):
 *   W[r][c] = scale[r][c / 64] * code[r][c] + bias[r][c / 64],  code in 0..15.
 * The caller owns all buffers (device memory). */
typedef struct {
  const void *q;       /* uint8 [rows, cols / 2]: byte j of a row holds column 2j in its low
                          nibble and column 2j + 1 in its high nibble; 16-byte aligned */
  const void *scales;  /* bf16 [rows, cols / 64] */
  const void *biases;  /* bf16 [rows, cols / 64] */
} compass_q4_matrix;

typedef struct {
  const void *ln_w;    /* bf16 [D] */
  compass_q4_matrix wq, wk, wv, wo, w_gate, w_up, w_down;  /* shapes of compass_layer_weights */
} compass_layer_weights_q4;

/* One decode step of one layer with 4-bit affine weights: compass_layer_decode's
 * arguments, workspace (compass_workspace_size(d, B, 1, kv->capacity, 1)), outputs and
 * errors, with every weight matrix read in the 4-bit form above. The result is the layer of
 * the dequantized weights; each dequantized weight is rounded once to bf16 before the
 * bf16 MFMA products (fp32 accumulation). Requires d->dtype == COMPASS_BF16 (else
 * COMPASS_E_UNSUPPORTED) and n_q_heads * head_dim a multiple of 64. */
int compass_layer_decode_q4(const compass_layer_desc *d, const compass_layer_weights_q4 *w,
                            int32_t B, const void *x, const int32_t *pos, const compass_kv *kv,
                            void *out, void *workspace, size_t ws_bytes, void *stream);

/* Tied-embedding head ("Text decoder forward": h = LayerNorm(h); logits =
 * embed_tokens.as_linear(h) * logit_scale), with the scale applied as the last fp32
 * operation on each logit (the in-place fp32 footer of the C-Kernel-Engine page,
 * section "1. Cohere2 Command R").
 *   h [R, D] (dtype)   norm_w [D]   embed [V, D] (dtype)   logits out [R, V] fp32
 *   workspace: compass_logits_workspace_size(R, D, dtype) bytes. */
size_t compass_logits_workspace_size(int32_t R, int32_t D, int32_t dtype);
int compass_logits(int32_t R, int32_t D, int32_t V, int32_t dtype, const void *h,
                   const void *norm_w, float ln_eps, const void *embed, float logit_scale,
                   float *logits, void *workspace, size_t ws_bytes, void *stream);

/* Token-id front end ("Text decoder forward" of the mlxcel Compass issue: the token
 * embedding, whose image-pad rows are then replaced by the vision merger's output rows;
 * FreeToken's "How it fits together" writes them with one indexed copy):
 *   h[r] = embed[tokens[r]] for r < R, then h[img_rows[i]] = img_feats[i] for i < n_img.
 *   tokens [R] int32 (device)   embed [V, D] (dtype)   img_rows [n_img] int32 (device;
 *   distinct rows; NULL when n_img = 0)   img_feats [n_img, D] (dtype)   h out [R, D].
 *   status (device int32, may be NULL): bit 0 set if a token id lies outside [0, V)
 *   (that row of h is zero), bit 1 if an image row lies outside [0, R) (skipped);
 *   read it after the stream has synchronized. D must be a multiple of 8; h must not
 *   overlap embed or img_feats. Stream-ordered, allocates nothing. */
int compass_embed(int32_t R, int32_t D, int32_t V, int32_t dtype, const int32_t *tokens,
                  const void *embed, const int32_t *img_rows, const void *img_feats,
                  int32_t n_img, void *h, int32_t *status, void *stream);

/* Decode positions ("Position ids": a generated token sits at its cache index plus the
 * row's rope_delta on all three axes). On the device: lens[b] += advance, then
 * pos[a * B + b] = lens[b] + rope_delta[b] for a = 0, 1, 2.
 *   lens [B] int32 (device, updated in place)   rope_delta [B] int32 (device, from
 *   compass_mrope_positions; NULL = zeros)   advance >= 0 (0 for the first decode step
 *   after a prefill whose lens the caller has set, 1 for each later step)
 *   pos out [3, B] int32, the pos argument of compass_layer_decode. */
int compass_decode_positions(int32_t B, int32_t *lens, const int32_t *rope_delta,
                             int32_t advance, int32_t *pos, void *stream);

/* Greedy head, the step that turns the tied-embedding logits of "Text decoder forward"
 * (mlxcel Compass issue) into the next token of greedy generation, as in that issue's
 * "Validation" text-generation check: token[r] = the vocabulary id of the largest logit
 * of compass_logits for row r (the same LayerNorm and logits GEMM, so the same fp32
 * values; the smallest id on ties), max_logit[r] (may be NULL) = that logit.
 *   h: R rows of D elements, row r at h + r * ldh (ldh = 0 means D; e.g. ldh = L * D
 *   with h pointing at row L - 1 picks the last token of every [L, D] batch row);
 *   ldh * element size must be a multiple of 16.   token out [R] int32 (device).
 *   R <= 65535. A NaN logit is never picked (a row of NaN / -inf logits gives id 0).
 *   norm_w NULL: the rows of h are already normalized (for instance the out_norm of a
 *   compass_layer_decode_chained call given the final norm weight as next_ln_w, which
 *   equals this call's own LayerNorm bit for bit); ln_eps is unused and R * ldh must stay
 *   below 2^31.
 *   workspace: compass_logits_argmax_workspace_size(R, D, V, dtype) bytes, 256-byte
 *   aligned. Other arguments and errors as compass_logits. */
size_t compass_logits_argmax_workspace_size(int32_t R, int32_t D, int32_t V, int32_t dtype);
int compass_logits_argmax(int32_t R, int32_t D, int32_t V, int32_t dtype, const void *h,
                          int64_t ldh, const void *norm_w, float ln_eps, const void *embed,
                          float logit_scale, int32_t *token, float *max_logit, void *workspace,
                          size_t ws_bytes, void *stream);

/* Message of the last failing call on this thread ("" if none). */
const char *compass_last_error(void);

/* Library version string (host). */
const char *compass_version(void);

/* Kernel timing with HIP events (host side; for measurement only).
 * compass_profile_enable(1) makes every later launch record a start/stop event pair
 * on its own stream; compass_profile_enable(0) stops recording. compass_profile_read
 * synchronizes the recorded events and returns, for kernels whose name equals
 * `kernel` (or all kernels if `kernel` is NULL), the launch count and the summed
 * duration in milliseconds. compass_profile_reset drops all records. The event pool
 * holds COMPASS_PROFILE_MAX launches; later launches are not recorded. */
#define COMPASS_PROFILE_MAX 65536
int compass_profile_enable(int on);
int compass_profile_reset(void);
int compass_profile_read(const char *kernel, int64_t *count, double *total_ms);
/* Name of the i-th distinct kernel name recorded so far (NULL past the end). */
const char *compass_profile_kernel_name(int32_t i);

#ifdef __cplusplus
}
#endif
#endif /* COMPASS_H */
