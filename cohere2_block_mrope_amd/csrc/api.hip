// extern "C" entry points of libcompass: argument validation (pure host code, run
// before any HIP call), workspace carving, and the launch sequence of each call.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/compass.h"
#include "launch.h"

using namespace compass;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return COMPASS_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// ----------------------------------------------------------------- kernel timing
struct ProfRec {
  const char* name;
  hipEvent_t e0, e1;
};
std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};  // read without the lock on every launch
std::vector<ProfRec> g_prof;
std::vector<std::pair<hipEvent_t, hipEvent_t>> g_prof_pool;
std::vector<std::string> g_prof_names;

struct KScope {
  int idx = -1;
  hipEvent_t stop = nullptr;
  hipStream_t s;
  KScope(const char* name, hipStream_t st) : s(st) {
    if (!g_prof_on.load(std::memory_order_relaxed)) return;  // profiling off: no lock, no events
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_on.load(std::memory_order_relaxed) || g_prof.size() >= COMPASS_PROFILE_MAX) return;
    const size_t i = g_prof.size();
    if (i >= g_prof_pool.size()) {
      hipEvent_t a, b;
      if (hipEventCreate(&a) != hipSuccess) return;
      if (hipEventCreate(&b) != hipSuccess) { (void)hipEventDestroy(a); return; }
      g_prof_pool.push_back({a, b});
    }
    ProfRec r{name, g_prof_pool[i].first, g_prof_pool[i].second};
    if (hipEventRecord(r.e0, s) != hipSuccess) return;
    g_prof.push_back(r);
    idx = (int)i;
    stop = r.e1;
    bool seen = false;
    for (auto& n : g_prof_names) seen |= (n == name);
    if (!seen) g_prof_names.push_back(name);
  }
  ~KScope() {
    if (idx >= 0) (void)hipEventRecord(stop, s);
  }
};

#define LAUNCH(name, stream, call)                                                   \
  do {                                                                               \
    hipError_t e_;                                                                   \
    {                                                                                \
      KScope ks_(name, stream);                                                      \
      e_ = (call);                                                                   \
    }                                                                                \
    if (e_ != hipSuccess)                                                            \
      return fail(COMPASS_E_DEVICE, "%s: launch failed: %s", name, hipGetErrorString(e_)); \
  } while (0)

// ----------------------------------------------------------------- validation
int check_desc(const compass_layer_desc* d) {
  if (!d) return fail(COMPASS_E_INVALID, "descriptor is NULL");
  if (d->hidden <= 0 || d->n_q_heads <= 0 || d->n_kv_heads <= 0 || d->head_dim <= 0 ||
      d->intermediate <= 0)
    return fail(COMPASS_E_INVALID, "non-positive width in descriptor");
  if (d->dtype != COMPASS_F32 && d->dtype != COMPASS_BF16)
    return fail(COMPASS_E_UNSUPPORTED, "dtype %d not supported", d->dtype);
  if (d->kind != COMPASS_SLIDING && d->kind != COMPASS_FULL)
    return fail(COMPASS_E_INVALID, "kind %d is neither SLIDING nor FULL", d->kind);
  if (d->n_q_heads % d->n_kv_heads)
    return fail(COMPASS_E_INVALID, "n_q_heads %d not a multiple of n_kv_heads %d", d->n_q_heads,
                d->n_kv_heads);
  const int g = d->n_q_heads / d->n_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return fail(COMPASS_E_UNSUPPORTED, "query heads per kv head %d not in {1,2,4,8}", g);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(COMPASS_E_UNSUPPORTED, "head_dim %d not in {64, 128}", d->head_dim);
  if (d->hidden % 64 || d->hidden > 8192)
    return fail(COMPASS_E_UNSUPPORTED, "hidden %d must be a multiple of 64 and <= 8192", d->hidden);
  if (d->intermediate % 64)
    return fail(COMPASS_E_UNSUPPORTED, "intermediate %d not a multiple of 64", d->intermediate);
  if (((long long)(d->n_q_heads + 2 * d->n_kv_heads) * d->head_dim) % 128)
    return fail(COMPASS_E_UNSUPPORTED, "(Hq + 2 Hkv) * head_dim must be a multiple of 128");
  if ((long long)(d->n_q_heads + 2 * d->n_kv_heads) * d->head_dim + 2LL * d->intermediate > (1LL << 30))
    return fail(COMPASS_E_UNSUPPORTED, "projection width too large");
  if (d->ln_fuse != 0 && d->ln_fuse != 1) return fail(COMPASS_E_INVALID, "ln_fuse %d is neither 0 nor 1", d->ln_fuse);
  if (d->rope_layout != COMPASS_ROPE_INTERLEAVED && d->rope_layout != COMPASS_ROPE_SECTIONS)
    return fail(COMPASS_E_INVALID, "rope_layout %d is neither INTERLEAVED nor SECTIONS", d->rope_layout);
  if (!(d->ln_eps >= 0.f) || !isfinite(d->ln_eps))
    return fail(COMPASS_E_INVALID, "ln_eps must be finite and >= 0");
  if (d->kind == COMPASS_SLIDING) {
    if (d->window < 1) return fail(COMPASS_E_INVALID, "window %d < 1 on a sliding layer", d->window);
    const int half = d->head_dim / 2;
    const int st = d->mrope_section[0], sh = d->mrope_section[1], sw = d->mrope_section[2];
    if (st < 0 || sh < 0 || sw < 0 || st + sh + sw != half)
      return fail(COMPASS_E_INVALID, "mrope_section {%d,%d,%d} must be >= 0 and sum to %d", st, sh,
                  sw, half);
    int ct = 0, ch = 0, cw = 0;
    for (int j = 0; j < half; ++j) {
      if (j % 3 == 1 && j < 3 * sh) ++ch;
      else if (j % 3 == 2 && j < 3 * sw) ++cw;
      else ++ct;
    }
    if (ct != st || ch != sh || cw != sw)
      return fail(COMPASS_E_INVALID, "mrope_section {%d,%d,%d} not realisable by the interleave", st,
                  sh, sw);
    if (!(d->rope_theta > 0.f) || !isfinite(d->rope_theta))
      return fail(COMPASS_E_INVALID, "rope_theta must be finite and > 0");
  }
  return COMPASS_OK;
}

int check_weights(const compass_layer_weights* w) {
  if (!w) return fail(COMPASS_E_INVALID, "weights struct is NULL");
  const void* p[8] = {w->ln_w, w->wq, w->wk, w->wv, w->wo, w->w_gate, w->w_up, w->w_down};
  const char* n[8] = {"ln_w", "wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"};
  for (int i = 0; i < 8; ++i) {
    if (!p[i]) return fail(COMPASS_E_INVALID, "weight %s is NULL", n[i]);
    if (!aligned16(p[i])) return fail(COMPASS_E_ALIGN, "weight %s not 16-byte aligned", n[i]);
  }
  return COMPASS_OK;
}

RopeTable rope_table(const compass_layer_desc* d) {
  RopeTable t;
  t.theta = d->rope_theta;
  t.sh3 = 3 * d->mrope_section[1];
  t.sw3 = 3 * d->mrope_section[2];
  t.layout = d->rope_layout;
  return t;
}

// ----------------------------------------------------------------- workspace
constexpr size_t kAlign = 256;
size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Dims {
  long long D, Hq, Hkv, hd, I, qd, Nv, K2;
  int esz;
};
Dims dims(const compass_layer_desc* d) {
  Dims m;
  m.D = d->hidden; m.Hq = d->n_q_heads; m.Hkv = d->n_kv_heads; m.hd = d->head_dim;
  m.I = d->intermediate;
  m.qd = m.Hq * m.hd;
  m.Nv = (m.Hq + 2 * m.Hkv) * m.hd + 2 * m.I;
  m.K2 = m.qd + m.I;
  m.esz = d->dtype == COMPASS_BF16 ? 2 : 4;
  return m;
}

struct PrefillWs {
  size_t a, q, kc, vc, a2, raw, row_seq, tiles, n_tiles, total;
  int max_tiles;
};
// Varlen prefill (n_seq > 0): B = 1, L = T packed rows, plus the plan's buffers.
// K splits of an fp32 prefill GEMM (64 x 64 tiles on the vector ALUs): enough for about one
// workgroup per CU when the tiles are few, at least 64 K elements per split.
int f32_prefill_splits(long long M, long long N, long long K) {
  const long long tiles = ((M + 63) / 64) * ((N + 63) / 64);
  long long sp = (256 + tiles - 1) / tiles;
  if (sp > K / 64) sp = K / 64;
  return sp < 1 ? 1 : (int)sp;
}

PrefillWs prefill_ws(const compass_layer_desc* d, long long B, long long L, long long n_seq = 0) {
  const Dims m = dims(d);
  const long long T = B * L;
  PrefillWs w;
  size_t off = 0;
  w.a = off; off += up(T * m.D * m.esz);
  w.q = off; off += up(T * m.qd * m.esz);
  w.kc = off; off += up(B * m.Hkv * L * m.hd * m.esz);
  w.vc = off; off += up(B * m.Hkv * L * m.hd * m.esz);
  w.a2 = off; off += up(T * m.K2 * m.esz);
  w.raw = off;
  if (d->dtype == COMPASS_F32) {
    const long long p1 = f32_prefill_splits(T, m.Nv, m.D) * m.Nv, p2 = f32_prefill_splits(T, m.D, m.K2) * m.D;
    off += up(T * (p1 > p2 ? p1 : p2) * 4);
  }
  else {
    const int so = gemm_bf16_resid_splits((int)T, (int)m.D, (int)m.K2);  // split-K output partials
    if (so > 1) off += up((long long)so * T * m.D * 4);
  }
  w.max_tiles = 0;
  w.row_seq = w.tiles = w.n_tiles = off;
  if (n_seq > 0) {
    const int tr = varlen_tile_rows(d->dtype);
    w.max_tiles = tr > 0 ? (int)((T + tr - 1) / tr + n_seq) : 0;
    w.row_seq = off; off += up(T * 4);
    w.tiles = off; off += up((long long)2 * w.max_tiles * 4 + 4);
    w.n_tiles = off; off += up(4);
  }
  w.total = off;
  return w;
}

// Split-K factor of the 64 x 64 decode GEMM tiles: about 512 workgroups in total (measured on
// MI355X: more splits cost more in the partial-sum traffic than they gain in
// parallelism), and at least 256 K elements per split.
int decode_splits(long long tiles, long long K) {
  if (tiles < 1) tiles = 1;
  long long s = (512 + tiles - 1) / tiles;
  if (s > K / 256) s = K / 256;
  if (s < 1) s = 1;
  return (int)s;
}

// Split-K factor of the bf16 decode output GEMM on the skinny kernel (batches of at most 64
// rows): about one workgroup per CU.
int skinny_splits(long long tiles, long long K) {
  if (tiles < 1) tiles = 1;
  long long s = (256 + tiles / 2) / tiles;
  if (s > K / 512) s = K / 512;
  if (s < 1) s = 1;
  return (int)s;
}

struct DecodeWs {
  size_t a, raw1, q, a2, part, raw2, total;
  int s1, s2, n_chunks;
  int k2;  // splits of the output GEMM on the skinny bf16 kernel (0: it does not apply)
};
DecodeWs decode_ws(const compass_layer_desc* d, long long B, long long cap) {
  const Dims m = dims(d);
  DecodeWs w;
  const long long tiles1 = ((B + 63) / 64) * ((m.Nv + 63) / 64);
  const long long tiles2 = ((B + 63) / 64) * ((m.D + 63) / 64);
  w.s1 = decode_splits(tiles1, m.D);
  w.s2 = decode_splits(tiles2, m.K2);
  w.k2 = skinny_splits((m.D + 63) / 64, m.K2);
  if (d->dtype != COMPASS_BF16 || !gemm_skinny_fits((int)B, (int)m.K2, (int)m.D, w.k2)) w.k2 = 0;
  const long long r2 = w.s2 > w.k2 ? w.s2 : w.k2;
  const long long keys = d->kind == COMPASS_SLIDING ? (cap < d->window ? cap : d->window) : cap;
  const int ck = decode_chunk_keys(d->dtype, d->head_dim);
  w.n_chunks = (int)((keys + ck - 1) / ck);
  if (w.n_chunks < 1) w.n_chunks = 1;
  size_t off = 0;
  w.a = off; off += up(B * m.D * m.esz);
  w.raw1 = off; off += up((long long)w.s1 * B * m.Nv * 4);
  w.q = off; off += up(B * m.qd * m.esz);
  w.a2 = off; off += up(B * m.K2 * m.esz);
  w.part = off; off += up(B * m.Hq * (long long)w.n_chunks * (m.hd + 2) * 4);
  w.raw2 = off; off += up(r2 * B * m.D * 4);
  w.total = off;
  return w;
}

BMap proj_bmap(const compass_layer_desc* d, const compass_layer_weights* w) {
  const Dims m = dims(d);
  BMap b{};
  b.kind = 1;
  b.p[0] = w->wq; b.p[1] = w->wk; b.p[2] = w->wv; b.p[3] = w->w_gate; b.p[4] = w->w_up;
  b.ld0 = (int)m.D;
  b.nq64 = (int)(m.qd / 64);
  b.nk64 = (int)(m.Hkv * m.hd / 64);
  return b;
}

BMap out_bmap(const compass_layer_desc* d, const compass_layer_weights* w) {
  const Dims m = dims(d);
  BMap b{};
  b.kind = 2;
  b.p[0] = w->wo; b.p[1] = w->w_down;
  b.ld0 = (int)m.qd; b.ld1 = (int)m.I;
  b.ksplit = (int)m.qd;
  return b;
}

int check_weights_q4(const compass_layer_desc* d, const compass_layer_weights_q4* w) {
  if (d->dtype != COMPASS_BF16) return fail(COMPASS_E_UNSUPPORTED, "4-bit weights need the bf16 dtype");
  if (!w->ln_w) return fail(COMPASS_E_INVALID, "weight ln_w is NULL");
  if (!aligned16(w->ln_w)) return fail(COMPASS_E_ALIGN, "weight ln_w not 16-byte aligned");
  const compass_q4_matrix* mats[7] = {&w->wq, &w->wk, &w->wv, &w->wo, &w->w_gate, &w->w_up, &w->w_down};
  const char* n[7] = {"wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"};
  for (int i = 0; i < 7; ++i) {
    if (!mats[i]->q || !mats[i]->scales || !mats[i]->biases)
      return fail(COMPASS_E_INVALID, "4-bit weight %s has a NULL pointer", n[i]);
    if (!aligned16(mats[i]->q)) return fail(COMPASS_E_ALIGN, "codes of %s not 16-byte aligned", n[i]);
    if (((uintptr_t)mats[i]->scales & 1) || ((uintptr_t)mats[i]->biases & 1))
      return fail(COMPASS_E_ALIGN, "scales/biases of %s not 2-byte aligned", n[i]);
  }
  const Dims m = dims(d);
  if (m.qd % 64) return fail(COMPASS_E_UNSUPPORTED, "n_q_heads * head_dim must be a multiple of 64 for 4-bit weights");
  return COMPASS_OK;
}

Q4Map proj_q4map(const compass_layer_desc* d, const compass_layer_weights_q4* w) {
  const Dims m = dims(d);
  Q4Map b{};
  b.kind = 1;
  const compass_q4_matrix* mats[5] = {&w->wq, &w->wk, &w->wv, &w->w_gate, &w->w_up};
  for (int i = 0; i < 5; ++i) {
    b.q[i] = mats[i]->q;
    b.s[i] = mats[i]->scales;
    b.b[i] = mats[i]->biases;
  }
  b.cols0 = (int)m.D;
  b.nq64 = (int)(m.qd / 64);
  b.nk64 = (int)(m.Hkv * m.hd / 64);
  return b;
}

Q4Map out_q4map(const compass_layer_desc* d, const compass_layer_weights_q4* w) {
  const Dims m = dims(d);
  Q4Map b{};
  b.kind = 2;
  b.q[0] = w->wo.q; b.s[0] = w->wo.scales; b.b[0] = w->wo.biases;
  b.q[1] = w->w_down.q; b.s[1] = w->w_down.scales; b.b[1] = w->w_down.biases;
  b.cols0 = (int)m.qd;
  b.cols1 = (int)m.I;
  b.ksplit = (int)m.qd;
  return b;
}

std::mutex g_lds_mu;
std::vector<std::pair<int, const void*>> g_lds_done;  // (device, kernel) pairs already raised

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// ----------------------------------------------------------------- no-allocation scratch
// Device memory of compass_layer_decode_noalloc: a file-scope device array that each GPU
// the library runs on holds from the loading of this code object until the process ends.
// In host code `scratch` names a host-side stand-in, not a device address: it is never
// passed to a kernel, a copy or a memset. Its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and kept in g_scratch.
static __device__ __align__(256) unsigned char scratch[COMPASS_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::vector<std::pair<int, void*>> g_scratch;  // (device, device address of scratch)

int scratch_address(void** p) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(COMPASS_E_DEVICE, "hipGetDevice failed: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  for (const auto& sc : g_scratch)
    if (sc.first == dev) {
      *p = sc.second;
      return COMPASS_OK;
    }
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || ptr == nullptr)
    return fail(COMPASS_E_DEVICE, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev,
                hipGetErrorString(e));
  if (((uintptr_t)ptr & (kAlign - 1)) != 0)
    return fail(COMPASS_E_DEVICE, "scratch on device %d is not 256-byte aligned", dev);
  g_scratch.emplace_back(dev, ptr);
  *p = ptr;
  return COMPASS_OK;
}

}  // namespace

hipError_t compass::ensure_dynamic_lds(const void* kernel, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_lds_mu);
  for (const auto& d : g_lds_done)
    if (d.first == dev && d.second == kernel) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) g_lds_done.emplace_back(dev, kernel);
  return e;
}

extern "C" {

const char* compass_last_error(void) { return g_err.c_str(); }

const char* compass_version(void) { return "compass-mi355x 0.1 (gfx950)"; }

int compass_mrope_positions(const int32_t* token_ids, int32_t B, int32_t L, int32_t image_token_id,
                            const int32_t* grid_thw, const int32_t* img_offset, int32_t spatial_merge,
                            int32_t* pos, int32_t* rope_delta, int32_t* status, void* stream) {
  if (B < 1 || L < 1) return fail(COMPASS_E_INVALID, "B=%d, L=%d must be >= 1", B, L);
  if ((long long)B * L * 3 > (1LL << 31) - 1) return fail(COMPASS_E_UNSUPPORTED, "B*L too large");
  if (L > COMPASS_MAX_TOKENS_PER_ROW)
    return fail(COMPASS_E_UNSUPPORTED, "L=%d exceeds COMPASS_MAX_TOKENS_PER_ROW=%d", L, COMPASS_MAX_TOKENS_PER_ROW);
  if (!token_ids || !img_offset || !pos || !rope_delta || !status)
    return fail(COMPASS_E_INVALID, "NULL pointer argument");
  if (spatial_merge < 1) return fail(COMPASS_E_INVALID, "spatial_merge %d < 1", spatial_merge);
  const hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  LAUNCH("positions", s, launch_positions(token_ids, B, L, image_token_id, grid_thw, img_offset,
                                          spatial_merge, pos, rope_delta, status, s));
  return ok();
}

size_t compass_workspace_size(const compass_layer_desc* d, int32_t B, int32_t L, int32_t capacity,
                              int32_t decode) {
  const std::string saved = g_err;
  if (check_desc(d) != COMPASS_OK || B < 1) { g_err = saved; return 0; }
  if (decode) {
    if (capacity < 1) return 0;
    return decode_ws(d, B, capacity).total;
  }
  if (L < 1) return 0;
  return prefill_ws(d, B, L).total;
}

// Varlen prefill: n_seq packed sequences with device offsets cu; status (device, may be
// NULL) receives the plan's status bits.
struct VarlenArgs {
  int n_seq;
  const int32_t* cu;
  int32_t* status;
};

// Prefill of a [B, L] chunk. start == NULL: plain prefill (K/V at cache rows [0, L) when a
// cache is given); start = kv->lens: the chunk continues the cache of each row. With va,
// B = 1 and L = T packed rows of va->n_seq sequences; start (may be NULL) then holds the
// tokens already cached per sequence.
static int prefill_impl(const compass_layer_desc* d, const compass_layer_weights* w, int32_t B,
                        int32_t L, const void* x, const int32_t* pos, const compass_kv* kv,
                        const int32_t* start, const int32_t* ds_rows, const void* ds, int32_t n_ds,
                        void* out, void* workspace, size_t ws_bytes, void* stream,
                        const VarlenArgs* va = nullptr) {
  int rc = check_desc(d);
  if (rc) return rc;
  if ((rc = check_weights(w))) return rc;
  if (B < 1 || L < 1) return fail(COMPASS_E_INVALID, "B=%d, L=%d must be >= 1", B, L);
  if (va) {
    if (va->n_seq < 1 || va->n_seq > kVarlenMaxSeqs)
      return fail(COMPASS_E_UNSUPPORTED, "n_seq=%d must be in [1, %d]", va->n_seq, kVarlenMaxSeqs);
    if (L > kVarlenMaxTokens)
      return fail(COMPASS_E_UNSUPPORTED, "T=%d packed rows exceed %d", L, kVarlenMaxTokens);
    if (!va->cu) return fail(COMPASS_E_INVALID, "cu_seqlens is NULL");
  }
  const Dims m = dims(d);
  const long long T = (long long)B * L;
  if (T * (m.K2 > m.Nv ? m.K2 : m.Nv) > (1LL << 31) - 1 || T > (1LL << 31) - 1)
    return fail(COMPASS_E_UNSUPPORTED, "B*L too large for 32-bit row indexing");
  if (!x || !out) return fail(COMPASS_E_INVALID, "x or out is NULL");
  if (!aligned16(x) || !aligned16(out)) return fail(COMPASS_E_ALIGN, "x/out not 16-byte aligned");
  const size_t xbytes = (size_t)T * m.D * m.esz;
  if (x != out && overlap(x, xbytes, out, xbytes))
    return fail(COMPASS_E_INVALID, "out partially overlaps x (only exact aliasing is allowed)");
  const bool sliding = d->kind == COMPASS_SLIDING;
  if (sliding && !pos) return fail(COMPASS_E_INVALID, "pos is NULL on a sliding layer");
  if (kv) {
    if (!kv->k || !kv->v) return fail(COMPASS_E_INVALID, "kv->k or kv->v is NULL");
    if (!aligned16(kv->k) || !aligned16(kv->v)) return fail(COMPASS_E_ALIGN, "kv not 16-byte aligned");
    if (va ? kv->capacity < 1 : kv->capacity < L)
      return fail(COMPASS_E_INVALID, "kv capacity %d < %d", kv->capacity, va ? 1 : L);
    // The attention kernels address one (row, kv head) slice of the cache with 32-bit byte
    // offsets.
    if ((long long)kv->capacity * m.hd * m.esz > (1LL << 31) - 1)
      return fail(COMPASS_E_UNSUPPORTED, "kv capacity %d x head_dim %lld: a (row, kv head) cache slice of 2 GiB or more",
                  kv->capacity, (long long)m.hd);
  }
  if (n_ds < 0) return fail(COMPASS_E_INVALID, "n_ds < 0");
  if (n_ds > 0) {
    if (!ds_rows || !ds) return fail(COMPASS_E_INVALID, "deepstack pointers NULL with n_ds > 0");
    if (!aligned16(ds)) return fail(COMPASS_E_ALIGN, "ds not 16-byte aligned");
  }
  const PrefillWs ws = prefill_ws(d, B, L, va ? va->n_seq : 0);
  if (!workspace || ws_bytes < ws.total)
    return fail(COMPASS_E_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, ws.total);
  if (((uintptr_t)workspace & (kAlign - 1)) != 0)
    return fail(COMPASS_E_ALIGN, "workspace not 256-byte aligned");

  char* wsb = (char*)workspace;
  VarlenPlan plan{};
  if (va) {
    plan.cu = va->cu;
    plan.n_seq = va->n_seq;
    plan.row_seq = (int32_t*)(wsb + ws.row_seq);
    plan.tiles = (int32_t*)(wsb + ws.tiles);
    plan.n_tiles = (int32_t*)(wsb + ws.n_tiles);
    plan.max_tiles = ws.max_tiles;
  }
  void* a = wsb + ws.a;
  void* q = wsb + ws.q;
  void* kc = kv ? kv->k : (void*)(wsb + ws.kc);
  void* vc = kv ? kv->v : (void*)(wsb + ws.vc);
  const int cap = kv ? kv->capacity : L;
  void* a2 = wsb + ws.a2;
  float* raw = (float*)(wsb + ws.raw);
  const hipStream_t s = (hipStream_t)stream;
  const int dt = d->dtype;

  ProjEpi ep{};
  ep.decode = 0;
  ep.L = L;
  ep.pos = pos;
  ep.pos_stride = (int)T;
  ep.rope = sliding ? 1 : 0;
  ep.Hq = (int)m.Hq; ep.Hkv = (int)m.Hkv; ep.hd = (int)m.hd;
  ep.q = q; ep.Lq = L;
  ep.kc = kc; ep.vc = vc; ep.cap = cap;
  ep.lens = nullptr;
  ep.kv_start = start;
  ep.row_seq = va ? plan.row_seq : nullptr;
  ep.cu = va ? va->cu : nullptr;
  ep.kv_by_seq = (va && kv) ? 1 : 0;
  ep.act = a2; ep.ldact = (int)m.K2; ep.act_col0 = (int)m.qd;
  ep.nq64 = (int)(m.qd / 64); ep.nk64 = (int)(m.Hkv * m.hd / 64);
  ep.I = (int)m.I;
  const RopeTable rt = rope_table(d);
  const BMap pb = proj_bmap(d, w), ob = out_bmap(d, w);
  const RowStart rs{va ? nullptr : start, L, cap, va ? plan.row_seq : nullptr};

  (void)hipGetLastError();
  if (va)
    LAUNCH("varlen_plan", s, launch_varlen_plan(plan, L, start, kv ? kv->capacity : 0,
                                                varlen_tile_rows(dt), va->status, s));
  if (dt == COMPASS_BF16 && d->ln_fuse) {
    float2* stats = (float2*)a;  // the LayerNorm output buffer holds the row statistics instead
    LAUNCH("ln_stats", s, launch_ln_stats(x, d->ln_eps, stats, (int)T, (int)m.D, s));
    LAUNCH("gemm_proj", s, launch_gemm_bf16_proj(x, (int)m.D, (int)T, (int)m.D, pb, (int)m.Nv, ep, rt, s, stats,
                                                 w->ln_w));
  } else if (dt == COMPASS_BF16) {
    LAUNCH("layernorm", s, launch_layernorm(dt, x, w->ln_w, d->ln_eps, a, (int)T, (int)m.D, s));
    LAUNCH("gemm_proj", s, launch_gemm_bf16_proj(a, (int)m.D, (int)T, (int)m.D, pb, (int)m.Nv, ep, rt, s));
  } else {
    LAUNCH("layernorm", s, launch_layernorm(dt, x, w->ln_w, d->ln_eps, a, (int)T, (int)m.D, s));
    const int sp = f32_prefill_splits(T, m.Nv, m.D);
    LAUNCH("gemm_proj_f32", s, launch_gemm_f32_raw(a, (int)m.D, (int)T, (int)m.D, pb, (int)m.Nv, sp, raw, 1.f, s));
    LAUNCH("proj_epilogue", s, launch_proj_epilogue(dt, raw, sp, (int)T, (int)m.Nv, ep, rt, s));
  }
  if (va)
    LAUNCH("attn_prefill", s, launch_attention_prefill_varlen(dt, q, kc, vc, L, (int)m.Hq, (int)m.Hkv, cap,
                                                              (int)m.hd, sliding, d->window, start, kv ? 1 : 0,
                                                              plan, a2, (int)m.K2, s));
  else
    LAUNCH("attn_prefill", s, launch_attention_prefill(dt, q, kc, vc, B, (int)m.Hq, (int)m.Hkv, L, cap,
                                                       (int)m.hd, sliding, d->window, start, a2, (int)m.K2, s));
  if (dt == COMPASS_BF16) {
    const int so = gemm_bf16_resid_splits((int)T, (int)m.D, (int)m.K2);
    if (so > 1) {  // too few output tiles to fill the CUs: split K, then reduce with the residual
      LAUNCH("gemm_out", s, launch_gemm_bf16_raw_wide(a2, (int)m.K2, (int)T, (int)m.K2, ob, (int)m.D, so, raw, s));
      LAUNCH("splitk_resid", s, launch_splitk_resid(dt, raw, so, (int)T, (int)m.D, x, out, rs, s));
    } else {
      LAUNCH("gemm_out", s, launch_gemm_bf16_resid(a2, (int)m.K2, (int)T, (int)m.K2, ob, (int)m.D, x, out,
                                                   (int)m.D, rs, s));
    }
  } else {
    const int so = f32_prefill_splits(T, m.D, m.K2);
    LAUNCH("gemm_out_f32", s, launch_gemm_f32_raw(a2, (int)m.K2, (int)T, (int)m.K2, ob, (int)m.D, so, raw, 1.f, s));
    LAUNCH("splitk_resid", s, launch_splitk_resid(dt, raw, so, (int)T, (int)m.D, x, out, rs, s));
  }
  if (n_ds > 0)
    LAUNCH("deepstack", s, launch_deepstack(dt, ds_rows, ds, n_ds, (int)m.D, (int)T, rs, out, s));
  return ok();
}

int compass_layer_prefill(const compass_layer_desc* d, const compass_layer_weights* w, int32_t B,
                          int32_t L, const void* x, const int32_t* pos, const compass_kv* kv,
                          const int32_t* ds_rows, const void* ds, int32_t n_ds, void* out,
                          void* workspace, size_t ws_bytes, void* stream) {
  return prefill_impl(d, w, B, L, x, pos, kv, nullptr, ds_rows, ds, n_ds, out, workspace, ws_bytes, stream);
}

int compass_layer_prefill_chunk(const compass_layer_desc* d, const compass_layer_weights* w, int32_t B,
                                int32_t L, const void* x, const int32_t* pos, const compass_kv* kv,
                                const int32_t* ds_rows, const void* ds, int32_t n_ds, void* out,
                                void* workspace, size_t ws_bytes, void* stream) {
  if (!kv || !kv->lens) return fail(COMPASS_E_INVALID, "chunked prefill needs kv with lens (tokens already cached)");
  return prefill_impl(d, w, B, L, x, pos, kv, kv->lens, ds_rows, ds, n_ds, out, workspace, ws_bytes, stream);
}

size_t compass_varlen_workspace_size(const compass_layer_desc* d, int32_t n_seq, int32_t T) {
  const std::string saved = g_err;
  if (check_desc(d) != COMPASS_OK || n_seq < 1 || T < 1) { g_err = saved; return 0; }
  return prefill_ws(d, 1, T, n_seq).total;
}

int compass_layer_prefill_varlen(const compass_layer_desc* d, const compass_layer_weights* w, int32_t n_seq,
                                 int32_t T, const int32_t* cu_seqlens, const void* x, const int32_t* pos,
                                 const compass_kv* kv, const int32_t* ds_rows, const void* ds, int32_t n_ds,
                                 void* out, int32_t* status, void* workspace, size_t ws_bytes, void* stream) {
  const VarlenArgs va{n_seq, cu_seqlens, status};
  return prefill_impl(d, w, 1, T, x, pos, kv, kv ? kv->lens : nullptr, ds_rows, ds, n_ds, out, workspace,
                      ws_bytes, stream, &va);
}

// One decode step; the GEMM weights are either bf16/fp32 (w) or 4-bit affine (wq). With
// need != NULL the call only validates its arguments (host code, no HIP call) and returns
// the workspace bytes it would use in *need.
static int decode_impl(const compass_layer_desc* d, const compass_layer_weights* w,
                       const compass_layer_weights_q4* wq, int32_t B, const void* x, const int32_t* pos,
                       const compass_kv* kv, void* out, void* workspace, size_t ws_bytes, void* stream,
                       size_t* need = nullptr, const void* x_norm = nullptr, const void* next_ln_w = nullptr,
                       float next_ln_eps = 0.f, void* out_norm = nullptr) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (wq) {
    if ((rc = check_weights_q4(d, wq))) return rc;
  } else if ((rc = check_weights(w))) {
    return rc;
  }
  if (B < 1) return fail(COMPASS_E_INVALID, "B=%d must be >= 1", B);
  const Dims m = dims(d);
  if ((long long)B * (m.K2 > m.Nv ? m.K2 : m.Nv) > (1LL << 31) - 1)
    return fail(COMPASS_E_UNSUPPORTED, "B too large");
  if (!x || !out) return fail(COMPASS_E_INVALID, "x or out is NULL");
  if (!aligned16(x) || !aligned16(out)) return fail(COMPASS_E_ALIGN, "x/out not 16-byte aligned");
  const size_t xbytes = (size_t)B * m.D * m.esz;
  if (x != out && overlap(x, xbytes, out, xbytes))
    return fail(COMPASS_E_INVALID, "out partially overlaps x (only exact aliasing is allowed)");
  const bool sliding = d->kind == COMPASS_SLIDING;
  if (sliding && !pos) return fail(COMPASS_E_INVALID, "pos is NULL on a sliding layer");
  if (!kv || !kv->k || !kv->v || !kv->lens) return fail(COMPASS_E_INVALID, "decode needs kv with k, v, lens");
  if (!aligned16(kv->k) || !aligned16(kv->v)) return fail(COMPASS_E_ALIGN, "kv not 16-byte aligned");
  if (kv->capacity < 1) return fail(COMPASS_E_INVALID, "kv capacity %d < 1", kv->capacity);
  if ((long long)B * m.Hkv * kv->capacity * m.hd > (1LL << 40))
    return fail(COMPASS_E_UNSUPPORTED, "kv cache too large");
  if (x_norm || out_norm) {
    if (d->dtype != COMPASS_BF16 || wq)
      return fail(COMPASS_E_UNSUPPORTED, "LayerNorm outputs are handed between bf16 layers only");
    if (out_norm && !next_ln_w) return fail(COMPASS_E_INVALID, "out_norm needs next_ln_w");
    if (!aligned16(x_norm) || !aligned16(out_norm) || !aligned16(next_ln_w))
      return fail(COMPASS_E_ALIGN, "x_norm / out_norm / next_ln_w not 16-byte aligned");
    if (out_norm && (overlap(out_norm, xbytes, x, xbytes) || overlap(out_norm, xbytes, out, xbytes)))
      return fail(COMPASS_E_INVALID, "out_norm overlaps x or out");
  }
  const DecodeWs ws = decode_ws(d, B, kv->capacity);
  if (need) {
    *need = ws.total;
    return ok();
  }
  if (!workspace || ws_bytes < ws.total)
    return fail(COMPASS_E_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, ws.total);
  if (((uintptr_t)workspace & (kAlign - 1)) != 0)
    return fail(COMPASS_E_ALIGN, "workspace not 256-byte aligned");

  char* wsb = (char*)workspace;
  void* a = wsb + ws.a;
  float* raw1 = (float*)(wsb + ws.raw1);
  void* q = wsb + ws.q;
  void* a2 = wsb + ws.a2;
  float* part = (float*)(wsb + ws.part);
  float* raw2 = (float*)(wsb + ws.raw2);
  const hipStream_t s = (hipStream_t)stream;
  const int dt = d->dtype;

  ProjEpi ep{};
  ep.decode = 1;
  ep.L = 1;
  ep.pos = pos;
  ep.pos_stride = B;
  ep.rope = sliding ? 1 : 0;
  ep.Hq = (int)m.Hq; ep.Hkv = (int)m.Hkv; ep.hd = (int)m.hd;
  ep.q = q; ep.Lq = 1;
  ep.kc = kv->k; ep.vc = kv->v; ep.cap = kv->capacity;
  ep.lens = kv->lens;
  ep.act = a2; ep.ldact = (int)m.K2; ep.act_col0 = (int)m.qd;
  ep.nq64 = (int)(m.qd / 64); ep.nk64 = (int)(m.Hkv * m.hd / 64);
  ep.I = (int)m.I;
  const RopeTable rt = rope_table(d);

  (void)hipGetLastError();
  if (x_norm)
    a = const_cast<void*>(x_norm);  // this layer's LayerNorm, written by the call that produced x
  else
    LAUNCH("layernorm", s, launch_layernorm(dt, x, wq ? wq->ln_w : w->ln_w, d->ln_eps, a, B, (int)m.D, s));
  // The output GEMM streams its weights through the skinny kernel when it applies (measured
  // faster there; the projection keeps the 64 x 64 split-K tiles).
  const bool skinny = !wq && ws.k2 > 0;
  const int s1 = ws.s1, s2 = skinny ? ws.k2 : ws.s2;
  if (wq)
    LAUNCH("gemm_proj_decode_q4", s, launch_gemm_q4_raw(a, (int)m.D, B, (int)m.D, proj_q4map(d, wq), (int)m.Nv, s1,
                                                        raw1, s));
  else if (dt == COMPASS_BF16)
    LAUNCH("gemm_proj_decode", s, launch_gemm_bf16_raw(a, (int)m.D, B, (int)m.D, proj_bmap(d, w), (int)m.Nv, s1,
                                                       raw1, s));
  else
    LAUNCH("gemm_proj_decode", s, launch_gemm_f32_raw(a, (int)m.D, B, (int)m.D, proj_bmap(d, w), (int)m.Nv, ws.s1,
                                                      raw1, 1.f, s));
  LAUNCH("proj_epilogue", s, launch_proj_epilogue(dt, raw1, s1, B, (int)m.Nv, ep, rt, s));
  LAUNCH("decode_attn", s, launch_decode_attention(dt, q, kv->k, kv->v, kv->lens, B, (int)m.Hq, (int)m.Hkv,
                                                   kv->capacity, (int)m.hd, sliding, d->window,
                                                   ws.n_chunks, part, s));
  LAUNCH("decode_combine", s, launch_decode_combine(dt, part, kv->lens, B, (int)m.Hq, kv->capacity,
                                                    (int)m.hd, ws.n_chunks, a2, (int)m.K2, s));
  if (wq)
    LAUNCH("gemm_out_decode_q4", s, launch_gemm_q4_raw(a2, (int)m.K2, B, (int)m.K2, out_q4map(d, wq), (int)m.D, s2,
                                                       raw2, s));
  else if (skinny)
    LAUNCH("gemm_out_decode", s, launch_gemm_skinny_raw(a2, (int)m.K2, B, (int)m.K2, out_bmap(d, w), (int)m.D, s2,
                                                        raw2, s));
  else if (dt == COMPASS_BF16)
    LAUNCH("gemm_out_decode", s, launch_gemm_bf16_raw(a2, (int)m.K2, B, (int)m.K2, out_bmap(d, w), (int)m.D, s2,
                                                      raw2, s));
  else
    LAUNCH("gemm_out_decode", s, launch_gemm_f32_raw(a2, (int)m.K2, B, (int)m.K2, out_bmap(d, w), (int)m.D, ws.s2,
                                                     raw2, 1.f, s));
  if (out_norm)
    LAUNCH("splitk_resid", s, launch_splitk_resid_ln(raw2, s2, B, (int)m.D, x, out, RowStart{kv->lens, 1, kv->capacity},
                                                     next_ln_w, next_ln_eps, out_norm, s));
  else
    LAUNCH("splitk_resid", s, launch_splitk_resid(dt, raw2, s2, B, (int)m.D, x, out,
                                                  RowStart{kv->lens, 1, kv->capacity}, s));
  return ok();
}

int compass_layer_decode(const compass_layer_desc* d, const compass_layer_weights* w, int32_t B,
                         const void* x, const int32_t* pos, const compass_kv* kv, void* out,
                         void* workspace, size_t ws_bytes, void* stream) {
  if (!w) return fail(COMPASS_E_INVALID, "weights struct is NULL");
  return decode_impl(d, w, nullptr, B, x, pos, kv, out, workspace, ws_bytes, stream);
}

int compass_layer_decode_chained(const compass_layer_desc* d, const compass_layer_weights* w, int32_t B,
                                 const void* x, const void* x_norm, const int32_t* pos, const compass_kv* kv,
                                 void* out, const void* next_ln_w, float next_ln_eps, void* out_norm,
                                 void* workspace, size_t ws_bytes, void* stream) {
  if (!w) return fail(COMPASS_E_INVALID, "weights struct is NULL");
  return decode_impl(d, w, nullptr, B, x, pos, kv, out, workspace, ws_bytes, stream, nullptr, x_norm, next_ln_w,
                     next_ln_eps, out_norm);
}

int compass_layer_decode_noalloc(const compass_layer_desc* d, const compass_layer_weights* w, int32_t B,
                                 const void* x, const int32_t* pos, const compass_kv* kv, void* out,
                                 void* stream) {
  if (!w) return fail(COMPASS_E_INVALID, "weights struct is NULL");
  size_t need = 0;
  int rc = decode_impl(d, w, nullptr, B, x, pos, kv, out, nullptr, 0, stream, &need);
  if (rc) return rc;
  if (need > (size_t)COMPASS_NOALLOC_SCRATCH_BYTES)
    return fail(COMPASS_E_WORKSPACE,
                "decode of B=%d over capacity %d needs %zu bytes of scratch, above the no-allocation "
                "maximum of %zu bytes (use compass_layer_decode with a caller workspace)",
                B, kv->capacity, need, (size_t)COMPASS_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  return decode_impl(d, w, nullptr, B, x, pos, kv, out, ws, (size_t)COMPASS_NOALLOC_SCRATCH_BYTES, stream);
}

int compass_layer_decode_q4(const compass_layer_desc* d, const compass_layer_weights_q4* w, int32_t B,
                            const void* x, const int32_t* pos, const compass_kv* kv, void* out,
                            void* workspace, size_t ws_bytes, void* stream) {
  if (!w) return fail(COMPASS_E_INVALID, "weights struct is NULL");
  return decode_impl(d, nullptr, w, B, x, pos, kv, out, workspace, ws_bytes, stream);
}

size_t compass_logits_workspace_size(int32_t R, int32_t D, int32_t dtype) {
  if (R < 1 || D < 1 || (dtype != COMPASS_F32 && dtype != COMPASS_BF16)) return 0;
  return up((size_t)R * D * (dtype == COMPASS_BF16 ? 2 : 4));
}

int compass_logits(int32_t R, int32_t D, int32_t V, int32_t dtype, const void* h, const void* norm_w,
                   float ln_eps, const void* embed, float logit_scale, float* logits, void* workspace,
                   size_t ws_bytes, void* stream) {
  if (R < 1 || D < 1 || V < 1) return fail(COMPASS_E_INVALID, "R=%d D=%d V=%d must be >= 1", R, D, V);
  if (dtype != COMPASS_F32 && dtype != COMPASS_BF16)
    return fail(COMPASS_E_UNSUPPORTED, "dtype %d not supported", dtype);
  if (D % 64 || D > 8192) return fail(COMPASS_E_UNSUPPORTED, "D=%d must be a multiple of 64, <= 8192", D);
  if ((long long)R * D > (1LL << 31) - 1 || (long long)V * D > (1LL << 31) - 1)
    return fail(COMPASS_E_UNSUPPORTED, "R*D or V*D too large");
  if (!h || !norm_w || !embed || !logits) return fail(COMPASS_E_INVALID, "NULL pointer argument");
  if (!aligned16(h) || !aligned16(norm_w) || !aligned16(embed) || !aligned16(logits))
    return fail(COMPASS_E_ALIGN, "tensor not 16-byte aligned");
  if (!(ln_eps >= 0.f) || !isfinite(ln_eps)) return fail(COMPASS_E_INVALID, "ln_eps must be finite and >= 0");
  const size_t need = compass_logits_workspace_size(R, D, dtype);
  if (!workspace || ws_bytes < need)
    return fail(COMPASS_E_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  if (((uintptr_t)workspace & (kAlign - 1)) != 0) return fail(COMPASS_E_ALIGN, "workspace not 256-byte aligned");
  const hipStream_t s = (hipStream_t)stream;
  BMap eb{};
  eb.kind = 0;
  eb.p[0] = embed;
  eb.ld0 = D;
  (void)hipGetLastError();
  LAUNCH("logits_layernorm", s, launch_layernorm(dtype, h, norm_w, ln_eps, workspace, R, D, s));
  if (dtype == COMPASS_BF16)
    LAUNCH("gemm_logits", s, launch_gemm_bf16_scaled_f32(workspace, D, R, D, eb, V, logit_scale, logits,
                                                          (long long)V, s));
  else
    LAUNCH("gemm_logits", s, launch_gemm_f32_raw(workspace, D, R, D, eb, V, 1, logits, logit_scale, s));
  return ok();
}

int compass_embed(int32_t R, int32_t D, int32_t V, int32_t dtype, const int32_t* tokens, const void* embed,
                  const int32_t* img_rows, const void* img_feats, int32_t n_img, void* h, int32_t* status,
                  void* stream) {
  if (R < 1 || D < 1 || V < 1) return fail(COMPASS_E_INVALID, "R=%d D=%d V=%d must be >= 1", R, D, V);
  if (dtype != COMPASS_F32 && dtype != COMPASS_BF16)
    return fail(COMPASS_E_UNSUPPORTED, "dtype %d not supported", dtype);
  if (D % 8) return fail(COMPASS_E_UNSUPPORTED, "D=%d must be a multiple of 8", D);
  if (n_img < 0) return fail(COMPASS_E_INVALID, "n_img=%d < 0", n_img);
  if (!tokens || !embed || !h) return fail(COMPASS_E_INVALID, "NULL pointer argument");
  if (n_img > 0 && (!img_rows || !img_feats))
    return fail(COMPASS_E_INVALID, "image pointers NULL with n_img > 0");
  if (!aligned16(embed) || !aligned16(h) || (n_img > 0 && !aligned16(img_feats)))
    return fail(COMPASS_E_ALIGN, "tensor not 16-byte aligned");
  const size_t esz = dtype == COMPASS_BF16 ? 2 : 4;
  const size_t hbytes = (size_t)R * D * esz;
  if (overlap(h, hbytes, embed, (size_t)V * D * esz) ||
      (n_img > 0 && overlap(h, hbytes, img_feats, (size_t)n_img * D * esz)))
    return fail(COMPASS_E_INVALID, "h overlaps an input");
  const hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  LAUNCH("embed", s, launch_embed(dtype, tokens, R, D, V, embed, img_rows, img_feats, n_img, h, status, s));
  return ok();
}

int compass_decode_positions(int32_t B, int32_t* lens, const int32_t* rope_delta, int32_t advance, int32_t* pos,
                             void* stream) {
  if (B < 1) return fail(COMPASS_E_INVALID, "B=%d must be >= 1", B);
  if (advance < 0) return fail(COMPASS_E_INVALID, "advance=%d < 0", advance);
  if (!lens || !pos) return fail(COMPASS_E_INVALID, "lens or pos is NULL");
  if (overlap(lens, (size_t)B * 4, pos, (size_t)B * 12)) return fail(COMPASS_E_INVALID, "pos overlaps lens");
  const hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  LAUNCH("decode_positions", s, launch_decode_positions(lens, rope_delta, B, pos, advance, s));
  return ok();
}

static int argmax_parts_bf16(int V) { return 2 * ((V + 255) / 256); }

size_t compass_logits_argmax_workspace_size(int32_t R, int32_t D, int32_t V, int32_t dtype) {
  if (R < 1 || D < 1 || V < 1 || (dtype != COMPASS_F32 && dtype != COMPASS_BF16)) return 0;
  if (dtype == COMPASS_BF16)  // LayerNorm rows, then per-row (max, id) partials of 128-column spans
    return up((size_t)R * D * 2) + 2 * up((size_t)R * argmax_parts_bf16(V) * 4);
  // fp32: LayerNorm rows, the logits, then per-row (max, id) winners of 4096-column chunks
  return up((size_t)R * D * 4) + up((size_t)R * V * 4) + 2 * up((size_t)R * argmax_chunks(V) * 4);
}

int compass_logits_argmax(int32_t R, int32_t D, int32_t V, int32_t dtype, const void* h, int64_t ldh,
                          const void* norm_w, float ln_eps, const void* embed, float logit_scale, int32_t* token,
                          float* max_logit, void* workspace, size_t ws_bytes, void* stream) {
  if (R < 1 || D < 1 || V < 1) return fail(COMPASS_E_INVALID, "R=%d D=%d V=%d must be >= 1", R, D, V);
  if (dtype != COMPASS_F32 && dtype != COMPASS_BF16)
    return fail(COMPASS_E_UNSUPPORTED, "dtype %d not supported", dtype);
  if (D % 64 || D > 8192) return fail(COMPASS_E_UNSUPPORTED, "D=%d must be a multiple of 64, <= 8192", D);
  if (ldh == 0) ldh = D;
  if (ldh < D) return fail(COMPASS_E_INVALID, "ldh=%lld < D=%d", (long long)ldh, D);
  if ((ldh * (dtype == COMPASS_BF16 ? 2 : 4)) % 16)
    return fail(COMPASS_E_ALIGN, "rows of h not 16-byte aligned (ldh=%lld)", (long long)ldh);
  if (R > 65535 || (long long)R * V > (1LL << 40) || (long long)V * D > (1LL << 31) - 1)
    return fail(COMPASS_E_UNSUPPORTED, "R > 65535, or R*V or V*D too large");
  if (!h || !embed || !token) return fail(COMPASS_E_INVALID, "NULL pointer argument");
  if (!aligned16(h) || !aligned16(norm_w) || !aligned16(embed))
    return fail(COMPASS_E_ALIGN, "tensor not 16-byte aligned");
  if (norm_w && (!(ln_eps >= 0.f) || !isfinite(ln_eps)))
    return fail(COMPASS_E_INVALID, "ln_eps must be finite and >= 0");
  if (!norm_w && (long long)R * ldh > (1LL << 31) - 1)  // the GEMM then reads h itself (32-bit offsets)
    return fail(COMPASS_E_UNSUPPORTED, "normalized rows: R * ldh above 2^31 - 1");
  const size_t need = compass_logits_argmax_workspace_size(R, D, V, dtype);
  if (!workspace || ws_bytes < need)
    return fail(COMPASS_E_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  if (((uintptr_t)workspace & (kAlign - 1)) != 0) return fail(COMPASS_E_ALIGN, "workspace not 256-byte aligned");
  const hipStream_t s = (hipStream_t)stream;
  const void* a = workspace;
  int lda = D;
  BMap eb{};
  eb.kind = 0;
  eb.p[0] = embed;
  eb.ld0 = D;
  (void)hipGetLastError();
  // Same LayerNorm and logits arithmetic as compass_logits (the maxima are bitwise those
  // of the logits it returns for the same rows). Without norm_w the rows of h are the
  // normalized rows already.
  if (norm_w)
    LAUNCH("logits_layernorm", s, launch_layernorm(dtype, h, norm_w, ln_eps, workspace, R, D, s, (long long)ldh));
  else {
    a = h;
    lda = (int)ldh;
  }
  if (dtype == COMPASS_BF16) {
    // The argmax is fused into the logits GEMM: only per-span partials reach memory.
    float* pv = (float*)((char*)workspace + up((size_t)R * D * 2));
    int* pi = (int*)((char*)pv + up((size_t)R * argmax_parts_bf16(V) * 4));
    int parts = 0;
    hipError_t ge = hipSuccess;
    LAUNCH("gemm_logits_argmax", s, (parts = gemm_bf16_argmax(a, lda, R, D, eb, V, logit_scale, pv, pi, s, &ge), ge));
    LAUNCH("argmax", s, launch_argmax_partials(pv, pi, R, parts, token, max_logit, s));
  } else {
    float* lg = (float*)((char*)workspace + up((size_t)R * D * 4));
    float* pv = (float*)((char*)lg + up((size_t)R * V * 4));
    int* pi = (int*)((char*)pv + up((size_t)R * argmax_chunks(V) * 4));
    LAUNCH("gemm_logits", s, launch_gemm_f32_raw(a, lda, R, D, eb, V, 1, lg, logit_scale, s));
    LAUNCH("argmax", s, launch_argmax(lg, R, V, (long long)V, 1.f, pv, pi, token, max_logit, s));
  }
  return ok();
}

int compass_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on.store(on != 0, std::memory_order_relaxed);
  return COMPASS_OK;
}

int compass_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof.clear();
  g_prof_names.clear();
  return COMPASS_OK;
}

int compass_profile_read(const char* kernel, int64_t* count, double* total_ms) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  int64_t c = 0;
  double t = 0.0;
  for (const ProfRec& r : g_prof) {
    if (kernel && strcmp(kernel, r.name) != 0) continue;
    hipError_t e = hipEventSynchronize(r.e1);
    if (e != hipSuccess) return fail(COMPASS_E_DEVICE, "event sync failed: %s", hipGetErrorString(e));
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.e0, r.e1);
    if (e != hipSuccess) return fail(COMPASS_E_DEVICE, "event time failed: %s", hipGetErrorString(e));
    ++c;
    t += ms;
  }
  if (count) *count = c;
  if (total_ms) *total_ms = t;
  return COMPASS_OK;
}

const char* compass_profile_kernel_name(int32_t i) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (i < 0 || (size_t)i >= g_prof_names.size()) return nullptr;
  return g_prof_names[i].c_str();
}

}  // extern "C"
