// The C ABI of lucev (see include/lucev.h): host-side validation, tree
// preparation, workspace carving and kernel dispatch.  Nothing here computes
// model math; every step of the forward runs in the kernels.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/lucev.h"
#include "internal.h"

using namespace lucev;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(LUCEV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_shape(const lucev_shape* s) {
  if (!s) return fail(LUCEV_ERR_NULL_ARG, "shape is NULL");
  if (s->hidden <= 0 || s->n_q_heads <= 0 || s->n_kv_heads <= 0 || s->head_dim <= 0 ||
      s->ffn <= 0 || s->vocab <= 0)
    return fail(LUCEV_ERR_BAD_SHAPE, "non-positive dimension");
  if (s->hidden % 128 || s->ffn % 128 || (s->n_q_heads * s->head_dim) % 128)
    return fail(LUCEV_ERR_BAD_SHAPE, "hidden, ffn and n_q_heads*head_dim must be multiples of 128");
  if (s->hidden > 8192) return fail(LUCEV_ERR_BAD_SHAPE, "hidden must be at most 8192 (got %d)", s->hidden);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(LUCEV_ERR_BAD_SHAPE, "head_dim must be 64 or 128 (got %d)", s->head_dim);
  if (s->n_q_heads % s->n_kv_heads)
    return fail(LUCEV_ERR_BAD_SHAPE, "n_q_heads must be a multiple of n_kv_heads");
  if (s->vocab % 16) return fail(LUCEV_ERR_BAD_SHAPE, "vocab must be a multiple of 16");
  if (!(s->rms_eps >= 0.f) || !(s->rope_base > 0.f))
    return fail(LUCEV_ERR_BAD_SHAPE, "rms_eps must be >= 0 and rope_base > 0");
  return LUCEV_OK;
}

// The tree attention holds at most kMaxAttnRows query rows (n * Hq / Hkv) per
// KV head: the limit the workspace and scratch sizes are quoted for.
int check_attn_rows(const lucev_shape* s, int n) {
  const int rows = n * (s->n_q_heads / s->n_kv_heads);
  if (rows > kMaxAttnRows)
    return fail(LUCEV_ERR_BAD_SHAPE, "tree attention: n * n_q_heads / n_kv_heads = %d query rows per KV head exceeds %d",
                rows, kMaxAttnRows);
  return LUCEV_OK;
}

// Depths, RoPE positions and ancestor masks of the draft tree.
int prep_tree(const lucev_tree* t, int vocab, int prefix_len, TreeArgs* out) {
  if (!t) return fail(LUCEV_ERR_NULL_ARG, "tree is NULL");
  if (t->n < 1 || t->n > LUCEV_MAX_NODES)
    return fail(LUCEV_ERR_BAD_TREE, "tree size %d outside [1, %d]", t->n, LUCEV_MAX_NODES);
  if (t->parent[0] != -1) return fail(LUCEV_ERR_BAD_TREE, "parent[0] must be -1");
  memset(out, 0, sizeof(*out));
  out->n = t->n;
  int depth[LUCEV_MAX_NODES];
  for (int i = 0; i < t->n; ++i) {
    const int p = t->parent[i];
    if (i > 0 && (p < 0 || p >= i))
      return fail(LUCEV_ERR_BAD_TREE, "parent[%d] = %d is not an earlier node", i, p);
    if (t->token[i] < 0 || t->token[i] >= vocab)
      return fail(LUCEV_ERR_BAD_TREE, "token[%d] = %d outside [0, vocab)", i, t->token[i]);
    depth[i] = i == 0 ? 0 : depth[p] + 1;
    out->parent[i] = p;
    out->token[i] = t->token[i];
    out->pos[i] = prefix_len + depth[i];
    out->anc[i] = (i == 0 ? 0ull : out->anc[p]) | (1ull << i);
  }
  return LUCEV_OK;
}

int check_q4(const lucev_q4& w, int64_t n_out, int64_t k_in, const char* name) {
  if (!w.packed) return fail(LUCEV_ERR_NULL_ARG, "%s.packed is NULL", name);
  if (w.n_out != n_out || w.k_in != k_in)
    return fail(LUCEV_ERR_BAD_SHAPE, "%s is [%lld, %lld], expected [%lld, %lld]", name,
                (long long)w.n_out, (long long)w.k_in, (long long)n_out, (long long)k_in);
  if (!aligned16(w.packed)) return fail(LUCEV_ERR_ALIGN, "%s.packed is not 16-byte aligned", name);
  return LUCEV_OK;
}

int check_kv(const lucev_kv* kv) {
  if (!kv) return fail(LUCEV_ERR_NULL_ARG, "kv is NULL");
  if (kv->prefix_len < 0 || kv->capacity < 0 || kv->prefix_len > kv->capacity)
    return fail(LUCEV_ERR_BAD_KV, "prefix_len %d / capacity %d invalid", kv->prefix_len, kv->capacity);
  if (kv->capacity % 8) return fail(LUCEV_ERR_BAD_KV, "capacity must be a multiple of 8");
  if (kv->prefix_len > 0 && (!kv->k || !kv->v)) return fail(LUCEV_ERR_NULL_ARG, "kv.k / kv.v is NULL");
  if (!aligned16(kv->k) || !aligned16(kv->v)) return fail(LUCEV_ERR_ALIGN, "kv buffers must be 16-byte aligned");
  return LUCEV_OK;
}

int check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  static int cache[128];  // 0 unknown, 1 gfx950, -1 other
  if (dev < 0 || dev >= 128) return fail(LUCEV_ERR_DEVICE, "device id %d out of range", dev);
  if (cache[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    cache[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
  }
  if (cache[dev] != 1) return fail(LUCEV_ERR_DEVICE, "device %d is not gfx950", dev);
  return LUCEV_OK;
}

// Scratch of lucev_tree_attention_noalloc (the chunk partials of the tree
// attention), for callers that cannot allocate.  Each GPU the library runs on
// holds its own copy of this array until the process ends.  In host code the
// name `scratch` is only a stand-in: the device address comes from
// hipGetSymbolAddress, looked up once per device (scratch_on_device).
constexpr size_t kNoAllocScratchBytes = (size_t)LUCEV_NOALLOC_SCRATCH_BYTES;
static __device__ __attribute__((aligned(256))) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 128;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // the array's device address on each device (NULL: not looked up yet)

// The device address of `scratch` on the current device, looked up on the
// first call on that device (with it current).
int scratch_on_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(LUCEV_ERR_DEVICE, "device id %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(LUCEV_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LUCEV_OK;
}

struct Ws {
  size_t xa, xm, q32, k32, v32, opart, ml, split, cand, total;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Which projections take their weights exactly (codes through the MFMA,
// block scale in fp32) with hi + lo operand rows: QKV and Wo, whose errors
// the later layers amplify; gate/up, down and the lm_head (after which
// nothing amplifies: its logits stay within a few 1e-4 of the exact ones)
// round the weights once to fp16 and read the hi rows alone.
constexpr bool kGemmExact[5] = {true, true, false, false, false};

// every GEMM of a layer and the head, for a tree of n nodes
void layer_gemms(const lucev_shape* s, int n, GemmPlan out[5]) {
  const int64_t H = s->hidden, F = s->ffn, Hq = s->n_q_heads, Hkv = s->n_kv_heads, d = s->head_dim;
  const int64_t dims[5][2] = {{(Hq + 2 * Hkv) * d, H}, {H, Hq * d}, {2 * F, H}, {H, F}, {s->vocab, H}};
  for (int i = 0; i < 5; ++i) out[i] = plan_gemm(dims[i][0], dims[i][1], n, kGemmExact[i]);
}

bool ws_layout(const lucev_shape* s, int nmax, int pmax, Ws* w) {
  if (check_shape(s) != LUCEV_OK || nmax < 1 || nmax > LUCEV_MAX_NODES || pmax < 0) return false;
  const int64_t H = s->hidden, F = s->ffn, Hq = s->n_q_heads, Hkv = s->n_kv_heads, d = s->head_dim;
  size_t split_floats = 0, cand = 0;
  for (int n = 1; n <= nmax; ++n) {
    GemmPlan g[5];
    layer_gemms(s, n, g);
    for (int i = 0; i < 5; ++i) {
      const size_t sf = (size_t)g[i].panels * g[i].c_max * g[i].tile_floats;
      if (sf > split_floats) split_floats = sf;
    }
    if ((size_t)g[4].panels * n > cand) cand = (size_t)g[4].panels * n;
  }
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at_ = off;
    off = align256(off + bytes);
    return at_;
  };
  // GEMM operands as fp16 hi/lo rows: normed inputs and the attention output
  // (xa), the SwiGLU product (xm)
  w->xa = take((size_t)2 * nmax * (H > Hq * d ? H : Hq * d) * 2);
  w->xm = take((size_t)2 * nmax * F * 2);
  w->q32 = take((size_t)nmax * Hq * d * 4);
  w->k32 = take((size_t)nmax * Hkv * d * 4);
  w->v32 = take((size_t)nmax * Hkv * d * 4);
  const int rows = nmax * (int)(Hq / Hkv);
  const int chunks = attention_max_chunks((int)Hkv);
  w->opart = take((size_t)chunks * Hkv * rows * d * 4);
  w->ml = take((size_t)chunks * Hkv * rows * 2 * sizeof(float));
  w->split = take(split_floats * sizeof(float));
  w->cand = take(cand * sizeof(f32x4));
  w->total = off;
  (void)pmax;
  return true;
}

int check_ws(const lucev_shape* s, int n, int prefix_len, void* ws, size_t ws_bytes, Ws* w) {
  if (!ws) return fail(LUCEV_ERR_NULL_ARG, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return fail(LUCEV_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (!ws_layout(s, n, prefix_len, w)) return fail(LUCEV_ERR_BAD_SHAPE, "unsupported workspace shape");
  if (ws_bytes < w->total)
    return fail(LUCEV_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, w->total);
  return LUCEV_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// X: the fp16 hi/lo operand rows [2n][k_in]; exact: weights enter exactly and
// both operand rows are used (else weights rounded once to fp16, hi rows only)
GemmParams gemm_params(const lucev_q4& w, const uint16_t* X, int n, bool exact, void* ws, const Ws& L) {
  GemmPlan pl = plan_gemm(w.n_out, w.k_in, n, exact);
  GemmParams p;
  memset(&p, 0, sizeof(p));
  p.X = X;
  p.n_nodes = n;
  p.wq = static_cast<const uint8_t*>(w.packed);
  p.wsc = reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(w.packed) + w.n_out * w.k_in / 2);
  p.n_out = w.n_out;
  p.k_in = w.k_in;
  p.n_tiles = pl.n_tiles;
  p.kgroups = pl.kgroups;
  p.panels = pl.panels;
  p.blocks = pl.blocks;
  p.units = pl.units;
  p.partials = at<float>(ws, L.split);
  p.c_max = pl.c_max;
  p.ug = pl.ug;
  p.ft = pl.ft;
  p.vr = pl.vr;
  return p;
}

// the same GEMM writing its per-block partial tiles into the split area
GemmParams gemm_params_split(const lucev_q4& w, const uint16_t* X, int n, bool exact, void* ws,
                             const Ws& L, SplitOut* so) {
  GemmParams p = gemm_params(w, X, n, exact, ws, L);
  p.partials = at<float>(ws, L.split);
  *so = split_out(plan_gemm(w.n_out, w.k_in, n, exact), p.partials);
  return p;
}

EpiArgs epi_blank() {
  EpiArgs e;
  memset(&e, 0, sizeof(e));
  return e;
}

// A quantised prefix as the attention reads it: int8 codes or packed
// nibbles (bits 8 or 4) with fp16 block-32 scales
struct KvQuant {
  const void* k_codes;
  const uint16_t* k_scales;
  const void* v_codes;
  const uint16_t* v_scales;
  int bits;
};

// q / k_tree / v_tree bf16 (always); q32 / k32 / v32 fp32 copies or NULL;
// out bf16 [n][Hq][d], or the Wo operand's fp16 hi/lo rows when out_hilo is
// set; out32 (fp32 [n][Hq][d]) instead of both when not NULL; kq a quantised
// prefix in place of kv's bf16 arrays, when not NULL
int run_attention(const lucev_shape* s, const TreeArgs& t, const lucev_kv* kv, const uint16_t* q,
                  const uint16_t* k_tree, const uint16_t* v_tree, const float* q32,
                  const float* k32, const float* v32, uint16_t* out, int out_hilo, float* o_part,
                  float* ml_part, hipStream_t st, const int32_t* table = nullptr, int n_phys = 0,
                  float* out32 = nullptr, const KvQuant* kq = nullptr) {
  AttnPlan plan = plan_attention(t.n, s->n_q_heads, s->n_kv_heads, s->head_dim, kv->prefix_len);
  if (table && plan.chunk / kPageTokens > kMaxChunkPagesHost)
    return fail(LUCEV_ERR_BAD_KV, "paged attention: %d-token prefix chunks exceed %d pages", plan.chunk,
                kMaxChunkPagesHost);
  AttnParams p;
  p.q = q;
  p.q32 = q32;
  p.kc = kv->k;
  p.vc = kv->v;
  p.cap = kv->capacity;
  p.prefix_len = kv->prefix_len;
  p.chunk = plan.chunk;
  p.n_chunks = plan.n_chunks;
  p.n = t.n;
  p.n_q_heads = s->n_q_heads;
  p.n_kv_heads = s->n_kv_heads;
  p.rows = plan.rows;
  p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)s->head_dim));
  p.o_part = o_part;
  p.table = table;
  p.n_phys = n_phys;
  p.ml_part = ml_part;
  p.kc8 = kq ? static_cast<const int8_t*>(kq->k_codes) : nullptr;
  p.ks16 = kq ? kq->k_scales : nullptr;
  p.vc8 = kq ? static_cast<const int8_t*>(kq->v_codes) : nullptr;
  p.vs16 = kq ? kq->v_scales : nullptr;
  CombineParams c;
  c.q = q;
  c.k_tree = k_tree;
  c.v_tree = v_tree;
  c.q32 = q32;
  c.k32 = k32;
  c.v32 = v32;
  c.o_part = p.o_part;
  c.ml_part = p.ml_part;
  c.n_chunks = plan.n_chunks;
  c.n = t.n;
  c.n_q_heads = s->n_q_heads;
  c.n_kv_heads = s->n_kv_heads;
  c.rows = plan.rows;
  c.scale_log2 = p.scale_log2;
  c.out = out;
  c.out_hilo = out_hilo;
  c.out32 = out32;
  hipError_t e = kq ? launch_attention_q8(plan, s->head_dim, kq->bits, p, c, t, st)
                    : launch_attention(plan, s->head_dim, p, c, t, st);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return LUCEV_OK;
}

// Final RMSNorm, lm_head (split-K partial tiles + consumer with the fp32
// top-2 per panel), then the per-row greedy token and gap; the acceptance
// walk too when path outputs are given.
int run_head(const lucev_shape* shape, const lucev_head_w* w, const TreeArgs& t, const float* x,
             uint16_t* logits_out, int32_t* argmax_out, float* gap_out, int32_t* path_out,
             int32_t* path_len_out, int32_t* committed_out, void* ws, const Ws& L, hipStream_t st) {
  const int n = t.n;
  const int H = shape->hidden;
  hipError_t e;
  uint16_t* xa = at<uint16_t>(ws, L.xa);
  if ((e = launch_norm_hilo(x, n, H, w->final_norm, shape->rms_eps, xa, kGemmExact[4], st)) != hipSuccess)
    return hip_fail(e, "final norm launch");
  SplitOut so;
  GemmParams p = gemm_params_split(w->lm_head, xa, n, kGemmExact[4], ws, L, &so);
  f32x4* cand = at<f32x4>(ws, L.cand);
  if ((e = launch_gemm(kGemmExact[4], p, st)) != hipSuccess) return hip_fail(e, "lm_head gemm launch");
  if ((e = launch_logits_finish(so, logits_out, shape->vocab, cand, n, st)) != hipSuccess)
    return hip_fail(e, "lm_head finish launch");
  if ((e = launch_finalize(cand, so.panels, t, argmax_out, gap_out, path_out, path_len_out,
                           committed_out, st)) != hipSuccess)
    return hip_fail(e, "finalize launch");
  return LUCEV_OK;
}

}  // namespace

extern "C" {

int lucev_abi_version(void) { return LUCEV_ABI_VERSION; }

const char* lucev_status_str(int status) {
  switch (status) {
    case LUCEV_OK: return "ok";
    case LUCEV_ERR_NULL_ARG: return "null argument";
    case LUCEV_ERR_BAD_SHAPE: return "unsupported shape";
    case LUCEV_ERR_BAD_TREE: return "malformed tree";
    case LUCEV_ERR_WORKSPACE: return "workspace too small";
    case LUCEV_ERR_ALIGN: return "misaligned pointer";
    case LUCEV_ERR_HIP: return "HIP error";
    case LUCEV_ERR_DEVICE: return "device is not gfx950";
    case LUCEV_ERR_BAD_KV: return "bad KV cache descriptor";
    default: return "unknown status";
  }
}

const char* lucev_last_error(void) { return g_err; }

size_t lucev_q4_packed_bytes(int64_t n_out, int64_t k_in) {
  if (n_out <= 0 || k_in <= 0 || n_out % 16 || k_in % 128) return 0;
  return (size_t)(n_out * k_in / 32 * 18);
}

static int check_pack(int kind, int32_t head_dim, const void* q, const void* d, int64_t n_out,
                      int64_t k_in, const void* dst, size_t dst_bytes) {
  if (!q || !d || !dst) return fail(LUCEV_ERR_NULL_ARG, "pack: NULL pointer");
  const size_t need = lucev_q4_packed_bytes(n_out, k_in);
  if (!need) return fail(LUCEV_ERR_BAD_SHAPE, "pack: n_out %% 16 and k_in %% 128 must be 0");
  if (kind < LUCEV_W_PLAIN || kind > LUCEV_W_GU) return fail(LUCEV_ERR_BAD_SHAPE, "pack: bad kind %d", kind);
  if (kind == LUCEV_W_QKV && (head_dim % 16 || head_dim <= 0 || n_out % head_dim))
    return fail(LUCEV_ERR_BAD_SHAPE, "pack: head_dim %d does not tile n_out", head_dim);
  if (kind == LUCEV_W_GU && n_out % 32) return fail(LUCEV_ERR_BAD_SHAPE, "pack: gate/up needs n_out %% 32 == 0");
  if (dst_bytes < need) return fail(LUCEV_ERR_WORKSPACE, "pack: dst %zu < %zu bytes", dst_bytes, need);
  return LUCEV_OK;
}

int lucev_q4_pack(int kind, int32_t head_dim, const uint8_t* q, const uint16_t* d, int64_t n_out,
                  int64_t k_in, void* dst, size_t dst_bytes) {
  int rc = check_pack(kind, head_dim, q, d, n_out, k_in, dst, dst_bytes);
  if (rc) return rc;
  pack_q4_host(q, d, n_out, k_in, kind, head_dim, dst);
  return LUCEV_OK;
}

int lucev_q4_pack_device(int kind, int32_t head_dim, const uint8_t* q, const uint16_t* d,
                         int64_t n_out, int64_t k_in, void* dst, size_t dst_bytes, void* stream) {
  int rc = check_pack(kind, head_dim, q, d, n_out, k_in, dst, dst_bytes);
  if (rc) return rc;
  if (!aligned16(dst) || !aligned16(q)) return fail(LUCEV_ERR_ALIGN, "pack: pointers must be 16-byte aligned");
  if ((rc = check_device())) return rc;
  hipError_t e = launch_pack_q4(q, d, n_out, k_in, kind, head_dim, dst, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "pack launch");
  return LUCEV_OK;
}

size_t lucev_workspace_bytes(const lucev_shape* shape, int32_t n_nodes, int32_t prefix_len) {
  Ws w;
  if (!ws_layout(shape, n_nodes, prefix_len, &w)) return 0;
  return w.total;
}

int lucev_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws) return fail(LUCEV_ERR_NULL_ARG, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(LUCEV_ERR_ALIGN, "workspace must be 256-byte aligned");
  int rc = check_device();
  if (rc) return rc;
  hipError_t e = launch_zero(ws, ws_bytes & ~size_t(15), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "zero launch");
  return LUCEV_OK;
}

int lucev_tree_attention(const lucev_shape* shape, const lucev_tree* tree, const lucev_kv* kv,
                         const uint16_t* q, const uint16_t* k_tree, const uint16_t* v_tree,
                         uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!q || !k_tree || !v_tree || !out) return fail(LUCEV_ERR_NULL_ARG, "tree_attention: NULL tensor");
  if ((rc = check_kv(kv))) return rc;
  TreeArgs t;
  if ((rc = prep_tree(tree, shape->vocab, kv->prefix_len, &t))) return rc;
  if ((rc = check_attn_rows(shape, t.n))) return rc;
  if (!aligned16(q) || !aligned16(k_tree) || !aligned16(v_tree) || !aligned16(out))
    return fail(LUCEV_ERR_ALIGN, "tree_attention: tensors must be 16-byte aligned");
  Ws L;
  if ((rc = check_ws(shape, t.n, kv->prefix_len, ws, ws_bytes, &L))) return rc;
  if ((rc = check_device())) return rc;
  return run_attention(shape, t, kv, q, k_tree, v_tree, nullptr, nullptr, nullptr, out, 0,
                       at<float>(ws, L.opart), at<float>(ws, L.ml), (hipStream_t)stream);
}

int lucev_tree_attention_f32(const lucev_shape* shape, const lucev_tree* tree, const lucev_kv* kv,
                             const float* q, const float* k_tree, const float* v_tree, float* out, void* ws,
                             size_t ws_bytes, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!q || !k_tree || !v_tree || !out) return fail(LUCEV_ERR_NULL_ARG, "tree_attention_f32: NULL tensor");
  if ((rc = check_kv(kv))) return rc;
  TreeArgs t;
  if ((rc = prep_tree(tree, shape->vocab, kv->prefix_len, &t))) return rc;
  if ((rc = check_attn_rows(shape, t.n))) return rc;
  if (!aligned16(q) || !aligned16(k_tree) || !aligned16(v_tree) || !aligned16(out))
    return fail(LUCEV_ERR_ALIGN, "tree_attention_f32: tensors must be 16-byte aligned");
  Ws L;
  if ((rc = check_ws(shape, t.n, kv->prefix_len, ws, ws_bytes, &L))) return rc;
  if ((rc = check_device())) return rc;
  // q, k_tree, v_tree as the fp32 inputs the verify step hands its attention
  return run_attention(shape, t, kv, nullptr, nullptr, nullptr, q, k_tree, v_tree, nullptr, 0,
                       at<float>(ws, L.opart), at<float>(ws, L.ml), (hipStream_t)stream, nullptr, 0, out);
}

// prefix_len / capacity / pointers / alignment of a quantised cache
static int check_kv_quant(int prefix_len, int capacity, const KvQuant& q, const char* what) {
  if (prefix_len < 0 || capacity < 0 || prefix_len > capacity)
    return fail(LUCEV_ERR_BAD_KV, "prefix_len %d / capacity %d invalid", prefix_len, capacity);
  if (capacity % 32) return fail(LUCEV_ERR_BAD_KV, "%s cache: capacity must be a multiple of 32", what);
  if (prefix_len > 0 && (!q.k_codes || !q.k_scales || !q.v_codes || !q.v_scales))
    return fail(LUCEV_ERR_NULL_ARG, "%s cache: NULL codes or scales", what);
  if (!aligned16(q.k_codes) || !aligned16(q.v_codes) || (reinterpret_cast<uintptr_t>(q.k_scales) & 7u) ||
      (reinterpret_cast<uintptr_t>(q.v_scales) & 3u))
    return fail(LUCEV_ERR_ALIGN, "%s cache: codes must be 16-byte, K scales 8-byte, V scales 4-byte aligned", what);
  return LUCEV_OK;
}

static int tree_attention_quant(const lucev_shape* shape, const lucev_tree* tree, int prefix_len, int capacity,
                                const KvQuant& kq, const uint16_t* q, const uint16_t* k_tree,
                                const uint16_t* v_tree, uint16_t* out, void* ws, size_t ws_bytes, void* stream,
                                const char* what) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!q || !k_tree || !v_tree || !out) return fail(LUCEV_ERR_NULL_ARG, "tree_attention_%s: NULL tensor", what);
  if ((rc = check_kv_quant(prefix_len, capacity, kq, what))) return rc;
  TreeArgs t;
  if ((rc = prep_tree(tree, shape->vocab, prefix_len, &t))) return rc;
  if ((rc = check_attn_rows(shape, t.n))) return rc;
  if (!aligned16(q) || !aligned16(k_tree) || !aligned16(v_tree) || !aligned16(out))
    return fail(LUCEV_ERR_ALIGN, "tree_attention_%s: tensors must be 16-byte aligned", what);
  Ws L;
  if ((rc = check_ws(shape, t.n, prefix_len, ws, ws_bytes, &L))) return rc;
  if ((rc = check_device())) return rc;
  lucev_kv flat;  // geometry only; the codes and scales come from kq
  flat.k = nullptr;
  flat.v = nullptr;
  flat.prefix_len = prefix_len;
  flat.capacity = capacity;
  return run_attention(shape, t, &flat, q, k_tree, v_tree, nullptr, nullptr, nullptr, out, 0,
                       at<float>(ws, L.opart), at<float>(ws, L.ml), (hipStream_t)stream, nullptr, 0, nullptr, &kq);
}

int lucev_tree_attention_q8(const lucev_shape* shape, const lucev_tree* tree, const lucev_kv_q8* kv,
                            const uint16_t* q, const uint16_t* k_tree, const uint16_t* v_tree, uint16_t* out,
                            void* ws, size_t ws_bytes, void* stream) {
  if (!kv) return fail(LUCEV_ERR_NULL_ARG, "kv is NULL");
  const KvQuant kq{kv->k_codes, kv->k_scales, kv->v_codes, kv->v_scales, 8};
  return tree_attention_quant(shape, tree, kv->prefix_len, kv->capacity, kq, q, k_tree, v_tree, out, ws, ws_bytes,
                              stream, "q8");
}

int lucev_tree_attention_q4(const lucev_shape* shape, const lucev_tree* tree, const lucev_kv_q4* kv,
                            const uint16_t* q, const uint16_t* k_tree, const uint16_t* v_tree, uint16_t* out,
                            void* ws, size_t ws_bytes, void* stream) {
  if (!kv) return fail(LUCEV_ERR_NULL_ARG, "kv is NULL");
  const KvQuant kq{kv->k_nibbles, kv->k_scales, kv->v_nibbles, kv->v_scales, 4};
  return tree_attention_quant(shape, tree, kv->prefix_len, kv->capacity, kq, q, k_tree, v_tree, out, ws, ws_bytes,
                              stream, "q4");
}

// shape, source cache and output pointers of a quantisation call
static int check_quantize(const lucev_shape* shape, const lucev_kv* src, const void* k_codes,
                          const uint16_t* k_scales, const void* v_codes, const uint16_t* v_scales, const char* what) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if ((rc = check_kv(src))) return rc;
  if (!src->k || !src->v || !k_codes || !k_scales || !v_codes || !v_scales)
    return fail(LUCEV_ERR_NULL_ARG, "kv_quantize_%s: NULL pointer", what);
  if (src->capacity % 32) return fail(LUCEV_ERR_BAD_KV, "kv_quantize_%s: capacity must be a multiple of 32", what);
  if (!aligned16(k_codes) || !aligned16(v_codes) || (reinterpret_cast<uintptr_t>(k_scales) & 1u) ||
      (reinterpret_cast<uintptr_t>(v_scales) & 1u))
    return fail(LUCEV_ERR_ALIGN, "kv_quantize_%s: codes must be 16-byte aligned", what);
  return check_device();
}

int lucev_kv_quantize_q8(const lucev_shape* shape, const lucev_kv* src, int8_t* k_codes, uint16_t* k_scales,
                         int8_t* v_codes, uint16_t* v_scales, void* stream) {
  int rc = check_quantize(shape, src, k_codes, k_scales, v_codes, v_scales, "q8");
  if (rc) return rc;
  hipError_t e = launch_quantize_q8(src->k, src->v, shape->n_kv_heads, src->capacity, shape->head_dim, k_codes,
                                    k_scales, v_codes, v_scales, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "quantize launch");
  return LUCEV_OK;
}

int lucev_kv_quantize_q4(const lucev_shape* shape, const lucev_kv* src, uint8_t* k_nibbles, uint16_t* k_scales,
                         uint8_t* v_nibbles, uint16_t* v_scales, void* stream) {
  int rc = check_quantize(shape, src, k_nibbles, k_scales, v_nibbles, v_scales, "q4");
  if (rc) return rc;
  hipError_t e = launch_quantize_q4(src->k, src->v, shape->n_kv_heads, src->capacity, shape->head_dim, k_nibbles,
                                    k_scales, v_nibbles, v_scales, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "quantize launch");
  return LUCEV_OK;
}

int lucev_tree_attention_noalloc(const lucev_shape* shape, const lucev_tree* tree, const lucev_kv* kv,
                                 const uint16_t* q, const uint16_t* k_tree, const uint16_t* v_tree,
                                 uint16_t* out, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!q || !k_tree || !v_tree || !out) return fail(LUCEV_ERR_NULL_ARG, "tree_attention_noalloc: NULL tensor");
  if ((rc = check_kv(kv))) return rc;
  TreeArgs t;
  if ((rc = prep_tree(tree, shape->vocab, kv->prefix_len, &t))) return rc;
  if ((rc = check_attn_rows(shape, t.n))) return rc;
  if (!aligned16(q) || !aligned16(k_tree) || !aligned16(v_tree) || !aligned16(out))
    return fail(LUCEV_ERR_ALIGN, "tree_attention_noalloc: tensors must be 16-byte aligned");
  // the chunk partials of this call: O [chunks][Hkv][rows][d], then (max, sum)
  // [chunks][Hkv][rows][2], all fp32
  const AttnPlan plan = plan_attention(t.n, shape->n_q_heads, shape->n_kv_heads, shape->head_dim, kv->prefix_len);
  const size_t o_bytes = align256((size_t)plan.n_chunks * shape->n_kv_heads * plan.rows * shape->head_dim * 4);
  const size_t need = o_bytes + (size_t)plan.n_chunks * shape->n_kv_heads * plan.rows * 2 * 4;
  if (need > kNoAllocScratchBytes)
    return fail(LUCEV_ERR_WORKSPACE,
                "tree_attention_noalloc: this call needs %zu bytes of scratch, more than the %zu the library holds "
                "(fewer nodes or a shorter prefix, or lucev_tree_attention with a workspace)",
                need, kNoAllocScratchBytes);
  if ((rc = check_device())) return rc;
  void* base = nullptr;
  if ((rc = scratch_on_device(&base))) return rc;
  float* o_part = static_cast<float*>(base);
  float* ml_part = reinterpret_cast<float*>(static_cast<uint8_t*>(base) + o_bytes);
  return run_attention(shape, t, kv, q, k_tree, v_tree, nullptr, nullptr, nullptr, out, 0, o_part, ml_part,
                       (hipStream_t)stream);
}

int lucev_tree_attention_paged(const lucev_shape* shape, const lucev_tree* tree,
                               const lucev_kv_paged* kv, const uint16_t* q, const uint16_t* k_tree,
                               const uint16_t* v_tree, uint16_t* out, void* ws, size_t ws_bytes,
                               void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!kv || !q || !k_tree || !v_tree || !out)
    return fail(LUCEV_ERR_NULL_ARG, "tree_attention_paged: NULL argument");
  if (kv->prefix_len < 0 || kv->n_pages < 0 || (kv->prefix_len > 0 && kv->n_pages < 1))
    return fail(LUCEV_ERR_BAD_KV, "tree_attention_paged: prefix_len %d, n_pages %d", kv->prefix_len,
                kv->n_pages);
  if (kv->prefix_len > 0 && (!kv->k_pages || !kv->v_pages || !kv->block_table))
    return fail(LUCEV_ERR_NULL_ARG, "tree_attention_paged: NULL page pool or block table");
  if (!aligned16(kv->k_pages) || !aligned16(kv->v_pages) || !aligned16(q) || !aligned16(k_tree) ||
      !aligned16(v_tree) || !aligned16(out))
    return fail(LUCEV_ERR_ALIGN, "tree_attention_paged: tensors must be 16-byte aligned");
  TreeArgs t;
  if ((rc = prep_tree(tree, shape->vocab, kv->prefix_len, &t))) return rc;
  if ((rc = check_attn_rows(shape, t.n))) return rc;
  Ws L;
  if ((rc = check_ws(shape, t.n, kv->prefix_len, ws, ws_bytes, &L))) return rc;
  if ((rc = check_device())) return rc;
  // the pool stands in for the contiguous cache; the table supplies every address
  lucev_kv flat;
  flat.k = kv->k_pages;
  flat.v = kv->v_pages;
  flat.prefix_len = kv->prefix_len;
  flat.capacity = 0;
  return run_attention(shape, t, &flat, q, k_tree, v_tree, nullptr, nullptr, nullptr, out, 0,
                       at<float>(ws, L.opart), at<float>(ws, L.ml), (hipStream_t)stream,
                       kv->prefix_len > 0 ? kv->block_table : nullptr, kv->n_pages);
}

// One layer over a bf16 prefix (kq NULL) or a quantised one (kq; kv then
// carries only prefix_len and capacity)
static int verify_layer_impl(const lucev_shape* shape, const lucev_layer_w* w, const lucev_tree* tree,
                             const lucev_kv* kv, const KvQuant* kq, float* resid_io, uint16_t* k_tree_out,
                             uint16_t* v_tree_out, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!w || !resid_io || !k_tree_out || !v_tree_out || !w->attn_norm || !w->ffn_norm)
    return fail(LUCEV_ERR_NULL_ARG, "verify_layer: NULL argument");
  if (kq) {
    if ((rc = check_kv_quant(kv->prefix_len, kv->capacity, *kq, kq->bits == 8 ? "q8" : "q4"))) return rc;
  } else if ((rc = check_kv(kv))) {
    return rc;
  }
  TreeArgs t;
  if ((rc = prep_tree(tree, shape->vocab, kv->prefix_len, &t))) return rc;
  if ((rc = check_attn_rows(shape, t.n))) return rc;
  const int64_t H = shape->hidden, F = shape->ffn, Hq = shape->n_q_heads, Hkv = shape->n_kv_heads,
                d = shape->head_dim;
  if ((rc = check_q4(w->wqkv, (Hq + 2 * Hkv) * d, H, "wqkv"))) return rc;
  if ((rc = check_q4(w->wo, H, Hq * d, "wo"))) return rc;
  if ((rc = check_q4(w->wgu, 2 * F, H, "wgu"))) return rc;
  if ((rc = check_q4(w->wd, H, F, "wd"))) return rc;
  if (!aligned16(resid_io) || !aligned16(k_tree_out) || !aligned16(v_tree_out))
    return fail(LUCEV_ERR_ALIGN, "verify_layer: tensors must be 16-byte aligned");
  Ws L;
  if ((rc = check_ws(shape, t.n, kv->prefix_len, ws, ws_bytes, &L))) return rc;
  if ((rc = check_device())) return rc;

  hipStream_t st = (hipStream_t)stream;
  const int n = t.n;
  const float eps = shape->rms_eps;
  uint16_t* xa = at<uint16_t>(ws, L.xa);
  uint16_t* xm = at<uint16_t>(ws, L.xm);
  float* q32 = at<float>(ws, L.q32);
  float* k32 = at<float>(ws, L.k32);
  float* v32 = at<float>(ws, L.v32);
  hipError_t e;

  // attention half: RMSNorm -> QKV (split) -> RoPE -> tree attention -> Wo (split)
  if ((e = launch_norm_hilo(resid_io, n, (int)H, w->attn_norm, eps, xa, kGemmExact[0], st)) != hipSuccess)
    return hip_fail(e, "attention norm launch");
  SplitOut so;
  {
    GemmParams p = gemm_params_split(w->wqkv, xa, n, true, ws, L, &so);
    if ((e = launch_gemm(true, p, st)) != hipSuccess)
      return hip_fail(e, "qkv gemm launch");
    EpiArgs ea = epi_blank();
    ea.k_out = k_tree_out;
    ea.v_out = v_tree_out;
    ea.q32 = q32;
    ea.k32 = k32;
    ea.v32 = v32;
    ea.n_q_heads = (int)Hq;
    ea.n_kv_heads = (int)Hkv;
    ea.head_dim = (int)d;
    for (int i = 0; i < n; ++i) ea.pos[i] = t.pos[i];
    for (int j = 0; j < d / 2; ++j) ea.inv_freq[j] = pow((double)shape->rope_base, -2.0 * j / (double)d);
    if ((e = launch_qkv_finish(so, ea, n, st)) != hipSuccess) return hip_fail(e, "qkv finish launch");
  }
  if ((rc = run_attention(shape, t, kv, nullptr, k_tree_out, v_tree_out, q32, k32, v32, xa, 1,
                          at<float>(ws, L.opart), at<float>(ws, L.ml), st, nullptr, 0, nullptr, kq)))
    return rc;
  {
    GemmParams p = gemm_params_split(w->wo, xa, n, true, ws, L, &so);
    if ((e = launch_gemm(true, p, st)) != hipSuccess)
      return hip_fail(e, "wo gemm launch");
    // residual += attention output projection, then the FFN RMSNorm (two
    // kernels: a fused one with one block per row, or with a cross-block
    // handoff of the row's sum of squares, measured slower)
    if ((e = launch_resid_finish(so, resid_io, (int)H, n, st)) != hipSuccess)
      return hip_fail(e, "wo finish launch");
    if ((e = launch_norm_hilo(resid_io, n, (int)H, w->ffn_norm, eps, xa, kGemmExact[2], st)) != hipSuccess)
      return hip_fail(e, "ffn norm launch");
  }
  // FFN half: gate/up (split) -> SwiGLU -> down (split) -> residual
  {
    GemmParams p = gemm_params_split(w->wgu, xa, n, false, ws, L, &so);
    if ((e = launch_gemm(false, p, st)) != hipSuccess)
      return hip_fail(e, "gate/up gemm launch");
    if ((e = launch_swiglu_finish(so, xm, (int)F, n, st)) != hipSuccess) return hip_fail(e, "swiglu launch");
  }
  {
    GemmParams p = gemm_params_split(w->wd, xm, n, false, ws, L, &so);
    if ((e = launch_gemm(false, p, st)) != hipSuccess)
      return hip_fail(e, "down gemm launch");
    if ((e = launch_resid_finish(so, resid_io, (int)H, n, st)) != hipSuccess)
      return hip_fail(e, "down finish launch");
  }
  return LUCEV_OK;
}

int lucev_verify_layer(const lucev_shape* shape, const lucev_layer_w* w, const lucev_tree* tree,
                       const lucev_kv* kv, float* resid_io, uint16_t* k_tree_out,
                       uint16_t* v_tree_out, void* ws, size_t ws_bytes, void* stream) {
  return verify_layer_impl(shape, w, tree, kv, nullptr, resid_io, k_tree_out, v_tree_out, ws, ws_bytes, stream);
}

int lucev_verify_layer_q8(const lucev_shape* shape, const lucev_layer_w* w, const lucev_tree* tree,
                          const lucev_kv_q8* kv, float* resid_io, uint16_t* k_tree_out, uint16_t* v_tree_out,
                          void* ws, size_t ws_bytes, void* stream) {
  if (!kv) return fail(LUCEV_ERR_NULL_ARG, "kv is NULL");
  const KvQuant kq{kv->k_codes, kv->k_scales, kv->v_codes, kv->v_scales, 8};
  lucev_kv geo;  // geometry only; the codes and scales come from kq
  geo.k = nullptr;
  geo.v = nullptr;
  geo.prefix_len = kv->prefix_len;
  geo.capacity = kv->capacity;
  return verify_layer_impl(shape, w, tree, &geo, &kq, resid_io, k_tree_out, v_tree_out, ws, ws_bytes, stream);
}

int lucev_verify_layer_q4(const lucev_shape* shape, const lucev_layer_w* w, const lucev_tree* tree,
                          const lucev_kv_q4* kv, float* resid_io, uint16_t* k_tree_out, uint16_t* v_tree_out,
                          void* ws, size_t ws_bytes, void* stream) {
  if (!kv) return fail(LUCEV_ERR_NULL_ARG, "kv is NULL");
  const KvQuant kq{kv->k_nibbles, kv->k_scales, kv->v_nibbles, kv->v_scales, 4};
  lucev_kv geo;
  geo.k = nullptr;
  geo.v = nullptr;
  geo.prefix_len = kv->prefix_len;
  geo.capacity = kv->capacity;
  return verify_layer_impl(shape, w, tree, &geo, &kq, resid_io, k_tree_out, v_tree_out, ws, ws_bytes, stream);
}

int lucev_accept_path(const lucev_shape* shape, const lucev_head_w* w, const lucev_tree* tree,
                      const float* resid, uint16_t* logits_out, int32_t* argmax_out, float* gap_out,
                      int32_t* path_out, int32_t* path_len_out, int32_t* committed_out, void* ws,
                      size_t ws_bytes, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!w || !w->final_norm || !resid || !argmax_out || !path_out || !path_len_out || !committed_out)
    return fail(LUCEV_ERR_NULL_ARG, "accept_path: NULL argument");
  TreeArgs t;
  if ((rc = prep_tree(tree, shape->vocab, 0, &t))) return rc;
  if ((rc = check_q4(w->lm_head, shape->vocab, shape->hidden, "lm_head"))) return rc;
  if (!aligned16(resid) || (logits_out && !aligned16(logits_out)))
    return fail(LUCEV_ERR_ALIGN, "accept_path: tensors must be 16-byte aligned");
  Ws L;
  if ((rc = check_ws(shape, t.n, 0, ws, ws_bytes, &L))) return rc;
  if ((rc = check_device())) return rc;

  return run_head(shape, w, t, resid, logits_out, argmax_out, gap_out, path_out, path_len_out,
                  committed_out, ws, L, (hipStream_t)stream);
}

int lucev_project_logits(const lucev_shape* shape, const lucev_head_w* w, int32_t n_rows,
                         const float* x, uint16_t* logits_out, int32_t* argmax_out, float* gap_out,
                         void* ws, size_t ws_bytes, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!w || !w->final_norm || !x || !argmax_out)
    return fail(LUCEV_ERR_NULL_ARG, "project_logits: NULL argument");
  if (n_rows < 1 || n_rows > LUCEV_MAX_NODES)
    return fail(LUCEV_ERR_BAD_TREE, "project_logits: n_rows %d outside [1, %d]", n_rows, LUCEV_MAX_NODES);
  if ((rc = check_q4(w->lm_head, shape->vocab, shape->hidden, "lm_head"))) return rc;
  if (!aligned16(x) || (logits_out && !aligned16(logits_out)))
    return fail(LUCEV_ERR_ALIGN, "project_logits: tensors must be 16-byte aligned");
  Ws L;
  if ((rc = check_ws(shape, n_rows, 0, ws, ws_bytes, &L))) return rc;
  if ((rc = check_device())) return rc;
  TreeArgs t;
  memset(&t, 0, sizeof(t));
  t.n = n_rows;
  return run_head(shape, w, t, x, logits_out, argmax_out, gap_out, nullptr, nullptr, nullptr, ws, L,
                  (hipStream_t)stream);
}

int lucev_commit_path(const lucev_shape* shape, int32_t n_layers, uint16_t* const* k_cache,
                      uint16_t* const* v_cache, const uint16_t* const* k_tree,
                      const uint16_t* const* v_tree, int32_t prefix_len, int32_t capacity,
                      int32_t n_nodes, const int32_t* path, const int32_t* path_len,
                      void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (n_layers < 1 || n_layers > LUCEV_MAX_COMMIT_LAYERS)
    return fail(LUCEV_ERR_BAD_SHAPE, "commit_path: n_layers %d outside [1, %d]", n_layers,
                LUCEV_MAX_COMMIT_LAYERS);
  if (n_nodes < 1 || n_nodes > LUCEV_MAX_NODES)
    return fail(LUCEV_ERR_BAD_TREE, "commit_path: n_nodes %d outside [1, %d]", n_nodes, LUCEV_MAX_NODES);
  if (!k_cache || !v_cache || !k_tree || !v_tree || !path || !path_len)
    return fail(LUCEV_ERR_NULL_ARG, "commit_path: NULL argument");
  if (prefix_len < 0 || capacity < 0 || (int64_t)prefix_len + n_nodes > capacity)
    return fail(LUCEV_ERR_BAD_KV, "commit_path: prefix_len %d + n_nodes %d exceeds capacity %d",
                prefix_len, n_nodes, capacity);
  CommitArgs a;
  memset(&a, 0, sizeof(a));
  for (int l = 0; l < n_layers; ++l) {
    if (!k_cache[l] || !v_cache[l] || !k_tree[l] || !v_tree[l])
      return fail(LUCEV_ERR_NULL_ARG, "commit_path: NULL pointer for layer %d", l);
    a.kc[l] = k_cache[l];
    a.vc[l] = v_cache[l];
    a.kt[l] = k_tree[l];
    a.vt[l] = v_tree[l];
  }
  a.path = path;
  a.path_len = path_len;
  a.n_layers = n_layers;
  a.n = n_nodes;
  a.prefix_len = prefix_len;
  a.cap = capacity;
  a.n_kv_heads = shape->n_kv_heads;
  a.head_dim = shape->head_dim;
  if ((rc = check_device())) return rc;
  hipError_t e = launch_commit(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "commit launch");
  return LUCEV_OK;
}

int lucev_describe_attention(const lucev_shape* shape, int32_t n_nodes, int32_t prefix_len, int32_t variant,
                             char* buf, size_t buf_len) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!buf || buf_len == 0) return fail(LUCEV_ERR_NULL_ARG, "describe_attention: NULL buffer");
  if (n_nodes < 1 || n_nodes > LUCEV_MAX_NODES || prefix_len < 0)
    return fail(LUCEV_ERR_BAD_TREE, "describe_attention: n_nodes %d / prefix_len %d invalid", n_nodes, prefix_len);
  if ((rc = check_attn_rows(shape, n_nodes))) return rc;
  if (variant < 0 || variant > 4) return fail(LUCEV_ERR_BAD_SHAPE, "describe_attention: variant %d", variant);
  const AttnPlan plan = plan_attention(n_nodes, shape->n_q_heads, shape->n_kv_heads, shape->head_dim, prefix_len);
  const int cb = n_nodes * shape->n_q_heads;
  if (variant >= 3)
    describe_attention_q8(plan, shape->head_dim, shape->n_kv_heads, cb, variant == 3 ? 8 : 4, buf, buf_len);
  else
    describe_attention(plan, shape->head_dim, shape->n_kv_heads, cb, variant == 1, variant == 2, buf, buf_len);
  return LUCEV_OK;
}

int lucev_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!sink || (bytes > 0 && !src)) return fail(LUCEV_ERR_NULL_ARG, "stream_read: NULL pointer");
  if (bytes % 16 || !aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3u))
    return fail(LUCEV_ERR_ALIGN, "stream_read: src must be 16-byte aligned, bytes a multiple of 16, sink 4-byte aligned");
  int rc = check_device();
  if (rc) return rc;
  hipError_t e = launch_stream_read(src, bytes, sink, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "stream read launch");
  return LUCEV_OK;
}

int lucev_set_gemv_max_rows(int32_t rows) {
  if (rows < 0 || rows > 8) return fail(LUCEV_ERR_BAD_SHAPE, "set_gemv_max_rows: %d outside [0, 8]", rows);
  g_gemv_max_rows = rows;
  return LUCEV_OK;
}

}  // extern "C"
