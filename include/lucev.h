/*
 * lucev.h -- C ABI of the tree-verification forward on one MI355X (gfx950).
 *
 * One step of tree-based speculative decoding on the target model: a tree of
 * drafted tokens is scored in ONE forward pass against a long KV cache, and
 * greedy acceptance keeps the longest accepted root path.
 *
 * Passages this interface follows (page title, section):
 *   - "Lucebox Hub", section "Speculative decoding 계층 (DFlash / DDTree /
 *     DSpark)": the target verifies a tree of candidates in one forward
 *     (verify_batch); the target adapter also projects hidden states through
 *     its lm_head and keeps the KV cache so rejected tokens can be dropped.
 *   - "Lucebox Hub", section "배경: 어떤 문제를 푸는가", item 1: decode reads
 *     every weight once per forward, so one forward that checks many drafted
 *     tokens amortises that read.
 *   - "Lucebox: 추측 디코딩과 전용 커널로 ..." (discuss.pytorch.kr), section
 *     "Lucebox 설치 및 실행": greedy decoding (temperature 0); tree budget 22
 *     nodes on an RTX 3090 and 40 on an RTX 5090.
 *
 * The layer is a pre-norm decoder layer: RMSNorm, GQA attention with RoPE at
 * position prefix_len + depth, SwiGLU FFN, all projections int4 block-32
 * (w = d * (q - 8), fp16 d per 32 consecutive inputs).
 *
 * Conventions for every entry point
 *   - Every tensor pointer is DEVICE memory owned by the caller and borrowed
 *     until the stream reaches the end of the call.  The library never
 *     allocates or frees device memory on these paths; scratch space is the
 *     caller's workspace (lucev_workspace_bytes).
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = default
 *     stream) with no implicit synchronisation.  Calls are graph-capturable.
 *   - Arguments are validated on the host BEFORE anything is launched.  On a
 *     non-zero return nothing was enqueued (except LUCEV_ERR_HIP, which
 *     reports a failed launch).  No C++ exception crosses the ABI.
 *   - Same inputs give bit-identical outputs (no floating-point atomics).
 *   - bf16 / fp16 tensors are passed as uint16_t bit patterns.
 *   - Shapes: hidden, ffn and n_q_heads*head_dim multiples of 128; hidden <= 8192;
 *     head_dim in {64, 128}; n_q_heads a multiple of n_kv_heads;
 *     vocab a multiple of 16; 1 <= tree nodes <= LUCEV_MAX_NODES.  Entry
 *     points that run the tree attention also need n * n_q_heads /
 *     n_kv_heads <= LUCEV_MAX_ATTN_ROWS (every query row of a KV head is held
 *     by one workgroup); larger trees return LUCEV_ERR_BAD_SHAPE.
 *   - KV cache descriptors (lucev_kv): 0 <= prefix_len <= capacity and
 *     capacity a multiple of 8 (each V^T row is read in 16-byte pieces), else
 *     LUCEV_ERR_BAD_KV; k and v non-NULL when prefix_len > 0
 *     (LUCEV_ERR_NULL_ARG) and 16-byte aligned (LUCEV_ERR_ALIGN).
 */
#ifndef LUCEV_H
#define LUCEV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LUCEV_ABI_VERSION 1
#define LUCEV_MAX_NODES 64
#define LUCEV_MAX_ATTN_ROWS 512  /* n * n_q_heads / n_kv_heads */

/* status codes */
#define LUCEV_OK 0
#define LUCEV_ERR_NULL_ARG -1   /* a required pointer is NULL */
#define LUCEV_ERR_BAD_SHAPE -2  /* unsupported dims (see conventions) */
#define LUCEV_ERR_BAD_TREE -3   /* n outside [1,64], parent[0] != -1,
                                   parent[i] outside [0,i), token outside [0,vocab) */
#define LUCEV_ERR_WORKSPACE -4  /* workspace smaller than lucev_workspace_bytes */
#define LUCEV_ERR_ALIGN -5      /* a pointer is not 16-byte aligned */
#define LUCEV_ERR_HIP -6        /* a HIP call failed; see lucev_last_error() */
#define LUCEV_ERR_DEVICE -7     /* current device is not gfx950 */
#define LUCEV_ERR_BAD_KV -8     /* prefix_len < 0 or > capacity, capacity < 0 or not a
                                   multiple of 8; paged: see lucev_tree_attention_paged;
                                   commit: prefix_len + n_nodes > capacity */

/* Model shape shared by every layer. */
typedef struct {
  int32_t hidden;      /* H */
  int32_t n_q_heads;   /* Hq */
  int32_t n_kv_heads;  /* Hkv; query head h reads KV head h / (Hq / Hkv) */
  int32_t head_dim;    /* d */
  int32_t ffn;         /* F (SwiGLU inner width) */
  int32_t vocab;       /* V */
  float rms_eps;       /* added to mean(x^2) inside RMSNorm */
  float rope_base;     /* RoPE: theta_j = pos * base^(-2j/d), rotate-half pairs (j, j+d/2) */
} lucev_shape;

/* One int4 matrix in the library's packed layout (lucev_q4_pack*).
 * Logical form: W[n, k] = d[n, k/32] * (q[n, k] - 8), n < n_out, k < k_in. */
typedef struct {
  const void* packed;  /* device, lucev_q4_packed_bytes(n_out, k_in) bytes */
  int64_t n_out;
  int64_t k_in;
} lucev_q4;

/* Weights of one layer.  Norm gains are bf16 [H] and multiply (x*g).
 *   wqkv: n_out = (Hq + 2 Hkv) d, k_in = H; logical rows [q heads; k heads; v heads]
 *   wo  : n_out = H, k_in = Hq d
 *   wgu : n_out = 2 F, k_in = H; logical rows [gate; up]
 *   wd  : n_out = H, k_in = F                                                */
typedef struct {
  const uint16_t* attn_norm;
  const uint16_t* ffn_norm;
  lucev_q4 wqkv, wo, wgu, wd;
} lucev_layer_w;

/* Final RMSNorm gain (bf16 [H]) and the lm_head (n_out = V, k_in = H). */
typedef struct {
  const uint16_t* final_norm;
  lucev_q4 lm_head;
} lucev_head_w;

/* One layer's bf16 KV cache for one sequence.
 *   k: [Hkv][capacity][d]  keys stored after RoPE (token t rotated at position t)
 *   v: [Hkv][d][capacity]  values stored dim-major (transposed), so the
 *                          attention reads consecutive tokens of one dim
 * Tokens 0 .. prefix_len-1 are the prefix every tree node attends to.        */
typedef struct {
  const uint16_t* k;
  const uint16_t* v;
  int32_t prefix_len;
  int32_t capacity;
} lucev_kv;

/* A paged bf16 KV cache for one layer: the prefix sits in a pool of
 * LUCEV_PAGE_TOKENS-token pages, and block_table maps prefix tokens to pages.
 *   k_pages     : bf16 [n_pages][Hkv][16][d]  keys after RoPE
 *   v_pages     : bf16 [n_pages][Hkv][d][16]  values, dim-major within a page
 *   block_table : DEVICE int32 [ceil(prefix_len / 16)]: the page holding
 *                 prefix tokens 16i .. 16i + 15 (entries are clamped to
 *                 [0, n_pages), so a bad entry cannot address outside the pool)
 * The prefix covered is tokens 0 .. prefix_len - 1, as in lucev_kv.          */
#define LUCEV_PAGE_TOKENS 16
typedef struct {
  const uint16_t* k_pages;
  const uint16_t* v_pages;
  const int32_t* block_table;
  int32_t n_pages;
  int32_t prefix_len;
} lucev_kv_paged;

/* The draft tree, in HOST memory, passed by value.  Node 0 is the root (the
 * last accepted token, not yet in the cache); parent[i] < i.  The library
 * derives depths, RoPE positions (prefix_len + depth) and ancestor masks into
 * kernel arguments, so no host->device copy is needed.  token[i] is node i's
 * drafted token (token[0] is not used by acceptance).                       */
typedef struct {
  int32_t n;
  int32_t parent[LUCEV_MAX_NODES];
  int32_t token[LUCEV_MAX_NODES];
} lucev_tree;

/* Matrix roles for packing (decides the library-private row order). */
#define LUCEV_W_PLAIN 0 /* wo, wd, lm_head */
#define LUCEV_W_QKV 1   /* needs head_dim (rotate-half pairs kept together) */
#define LUCEV_W_GU 2    /* gate and up rows interleaved so SwiGLU pairs meet */

/* ------------------------------------------------------------ helpers */

int lucev_abi_version(void);
const char* lucev_status_str(int status);
/* Thread-local text of the last error on this thread ("" if none). */
const char* lucev_last_error(void);

/* Bytes of the packed layout: n_out * k_in * 9 / 16 (18 B per 32 weights).
 * Returns 0 if n_out % 16 or k_in % 128 is non-zero. */
size_t lucev_q4_packed_bytes(int64_t n_out, int64_t k_in);

/* Pack logical codes q (uint8 [n_out][k_in], values 0..15) and scales d
 * (fp16 bits [n_out][k_in/32]) into `dst`.  HOST pointers.  `kind` is one of
 * LUCEV_W_*; head_dim is read only for LUCEV_W_QKV.  Returns LUCEV_OK,
 * LUCEV_ERR_NULL_ARG, LUCEV_ERR_BAD_SHAPE or LUCEV_ERR_WORKSPACE (dst_bytes
 * too small). */
int lucev_q4_pack(int kind, int32_t head_dim, const uint8_t* q, const uint16_t* d,
                  int64_t n_out, int64_t k_in, void* dst, size_t dst_bytes);

/* Same packing with DEVICE pointers, enqueued on `stream`. */
int lucev_q4_pack_device(int kind, int32_t head_dim, const uint8_t* q, const uint16_t* d,
                         int64_t n_out, int64_t k_in, void* dst, size_t dst_bytes,
                         void* stream);

/* Workspace bytes needed by every entry point below for a tree of up to
 * `n_nodes` nodes against a prefix of up to `prefix_len` tokens.  Returns 0
 * for an unsupported shape. */
size_t lucev_workspace_bytes(const lucev_shape* shape, int32_t n_nodes, int32_t prefix_len);

/* Zero-fill a workspace (once before its first use; no call depends on
 * what an earlier call left in it). */
int lucev_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------ the step */

/* One decoder layer over all tree nodes (RMSNorm, fused QKV projection, RoPE
 * at prefix_len + depth, tree-masked GQA attention over the prefix and each
 * node's ancestors, output projection + residual, RMSNorm, SwiGLU FFN +
 * residual).  The target verifies the whole drafted tree in one forward
 * ("Lucebox Hub", section "Speculative decoding 계층 (DFlash / DDTree /
 * DSpark)"), and that forward reads every weight once for all nodes (same
 * page, section "배경: 어떤 문제를 푸는가", item 1).
 *   resid_io   : fp32 [n][H] residual stream, updated in place
 *   k_tree_out : bf16 [n][Hkv][d] this layer's tree keys after RoPE
 *   v_tree_out : bf16 [n][Hkv][d] this layer's tree values
 * Attention inside uses the workspace; outputs must not alias inputs.
 * Returns LUCEV_OK, LUCEV_ERR_NULL_ARG, LUCEV_ERR_BAD_SHAPE (dims, weight
 * shapes, attention rows), LUCEV_ERR_BAD_TREE, LUCEV_ERR_BAD_KV,
 * LUCEV_ERR_ALIGN, LUCEV_ERR_WORKSPACE, LUCEV_ERR_DEVICE or LUCEV_ERR_HIP. */
int lucev_verify_layer(const lucev_shape* shape, const lucev_layer_w* w, const lucev_tree* tree,
                       const lucev_kv* kv, float* resid_io, uint16_t* k_tree_out,
                       uint16_t* v_tree_out, void* ws, size_t ws_bytes, void* stream);

/* Tree-masked GQA attention alone.  Node i, query head h attends with scale
 * 1/sqrt(d) to all prefix keys of KV head h/(Hq/Hkv) and to the tree keys of
 * i's ancestors and itself: one forward over the tree gives each node what
 * decoding its own root path would ("Lucebox Hub", section "Speculative
 * decoding 계층 (DFlash / DDTree / DSpark)"), and a long context makes the
 * KV prefix the bulk of the bytes (same page, section "KVFlash").
 *   q      : bf16 [n][Hq][d] after RoPE
 *   k_tree : bf16 [n][Hkv][d] after RoPE;  v_tree : bf16 [n][Hkv][d]
 *   out    : bf16 [n][Hq][d]
 * Returns LUCEV_OK, LUCEV_ERR_NULL_ARG, LUCEV_ERR_BAD_SHAPE (dims, or more
 * than LUCEV_MAX_ATTN_ROWS query rows per KV head), LUCEV_ERR_BAD_TREE,
 * LUCEV_ERR_BAD_KV, LUCEV_ERR_ALIGN, LUCEV_ERR_WORKSPACE, LUCEV_ERR_DEVICE or
 * LUCEV_ERR_HIP. */
int lucev_tree_attention(const lucev_shape* shape, const lucev_tree* tree, const lucev_kv* kv,
                         const uint16_t* q, const uint16_t* k_tree, const uint16_t* v_tree,
                         uint16_t* out, void* ws, size_t ws_bytes, void* stream);

/* The same attention on fp32 inputs and output, exactly as lucev_verify_layer
 * runs it inside the step (queries carried at about 16 significant bits in
 * the prefix pass, tree keys and values in fp32):
 *   q      : fp32 [n][Hq][d] after RoPE
 *   k_tree : fp32 [n][Hkv][d] after RoPE;  v_tree : fp32 [n][Hkv][d]
 *   out    : fp32 [n][Hq][d]
 * Returns the codes of lucev_tree_attention. */
int lucev_tree_attention_f32(const lucev_shape* shape, const lucev_tree* tree, const lucev_kv* kv,
                             const float* q, const float* k_tree, const float* v_tree, float* out, void* ws,
                             size_t ws_bytes, void* stream);

/* lucev_tree_attention without a workspace, for callers that cannot allocate
 * device memory or hand the library a buffer (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments,
 * kernels and results as lucev_tree_attention (bit-identical).  Its chunk
 * partials live in one scratch array of LUCEV_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, held until the process ends; a call needs
 * about 256 * n * (n_q_heads / n_kv_heads) * (4 * head_dim + 8) bytes of it
 * (a 22-node tree of 48/8 heads, d = 128: 17.6 MB; 40 nodes: 31.9 MB) and
 * returns LUCEV_ERR_WORKSPACE when that exceeds the array.  Every call on one
 * GPU shares the array: calls that overlap on one GPU (other streams, other
 * host threads) race and must be serialised by the caller.  Nothing in the
 * array needs clearing between calls.  Otherwise returns the codes of
 * lucev_tree_attention. */
#define LUCEV_NOALLOC_SCRATCH_BYTES (32u << 20)
int lucev_tree_attention_noalloc(const lucev_shape* shape, const lucev_tree* tree, const lucev_kv* kv,
                                 const uint16_t* q, const uint16_t* k_tree, const uint16_t* v_tree,
                                 uint16_t* out, void* stream);

/* The same attention over a paged prefix: a pool of 16-token physical blocks
 * and a block table per sequence, which changes layout and allocation only,
 * with no approximation ("Lucebox Hub", section "Paged attention +
 * continuous batching").  Results are bit-identical to lucev_tree_attention
 * on the same keys and values stored contiguously.
 * Requires each prefix chunk a block reads (about prefix_len * Hkv / 256
 * tokens) to span at most 1024 pages.  Returns the codes of
 * lucev_tree_attention; LUCEV_ERR_BAD_KV also for prefix_len < 0, n_pages < 1
 * with a non-empty prefix, or chunks of more than 1024 pages. */
int lucev_tree_attention_paged(const lucev_shape* shape, const lucev_tree* tree,
                               const lucev_kv_paged* kv, const uint16_t* q, const uint16_t* k_tree,
                               const uint16_t* v_tree, uint16_t* out, void* ws, size_t ws_bytes,
                               void* stream);

/* ------------------------------------------------------------ int8 KV prefix */

/* One layer's KV cache held as int8 codes with one fp16 scale per block of 32
 * values: the q8_0 cache type the pages run beside F16 and Q4_0 ("Lucebox
 * Hub", sections "Paged attention + continuous batching" and "설치·사용법"),
 * read here as value = d * code, code in [-127, 127], d = fp16(amax / 127).
 * Keys are blocked along the head dim of each token, values along the tokens
 * of each dim (the cache keeps V dim-major):
 *   k_codes  : int8 [Hkv][capacity][d]        (16-byte aligned)
 *   k_scales : fp16 [Hkv][capacity][d / 32]   (8-byte aligned)
 *   v_codes  : int8 [Hkv][d][capacity]        (16-byte aligned)
 *   v_scales : fp16 [Hkv][d][capacity / 32]   (4-byte aligned)
 * capacity is a multiple of 32; tokens 0 .. prefix_len - 1 are the prefix. */
typedef struct {
  const int8_t* k_codes;
  const uint16_t* k_scales;
  const int8_t* v_codes;
  const uint16_t* v_scales;
  int32_t prefix_len;
  int32_t capacity;
} lucev_kv_q8;

/* Quantise every token (0 .. capacity - 1) of a bf16 cache (lucev_kv layout)
 * into the int8 layout above: per block, amax, d = fp16(amax / 127) from an
 * fp32 division, code = rint(x / d) from an fp32 division (ties to even)
 * clamped to [-127, 127]; a block of zeros gets d = 0.  All pointers DEVICE.
 * Requires src->capacity % 32 == 0.  Returns LUCEV_OK, LUCEV_ERR_NULL_ARG,
 * LUCEV_ERR_BAD_SHAPE, LUCEV_ERR_BAD_KV, LUCEV_ERR_ALIGN, LUCEV_ERR_DEVICE or
 * LUCEV_ERR_HIP. */
int lucev_kv_quantize_q8(const lucev_shape* shape, const lucev_kv* src, int8_t* k_codes, uint16_t* k_scales,
                         int8_t* v_codes, uint16_t* v_scales, void* stream);

/* lucev_tree_attention over an int8 prefix: every prefix key and value enters
 * as the nearest fp16 of d * code (one rounding, within 2^-11 of itself, 16
 * times finer than the int8 step), queries and P as nearest fp16, all
 * products and sums in fp32 (fp16 MFMAs).  Prefix values must lie within the
 * fp16 range (|x| <= 65504).  q, k_tree, v_tree and out as in
 * lucev_tree_attention.  Returns its codes; LUCEV_ERR_BAD_KV also for a
 * capacity that is not a multiple of 32, LUCEV_ERR_ALIGN for the alignments
 * above. */
int lucev_tree_attention_q8(const lucev_shape* shape, const lucev_tree* tree, const lucev_kv_q8* kv,
                            const uint16_t* q, const uint16_t* k_tree, const uint16_t* v_tree, uint16_t* out,
                            void* ws, size_t ws_bytes, void* stream);

/* ----------------------------------------------------------- 4-bit KV prefix */

/* One layer's KV cache held as 4-bit codes with one fp16 scale per block of
 * 32 values: the Q4_0 cache type of the same passages ("Lucebox Hub",
 * sections "Paged attention + continuous batching" and "설치·사용법"), read
 * here as value = d * (q - 8), nibble q in [0, 15] (q = 0 never written),
 * d = fp16(amax / 7).  Blocks as in lucev_kv_q8 (K along the head dim of each
 * token, V along the tokens of each dim); each block's 32 nibbles fill 16
 * bytes, as four little-endian dwords of 8 values each, value e (0..7) of a
 * dword at bits 4 (e / 2) + 16 (e % 2) .. +3 (the order a bit-field insert
 * under an fp16 exponent decodes two at a time):
 *   k_nibbles : [Hkv][capacity][d / 2] bytes   (16-byte aligned)
 *   k_scales  : fp16 [Hkv][capacity][d / 32]   (8-byte aligned)
 *   v_nibbles : [Hkv][d][capacity / 2] bytes   (16-byte aligned)
 *   v_scales  : fp16 [Hkv][d][capacity / 32]   (4-byte aligned)
 * capacity is a multiple of 32; tokens 0 .. prefix_len - 1 are the prefix. */
typedef struct {
  const uint8_t* k_nibbles;
  const uint16_t* k_scales;
  const uint8_t* v_nibbles;
  const uint16_t* v_scales;
  int32_t prefix_len;
  int32_t capacity;
} lucev_kv_q4;

/* Quantise every token (0 .. capacity - 1) of a bf16 cache (lucev_kv layout)
 * into the 4-bit layout above: per block, amax, d = fp16(amax / 7) from an
 * fp32 division, code = rint(x / d) from an fp32 division (ties to even)
 * clamped to [-7, 7], nibble code + 8; a block of zeros gets d = 0 and
 * nibbles 8.  All pointers DEVICE.  Requires src->capacity % 32 == 0.
 * Returns the codes of lucev_kv_quantize_q8. */
int lucev_kv_quantize_q4(const lucev_shape* shape, const lucev_kv* src, uint8_t* k_nibbles, uint16_t* k_scales,
                         uint8_t* v_nibbles, uint16_t* v_scales, void* stream);

/* lucev_tree_attention over a 4-bit prefix: every prefix key and value
 * enters as the nearest fp16 of d * (q - 8), queries and P as nearest fp16,
 * all products and sums in fp32 (fp16 MFMAs), exactly as
 * lucev_tree_attention_q8 does with its codes.  Prefix values must lie within
 * the fp16 range.  Returns the codes of lucev_tree_attention_q8. */
int lucev_tree_attention_q4(const lucev_shape* shape, const lucev_tree* tree, const lucev_kv_q4* kv,
                            const uint16_t* q, const uint16_t* k_tree, const uint16_t* v_tree, uint16_t* out,
                            void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------- the step over a quantised prefix */

/* lucev_verify_layer with the layer's prefix held as int8 (lucev_kv_q8) or
 * 4-bit (lucev_kv_q4) codes: the pages run the target with q8_0 or Q4_0 K/V
 * ("Lucebox Hub", sections "Paged attention + continuous batching" and
 * "설치·사용법").  Everything but the attention's prefix part is
 * lucev_verify_layer's; that part is lucev_tree_attention_q8 / _q4's (prefix
 * keys and values as the nearest fp16 of their dequantised values, q -- the
 * layer's fp32 q -- and P as nearest fp16, fp32 sums), while the tree keys
 * and the merge stay in fp32 as in lucev_verify_layer.  Other arguments,
 * outputs and workspace as lucev_verify_layer; the cache layouts, alignments
 * and capacity % 32 as lucev_tree_attention_q8 / _q4.  Returns the codes of
 * lucev_verify_layer. */
int lucev_verify_layer_q8(const lucev_shape* shape, const lucev_layer_w* w, const lucev_tree* tree,
                          const lucev_kv_q8* kv, float* resid_io, uint16_t* k_tree_out, uint16_t* v_tree_out,
                          void* ws, size_t ws_bytes, void* stream);
int lucev_verify_layer_q4(const lucev_shape* shape, const lucev_layer_w* w, const lucev_tree* tree,
                          const lucev_kv_q4* kv, float* resid_io, uint16_t* k_tree_out, uint16_t* v_tree_out,
                          void* ws, size_t ws_bytes, void* stream);

/* Final RMSNorm, lm_head, greedy token and top1-top2 gap per node (taken on
 * the fp32 logits), then greedy acceptance over the tree: a node is accepted
 * when its parent is accepted and its drafted token equals the parent's
 * greedy token; the path ends at the deepest accepted node (lowest index on
 * ties).  Decoding is greedy at temperature 0 and the tree keeps the longest
 * accepted path ("Lucebox: 추측 디코딩과 전용 커널로 ...", section "Lucebox
 * 설치 및 실행"); the target adapter projects through its lm_head ("Lucebox
 * Hub", section "Speculative decoding 계층 (DFlash / DDTree / DSpark)").
 * All outputs are DEVICE buffers:
 *   resid         : fp32 [n][H] final residual stream (input)
 *   logits_out    : bf16 [n][V] or NULL
 *   argmax_out    : int32 [n]
 *   gap_out       : fp32 [n] or NULL
 *   path_out      : int32 [n]; path_len_out: int32 [1]
 *   committed_out : int32 [n]: accepted drafted tokens along the path, then
 *                   the greedy token at its end (path_len entries)
 * Returns LUCEV_OK, LUCEV_ERR_NULL_ARG, LUCEV_ERR_BAD_SHAPE, LUCEV_ERR_BAD_TREE,
 * LUCEV_ERR_ALIGN, LUCEV_ERR_WORKSPACE, LUCEV_ERR_DEVICE or LUCEV_ERR_HIP. */
int lucev_accept_path(const lucev_shape* shape, const lucev_head_w* w, const lucev_tree* tree,
                      const float* resid, uint16_t* logits_out, int32_t* argmax_out,
                      float* gap_out, int32_t* path_out, int32_t* path_len_out,
                      int32_t* committed_out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------ draft hooks */

/* The target's lm_head over arbitrary hidden rows: final RMSNorm, lm_head,
 * greedy token and top1-top2 gap per row (fp32 logits), with no tree.  The
 * target adapter projects the drafter's hidden states through the target's
 * lm_head ("Lucebox Hub", section "Speculative decoding 계층 (DFlash /
 * DDTree / DSpark)": the adapter's lm_head projection duty).  The other
 * adapter duty, capture of chosen layers' activations, needs no entry point:
 * resid_io after lucev_verify_layer of layer l IS layer l's output, and a
 * caller copies it on the same stream (or inside the same graph).
 *   x          : fp32 [n_rows][H] hidden rows (DEVICE)
 *   logits_out : bf16 [n_rows][V] or NULL
 *   argmax_out : int32 [n_rows];  gap_out: fp32 [n_rows] or NULL
 * 1 <= n_rows <= LUCEV_MAX_NODES; the workspace is sized by
 * lucev_workspace_bytes(shape, n_rows, 0) or larger.  Returns LUCEV_OK,
 * LUCEV_ERR_NULL_ARG, LUCEV_ERR_BAD_SHAPE, LUCEV_ERR_BAD_TREE (n_rows),
 * LUCEV_ERR_ALIGN, LUCEV_ERR_WORKSPACE, LUCEV_ERR_DEVICE or LUCEV_ERR_HIP. */
int lucev_project_logits(const lucev_shape* shape, const lucev_head_w* w, int32_t n_rows,
                         const float* x, uint16_t* logits_out, int32_t* argmax_out,
                         float* gap_out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------ after the step */

#define LUCEV_MAX_COMMIT_LAYERS 64

/* Commit the accepted path into the KV caches, so the next step's prefix is
 * this step's prefix plus the accepted tokens.  The target keeps its KV cache
 * and drops what the tree rejected ("Lucebox Hub", section "Speculative
 * decoding 계층 (DFlash / DDTree / DSpark)": the target adapter's KV
 * snapshot / restore duty); here that is an append of the kept nodes only.
 * Path node path[j] (root first) sits at depth j, so its key was rotated at
 * position prefix_len + j; its key and value rows are written at cache token
 * prefix_len + j of every listed layer.  The caller then advances prefix_len
 * by *path_len.  The bonus token (the greedy token at the path's end) is not
 * in the tree: it is the next step's root.
 *   k_cache, v_cache : HOST arrays of n_layers DEVICE pointers, one layer's
 *                      bf16 cache each (lucev_kv layout, written)
 *   k_tree, v_tree   : HOST arrays of n_layers DEVICE pointers, one layer's
 *                      bf16 [n_nodes][Hkv][d] tree K (after RoPE) / V as
 *                      written by lucev_verify_layer (read)
 *   path, path_len   : DEVICE outputs of lucev_accept_path (int32 [n_nodes],
 *                      int32 [1]), read on the device, so no host round trip
 *                      sits between acceptance and commit
 * Requires 1 <= n_layers <= LUCEV_MAX_COMMIT_LAYERS, 1 <= n_nodes <=
 * LUCEV_MAX_NODES and prefix_len + n_nodes <= capacity (room for the longest
 * path); path entries outside [0, n_nodes) are skipped.  Returns LUCEV_OK,
 * LUCEV_ERR_NULL_ARG, LUCEV_ERR_BAD_SHAPE, LUCEV_ERR_BAD_TREE (n_nodes),
 * LUCEV_ERR_BAD_KV (capacity) or LUCEV_ERR_HIP. */
int lucev_commit_path(const lucev_shape* shape, int32_t n_layers, uint16_t* const* k_cache,
                      uint16_t* const* v_cache, const uint16_t* const* k_tree,
                      const uint16_t* const* v_tree, int32_t prefix_len, int32_t capacity,
                      int32_t n_nodes, const int32_t* path, const int32_t* path_len,
                      void* stream);

/*
 * lucev_set_gemv_max_rows: GEMM operand rows (two per node for the QKV and
 * Wo projections, whose activations travel as fp16 hi + lo rows; one per node
 * for gate/up, down and the lm_head) at or below which the int4 projections take
 * dot products on the vector ALUs (v_dot2_f32_f16) instead of MFMA, for
 * trees too small to make a dense contraction.  Measured on MI355X, MFMA is
 * no slower at any node count (the dot products come within 5 % at one or
 * two operand rows and lose from four on), so the default is 0.  rows in [0, 8], else LUCEV_ERR_BAD_SHAPE.  Process-wide; applies to
 * calls made (and workspaces sized) afterwards, not to captured graphs.
 */
int lucev_set_gemv_max_rows(int32_t rows);

/*
 * Measurement helpers (not part of the verify step).
 *
 * lucev_describe_attention: the kernels the tree attention launches for this
 * shape, tree size and prefix length -- the same plan every attention entry
 * point uses -- as text: each kernel's template, grid and block, the
 * prefix chunk per workgroup and the query row groups (past 16 query tiles
 * per KV head, one workgroup per chunk and group).  variant 0 =
 * lucev_tree_attention (bf16 q),
 * 1 = lucev_tree_attention_f32 and the verify step (fp32 q, split into bf16
 * hi + lo), 2 = lucev_tree_attention_paged, 3 = lucev_tree_attention_q8,
 * 4 = lucev_tree_attention_q4.
 * Writes at most buf_len bytes, NUL-terminated (truncated if longer).
 * Errors as lucev_tree_attention for the shape and tree size
 * (LUCEV_ERR_BAD_SHAPE, LUCEV_ERR_BAD_TREE); LUCEV_ERR_NULL_ARG for a NULL or
 * empty buf.  Host only: enqueues nothing.
 *
 * lucev_stream_read: reads `bytes` of device memory at src once, with
 * non-temporal 16-byte loads spread over every CU, and enqueues nothing else;
 * sink (device, 4 bytes) is written only when the loads' XOR fold hits one
 * fixed value.  Its duration at a given size is the read rate a kernel that
 * streams that many bytes can reach on this device (launch, ramp-up and tail
 * included), the practical ceiling beside the 8 TB/s peak.  src 16-byte
 * aligned and bytes a multiple of 16 (LUCEV_ERR_ALIGN), src and sink non-NULL
 * (LUCEV_ERR_NULL_ARG).
 */
int lucev_describe_attention(const lucev_shape* shape, int32_t n_nodes, int32_t prefix_len, int32_t variant,
                             char* buf, size_t buf_len);
int lucev_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LUCEV_H */
