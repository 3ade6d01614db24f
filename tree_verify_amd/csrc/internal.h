// Internal interfaces between the C ABI (api.hip) and the kernel files.
#pragma once

#include "common.h"

namespace lucev {

enum { W_PLAIN = 0, W_QKV = 1, W_GU = 2 };  // same values as LUCEV_W_*

// GEMM partition: blocks of kGemmWaves waves own panels of kGemmWaves *
// kGemmFT 16-row tiles; the flat list of units (panel, one or two 128-column
// groups), panel-major, is split evenly over the blocks (block-level
// stream-K).
#ifndef LUCEV_GEMM_WAVES
#define LUCEV_GEMM_WAVES 8
#endif
#ifndef LUCEV_GEMM_FT
#define LUCEV_GEMM_FT 2
#endif
#ifndef LUCEV_GEMM_BPC
#define LUCEV_GEMM_BPC 1
#endif
constexpr int kGemmWaves = LUCEV_GEMM_WAVES;     // waves per block
constexpr int kGemmFT = LUCEV_GEMM_FT;           // 16-row tiles per wave
constexpr int kGemmBlocksPerCU = LUCEV_GEMM_BPC;  // grid = 256 CUs x this (at most)
// What the GEMM's scheduling fences let the compiler move across them (the
// sched_barrier mask): all but the vector-memory loads they pin in place.
#ifndef LUCEV_GEMM_SCHED_MASK
#define LUCEV_GEMM_SCHED_MASK 0x78F
#endif
constexpr int kGemmSchedMask = LUCEV_GEMM_SCHED_MASK;

struct GemmPlan {
  int ft, ntx, ug, n_tiles, kgroups, panels, blocks, tile_floats;
  int vr;      // dot-product path: operand rows it covers (0: MFMA)
  int tile_n;  // nodes per partial tile
  int64_t units;
  int c_max;  // most blocks sharing one panel (partial-tile slots per panel)
};

// Blocks take contiguous ranges of the flat unit list [0, U): block b starts
// at floor(b U / B), so range lengths differ by at most one unit (B <= U).
__host__ __device__ inline int64_t range_start(int b, int64_t U, int B) {
  return (int64_t)b * U / B;
}
// the block whose range holds unit u: the largest b with floor(b U / B) <= u
__host__ __device__ inline int block_of_unit(int64_t u, int64_t U, int B) {
  return (int)(((u + 1) * B - 1) / U);
}

// Where a GEMM left its partial tiles: panel p's
// contributors are blocks bf..bl (bf = block_of_unit(p * gu), bl =
// block_of_unit(p * gu + gu - 1)); contributor c = b - bf wrote fp32
// [tile_n][tile_f] at part + (p * c_max + c) * tile_n * tile_f.  Output
// feature f of the GEMM is panel f / tile_f, column f % tile_f.
struct SplitOut {
  const float* part;
  int64_t units;
  int blocks, gu, c_max, tile_f, tile_n, panels;
};

struct GemmParams {
  const uint16_t* X;        // fp16 [2 * n_nodes][k_in]: row 2i = hi(x_i), row 2i+1 = lo(x_i)
                            // (the non-exact kernel reads the hi rows only)
  int n_nodes;
  const uint8_t* wq;        // nibble region of the packed matrix
  const uint16_t* wsc;      // scale region (fp16 bits)
  int64_t n_out, k_in;
  int n_tiles, kgroups, panels, blocks;
  int64_t units;
  float* partials;          // per-block partial tiles (see SplitOut)
  int c_max;                // partial-tile slots per panel
  int ug;                   // 128-column groups per unit (the plan's)
  int ft;                   // 16-row tiles per wave (the plan's)
  int vr;                   // operand rows of the dot-product path, 0 for MFMA (the plan's)
};

// Arguments of the QKV consumer (RoPE, q/k/v outputs).
struct EpiArgs {
  uint16_t* out16;          // bf16 q, may be NULL
  uint16_t* k_out;          // QKV consumer: bf16 [n][Hkv][d]
  uint16_t* v_out;
  float* q32;               // QKV consumer: fp32 q [n][Hq][d], k and v [n][Hkv][d]
  float* k32;
  float* v32;
  int n_q_heads, n_kv_heads, head_dim;
  int32_t pos[kMaxNodes];
  double inv_freq[kMaxNodes];  // base^(-2j/d), j < d/2
};

// 16-row MFMA tiles of the operand: the 2n hi/lo rows (exact projections) or
// the n hi rows (gate/up, down)
int gemm_ntx(int n_nodes, bool exact);
int gemm_ug(int kgroups, int ntx, int vr);  // 128-column groups per unit
// tiles per wave: fewer when many node tiles already fill the registers
constexpr int gemm_ft_for(int ntx) { return ntx <= 4 ? kGemmFT : (kGemmFT > 1 ? kGemmFT / 2 : 1); }
// A matrix whose wide plan (gemm_ft_for tiles per wave, gemm_ug groups per
// unit) gives fewer units than kGemmNarrowUnits per block takes one tile per
// wave and one column group per unit (four times the units, so the blocks'
// shares even out); one with fewer than kGemmMidUnits takes one tile per wave
// and keeps its column groups (twice the units).
constexpr int kGemmNarrowUnits = 4;
constexpr int kGemmMidUnits = 12;
// Most operand rows (hi and lo rows of the exact projections, hi rows of the
// others) that take the VALU dot-product path instead of MFMA: 0 by default
// (MFMA measured no slower at any node count), at most 8 (lucev_set_gemv_max_rows).
extern int g_gemv_max_rows;
int gemm_vr(int n_nodes, bool exact);
GemmPlan plan_gemm(int64_t n_out, int64_t k_in, int n_nodes, bool exact);
// Every block writes its share of each panel it touches as a partial tile;
// a consumer kernel sums them.  exact: weights enter exactly (QKV, Wo,
// lm_head), else rounded once to fp16.
hipError_t launch_gemm(bool exact, const GemmParams& p, hipStream_t s);
hipError_t launch_pack_q4(const uint8_t* q, const uint16_t* d, int64_t n_out, int64_t k_in,
                          int kind, int head_dim, void* dst, hipStream_t s);
void pack_q4_host(const uint8_t* q, const uint16_t* d, int64_t n_out, int64_t k_in, int kind,
                  int head_dim, void* dst);

// ---------------------------------------------------------------- attention

struct AttnPlan {
  int chunk;     // prefix tokens per block (multiple of 64)
  int n_chunks;  // ceil(prefix_len / chunk); 0 when the prefix is empty
  int rows;      // n * (Hq / Hkv) query rows per KV head
  int roww;      // row waves per block (4 or 8)
  int qpw;       // query tiles (16 rows) per row wave
  int waves;     // waves per block (row waves + 4 quarter waves when split)
  bool split;    // the ragged last query tile is shared by four waves (by key quarter)
};

struct AttnParams {
  const uint16_t* q;   // bf16 [n][Hq][d], after RoPE (used when q32 is NULL)
  const float* q32;    // fp32 [n][Hq][d] or NULL
  const uint16_t* kc;  // bf16 [Hkv][cap][d]
  const uint16_t* vc;  // bf16 [Hkv][d][cap]
  int cap, prefix_len, chunk, n_chunks;
  int n, n_q_heads, n_kv_heads, rows;
  float scale_log2;    // log2(e) / sqrt(d)
  float* o_part;       // fp32 [n_chunks][Hkv][rows][d], normalised per chunk
  float* ml_part;      // fp32 [n_chunks][Hkv][rows][2]: (max, sum) in log2 units
  const int32_t* table;  // paged cache: page of each 16 prefix tokens, or NULL (contiguous)
  int n_phys;            // pages in the pool (paged cache)
  // quantised cache (attention_kvq.hip): int8 codes or packed nibbles and fp16 scales, K blocked along the
  // head dim of a token, V along the tokens of a dim
  const int8_t* kc8;     // [Hkv][cap][d]
  const uint16_t* ks16;  // [Hkv][cap][d / 32]
  const int8_t* vc8;     // [Hkv][d][cap]
  const uint16_t* vs16;  // [Hkv][d][cap / 32]
  int row_groups;        // row groups per (chunk, KV head), set by the partial kernels' launches
  int group_tiles;       // query tiles per row group
};
constexpr int kPageTokens = 16;
constexpr int kMaxChunkPagesHost = 1024;  // pages of one block's prefix chunk

struct CombineParams {
  const uint16_t* q;       // bf16 inputs, used when the fp32 ones are NULL
  const uint16_t* k_tree;  // bf16 [n][Hkv][d]
  const uint16_t* v_tree;
  const float* q32;        // fp32 q / tree K / tree V or NULL
  const float* k32;
  const float* v32;
  const float* o_part;
  const float* ml_part;
  int n_chunks, n, n_q_heads, n_kv_heads, rows;
  float scale_log2;
  uint16_t* out;      // bf16 [n][Hq][d], or fp16 hi/lo rows [2n][Hq * d] when out_hilo
  int out_hilo;
  float* out32;       // fp32 [n][Hq][d] instead of `out`, when not NULL
};

// Every query row of a KV head lives in one block of the partial kernel: at
// most 8 row waves x 4 tiles x 16 rows.
constexpr int kMaxAttnRows = 512;
// compute units of the current device (256 on MI355X; that figure when no
// device can be queried), cached per device: grids and prefix chunks are
// sized to it
int device_cu_count();
AttnPlan plan_attention(int n_nodes, int n_q_heads, int n_kv_heads, int head_dim, int prefix_len);
int attention_max_chunks(int n_kv_heads);
hipError_t launch_attention(const AttnPlan& plan, int head_dim, const AttnParams& p,
                            const CombineParams& c, const TreeArgs& t, hipStream_t s);
// the same over an int8 prefix (p.kc8 ..), and the merge both end with
hipError_t launch_attention_q8(const AttnPlan& plan, int head_dim, int bits, const AttnParams& p,
                               const CombineParams& c, const TreeArgs& t, hipStream_t s);
hipError_t launch_combine(int head_dim, const CombineParams& c, const TreeArgs& t, hipStream_t s);
// the kernels, grids and blocks the attention launches for a plan (snprintf semantics)
int describe_attention(const AttnPlan& plan, int head_dim, int n_kv_heads, int combine_blocks, bool fp32_q,
                       bool paged, char* buf, size_t len);
int describe_attention_q8(const AttnPlan& plan, int head_dim, int n_kv_heads, int combine_blocks, int bits,
                          char* buf, size_t len);
// one non-temporal read of `bytes` (multiple of 16) over the whole device
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s);
// int8 block-32 quantisation of a bf16 cache's first cap tokens
hipError_t launch_quantize_q8(const uint16_t* kc, const uint16_t* vc, int hkv, int cap, int d, int8_t* k_codes,
                              uint16_t* k_scales, int8_t* v_codes, uint16_t* v_scales, hipStream_t s);
// 4-bit block-32 quantisation (nibbles packed two to a byte)
hipError_t launch_quantize_q4(const uint16_t* kc, const uint16_t* vc, int hkv, int cap, int d, uint8_t* k_nib,
                              uint16_t* k_scales, uint8_t* v_nib, uint16_t* v_scales, hipStream_t s);

// ---------------------------------------------------------------- small kernels

// ---------------------------------------------------------------- split-K consumers
// Each sums a GEMM's partial tiles in contributor order and applies the
// projection's epilogue.
SplitOut split_out(const GemmPlan& g, const float* part);
// QKV: RoPE (rotate-half pairs sit 8 rows apart in one tile) -> fp32 q/k/v
// and bf16 tree K/V
hipError_t launch_qkv_finish(const SplitOut& so, const EpiArgs& e, int n, hipStream_t s);
// gate/up: silu(gate) * up -> fp16 rows 2i of [2n][ffn] (hi rows; the down
// projection reads no lo rows)
hipError_t launch_swiglu_finish(const SplitOut& so, uint16_t* m, int ffn, int n, hipStream_t s);
// residual: resid[n][hidden] += y
hipError_t launch_resid_finish(const SplitOut& so, float* resid, int hidden, int n, hipStream_t s);
// lm_head: bf16 logits [n][vocab] (if logits is not NULL) and each panel's
// top-2 per node, cand[panel][node] = {best, index bits, second, 0}
hipError_t launch_logits_finish(const SplitOut& so, uint16_t* logits, int64_t vocab, f32x4* cand, int n,
                                hipStream_t s);

// RMSNorm of each row into the GEMM operand: u = x / sqrt(mean(x^2) + eps) * g
// as fp16 hi/lo rows [2n][hidden]
hipError_t launch_norm_hilo(const float* x, int n, int hidden, const uint16_t* g, float eps,
                            uint16_t* out, bool write_lo, hipStream_t s);
hipError_t launch_finalize(const f32x4* cand, int n_cand, const TreeArgs& t, int32_t* argmax,
                           float* gap, int32_t* path, int32_t* path_len, int32_t* committed,
                           hipStream_t s);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

// accepted-path commit into the KV caches of up to kMaxCommitLayers layers
constexpr int kMaxCommitLayers = 64;
struct CommitArgs {
  uint16_t* kc[kMaxCommitLayers];
  uint16_t* vc[kMaxCommitLayers];
  const uint16_t* kt[kMaxCommitLayers];
  const uint16_t* vt[kMaxCommitLayers];
  const int32_t* path;
  const int32_t* path_len;
  int n_layers, n, prefix_len, cap, n_kv_heads, head_dim;
};
hipError_t launch_commit(const CommitArgs& a, hipStream_t s);

}  // namespace lucev
