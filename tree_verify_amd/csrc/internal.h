// Internal interfaces between the C ABI (api.hip) and the kernel files.
#pragma once

#include "common.h"

namespace lucev {

enum { W_PLAIN = 0, W_QKV = 1, W_GU = 2 };  // same values as LUCEV_W_*
enum { EPI_RESID = 0, EPI_SWIGLU = 1, EPI_QKV = 2, EPI_LOGITS = 3 };
enum { A_F16HL = 0, A_F32N = 1 };

// GEMM partition: a flat list of units (4-tile feature group fg, 128-column
// group c), fg-major, split evenly over the blocks (block-level stream-K).
struct GemmPlan {
  int ft, nt, n_tiles, kgroups, fgroups, blocks, tile_floats;
  int64_t units;
};

struct GemmParams {
  int a_mode;               // A_F16HL or A_F32N
  const uint16_t* Xhi;      // A_F16HL: fp16 high / low planes [n_nodes][ldx], x = hi + lo
  const uint16_t* Xlo;
  const float* Xf;          // A_F32N: fp32 residual [n_nodes][ldx]
  const uint16_t* g;        // A_F32N: bf16 RMSNorm gain [k_in]
  const float* ssq;         // A_F32N: row sums of x^2 as [ssq_groups][n_nodes] partials
  int ssq_groups;
  int ldx;
  int n_nodes;
  const uint8_t* wq;        // nibble region of the packed matrix
  const uint16_t* wsc;      // scale region (fp16 bits)
  int64_t n_out, k_in;
  int n_tiles, kgroups, fgroups, blocks;
  int64_t units;
  float* partials;          // [blocks][2][tile]: split-segment partial tiles
  uint32_t* counters;       // [fgroups], zero between calls
  float rms_eps;
};

struct EpiArgs {
  float* resid;             // EPI_RESID: fp32 [n][ld_out], updated in place
  float* ssq_out;           // EPI_RESID: per feature group sum of x_new^2, [fgroups][n], or NULL
  uint16_t* out16;          // bf16 q / logits (may be NULL) / fp16 high plane of SwiGLU m
  uint16_t* out16_lo;       // fp16 low plane of SwiGLU m
  int ld_out;
  uint16_t* k_out;          // EPI_QKV: bf16 [n][Hkv][d]
  uint16_t* v_out;
  float* q32;               // EPI_QKV: fp32 q [n][Hq][d], k and v [n][Hkv][d]
  float* k32;
  float* v32;
  int n_q_heads, n_kv_heads, head_dim;
  f32x4* cand;              // EPI_LOGITS: per (block, node) {best, idx, second, 0}
  int32_t pos[kMaxNodes];
  double inv_freq[kMaxNodes];  // base^(-2j/d), j < d/2
};

GemmPlan plan_gemm(int64_t n_out, int64_t k_in, int n_nodes);
hipError_t launch_gemm(int epi, const GemmParams& p, const EpiArgs& e, hipStream_t s);
hipError_t launch_pack_q4(const uint8_t* q, const uint16_t* d, int64_t n_out, int64_t k_in,
                          int kind, int head_dim, void* dst, hipStream_t s);
void pack_q4_host(const uint8_t* q, const uint16_t* d, int64_t n_out, int64_t k_in, int kind,
                  int head_dim, void* dst);

// ---------------------------------------------------------------- attention

struct AttnPlan {
  int chunk;     // prefix tokens per block (multiple of 64)
  int n_chunks;  // ceil(prefix_len / chunk); 0 when the prefix is empty
  int rows;      // n * (Hq / Hkv) query rows per KV head
  int qpw;       // query tiles (16 rows) per wave
  int waves;     // waves per block
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
};

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
  uint16_t* out;      // [n][Hq][d]: bf16, or the fp16 high plane when out_lo is set
  uint16_t* out_lo;   // fp16 low plane (o = hi + lo) or NULL
};

AttnPlan plan_attention(int n_nodes, int n_q_heads, int n_kv_heads, int head_dim, int prefix_len);
int attention_max_chunks(int n_kv_heads);
hipError_t launch_attention(const AttnPlan& plan, int head_dim, const AttnParams& p,
                            const CombineParams& c, const TreeArgs& t, hipStream_t s);

// ---------------------------------------------------------------- small kernels

hipError_t launch_row_ssq(const float* x, int n, int hidden, float* ssq, hipStream_t s);
hipError_t launch_finalize(const f32x4* cand, int n_cand, const TreeArgs& t, int32_t* argmax,
                           float* gap, int32_t* path, int32_t* path_len, int32_t* committed,
                           hipStream_t s);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

}  // namespace lucev
