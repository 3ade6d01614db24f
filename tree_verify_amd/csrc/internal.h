// Internal interfaces between the C ABI (api.hip) and the kernel files.
#pragma once

#include "common.h"

namespace lucev {

enum { W_PLAIN = 0, W_QKV = 1, W_GU = 2 };  // same values as LUCEV_W_*
enum { EPI_RESID = 0, EPI_SWIGLU = 1, EPI_QKV = 2, EPI_LOGITS = 3 };

struct GemmPlan {
  int ft, nt, n_tiles, kgroups, fgroups, ksplit, gps, tile_floats;
};

struct GemmParams {
  const uint16_t* X;  // fp16 activations [n_nodes][ldx]
  int ldx;
  int n_nodes;
  const uint8_t* wq;     // nibble region of the packed matrix
  const uint16_t* wsc;   // scale region (fp16 bits)
  int64_t n_out;
  int n_tiles, kgroups, fgroups, ksplit, gps;
  float* partials;       // split-K partial tiles (workspace)
  uint32_t* counters;    // one per feature group, zero between calls
};

struct EpiArgs {
  float* resid;        // EPI_RESID: fp32 [n][ld_out]
  uint16_t* out16;     // q (bf16) / swiglu m (fp16) / logits (bf16, may be NULL)
  int ld_out;
  uint16_t* k_out;     // EPI_QKV: bf16 [n][Hkv][d]
  uint16_t* v_out;
  int n_q_heads, n_kv_heads, head_dim;
  f32x4* cand;         // EPI_LOGITS: per (feature group, node) {best, idx, second, 0}
  int cand_stride;
  int32_t pos[kMaxNodes];
  double inv_freq[kMaxNodes];  // base^(-2j/d), j < d/2
};

GemmPlan plan_gemm(int64_t n_out, int64_t k_in, int n_nodes, int max_ksplit);
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
  const uint16_t* q;   // bf16 [n][Hq][d], after RoPE
  const uint16_t* kc;  // bf16 [Hkv][cap][d]
  const uint16_t* vc;  // bf16 [Hkv][d][cap]
  int cap, prefix_len, chunk, n_chunks;
  int n, n_q_heads, n_kv_heads, rows;
  float scale_log2;    // log2(e) / sqrt(d)
  uint16_t* o_part;    // fp16 [n_chunks][Hkv][rows][d], normalised per chunk
  float* ml_part;      // fp32 [n_chunks][Hkv][rows][2]: (max, sum) in log2 units
};

struct CombineParams {
  const uint16_t* q;
  const uint16_t* k_tree;  // bf16 [n][Hkv][d]
  const uint16_t* v_tree;
  const uint16_t* o_part;
  const float* ml_part;
  int n_chunks, n, n_q_heads, n_kv_heads, rows;
  float scale_log2;
  uint16_t* out;      // [n][Hq][d], bf16 or fp16 bits
  int out_f16;
};

AttnPlan plan_attention(int n_nodes, int n_q_heads, int n_kv_heads, int head_dim, int prefix_len);
int attention_max_chunks(int n_kv_heads);
hipError_t launch_attention(const AttnPlan& plan, int head_dim, const AttnParams& p,
                            const CombineParams& c, const TreeArgs& t, hipStream_t s);

// ---------------------------------------------------------------- small kernels

hipError_t launch_rmsnorm(const float* x, int n, int hidden, const uint16_t* g, float eps,
                          uint16_t* out_f16, int ld_out, hipStream_t s);
hipError_t launch_finalize(const f32x4* cand, int n_fg, int cand_stride, const TreeArgs& t,
                           int32_t* argmax, float* gap, int32_t* path, int32_t* path_len,
                           int32_t* committed, uint32_t* counter, hipStream_t s);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

}  // namespace lucev
