// Internal interface between the C-ABI layer (fa_api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Geometry shared by host and device code.
constexpr int kFwdTileRows = 128;  // query rows per tile (4 waves x 32 rows)
constexpr int kFwdBlockN = 64;     // keys per K/V stage in the forward
constexpr int kBwdBlockN = 128;    // keys per backward work item (4 waves x 32 keys)
constexpr int kBwdBlockM = 64;     // query rows per backward step
constexpr int kDqTileRows = 256;   // query rows per dQ work item (deterministic mode)
constexpr int kSchedMaxCost = 8192;  // histogram bins of the longest-first sort
constexpr int kBwdPreBlocks = 8192;  // most workgroups of the backward's pre pass

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int o_f32;           // O is fp32 (strides in fp32 elements), else bf16
  int batch, seqlen_q, seqlen_k, heads;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int total_q;
  int n_qtiles;        // fixed length: work items per (batch, head)
  const int32_t* sched;  // variable length: {count, (seq, tile) pairs...}
  float scale;         // softmax scale
  float scale_log2;    // softmax scale * log2(e)
  // key split (n_split > 1): chunk c of every sequence's keys writes its partial
  // LSE to part_lse[(c*heads + h)*total_q + row] and its partial O (fp32) to
  // part_o[((c*heads + h)*total_q + row)*D]; row counts through the packed or
  // batched query rows (b*seqlen_q + i for fixed length)
  int n_split;
  float* part_lse;
  float* part_o;
  // fp16 copy of V for the PV product, [H, total_k, D] over the packed or batched key
  // rows (b*seqlen_k + j for fixed length), each 64-key tile of a sequence scaled by
  // 2^-e with e = v_exp[h*total_k + first row of the tile] (see vprep_kernel)
  int total_k;
  uint16_t* v16;
  int32_t* v_exp;
};

struct FwdConfig {
  int head_dim;     // 64 or 128
  int q_tiles;      // 1 or 2 query tiles per workgroup
  bool causal;
  bool varlen;
  int poly_per16;   // 0, 2, 4
  int tau;          // 8 or 0
  int key_splits;     // 1, or > 1 for the split forward (q_tiles == 1) + merge
};

// Returns hipSuccess or the launch error.  Grid size is derived from p and cfg.
hipError_t launch_fwd(const FwdParams& p, const FwdConfig& cfg, hipStream_t stream);

// Writes the fp16 copy of V and the per-tile exponents into p.v16 / p.v_exp.
hipError_t launch_fwd_vprep(const FwdParams& p, int head_dim, bool varlen, hipStream_t stream);

// Builds the longest-first list {count, (seq, tile)...} for variable length.
hipError_t launch_fwd_schedule(const int32_t* cu_q, const int32_t* cu_k, int batch, int tile_rows,
                               int block_n, bool causal, int32_t* out, hipStream_t stream);

// Evaluates the forward's software and hardware 2^x on n device values.
hipError_t launch_exp2_probe(const float* x, float* y_poly, float* y_hw, int64_t n, hipStream_t stream);

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int64_t do_sb, do_ss, do_sh;
  int64_t dq_sb, dq_ss, dq_sh;
  int64_t dk_sb, dk_ss, dk_sh;
  int64_t dv_sb, dv_ss, dv_sh;
  int batch, seqlen_q, seqlen_k, heads;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int total_q, total_k;
  int max_seqlen_q, max_seqlen_k;
  float scale;
  float scale_log2;
  bool causal;
  bool varlen;
  bool deterministic;
  bool grad_bf16;
  int head_dim;
  // workspace carve-up
  float* dq_acc;      // [H, total_q, D] fp32 (fixed length: total_q = B*S_q)
  float* dvec;        // [H, total_q] fp32, D_i = sum_d dO_id O_id
  int32_t* sched;     // variable length work list for the key-tile kernel
  // fp16 copies of Q and K for the fp16 products (dS enters dK = dS^T Q and dQ = dS K
  // in fp16, so Q and K must be fp16 there, and S = Q K^T then uses the same copies):
  // Q16 = Q 2^-a, K16 = K 2^-b, [H, total_q, D] and [H, total_k, D]
  uint16_t* q16;
  uint16_t* k16;
  // maxima found by the pre pass (float bit patterns, so unsigned order = value order):
  // stats[0..3] = {max |q|, max |k|, max ||dO_i||^2, max ||v_j||^2}, followed by four
  // per-block slots for each of up to kBwdPreBlocks blocks; the exponents a, b and the
  // dS exponent f are derived from stats[0..3] by every kernel (bwd_exponents)
  uint32_t* stats;
};

// Power-of-two exponents of the backward's fp16 operands, the same in every kernel.
struct BwdExp {
  int a, b, f;    // Q16 = Q 2^-a, K16 = K 2^-b, dS16 = dS 2^-f
};

hipError_t launch_bwd(const BwdParams& p, int phases, hipStream_t stream);  // phases: 1 pre, 2 main, 4 post

}  // namespace fa
