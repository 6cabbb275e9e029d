// Backward pass of exact tiled attention for gfx950.
//
// The pages name a backward pass that works from the saved log-sum-exp, adds dQ
// contributions with global atomic adds, and offers a deterministic mode
// (fdeinterviews.com FA4 summary, "Paired-CTA backward pass" bullet and features
// paragraph); the gradient itself is the textbook one of softmax attention:
//   P  = exp(scale*QK^T - LSE)         (recomputed, never stored)
//   dV = P^T dO
//   dP = dO V^T,  D_i = sum_d dO_id O_id,  dS = P o (dP - D)
//   dK = scale * dS^T Q,   dQ = scale * dS K
//
// Kernels (all on the caller's stream):
//   bwd_pre:  D_i for every row and head; the maxima behind the fp16 exponents;
//             zeroes the fp32 dQ accumulator.  bwd_convert then writes Q16 and K16.
//   bwd_kv:   one workgroup per block of 128 keys (4 waves x 32 keys) keeps dK and
//             dV in registers and walks the query tiles of 64 rows that can see
//             its keys.  Atomic mode: dS goes through LDS (transposed by the
//             transpose reads) and each wave adds its share of dQ with fp32
//             global atomics.
//   bwd_dq:   deterministic mode only: one workgroup per 128 query rows keeps dQ
//             in registers and walks the key tiles (recomputing P and dP), so dQ
//             is reduced in a fixed order with no atomics.
//   bwd_post: atomic mode: copies the scaled fp32 accumulator into dQ's layout and
//             dtype.
// dS enters the dQ and dK products in fp16 (11 significant bits; bf16's 8 would leave
// up to ~8e-3 of error on config 5's gradients), so Q and K enter those products --
// and, to share one copy, S = Q K^T -- as exact fp16 copies made by the pre phase.
// Three power-of-two exponents keep every fp16 operand in range: Q16 = Q 2^-a and
// K16 = K 2^-b from the largest |q| and |k|, dS16 = dS 2^-f from the bound
// |dS_ij| <= scale |dO_i . (v_j - O_i)| <= 2 scale max_i ||dO_i|| max_j ||v_j||;
// S picks up 2^(a+b) in the exponent's multiplier and dK, dQ are scaled back by
// 2^(f+a), 2^(f+b) when written.  dP = dO V^T and dV = P^T dO stay BF16.
#include <algorithm>

#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

constexpr float kLog2e = 1.4426950408889634f;

// Per (sequence, head) view used by the backward kernels.
struct BwdSeq {
  int Lq, Lk;
  int64_t qoff, koff, voff, ooff, dooff, dqoff, dkoff, dvoff;  // element offsets
  int64_t lseoff;   // offset of row 0 in the LSE array
  int64_t rowbase;  // row index of row 0 in the [H, total_q] row-term arrays (and Q16)
  int64_t krowbase; // row index of key 0 in the [H, total_k] rows of K16
};

__device__ __forceinline__ BwdSeq bwd_seq(const BwdParams& p, int b, int h) {
  BwdSeq s;
  if (p.varlen) {
    const int sq = p.cu_q[b], sk = p.cu_k[b];
    s.Lq = p.cu_q[b + 1] - sq;
    s.Lk = p.cu_k[b + 1] - sk;
    s.qoff = sq * p.q_ss + h * p.q_sh;
    s.ooff = sq * p.o_ss + h * p.o_sh;
    s.dooff = sq * p.do_ss + h * p.do_sh;
    s.dqoff = sq * p.dq_ss + h * p.dq_sh;
    s.koff = sk * p.k_ss + h * p.k_sh;
    s.voff = sk * p.v_ss + h * p.v_sh;
    s.dkoff = sk * p.dk_ss + h * p.dk_sh;
    s.dvoff = sk * p.dv_ss + h * p.dv_sh;
    s.lseoff = (int64_t)h * p.total_q + sq;
    s.rowbase = (int64_t)h * p.total_q + sq;
    s.krowbase = (int64_t)h * p.total_k + sk;
  } else {
    s.Lq = p.seqlen_q;
    s.Lk = p.seqlen_k;
    s.qoff = b * p.q_sb + h * p.q_sh;
    s.ooff = b * p.o_sb + h * p.o_sh;
    s.dooff = b * p.do_sb + h * p.do_sh;
    s.dqoff = b * p.dq_sb + h * p.dq_sh;
    s.koff = b * p.k_sb + h * p.k_sh;
    s.voff = b * p.v_sb + h * p.v_sh;
    s.dkoff = b * p.dk_sb + h * p.dk_sh;
    s.dvoff = b * p.dv_sb + h * p.dv_sh;
    s.lseoff = ((int64_t)b * p.heads + h) * p.seqlen_q;
    s.rowbase = (int64_t)h * p.total_q + (int64_t)b * p.seqlen_q;
    s.krowbase = (int64_t)h * p.total_k + (int64_t)b * p.seqlen_k;
  }
  return s;
}

// floor(log2 x) of a non-negative float given by its bits; -127 for 0
__device__ __forceinline__ int exp_of(uint32_t bits) { return (int)((bits >> 23) & 0xFFu) - 127; }

__device__ __forceinline__ float pow2f(int e) { return __int_as_float((127 + e) << 23); }  // |e| <= 126

// The fp16 exponents from the pre pass's maxima: the largest |q| (|k|) lands in
// [2^14, 2^15) of Q16 (K16), and the dS bound below 2^15, so nothing can overflow
// fp16 (largest 65504) and only values 2^28 below the largest become subnormal.
__device__ __forceinline__ BwdExp bwd_exponents(const BwdParams& p) {
  const FA_CONST uint32_t* st = (const FA_CONST uint32_t*)p.stats;
  BwdExp e;
  e.a = min(max(exp_of(st[0]) - 14, -100), 100);
  e.b = min(max(exp_of(st[1]) - 14, -100), 100);
  const float bound = 2.0f * p.scale * __builtin_sqrtf(__uint_as_float(st[2])) * __builtin_sqrtf(__uint_as_float(st[3]));
  e.f = min(max(exp_of(__float_as_uint(bound)) - 14, -100), 100);
  e.a = __builtin_amdgcn_readfirstlane(e.a);
  e.b = __builtin_amdgcn_readfirstlane(e.b);
  e.f = __builtin_amdgcn_readfirstlane(e.f);
  return e;
}

// stats[4 + 4g + i] holds block g's maximum of quantity i; one workgroup reduces them
// into stats[0..3] (every block of the pre pass writes its four slots, so nothing
// needs clearing between calls)
__global__ __launch_bounds__(1024) void bwd_reduce_stats_kernel(uint32_t* stats, int blocks) {
  __shared__ uint32_t red[16][4];
  uint32_t m[4] = {0u, 0u, 0u, 0u};
  for (int g = threadIdx.x; g < blocks; g += 1024)
#pragma unroll
    for (int i = 0; i < 4; ++i) m[i] = max(m[i], stats[4 + 4 * g + i]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m[i] = max(m[i], (uint32_t)__shfl_xor((int)m[i], o, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6][i] = m[i];
  }
  __syncthreads();
  if (threadIdx.x < 4) {
    uint32_t r = 0;
    for (int w = 0; w < 16; ++w) r = max(r, red[w][threadIdx.x]);
    stats[threadIdx.x] = r;
  }
}

// Largest bf16 magnitude among 8 values, as float bits (ordered like the values).
__device__ __forceinline__ uint32_t max_mag8(u32x4 v) {
  uint32_t m = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) m = max(m, max(v[w] & 0x7FFFu, (v[w] >> 16) & 0x7FFFu));
  return m << 16;
}

__device__ __forceinline__ float sumsq8(u32x4 v) {
  float acc = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    acc = __builtin_fmaf(bf16_lo(v[w]), bf16_lo(v[w]), acc);
    acc = __builtin_fmaf(bf16_hi(v[w]), bf16_hi(v[w]), acc);
  }
  return acc;
}

// Block-wide maximum of one value per thread (256 threads), written by thread 0.
__device__ __forceinline__ void block_max_store(uint32_t v, uint32_t* dst, uint32_t* lds4) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, m, 64));
  if ((threadIdx.x & 63) == 0) lds4[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) *dst = max(max(lds4[0], lds4[1]), max(lds4[2], lds4[3]));
  __syncthreads();
}

__device__ __forceinline__ uint32_t rows_bytes(int rows, int64_t stride_elems, int row_bytes) {
  return rows > 0 ? (uint32_t)(rows - 1) * (uint32_t)(stride_elems * 2) + (uint32_t)row_bytes : 0u;
}

// ---------------------------------------------------------------------------
// bwd_pre: D_i = sum_d dO_id O_id (fp32), each block's maxima behind the fp16
// exponents (|q|, |k|, ||dO_i||^2, ||v_j||^2, reduced afterwards by bwd_reduce_stats)
// and zeroing of the dQ accumulator.  16-byte chunks: D/8 lanes per (row, head), reduced
// with xor shuffles.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p, int zero_acc) {
  constexpr int CPR = D / 8;  // chunks per row
  __shared__ uint32_t red[4];
  const int64_t total_rows = (int64_t)p.total_q * p.heads;
  const int64_t total_krows = (int64_t)p.total_k * p.heads;
  const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  // element offset of (row, head) in a [B,S,H,D] / [T,H,D] tensor; row counts the
  // packed or batched rows (b * seqlen + s for fixed length)
  auto offs = [&](int64_t row, int h, int64_t sb, int64_t ss, int64_t sh, int seqlen) {
    if (p.varlen) return row * ss + h * sh;
    const int64_t b = row / seqlen, t = row - b * seqlen;
    return b * sb + t * ss + h * sh;
  };
  float do2 = 0.0f;
  uint32_t qmax = 0;
  // loops sized to a whole number of rows per pass, so the xor reductions see full rows
  for (int64_t w = tid; w < ((total_rows * CPR + 63) / 64) * 64; w += nthreads) {
    const int64_t rh = w / CPR;
    const int chunk = (int)(w - rh * CPR);
    float acc = 0.0f, sq = 0.0f;
    bool live = rh < total_rows;
    int h = 0;
    int64_t row = 0;
    if (live) {
      // rows in memory order (the head inside the row), so that a wave reads contiguous bytes
      row = rh / p.heads;
      h = (int)(rh - row * p.heads);
      const u32x4 ov = *(const u32x4*)((const uint16_t*)p.o + offs(row, h, p.o_sb, p.o_ss, p.o_sh, p.seqlen_q) + chunk * 8);
      const u32x4 dv = *(const u32x4*)((const uint16_t*)p.dout + offs(row, h, p.do_sb, p.do_ss, p.do_sh, p.seqlen_q) + chunk * 8);
      const u32x4 qv = *(const u32x4*)((const uint16_t*)p.q + offs(row, h, p.q_sb, p.q_ss, p.q_sh, p.seqlen_q) + chunk * 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc = __builtin_fmaf(bf16_lo(ov[j]), bf16_lo(dv[j]), acc);
        acc = __builtin_fmaf(bf16_hi(ov[j]), bf16_hi(dv[j]), acc);
      }
      sq = sumsq8(dv);
      qmax = max(qmax, max_mag8(qv));
    }
#pragma unroll
    for (int m = CPR / 2; m >= 1; m >>= 1) {
      acc += __shfl_xor(acc, m, CPR);
      sq += __shfl_xor(sq, m, CPR);
    }
    if (live && chunk == 0) p.dvec[(int64_t)h * p.total_q + row] = acc;
    if (live) do2 = fmaxf(do2, sq);
  }
  uint32_t kmax = 0;
  float v2 = 0.0f;
  for (int64_t w = tid; w < ((total_krows * CPR + 63) / 64) * 64; w += nthreads) {
    const int64_t rh = w / CPR;
    const int chunk = (int)(w - rh * CPR);
    float sq = 0.0f;
    const bool live = rh < total_krows;
    if (live) {
      const int64_t row = rh / p.heads;
      const int h = (int)(rh - row * p.heads);
      const u32x4 kv = *(const u32x4*)((const uint16_t*)p.k + offs(row, h, p.k_sb, p.k_ss, p.k_sh, p.seqlen_k) + chunk * 8);
      const u32x4 vv = *(const u32x4*)((const uint16_t*)p.v + offs(row, h, p.v_sb, p.v_ss, p.v_sh, p.seqlen_k) + chunk * 8);
      kmax = max(kmax, max_mag8(kv));
      sq = sumsq8(vv);
    }
#pragma unroll
    for (int m = CPR / 2; m >= 1; m >>= 1) sq += __shfl_xor(sq, m, CPR);
    if (live) v2 = fmaxf(v2, sq);
  }
  uint32_t* mine = p.stats + 4 + 4 * blockIdx.x;
  block_max_store(qmax, mine + 0, red);
  block_max_store(kmax, mine + 1, red);
  block_max_store(__float_as_uint(do2), mine + 2, red);
  block_max_store(__float_as_uint(v2), mine + 3, red);
  if (zero_acc) {
    float4* acc4 = (float4*)p.dq_acc;
    const int64_t n4 = total_rows * D / 4;
    for (int64_t i = tid; i < n4; i += nthreads) acc4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// ---------------------------------------------------------------------------
// bwd_convert: Q16 = Q 2^-a and K16 = K 2^-b in [H, rows, D] layout (exact: a bf16 value
// has 8 significant bits and the fp16 copy 11, and the scaled values stay in fp16's
// normal range down to 2^-28 of the largest).
template <int D>
__global__ __launch_bounds__(256) void bwd_convert_kernel(BwdParams p) {
  constexpr int CPR = D / 8;
  const BwdExp ex = bwd_exponents(p);
  const float sa = pow2f(-ex.a), sb = pow2f(-ex.b);
  const int64_t nq = (int64_t)p.total_q * p.heads * CPR, nk = (int64_t)p.total_k * p.heads * CPR;
  const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < nq + nk; w += nthreads) {
    const bool isq = w < nq;
    const int64_t ww = isq ? w : w - nq;
    const int64_t rh = ww / CPR;  // row of the [H, rows] layout
    const int chunk = (int)(ww - rh * CPR);
    const int rows = isq ? p.total_q : p.total_k;
    const int h = (int)(rh / rows);
    const int64_t row = rh - (int64_t)h * rows;
    int64_t off;
    if (p.varlen) {
      off = isq ? row * p.q_ss + h * p.q_sh : row * p.k_ss + h * p.k_sh;
    } else {
      const int seqlen = isq ? p.seqlen_q : p.seqlen_k;
      const int64_t b = row / seqlen, t = row - b * seqlen;
      off = isq ? b * p.q_sb + t * p.q_ss + h * p.q_sh : b * p.k_sb + t * p.k_ss + h * p.k_sh;
    }
    const u32x4 v = *(const u32x4*)((const uint16_t*)(isq ? p.q : p.k) + off + chunk * 8);
    const float sc = isq ? sa : sb;
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack_f16(bf16_lo(v[j]) * sc, bf16_hi(v[j]) * sc);
    *(u32x4*)((isq ? p.q16 : p.k16) + rh * D + chunk * 8) = o;
  }
}

// ---------------------------------------------------------------------------
// bwd_post: dQ (given layout and dtype) <- fp32 accumulator times 2^(f+b).
template <int D>
__global__ __launch_bounds__(256) void bwd_post_kernel(BwdParams p) {
  const BwdExp ex = bwd_exponents(p);
  const float qs = pow2f(ex.f + ex.b);  // the accumulator holds dQ 2^-(f+b)
  const int64_t total = (int64_t)p.total_q * p.heads * (D / 4);
  const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += nthreads) {
    const int64_t rh = i / (D / 4);
    const int c4 = (int)(i - rh * (D / 4));
    const int h = (int)(rh / p.total_q);
    const int64_t row = rh - (int64_t)h * p.total_q;
    int64_t base;
    if (p.varlen) {
      base = row * p.dq_ss + h * p.dq_sh;
    } else {
      const int64_t b = row / p.seqlen_q, s = row - b * p.seqlen_q;
      base = b * p.dq_sb + s * p.dq_ss + h * p.dq_sh;
    }
    float4 v = ((const float4*)p.dq_acc)[i];
    v.x *= qs;
    v.y *= qs;
    v.z *= qs;
    v.w *= qs;
    if (p.grad_bf16) {
      u32x2 w = {pack_bf16(v.x, v.y), pack_bf16(v.z, v.w)};
      *(u32x2*)((uint16_t*)p.dq + base + c4 * 4) = w;
    } else {
      *(float4*)((float*)p.dq + base + c4 * 4) = v;
    }
  }
}

// Store 4 consecutive gradient values (fp32 or bf16) through a buffer resource.
__device__ __forceinline__ void store_grad4(rsrc_t r, uint32_t byte_off_f32, uint32_t byte_off_bf16, bool bf16,
                                            float a, float b, float c, float d) {
  if (bf16) {
    buf_store8(r, byte_off_bf16, u32x2{pack_bf16(a, b), pack_bf16(c, d)});
  } else {
    buf_store16(r, byte_off_f32, u32x4{__float_as_uint(a), __float_as_uint(b), __float_as_uint(c), __float_as_uint(d)});
  }
}

// ---------------------------------------------------------------------------
// bwd_kv: dK, dV (and atomic dQ) for one block of 128 keys.
//
// Eight waves, two per SIMD: wave w owns the 32 keys k_blk0 + 32*(w&3) + (lane&31)
// and, of every 64-row query step, the 32-row half w>>2.  The two waves of a SIMD
// therefore work on the same keys with independent rows, which lets the hardware
// overlap one wave's softmax arithmetic with the other's matrix products; each keeps
// a partial dK^T/dV^T that is summed through LDS at the end.  K and V stay in LDS
// (row reads feed S = Q K^T and dP = dO V^T; transpose reads feed dQ = dS K).
//
// Per step and wave:
//   S = Q16 K16^T (fp16), dP = dO V^T (bf16)   (C layout: lane = key, registers = 16 rows)
//   P = 2^(S*c 2^(a+b) - LSE*log2 e),  dS16 = scale 2^-f P (dP - D)  (fp16)
//   dV^T += dO^T P (bf16),  dK^T += Q16^T dS16 (fp16)   (A operands by transpose reads)
// Atomic mode: dS16^T goes to LDS; after a barrier each wave computes one 32x32 block
// of dQ 2^-(f+b) = dS16 K16 and adds it with fp32 buffer atomics (rows past the end
// are dropped by the buffer range check).
//
// The Q/dO stage is double-buffered in deterministic mode (the next step streams in
// while the current one is used).  In atomic mode the dS' staging leaves room for a
// single stage only: its refill is issued after the second barrier (once every wave
// has finished reading it) and overlaps the dQ part.
//
// dS16^T LDS layout: [128 keys][64 queries] fp16, 128-byte rows of sixteen 8-byte
// granules; granule g of row r is stored at g ^ ds_swizzle(r), which keeps both the
// 32-row column writes and the 4-row transpose reads free of bank conflicts.
__device__ __forceinline__ int ds_swizzle(int row) { return (((row >> 1) & 3) << 2) | ((row >> 3) & 3); }

template <int D, bool CAUSAL, bool VARLEN, bool DQ_ATOMIC>
__global__ __launch_bounds__(512) void bwd_kv_kernel(BwdParams p) {
  constexpr int BM = kBwdBlockM;    // query rows per step (two 32-row halves)
  constexpr int BNK = kBwdBlockN;   // keys per workgroup (four 32-key groups)
  constexpr int ROWB = D * 2;
  constexpr int QT_BYTES = BM * ROWB;
  constexpr int STAGE = 2 * QT_BYTES + 2 * BM * 4;  // Q, dO, LSE*log2e, scale*D
  constexpr int KT_BYTES = BNK * ROWB;
  constexpr int DS_ROWB = BM * 2;                   // one key row of dS^T
  constexpr int DS_BYTES = DQ_ATOMIC ? BNK * DS_ROWB : 0;
  constexpr int SLOTS = D / 8, NDS = D / 16, NDB = D / 32;
  // Deterministic mode needs no dS staging, which leaves room to double-buffer the
  // Q/dO stage; the atomic mode's single stage is refilled during its dQ part.
  constexpr int NSTAGE = DQ_ATOMIC ? 1 : 2;
  // Every buffer is its own object, so that the compiler can tell the stage a step
  // reads from the one the next step's DMA loads fill (and does not make the reads
  // wait for those loads).  The final dK/dV reduction reuses the K and V buffers.
  __shared__ __attribute__((aligned(1024))) char stage0[STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1[NSTAGE == 2 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) char k_lds_raw[KT_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds_raw[KT_BYTES];
  __shared__ __attribute__((aligned(1024))) char dsh_raw[DQ_ATOMIC ? DS_BYTES : 16];
  auto stage_buf = [&](int st) { return (FA_LDS char*)(st ? stage1 : stage0); };
  FA_LDS char* k_lds = (FA_LDS char*)k_lds_raw;
  FA_LDS char* v_lds = (FA_LDS char*)v_lds_raw;
  FA_LDS char* dsh_lds = (FA_LDS char*)dsh_raw;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kw = wave & 3;   // key group
  const int qh = wave >> 2;  // row half of each step
  const int hl = lane >> 5;
  const int i16 = lane & 15;

  int b, h, kblk;
  if constexpr (VARLEN) {
    const int item = blockIdx.x / p.heads;
    h = blockIdx.x - item * p.heads;
    if (item >= p.sched[0]) return;
    b = p.sched[1 + 2 * item];
    kblk = p.sched[2 + 2 * item];
  } else {
    const int bh_count = p.batch * p.heads;
    kblk = blockIdx.x / bh_count;  // ascending: longest first under the causal mask
    const int bh = blockIdx.x - kblk * bh_count;
    b = bh / p.heads;
    h = bh - b * p.heads;
  }
  const BwdSeq sq = bwd_seq(p, b, h);
  const int Lq = sq.Lq, Lk = sq.Lk;
  const int k_blk0 = kblk * BNK;
  if (k_blk0 >= Lk) return;

  // Q and K come from their fp16 copies (rows ROWB bytes apart)
  const uint32_t q_ss2 = (uint32_t)ROWB, do_ss2 = (uint32_t)(p.do_ss * 2);
  const uint32_t k_ss2 = (uint32_t)ROWB, v_ss2 = (uint32_t)(p.v_ss * 2);
  const rsrc_t rq = make_rsrc(p.q16 + sq.rowbase * D, (uint32_t)Lq * ROWB);
  const rsrc_t rdo = make_rsrc((const uint16_t*)p.dout + sq.dooff, rows_bytes(Lq, p.do_ss, ROWB));
  const rsrc_t rk = make_rsrc(p.k16 + sq.krowbase * D, (uint32_t)Lk * ROWB);
  const rsrc_t rv = make_rsrc((const uint16_t*)p.v + sq.voff, rows_bytes(Lk, p.v_ss, ROWB));
  const rsrc_t racc = make_rsrc(p.dq_acc + (DQ_ATOMIC ? sq.rowbase * D : 0), DQ_ATOMIC ? (uint32_t)Lq * D * 4 : 0u);
  const BwdExp ex = bwd_exponents(p);
  const float sc16 = p.scale * pow2f(-ex.f);  // dS16 = sc16 * P (dP - D)

  // K and V tiles of the block (rows past the end read as zero)
#pragma unroll
  for (int i = wave; i < KT_BYTES / 1024; i += 8) {
    const int idx = i * 64 + lane;
    const int r = idx / SLOTS;
    const int cc = (idx % SLOTS) ^ slot_swizzle<D>(r);
    buf_load_lds16(rk, k_lds + i * 1024, (uint32_t)(k_blk0 + r) * k_ss2 + cc * 16);
    buf_load_lds16(rv, v_lds + i * 1024, (uint32_t)(k_blk0 + r) * v_ss2 + cc * 16);
  }
  dma_issued();

  // causal: row i sees keys j <= i + coff (bottom-right alignment; 0 for equal lengths)
  const int coff = Lk - Lq;
  const int i_start = CAUSAL ? max(0, k_blk0 - coff) / BM : 0;
  const int i_end = (Lq + BM - 1) / BM;
  const int n_steps = i_end > i_start ? i_end - i_start : 0;
  const float c = p.scale_log2 * pow2f(ex.a + ex.b);  // S16 = S 2^-(a+b)

  auto issue_q = [&](int i, int stage) {
    FA_LDS char* qt = stage_buf(stage);
    FA_LDS char* dot = qt + QT_BYTES;
#pragma unroll
    for (int j = wave; j < QT_BYTES / 1024; j += 8) {
      const int idx = j * 64 + lane;
      const int r = idx / SLOTS;
      const int cc = (idx % SLOTS) ^ slot_swizzle<D>(r);
      buf_load_lds16(rq, qt + j * 1024, (uint32_t)(i * BM + r) * q_ss2 + cc * 16);
      buf_load_lds16(rdo, dot + j * 1024, (uint32_t)(i * BM + r) * do_ss2 + cc * 16);
    }
    dma_issued();
  };
  float lse_next = 0.0f, dvec_next = 0.0f;
  auto load_terms = [&](int i) {
    if (threadIdx.x < BM) {
      const int row = i * BM + threadIdx.x;
      if (row < Lq) {
        lse_next = p.lse[sq.lseoff + row];
        dvec_next = p.dvec[sq.rowbase + row];
      } else {
        lse_next = INFINITY;  // makes P = 0 for rows past the end
        dvec_next = 0.0f;
      }
    }
  };

  // lane-constant operand address parts
  const int my_key = k_blk0 + 32 * kw + (lane & 31);
  const int sw_row = slot_swizzle<D>(lane & 15);
  const int arow = (32 * qh + (lane & 31)) * ROWB;   // Q/dO row of the A operand
  const int brow = (32 * kw + (lane & 31)) * ROWB;   // K/V row of the B operand
  const int tr_r1 = 4 * hl + (i16 >> 2);
  const int sw_t1 = slot_swizzle<D>(tr_r1), sw_t2 = slot_swizzle<D>(tr_r1 + 8);
  const int tr_clo = 2 * ((lane >> 4) & 1) + ((i16 & 3) >> 1);
  const int tr_half = (i16 & 1) * 8;
  const int krow = 32 * kw + (lane & 31);                  // this lane's key row of dS^T
  const int ds_sw_w = ds_swizzle(krow);
  const int ds_gcol = 4 * ((lane >> 4) & 1) + (i16 & 3);   // granule within a 32-query block

  f32x16 dvacc[NDB], dkacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dvacc[db] = f32x16{};
    dkacc[db] = f32x16{};
  }

  if (n_steps > 0) {
    issue_q(i_start, 0);
    load_terms(i_start);
  }
  // one step: the 64 query rows i_start + it; the stage is a compile-time constant
  auto step = [&](const int it, auto stage_c) {
    constexpr int stage = decltype(stage_c)::value;
    const int i = i_start + it;
    const int q0 = i * BM;
    FA_LDS char* qt = stage_buf(stage);
    FA_LDS char* dot = qt + QT_BYTES;
    FA_LDS float* lse_l = (FA_LDS float*)(dot + QT_BYTES);
    FA_LDS float* dvec_l = lse_l + BM;
    // wait for this stage's loads; the previous step's 16 dQ atomics (issued after
    // them) may still be in flight
    if (DQ_ATOMIC && it > 0 && kw < NDB) wait_vmem_keep16();
    else wait_vmem();
    if (threadIdx.x < BM) {
      lse_l[threadIdx.x] = (lse_next == -INFINITY) ? INFINITY : lse_next * kLog2e;
      dvec_l[threadIdx.x] = dvec_next * sc16;
    }
    __syncthreads();
    if (NSTAGE == 2 && it + 1 < n_steps) {
      // the other stage was consumed in the previous step (before the barrier above)
      issue_q(i + 1, stage ^ 1);
      load_terms(i + 1);
    }

    const int row0 = q0 + 32 * qh;   // first row of this wave's half
    // every key of the wave after every row of its half: nothing visible
    const bool skip = CAUSAL && (k_blk0 + 32 * kw > row0 + 31 + coff);
    bool need_mask = (k_blk0 + BNK > Lk);
    if constexpr (CAUSAL) need_mask = need_mask || (k_blk0 + 32 * kw + 31 > row0 + coff);
    u32x4 dsh[2];
    if (!skip) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const int co = ((2 * ds + hl) ^ sw_row) << 4;
        s = mfma_f16(lds_read16(qt + arow + co), lds_read16(k_lds + brow + co), s);
        dp = mfma_bf16(lds_read16(dot + arow + co), lds_read16(v_lds + brow + co), dp);
      }
      // hidden keys (the causal diagonal, the ragged last block): their scores become
      // -inf, so P and dS' are exactly 0.  A wave-uniform branch, so that the other
      // steps carry no mask arithmetic.
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int query = row0 + 8 * (r >> 2) + 4 * hl + (r & 3);
          bool hide = my_key >= Lk;
          if constexpr (CAUSAL) hide = hide || my_key > query + coff;
          s[r] = hide ? -INFINITY : s[r];
        }
      }
      u32x4 pb[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint32_t ph[4], hh[4];
#pragma unroll
        for (int r4h = 0; r4h < 2; ++r4h) {
          const int r4 = 2 * half + r4h;
          const f32x4 l2 = *(const FA_LDS f32x4*)(lse_l + 32 * qh + 8 * r4 + 4 * hl);
          const f32x4 dd = *(const FA_LDS f32x4*)(dvec_l + 32 * qh + 8 * r4 + 4 * hl);
          float pv[4], dsv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float pe = exp2_hw(__builtin_fmaf(s[4 * r4 + j], c, -l2[j]));
            pv[j] = pe;
            dsv[j] = pe * __builtin_fmaf(dp[4 * r4 + j], sc16, -dd[j]);  // scale 2^-f P (dP - D)
          }
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int k = 2 * r4h + e;
            ph[k] = pack_bf16(pv[2 * e], pv[2 * e + 1]);
            hh[k] = pack_f16(dsv[2 * e], dsv[2 * e + 1]);
          }
        }
        pb[half] = u32x4{ph[0], ph[1], ph[2], ph[3]};
        dsh[half] = u32x4{hh[0], hh[1], hh[2], hh[3]};
      }
      // dV^T += dO^T P ; dK^T += Q16^T dS16  (16-row groups of this half)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int r1 = 32 * qh + 16 * half + tr_r1;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int cc = 4 * db + tr_clo;
          const int o1 = r1 * ROWB + ((cc ^ sw_t1) << 4) + tr_half;
          const int o2 = (r1 + 8) * ROWB + ((cc ^ sw_t2) << 4) + tr_half;
          const u32x2 a_lo = lds_read_tr16(dot + o1), a_hi = lds_read_tr16(dot + o2);
          dvacc[db] = mfma_bf16(u32x4{a_lo[0], a_lo[1], a_hi[0], a_hi[1]}, pb[half], dvacc[db]);
          const u32x2 q_lo = lds_read_tr16(qt + o1), q_hi = lds_read_tr16(qt + o2);
          dkacc[db] = mfma_f16(u32x4{q_lo[0], q_lo[1], q_hi[0], q_hi[1]}, dsh[half], dkacc[db]);
        }
      }
    } else {
      dsh[0] = dsh[1] = u32x4{0u, 0u, 0u, 0u};
    }
    if constexpr (DQ_ATOMIC) {
      // dS16^T to LDS: granule (8qh + 2r4 + hl) of row krow holds rows 32qh + 8r4 + 4hl + 0..3
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int half = r4 >> 1, e = 2 * (r4 & 1);
        const int off = krow * DS_ROWB + (((8 * qh + 2 * r4 + hl) ^ ds_sw_w) << 3);
        *(FA_LDS u32x2*)(dsh_lds + off) = u32x2{dsh[half][e], dsh[half][e + 1]};
      }
    }
    if constexpr (DQ_ATOMIC) {
      __syncthreads();  // stage consumed by every wave and dS16 complete
      if (it + 1 < n_steps) {
        issue_q(i + 1, 0);
        load_terms(i + 1);
      }
      // this wave's dQ block: rows q0 + 32qh + ..., columns 32kw + (lane & 31)
      if (kw < NDB) {
        f32x16 acc = f32x16{};
        const int cc = 4 * kw + tr_clo;
#pragma unroll
        for (int g = 0; g < BNK / 16; ++g) {
          const int r1 = 16 * g + tr_r1;
          const u32x2 k1 = lds_read_tr16(k_lds + r1 * ROWB + ((cc ^ sw_t1) << 4) + tr_half);
          const u32x2 k2 = lds_read_tr16(k_lds + (r1 + 8) * ROWB + ((cc ^ sw_t2) << 4) + tr_half);
          const u32x4 kb = u32x4{k1[0], k1[1], k2[0], k2[1]};
          const int c8 = 8 * qh + ds_gcol;
          const int oa = r1 * DS_ROWB + ((c8 ^ ds_swizzle(r1)) << 3);
          const int ob = (r1 + 8) * DS_ROWB + ((c8 ^ ds_swizzle(r1 + 8)) << 3);
          const u32x2 h1 = lds_read_tr16(dsh_lds + oa), h2 = lds_read_tr16(dsh_lds + ob);
          acc = mfma_f16(u32x4{h1[0], h1[1], h2[0], h2[1]}, kb, acc);
        }
        const uint32_t rowb = (uint32_t)(row0 + 4 * hl) * (D * 4) + (uint32_t)(32 * kw + (lane & 31)) * 4;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[r], racc, rowb + (uint32_t)(8 * (r >> 2) + (r & 3)) * (D * 4),
                                                          0, 0);
      }
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  if constexpr (NSTAGE == 2) {
    int it = 0;
    for (; it + 1 < n_steps; it += 2) {
      step(it, I0{});
      step(it + 1, I1{});
    }
    if (it < n_steps) step(it, I0{});
  } else {
    for (int it = 0; it < n_steps; ++it) step(it, I0{});
  }

  // ---- sum the two row-half partials of each key group, then store dK, dV ----
  // One 32-column block of d per round through the (now free) K and V buffers:
  // [key group][4 rows of 4][64 lanes] f32x4 each, dK in k_lds and dV in v_lds.
  const float ks = pow2f(ex.f + ex.a);  // the accumulators hold dK 2^-(f+a)
  const int gb = p.grad_bf16 ? 2 : 4;
  const rsrc_t rdk = make_rsrc((char*)p.dk + sq.dkoff * gb, Lk > 0 ? (uint32_t)(Lk - 1) * (uint32_t)(p.dk_ss * gb) + D * gb : 0u);
  const rsrc_t rdv = make_rsrc((char*)p.dv + sq.dvoff * gb, Lk > 0 ? (uint32_t)(Lk - 1) * (uint32_t)(p.dv_ss * gb) + D * gb : 0u);
  const uint32_t dk_row = (uint32_t)my_key * (uint32_t)(p.dk_ss * gb);
  const uint32_t dv_row = (uint32_t)my_key * (uint32_t)(p.dv_ss * gb);
  FA_LDS f32x4* red_k = (FA_LDS f32x4*)k_lds + kw * (4 * 64);
  FA_LDS f32x4* red_v = (FA_LDS f32x4*)v_lds + kw * (4 * 64);
  static_assert(4 * 4 * 64 * 16 <= KT_BYTES, "one reduction round must fit a K/V buffer");
  wait_vmem();  // with no query step the K/V loads were never waited for
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    __syncthreads();  // the buffers are free (main loop or the previous round done)
    if (qh == 1) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        red_k[r4 * 64 + lane] = f32x4{dkacc[db][4 * r4], dkacc[db][4 * r4 + 1], dkacc[db][4 * r4 + 2], dkacc[db][4 * r4 + 3]};
        red_v[r4 * 64 + lane] = f32x4{dvacc[db][4 * r4], dvacc[db][4 * r4 + 1], dvacc[db][4 * r4 + 2], dvacc[db][4 * r4 + 3]};
      }
    }
    __syncthreads();
    if (qh == 0) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * db + 8 * r4 + 4 * hl;
        const f32x4 ok = red_k[r4 * 64 + lane];
        const f32x4 ov = red_v[r4 * 64 + lane];
        store_grad4(rdk, dk_row + d * 4, dk_row + d * 2, p.grad_bf16, (dkacc[db][4 * r4] + ok[0]) * ks,
                    (dkacc[db][4 * r4 + 1] + ok[1]) * ks, (dkacc[db][4 * r4 + 2] + ok[2]) * ks,
                    (dkacc[db][4 * r4 + 3] + ok[3]) * ks);
        store_grad4(rdv, dv_row + d * 4, dv_row + d * 2, p.grad_bf16, dvacc[db][4 * r4] + ov[0],
                    dvacc[db][4 * r4 + 1] + ov[1], dvacc[db][4 * r4 + 2] + ov[2], dvacc[db][4 * r4 + 3] + ov[3]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bwd_dq (deterministic mode): dQ for 256 query rows, no atomics.
//
// Shaped like the forward: eight waves (two per SIMD) of 32 rows each keep Q and
// dO in registers as B operands; K and V tiles of 64 keys stream through a
// double-buffered LDS stage.  Per tile and 32-key block:
//   S^T = K16 Q16^T (fp16), dP^T = V dO^T (bf16)   (lane = query row, registers = keys)
//   dS16^T = scale 2^-f P^T (dP^T - D)  with P^T = 2^(S^T*c 2^(a+b) - LSE*log2 e)
//   dQ^T 2^-(f+b) += K16^T dS16^T (fp16)            (A = K16^T by transpose reads)
// dQ is reduced in registers in a fixed order and written once.
template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(512) void bwd_dq_kernel(BwdParams p) {
  constexpr int BN = kFwdBlockN;
  constexpr int NW = 8;
  constexpr int WG_ROWS = 32 * NW;
  constexpr int ROWB = D * 2;
  constexpr int TILE_BYTES = BN * ROWB;
  constexpr int SLOTS = D / 8, NKB = BN / 32, NDS = D / 16, NDB = D / 32;
  // K and V of the two stages as separate objects, so that the compiler can tell the
  // buffers a tile reads from the ones the next tile's DMA loads fill
  __shared__ __attribute__((aligned(1024))) char k_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char k_lds1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds1[TILE_BYTES];
  auto kbuf = [&](int st) { return (FA_LDS char*)(st ? k_lds1 : k_lds0); };
  auto vbuf = [&](int st) { return (FA_LDS char*)(st ? v_lds1 : v_lds0); };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane >> 5;
  const int i16 = lane & 15;

  int b, h, qtile;
  if constexpr (VARLEN) {
    const int item = blockIdx.x / p.heads;
    h = blockIdx.x - item * p.heads;
    if (item >= p.sched[0]) return;
    b = p.sched[1 + 2 * item];
    qtile = p.sched[2 + 2 * item];
  } else {
    const int bh_count = p.batch * p.heads;
    const int t = blockIdx.x / bh_count;
    const int bh = blockIdx.x - t * bh_count;
    const int n_qt = (p.seqlen_q + WG_ROWS - 1) / WG_ROWS;
    qtile = CAUSAL ? (n_qt - 1 - t) : t;
    b = bh / p.heads;
    h = bh - b * p.heads;
  }
  const BwdSeq sq = bwd_seq(p, b, h);
  const int Lq = sq.Lq, Lk = sq.Lk;
  const int wg_q0 = qtile * WG_ROWS;
  if (wg_q0 >= Lq) return;

  // Q and K come from their fp16 copies (rows ROWB bytes apart)
  const uint32_t q_ss2 = (uint32_t)ROWB, do_ss2 = (uint32_t)(p.do_ss * 2);
  const uint32_t k_ss2 = (uint32_t)ROWB, v_ss2 = (uint32_t)(p.v_ss * 2);
  const rsrc_t rq = make_rsrc(p.q16 + sq.rowbase * D, (uint32_t)Lq * ROWB);
  const rsrc_t rdo = make_rsrc((const uint16_t*)p.dout + sq.dooff, rows_bytes(Lq, p.do_ss, ROWB));
  const rsrc_t rk = make_rsrc(p.k16 + sq.krowbase * D, (uint32_t)Lk * ROWB);
  const rsrc_t rv = make_rsrc((const uint16_t*)p.v + sq.voff, rows_bytes(Lk, p.v_ss, ROWB));
  const BwdExp ex = bwd_exponents(p);
  const float sc16 = p.scale * pow2f(-ex.f);  // dS16 = sc16 * P (dP - D)

  // rows of this wave: two 128-row tiles interleaved so that the two waves of a
  // SIMD hold neighbouring row blocks
  const int q0 = wg_q0 + 32 * wave;
  const int my_row = q0 + (lane & 31);
  u32x4 qreg[NDS], doreg[NDS];
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) {
    qreg[ds] = buf_load16(rq, (uint32_t)my_row * q_ss2 + (2 * ds + hl) * 16);
    doreg[ds] = buf_load16(rdo, (uint32_t)my_row * do_ss2 + (2 * ds + hl) * 16);
  }
  float lse2 = INFINITY, dvs = 0.0f;
  if (my_row < Lq) {
    const float l = p.lse[sq.lseoff + my_row];
    lse2 = (l == -INFINITY) ? INFINITY : l * kLog2e;
    dvs = p.dvec[sq.rowbase + my_row] * sc16;
  }

  int kv_end = Lk;
  const int coff = Lk - Lq;  // causal: row i sees keys j <= i + coff
  if constexpr (CAUSAL) kv_end = max(0, min(Lk, min(Lq, wg_q0 + WG_ROWS) + coff));
  const int n_tiles = (kv_end + BN - 1) / BN;
  int n_mine = q0 < Lq ? n_tiles : 0;  // a wave whose rows are all past the end only helps stage K/V
  if constexpr (CAUSAL) n_mine = (q0 >= Lq || q0 + 31 + coff < 0) ? 0 : min(n_tiles, (q0 + 31 + coff) / BN + 1);

  auto issue_tile = [&](int t, int stage) {
    const int k0 = t * BN;
    FA_LDS char* kd = kbuf(stage);
    FA_LDS char* vd = vbuf(stage);
#pragma unroll
    for (int i = wave; i < TILE_BYTES / 1024; i += NW) {
      const int idx = i * 64 + lane;
      const int r = idx / SLOTS;
      const int cc = (idx % SLOTS) ^ slot_swizzle<D>(r);
      buf_load_lds16(rk, kd + i * 1024, (uint32_t)(k0 + r) * k_ss2 + cc * 16);
      buf_load_lds16(rv, vd + i * 1024, (uint32_t)(k0 + r) * v_ss2 + cc * 16);
    }
    dma_issued();
  };

  // part u of this wave's share of tile t's loads: packet wave + NW (u % PPW) of K
  // (u < PPW) or of V; the packets of a wave start a multiple of 16 rows apart, so
  // that each lane's offset is one register per tensor plus a wave-uniform row term
  constexpr int PPW = TILE_BYTES / 1024 / NW;
  constexpr int NPART = 2 * PPW;
  static_assert(PPW * NW * 1024 == TILE_BYTES && (NW * 64 / SLOTS) % 16 == 0, "packet layout");
  const int l_row = (wave * 64 + lane) / SLOTS;
  const int l_cs = ((wave * 64 + lane) % SLOTS) ^ slot_swizzle<D>(l_row);
  const uint32_t k_lane = (uint32_t)l_row * k_ss2 + l_cs * 16, v_lane = (uint32_t)l_row * v_ss2 + l_cs * 16;
  auto dma_part = [&](const int t, const int stage, const int u) __attribute__((always_inline)) {
    const int k = u % PPW;
    const uint32_t row = (uint32_t)(t * BN + k * (NW * 64 / SLOTS));
    if (u < PPW) buf_load_lds16(rk, kbuf(stage) + (wave + NW * k) * 1024, k_lane + row * k_ss2);
    else buf_load_lds16(rv, vbuf(stage) + (wave + NW * k) * 1024, v_lane + row * v_ss2);
    dma_issued();
  };

  // lane-constant LDS offsets within a tile: with the stage a compile-time constant
  // every operand read is one register plus an immediate
  const int sw_row = slot_swizzle<D>(lane & 15);
  const int tr_r1 = 4 * hl + (i16 >> 2);
  const int sw_t1 = slot_swizzle<D>(tr_r1), sw_t2 = slot_swizzle<D>(tr_r1 + 8);
  const int tr_clo = 2 * ((lane >> 4) & 1) + ((i16 & 3) >> 1);
  const int tr_half = (i16 & 1) * 8;
  int off_r[NDS], off_t1[NDB], off_t2[NDB];
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) off_r[ds] = (lane & 31) * ROWB + (((2 * ds + hl) ^ sw_row) << 4);
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int cc = 4 * db + tr_clo;
    off_t1[db] = tr_r1 * ROWB + ((cc ^ sw_t1) << 4) + tr_half;
    off_t2[db] = (tr_r1 + 8) * ROWB + ((cc ^ sw_t2) << 4) + tr_half;
  }
  const float c = p.scale_log2 * pow2f(ex.a + ex.b);  // S16 = S 2^-(a+b)

  f32x16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqacc[db] = f32x16{};

  // one tile of 64 keys; MASK: the tile may hold keys this wave must not see
  auto tile = [&](const int t, auto stage_c, auto mask_c) {
    constexpr int STAGE = decltype(stage_c)::value;
    constexpr bool MASK = decltype(mask_c)::value;
    wait_vmem();
    __syncthreads();
    // tile t+1's loads go out one packet per two MFMAs of the first score block
    // (issued together at the barrier they queue at the CU's address unit); past the
    // last tile the last tile is loaded again into the free stage, without a branch
    const int t_next = min(t + 1, n_tiles - 1);
    const int k0 = t * BN;
    const FA_LDS char* kt = kbuf(STAGE);
    const FA_LDS char* vt = vbuf(STAGE);
    // key k0 + rel is hidden from this lane's row when rel >= lim
    int lim = Lk;
    if constexpr (CAUSAL) lim = min(lim, my_row + 1 + coff);
    lim -= k0 + 4 * hl;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      f32x16 s = f32x16{}, dp = f32x16{};
      // raised priority: these products issue ahead of the other wave's vector work
      // on the SIMD, so that the vector work of one wave runs beside the products of
      // the other more often
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        s = mfma_f16(lds_read16(kt + 32 * kb * ROWB + off_r[ds]), qreg[ds], s);
        dp = mfma_bf16(lds_read16(vt + 32 * kb * ROWB + off_r[ds]), doreg[ds], dp);
        if (kb == 0 && ds * NPART / NDS * NDS == ds * NPART) dma_part(t_next, STAGE ^ 1, ds * NPART / NDS);
      }
      __builtin_amdgcn_s_setprio(0);
      u32x4 dsh[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint32_t hh[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float dv2[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int r = 8 * half + 2 * e + u;
            float pe = exp2_hw(__builtin_fmaf(s[r], c, -lse2));
            if constexpr (MASK) pe = (32 * kb + 8 * (r >> 2) + (r & 3) >= lim) ? 0.0f : pe;
            dv2[u] = pe * __builtin_fmaf(dp[r], sc16, -dvs);   // scale 2^-f P (dP - D)
          }
          hh[e] = pack_f16(dv2[0], dv2[1]);
        }
        dsh[half] = u32x4{hh[0], hh[1], hh[2], hh[3]};
      }
      // dQ^T += K16^T dS16^T  (A = K16^T through the transpose reads, 16-key groups)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int rb = (32 * kb + 16 * half) * ROWB;
          const u32x2 lo = lds_read_tr16(kt + rb + off_t1[db]);
          const u32x2 hi = lds_read_tr16(kt + rb + off_t2[db]);
          dqacc[db] = mfma_f16(u32x4{lo[0], lo[1], hi[0], hi[1]}, dsh[half], dqacc[db]);
        }
      }
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using MF = std::false_type;
  using MT = std::true_type;
  // tiles before t_plain need no mask for this wave's rows
  int t_plain = Lk / BN;
  if constexpr (CAUSAL) t_plain = min(t_plain, max(0, q0 + 1 + coff) / BN);
  const int t_lim = min(n_mine, t_plain);
  if (n_tiles > 0) issue_tile(0, 0);
  int t = 0;
  for (; t + 1 < t_lim; t += 2) {
    tile(t, I0{}, MF{});
    tile(t + 1, I1{}, MF{});
  }
  for (; t + 1 < n_mine; t += 2) {
    tile(t, I0{}, MT{});
    tile(t + 1, I1{}, MT{});
  }
  if (t < n_mine) {
    tile(t, I0{}, MT{});
    ++t;
  }
  for (; t < n_tiles; ++t) {
    wait_vmem();
    __syncthreads();
    if (t + 1 < n_tiles) issue_tile(t + 1, (t & 1) ^ 1);
  }
  wait_vmem();  // the last tile's repeated loads land before the LDS is released

  const float qs = pow2f(ex.f + ex.b);  // the accumulators hold dQ 2^-(f+b)
  const int gb = p.grad_bf16 ? 2 : 4;
  const rsrc_t rdq = make_rsrc((char*)p.dq + sq.dqoff * gb, (uint32_t)(Lq - 1) * (uint32_t)(p.dq_ss * gb) + D * gb);
  const uint32_t row_off = (uint32_t)my_row * (uint32_t)(p.dq_ss * gb);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = 32 * db + 8 * r4 + 4 * hl;
      store_grad4(rdq, row_off + d * 4, row_off + d * 2, p.grad_bf16, dqacc[db][4 * r4] * qs,
                  dqacc[db][4 * r4 + 1] * qs, dqacc[db][4 * r4 + 2] * qs, dqacc[db][4 * r4 + 3] * qs);
    }
}

// ---------------------------------------------------------------------------
// Longest-first list of key blocks for variable-length batches: cost of key block
// j of sequence b = number of 64-row query steps it visits.
__global__ __launch_bounds__(1024) void sched_kv_kernel(const int32_t* cu_q, const int32_t* cu_k, int batch,
                                                        int causal, int32_t* out) {
  __shared__ int hist[kSchedMaxCost + 1];
  __shared__ int wsum[16];
  __shared__ int total;
  for (int i = threadIdx.x; i <= kSchedMaxCost; i += blockDim.x) hist[i] = 0;
  if (threadIdx.x == 0) total = 0;
  __syncthreads();
  auto cost_of = [&](int b, int j) {
    const int lq = cu_q[b + 1] - cu_q[b];
    const int lk = cu_k[b + 1] - cu_k[b];
    const int steps = (lq + kBwdBlockM - 1) / kBwdBlockM;
    const int first = causal ? max(0, j * kBwdBlockN - (lk - lq)) / kBwdBlockM : 0;
    return min(max(steps - first, 0), kSchedMaxCost);
  };
  // Longest first by cost bucket: a bucket spans the cost change of 16 neighbouring
  // causal key blocks, and within a bucket each sequence's blocks stay together, longest
  // first, so that the workgroups running at one time read the same sequences' Q and
  // dO and find them in L2
  constexpr int bw = 16 * kBwdBlockN / kBwdBlockM;
  for (int b = threadIdx.x; b < batch; b += blockDim.x) {
    const int lk = cu_k[b + 1] - cu_k[b];
    const int nb = (lk + kBwdBlockN - 1) / kBwdBlockN;
    for (int j = 0; j < nb;) {
      const int bk = cost_of(b, j) / bw;
      int j1 = j + 1;
      while (j1 < nb && cost_of(b, j1) / bw == bk) ++j1;
      atomicAdd(&hist[bk], j1 - j);
      j = j1;
    }
    atomicAdd(&total, nb);
  }
  __syncthreads();
  scan_bins_descending<kSchedMaxCost + 1>(hist, wsum);
  if (threadIdx.x == 0) out[0] = total;
  for (int b = threadIdx.x; b < batch; b += blockDim.x) {
    const int lk = cu_k[b + 1] - cu_k[b];
    const int nb = (lk + kBwdBlockN - 1) / kBwdBlockN;
    for (int j = 0; j < nb;) {
      const int bk = cost_of(b, j) / bw;
      int j1 = j + 1;
      while (j1 < nb && cost_of(b, j1) / bw == bk) ++j1;
      int pos = atomicAdd(&hist[bk], j1 - j);
      for (int u = j; u < j1; ++u, ++pos) {
        out[1 + 2 * pos] = b;
        out[2 + 2 * pos] = u;
      }
      j = j1;
    }
  }
}

template <int D>
static hipError_t launch_bwd_d(const BwdParams& p, int phases, hipStream_t stream) {
  const bool atomic = !p.deterministic;
  const int64_t rows = (int64_t)p.total_q * p.heads;
  if (phases & 1) {
    const int64_t work = std::max(rows, (int64_t)p.total_k * p.heads) * (D / 8);
    int grid = (int)std::min<int64_t>((work + 255) / 256, kBwdPreBlocks);
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3(grid), dim3(256), 0, stream, p, atomic ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_reduce_stats_kernel, dim3(1), dim3(1024), 0, stream, p.stats, grid);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t cwork = ((int64_t)p.total_q + p.total_k) * p.heads * (D / 8);
    int cgrid = (int)std::min<int64_t>((cwork + 255) / 256, 2048 * 4);
    if (cgrid < 1) cgrid = 1;
    hipLaunchKernelGGL(bwd_convert_kernel<D>, dim3(cgrid), dim3(256), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // key-block kernel
  if (phases & 2) {
    unsigned grid;
    if (p.varlen) {
      hipError_t e = hipSuccess;
      hipLaunchKernelGGL(sched_kv_kernel, dim3(1), dim3(1024), 0, stream, p.cu_q, p.cu_k, p.batch,
                         p.causal ? 1 : 0, p.sched);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      grid = (unsigned)((p.total_k + kBwdBlockN - 1) / kBwdBlockN + p.batch) * (unsigned)p.heads;
    } else {
      grid = (unsigned)((p.seqlen_k + kBwdBlockN - 1) / kBwdBlockN) * (unsigned)(p.batch * p.heads);
    }
    if (grid > 0) {
#define FA_KV(C, V, A) hipLaunchKernelGGL((bwd_kv_kernel<D, C, V, A>), dim3(grid), dim3(512), 0, stream, p)
      if (p.causal) {
        if (p.varlen) { if (atomic) FA_KV(true, true, true); else FA_KV(true, true, false); }
        else { if (atomic) FA_KV(true, false, true); else FA_KV(true, false, false); }
      } else {
        if (p.varlen) { if (atomic) FA_KV(false, true, true); else FA_KV(false, true, false); }
        else { if (atomic) FA_KV(false, false, true); else FA_KV(false, false, false); }
      }
#undef FA_KV
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (!(phases & 4)) return hipSuccess;
  if (atomic) {
    int64_t work = rows * (D / 4);
    int grid = (int)std::min<int64_t>((work + 255) / 256, 2048 * 4);
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(bwd_post_kernel<D>, dim3(grid), dim3(256), 0, stream, p);
    return hipGetLastError();
  }
  // deterministic: query-major dQ kernel; its list reuses the forward's query-tile order
  unsigned grid;
  int32_t* qsched = p.sched + 1 + 2 * ((p.total_k + kBwdBlockN - 1) / kBwdBlockN + p.batch);
  if (p.varlen) {
    hipError_t e = launch_fwd_schedule(p.cu_q, p.cu_k, p.batch, kDqTileRows, kFwdBlockN, p.causal, qsched, stream);
    if (e != hipSuccess) return e;
    grid = (unsigned)((p.total_q + kDqTileRows - 1) / kDqTileRows + p.batch) * (unsigned)p.heads;
  } else {
    grid = (unsigned)((p.seqlen_q + kDqTileRows - 1) / kDqTileRows) * (unsigned)(p.batch * p.heads);
  }
  if (grid == 0) return hipSuccess;
  BwdParams pq = p;
  pq.sched = qsched;
#define FA_DQ(C, V) hipLaunchKernelGGL((bwd_dq_kernel<D, C, V>), dim3(grid), dim3(512), 0, stream, pq)
  if (p.causal) { if (p.varlen) FA_DQ(true, true); else FA_DQ(true, false); }
  else { if (p.varlen) FA_DQ(false, true); else FA_DQ(false, false); }
#undef FA_DQ
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdParams& p, int phases, hipStream_t stream) {
  return p.head_dim == 128 ? launch_bwd_d<128>(p, phases, stream) : launch_bwd_d<64>(p, phases, stream);
}

}  // namespace fa
