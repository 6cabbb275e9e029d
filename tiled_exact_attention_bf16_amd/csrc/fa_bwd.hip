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
//   bwd_pre:  D_i for every row and head; zeroes the fp32 dQ accumulator.
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
// dS is split into a bf16 high part and a bf16 low part (dS - hi) before the dQ
// and dK products, so those products see dS to about 16 significant bits while
// every matrix-core operation stays BF16.
#include <algorithm>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

constexpr float kLog2e = 1.4426950408889634f;

// Per (sequence, head) view used by the backward kernels.
struct BwdSeq {
  int Lq, Lk;
  int64_t qoff, koff, voff, ooff, dooff, dqoff, dkoff, dvoff;  // element offsets
  int64_t lseoff;   // offset of row 0 in the LSE array
  int64_t rowbase;  // row index of row 0 in the [H, total_q] row-term arrays
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
  }
  return s;
}

__device__ __forceinline__ uint32_t rows_bytes(int rows, int64_t stride_elems, int row_bytes) {
  return rows > 0 ? (uint32_t)(rows - 1) * (uint32_t)(stride_elems * 2) + (uint32_t)row_bytes : 0u;
}

// ---------------------------------------------------------------------------
// bwd_pre: D_i = sum_d dO_id O_id (fp32) and zeroing of the dQ accumulator.
// 16-byte chunks: D/8 lanes per (row, head), reduced with xor shuffles.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p, int zero_acc) {
  constexpr int CPR = D / 8;  // chunks per row
  const int64_t total_rows = (int64_t)p.total_q * p.heads;
  const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int64_t w = tid; w < total_rows * CPR; w += nthreads) {
    const int64_t rh = w / CPR;
    const int chunk = (int)(w - rh * CPR);
    const int h = (int)(rh / p.total_q);
    const int64_t row = rh - (int64_t)h * p.total_q;  // global packed row (b*S + s for fixed)
    int64_t obase, dobase;
    if (p.varlen) {
      obase = row * p.o_ss + h * p.o_sh;
      dobase = row * p.do_ss + h * p.do_sh;
    } else {
      const int64_t b = row / p.seqlen_q, s = row - b * p.seqlen_q;
      obase = b * p.o_sb + s * p.o_ss + h * p.o_sh;
      dobase = b * p.do_sb + s * p.do_ss + h * p.do_sh;
    }
    const u32x4 ov = *(const u32x4*)((const uint16_t*)p.o + obase + chunk * 8);
    const u32x4 dv = *(const u32x4*)((const uint16_t*)p.dout + dobase + chunk * 8);
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc = __builtin_fmaf(bf16_lo(ov[j]), bf16_lo(dv[j]), acc);
      acc = __builtin_fmaf(bf16_hi(ov[j]), bf16_hi(dv[j]), acc);
    }
#pragma unroll
    for (int m = CPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, CPR);
    if (chunk == 0) p.dvec[(int64_t)h * p.total_q + row] = acc;
  }
  if (zero_acc) {
    float4* acc4 = (float4*)p.dq_acc;
    const int64_t n4 = total_rows * D / 4;
    for (int64_t i = tid; i < n4; i += nthreads) acc4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// ---------------------------------------------------------------------------
// bwd_post: dQ (given layout and dtype) <- fp32 accumulator (already scaled).
template <int D>
__global__ __launch_bounds__(256) void bwd_post_kernel(BwdParams p) {
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
    const float4 v = ((const float4*)p.dq_acc)[i];
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
template <int D, bool CAUSAL, bool VARLEN, bool DQ_ATOMIC>
__global__ __launch_bounds__(256) void bwd_kv_kernel(BwdParams p) {
  constexpr int BM = kBwdBlockM;    // query rows per step
  constexpr int BNK = kBwdBlockN;   // keys per workgroup
  constexpr int ROWB = D * 2;
  constexpr int QT_BYTES = BM * ROWB;
  constexpr int STAGE = 2 * QT_BYTES + 2 * BM * 4;  // Q, dO, LSE*log2e, D
  constexpr int KT_BYTES = DQ_ATOMIC ? BNK * ROWB : 0;
  constexpr int DS_PITCH = BM * 2 + 8;              // bytes per key row of dS^T (padded)
  constexpr int DS_BYTES = DQ_ATOMIC ? BNK * DS_PITCH : 0;
  constexpr int SLOTS = D / 8, NDS = D / 16, NDB = D / 32;
  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * STAGE + KT_BYTES + 2 * DS_BYTES];
  FA_LDS char* smem = (FA_LDS char*)smem_raw;
  FA_LDS char* k_lds = smem + 2 * STAGE;
  FA_LDS char* dsh_lds = k_lds + KT_BYTES;
  FA_LDS char* dsl_lds = dsh_lds + DS_BYTES;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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

  const uint32_t q_ss2 = (uint32_t)(p.q_ss * 2), do_ss2 = (uint32_t)(p.do_ss * 2);
  const uint32_t k_ss2 = (uint32_t)(p.k_ss * 2), v_ss2 = (uint32_t)(p.v_ss * 2);
  const rsrc_t rq = make_rsrc((const uint16_t*)p.q + sq.qoff, rows_bytes(Lq, p.q_ss, ROWB));
  const rsrc_t rdo = make_rsrc((const uint16_t*)p.dout + sq.dooff, rows_bytes(Lq, p.do_ss, ROWB));
  const rsrc_t rk = make_rsrc((const uint16_t*)p.k + sq.koff, rows_bytes(Lk, p.k_ss, ROWB));
  const rsrc_t rv = make_rsrc((const uint16_t*)p.v + sq.voff, rows_bytes(Lk, p.v_ss, ROWB));

  const int my_key = k_blk0 + 32 * wave + (lane & 31);
  u32x4 kreg[NDS], vreg[NDS];
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) {
    kreg[ds] = buf_load16(rk, (uint32_t)my_key * k_ss2 + (2 * ds + hl) * 16);
    vreg[ds] = buf_load16(rv, (uint32_t)my_key * v_ss2 + (2 * ds + hl) * 16);
  }
  if constexpr (DQ_ATOMIC) {
#pragma unroll
    for (int i = wave; i < KT_BYTES / 1024; i += 4) {
      const int idx = i * 64 + lane;
      const int r = idx / SLOTS;
      const int c = (idx % SLOTS) ^ slot_swizzle<D>(r);
      buf_load_lds16(rk, k_lds + i * 1024, (uint32_t)(k_blk0 + r) * k_ss2 + c * 16);
    }
  }

  const int i_start = CAUSAL ? k_blk0 / BM : 0;
  const int i_end = (Lq + BM - 1) / BM;
  const int n_steps = i_end > i_start ? i_end - i_start : 0;
  const float c = p.scale_log2;

  // Q/dO stage loader (DMA) and row terms (registers of threads 0..63)
  auto issue_q = [&](int i, int stage) {
    FA_LDS char* qd = smem + stage * STAGE;
    FA_LDS char* dod = qd + QT_BYTES;
#pragma unroll
    for (int j = wave; j < QT_BYTES / 1024; j += 4) {
      const int idx = j * 64 + lane;
      const int r = idx / SLOTS;
      const int cc = (idx % SLOTS) ^ slot_swizzle<D>(r);
      buf_load_lds16(rq, qd + j * 1024, (uint32_t)(i * BM + r) * q_ss2 + cc * 16);
      buf_load_lds16(rdo, dod + j * 1024, (uint32_t)(i * BM + r) * do_ss2 + cc * 16);
    }
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

  // lane-constant operand address parts (see fa_device.h for the layouts)
  const int sw_row = slot_swizzle<D>(lane & 15);
  const int tr_r1 = 4 * hl + (i16 >> 2);
  const int sw_t1 = slot_swizzle<D>(tr_r1), sw_t2 = slot_swizzle<D>(tr_r1 + 8);
  const int tr_clo = 2 * ((lane >> 4) & 1) + ((i16 & 3) >> 1);
  const int tr_half = (i16 & 1) * 8;

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
  for (int it = 0; it < n_steps; ++it) {
    const int i = i_start + it;
    const int stage = it & 1;
    const int q0 = i * BM;
    FA_LDS char* qt = smem + stage * STAGE;
    FA_LDS char* dot = qt + QT_BYTES;
    FA_LDS float* lse_l = (FA_LDS float*)(dot + QT_BYTES);
    FA_LDS float* dvec_l = lse_l + BM;
    wait_vmem();
    if (threadIdx.x < BM) {
      lse_l[threadIdx.x] = (lse_next == -INFINITY) ? INFINITY : lse_next * kLog2e;
      dvec_l[threadIdx.x] = dvec_next;
    }
    __syncthreads();
    if (it + 1 < n_steps) {
      issue_q(i + 1, stage ^ 1);
      load_terms(i + 1);
    }

    // S = Q K^T (lane: key my_key; rows: queries q0 + 32qb + 8(r/4) + 4hl + (r&3))
    f32x16 s[2], dp[2];
    s[0] = s[1] = dp[0] = dp[1] = f32x16{};
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const int coff = ((2 * ds + hl) ^ sw_row) << 4;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const u32x4 a = lds_read16(qt + (32 * qb + (lane & 31)) * ROWB + coff);
        s[qb] = mfma_bf16(a, kreg[ds], s[qb]);
        const u32x4 ad = lds_read16(dot + (32 * qb + (lane & 31)) * ROWB + coff);
        dp[qb] = mfma_bf16(ad, vreg[ds], dp[qb]);
      }
    }

    // P = 2^(s*c - LSE*log2 e), masked; dS = P (dP - D)
    bool need_mask = (k_blk0 + BNK > Lk);
    if constexpr (CAUSAL) need_mask = need_mask || (q0 < k_blk0 + BNK);
    u32x4 pb[4], dsh[4], dsl[4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float pv[16], dsv[16];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 l2 = *(const FA_LDS f32x4*)(lse_l + 32 * qb + 8 * r4 + 4 * hl);
        const f32x4 dd = *(const FA_LDS f32x4*)(dvec_l + 32 * qb + 8 * r4 + 4 * hl);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * r4 + j;
          float pe = exp2_hw(__builtin_fmaf(s[qb][r], c, -l2[j]));
          if (need_mask) {
            const int query = q0 + 32 * qb + 8 * r4 + 4 * hl + j;
            bool hide = my_key >= Lk;
            if constexpr (CAUSAL) hide = hide || my_key > query;
            if (hide) pe = 0.0f;
          }
          pv[r] = pe;
          dsv[r] = pe * (dp[qb][r] - dd[j]);
        }
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int g = 2 * qb + half;
        uint32_t ph[4], hh[4], ll[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a0 = dsv[8 * half + 2 * e], a1 = dsv[8 * half + 2 * e + 1];
          ph[e] = pack_bf16(pv[8 * half + 2 * e], pv[8 * half + 2 * e + 1]);
          hh[e] = pack_bf16(a0, a1);
          ll[e] = pack_bf16(a0 - bf16_lo(hh[e]), a1 - bf16_hi(hh[e]));
        }
        pb[g] = u32x4{ph[0], ph[1], ph[2], ph[3]};
        dsh[g] = u32x4{hh[0], hh[1], hh[2], hh[3]};
        dsl[g] = u32x4{ll[0], ll[1], ll[2], ll[3]};
      }
    }

    // dV^T += dO^T P ; dK^T += Q^T dS  (A operands through the transpose reads)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int r1 = 16 * g + tr_r1;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int cc = 4 * db + tr_clo;
        const int o1 = r1 * ROWB + ((cc ^ sw_t1) << 4) + tr_half;
        const int o2 = (r1 + 8) * ROWB + ((cc ^ sw_t2) << 4) + tr_half;
        const u32x2 a_lo = lds_read_tr16(dot + o1), a_hi = lds_read_tr16(dot + o2);
        dvacc[db] = mfma_bf16(u32x4{a_lo[0], a_lo[1], a_hi[0], a_hi[1]}, pb[g], dvacc[db]);
        const u32x2 q_lo = lds_read_tr16(qt + o1), q_hi = lds_read_tr16(qt + o2);
        const u32x4 qa = u32x4{q_lo[0], q_lo[1], q_hi[0], q_hi[1]};
        dkacc[db] = mfma_bf16(qa, dsh[g], dkacc[db]);
        dkacc[db] = mfma_bf16(qa, dsl[g], dkacc[db]);
      }
    }

    if constexpr (DQ_ATOMIC) {
      // dS^T rows (keys) to LDS: 4 consecutive queries per 8-byte write
      const int krow = 32 * wave + (lane & 31);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int g = 2 * qb + (r4 >> 1);
          const int e = 2 * (r4 & 1);
          const int off = krow * DS_PITCH + (32 * qb + 8 * r4 + 4 * hl) * 2;
          *(FA_LDS u32x2*)(dsh_lds + off) = u32x2{dsh[g][e], dsh[g][e + 1]};
          *(FA_LDS u32x2*)(dsl_lds + off) = u32x2{dsl[g][e], dsl[g][e + 1]};
        }
      __syncthreads();
      // dQ (64 x D) = dS (64 x 128) K (128 x D): blocks (qb, db) spread over the 4 waves
      for (int blk = wave; blk < 2 * NDB; blk += 4) {
        const int qb = blk / NDB, db = blk - qb * NDB;
        f32x16 acc = f32x16{};
        const int dcol = (32 * qb + 16 * ((lane >> 4) & 1) + 4 * (i16 & 3)) * 2;
        const int cc = 4 * db + tr_clo;
#pragma unroll
        for (int g = 0; g < BNK / 16; ++g) {
          const int r1 = 16 * g + tr_r1;
          const u32x2 h1 = lds_read_tr16(dsh_lds + r1 * DS_PITCH + dcol);
          const u32x2 h2 = lds_read_tr16(dsh_lds + (r1 + 8) * DS_PITCH + dcol);
          const u32x2 l1 = lds_read_tr16(dsl_lds + r1 * DS_PITCH + dcol);
          const u32x2 l2 = lds_read_tr16(dsl_lds + (r1 + 8) * DS_PITCH + dcol);
          const u32x2 k1 = lds_read_tr16(k_lds + r1 * ROWB + ((cc ^ sw_t1) << 4) + tr_half);
          const u32x2 k2 = lds_read_tr16(k_lds + (r1 + 8) * ROWB + ((cc ^ sw_t2) << 4) + tr_half);
          const u32x4 kb = u32x4{k1[0], k1[1], k2[0], k2[1]};
          acc = mfma_bf16(u32x4{h1[0], h1[1], h2[0], h2[1]}, kb, acc);
          acc = mfma_bf16(u32x4{l1[0], l1[1], l2[0], l2[1]}, kb, acc);
        }
        const int d = 32 * db + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int query = q0 + 32 * qb + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (query < Lq) atomicAdd(p.dq_acc + (sq.rowbase + query) * D + d, acc[r] * p.scale);
        }
      }
    }
  }

  // ---- write dK = scale * dK^T acc, dV ----
  const int gb = p.grad_bf16 ? 2 : 4;
  const rsrc_t rdk = make_rsrc((char*)p.dk + sq.dkoff * gb, Lk > 0 ? (uint32_t)(Lk - 1) * (uint32_t)(p.dk_ss * gb) + D * gb : 0u);
  const rsrc_t rdv = make_rsrc((char*)p.dv + sq.dvoff * gb, Lk > 0 ? (uint32_t)(Lk - 1) * (uint32_t)(p.dv_ss * gb) + D * gb : 0u);
  const uint32_t dk_row = (uint32_t)my_key * (uint32_t)(p.dk_ss * gb);
  const uint32_t dv_row = (uint32_t)my_key * (uint32_t)(p.dv_ss * gb);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = 32 * db + 8 * r4 + 4 * hl;
      store_grad4(rdk, dk_row + d * 4, dk_row + d * 2, p.grad_bf16, dkacc[db][4 * r4] * p.scale,
                  dkacc[db][4 * r4 + 1] * p.scale, dkacc[db][4 * r4 + 2] * p.scale, dkacc[db][4 * r4 + 3] * p.scale);
      store_grad4(rdv, dv_row + d * 4, dv_row + d * 2, p.grad_bf16, dvacc[db][4 * r4], dvacc[db][4 * r4 + 1],
                  dvacc[db][4 * r4 + 2], dvacc[db][4 * r4 + 3]);
    }
}

// ---------------------------------------------------------------------------
// bwd_dq (deterministic mode): dQ for 128 query rows, no atomics.
template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdParams p) {
  constexpr int BN = kFwdBlockN;
  constexpr int ROWB = D * 2;
  constexpr int TILE_BYTES = BN * ROWB;
  constexpr int STAGE_BYTES = 2 * TILE_BYTES;
  constexpr int SLOTS = D / 8, NKB = BN / 32, NDS = D / 16, NDB = D / 32;
  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * STAGE_BYTES];
  FA_LDS char* smem = (FA_LDS char*)smem_raw;

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
    const int n_qt = (p.seqlen_q + kFwdTileRows - 1) / kFwdTileRows;
    qtile = CAUSAL ? (n_qt - 1 - t) : t;
    b = bh / p.heads;
    h = bh - b * p.heads;
  }
  const BwdSeq sq = bwd_seq(p, b, h);
  const int Lq = sq.Lq, Lk = sq.Lk;
  const int wg_q0 = qtile * kFwdTileRows;
  if (wg_q0 >= Lq) return;

  const uint32_t q_ss2 = (uint32_t)(p.q_ss * 2), do_ss2 = (uint32_t)(p.do_ss * 2);
  const uint32_t k_ss2 = (uint32_t)(p.k_ss * 2), v_ss2 = (uint32_t)(p.v_ss * 2);
  const rsrc_t rq = make_rsrc((const uint16_t*)p.q + sq.qoff, rows_bytes(Lq, p.q_ss, ROWB));
  const rsrc_t rdo = make_rsrc((const uint16_t*)p.dout + sq.dooff, rows_bytes(Lq, p.do_ss, ROWB));
  const rsrc_t rk = make_rsrc((const uint16_t*)p.k + sq.koff, rows_bytes(Lk, p.k_ss, ROWB));
  const rsrc_t rv = make_rsrc((const uint16_t*)p.v + sq.voff, rows_bytes(Lk, p.v_ss, ROWB));

  const int q0 = wg_q0 + wave * 32;
  const int my_row = q0 + (lane & 31);
  u32x4 qreg[NDS], doreg[NDS];
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) {
    qreg[ds] = buf_load16(rq, (uint32_t)my_row * q_ss2 + (2 * ds + hl) * 16);
    doreg[ds] = buf_load16(rdo, (uint32_t)my_row * do_ss2 + (2 * ds + hl) * 16);
  }
  float lse2 = INFINITY, dvec = 0.0f;
  if (my_row < Lq) {
    const float l = p.lse[sq.lseoff + my_row];
    lse2 = (l == -INFINITY) ? INFINITY : l * kLog2e;
    dvec = p.dvec[sq.rowbase + my_row];
  }

  int kv_end = Lk;
  if constexpr (CAUSAL) kv_end = min(Lk, min(Lq, wg_q0 + kFwdTileRows));
  const int n_tiles = (kv_end + BN - 1) / BN;

  auto issue_tile = [&](int t, int stage) {
    const int k0 = t * BN;
    FA_LDS char* kd = smem + stage * STAGE_BYTES;
    FA_LDS char* vd = kd + TILE_BYTES;
#pragma unroll
    for (int i = wave; i < TILE_BYTES / 1024; i += 4) {
      const int idx = i * 64 + lane;
      const int r = idx / SLOTS;
      const int cc = (idx % SLOTS) ^ slot_swizzle<D>(r);
      buf_load_lds16(rk, kd + i * 1024, (uint32_t)(k0 + r) * k_ss2 + cc * 16);
      buf_load_lds16(rv, vd + i * 1024, (uint32_t)(k0 + r) * v_ss2 + cc * 16);
    }
  };

  const int sw_row = slot_swizzle<D>(lane & 15);
  const int tr_r1 = 4 * hl + (i16 >> 2);
  const int sw_t1 = slot_swizzle<D>(tr_r1), sw_t2 = slot_swizzle<D>(tr_r1 + 8);
  const int tr_clo = 2 * ((lane >> 4) & 1) + ((i16 & 3) >> 1);
  const int tr_half = (i16 & 1) * 8;
  const float c = p.scale_log2;

  f32x16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqacc[db] = f32x16{};

  if (n_tiles > 0) issue_tile(0, 0);
  for (int t = 0; t < n_tiles; ++t) {
    const int stage = t & 1;
    wait_vmem();
    __syncthreads();
    if (t + 1 < n_tiles) issue_tile(t + 1, stage ^ 1);
    const int k0 = t * BN;
    if (CAUSAL && k0 > q0 + 31) continue;
    const FA_LDS char* kt = smem + stage * STAGE_BYTES;
    const FA_LDS char* vt = kt + TILE_BYTES;

    // S^T = K Q^T and dP^T = V dO^T (lane: query my_row; regs: keys)
    f32x16 s[NKB], dp[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = dp[kb] = f32x16{};
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const int coff = ((2 * ds + hl) ^ sw_row) << 4;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int ro = (32 * kb + (lane & 31)) * ROWB + coff;
        s[kb] = mfma_bf16(lds_read16(kt + ro), qreg[ds], s[kb]);
        dp[kb] = mfma_bf16(lds_read16(vt + ro), doreg[ds], dp[kb]);
      }
    }
    bool need_mask = (k0 + BN > Lk);
    if constexpr (CAUSAL) need_mask = need_mask || (k0 + BN - 1 > q0);
    u32x4 dsh[2 * NKB], dsl[2 * NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      float dsv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pe = exp2_hw(__builtin_fmaf(s[kb][r], c, -lse2));
        if (need_mask) {
          const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * hl + (r & 3);
          bool hide = key >= Lk;
          if constexpr (CAUSAL) hide = hide || key > my_row;
          if (hide) pe = 0.0f;
        }
        dsv[r] = pe * (dp[kb][r] - dvec);
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint32_t hh[4], ll[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a0 = dsv[8 * half + 2 * e], a1 = dsv[8 * half + 2 * e + 1];
          hh[e] = pack_bf16(a0, a1);
          ll[e] = pack_bf16(a0 - bf16_lo(hh[e]), a1 - bf16_hi(hh[e]));
        }
        dsh[2 * kb + half] = u32x4{hh[0], hh[1], hh[2], hh[3]};
        dsl[2 * kb + half] = u32x4{ll[0], ll[1], ll[2], ll[3]};
      }
    }
    // dQ^T += K^T dS^T (A = K^T through the transpose reads)
#pragma unroll
    for (int g = 0; g < BN / 16; ++g) {
      const int r1 = 16 * g + tr_r1;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int cc = 4 * db + tr_clo;
        const u32x2 lo = lds_read_tr16(kt + r1 * ROWB + ((cc ^ sw_t1) << 4) + tr_half);
        const u32x2 hi = lds_read_tr16(kt + (r1 + 8) * ROWB + ((cc ^ sw_t2) << 4) + tr_half);
        const u32x4 a = u32x4{lo[0], lo[1], hi[0], hi[1]};
        dqacc[db] = mfma_bf16(a, dsh[g], dqacc[db]);
        dqacc[db] = mfma_bf16(a, dsl[g], dqacc[db]);
      }
    }
  }

  const int gb = p.grad_bf16 ? 2 : 4;
  const rsrc_t rdq = make_rsrc((char*)p.dq + sq.dqoff * gb, (uint32_t)(Lq - 1) * (uint32_t)(p.dq_ss * gb) + D * gb);
  const uint32_t row_off = (uint32_t)my_row * (uint32_t)(p.dq_ss * gb);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = 32 * db + 8 * r4 + 4 * hl;
      store_grad4(rdq, row_off + d * 4, row_off + d * 2, p.grad_bf16, dqacc[db][4 * r4] * p.scale,
                  dqacc[db][4 * r4 + 1] * p.scale, dqacc[db][4 * r4 + 2] * p.scale, dqacc[db][4 * r4 + 3] * p.scale);
    }
}

// ---------------------------------------------------------------------------
// Longest-first list of key blocks for variable-length batches: cost of key block
// j of sequence b = number of 64-row query steps it visits.
__global__ __launch_bounds__(1024) void sched_kv_kernel(const int32_t* cu_q, const int32_t* cu_k, int batch,
                                                        int causal, int32_t* out) {
  __shared__ int hist[kSchedMaxCost + 1];
  __shared__ int total;
  for (int i = threadIdx.x; i <= kSchedMaxCost; i += blockDim.x) hist[i] = 0;
  if (threadIdx.x == 0) total = 0;
  __syncthreads();
  auto cost_of = [&](int b, int j) {
    const int lq = cu_q[b + 1] - cu_q[b];
    const int steps = (lq + kBwdBlockM - 1) / kBwdBlockM;
    const int first = causal ? (j * kBwdBlockN) / kBwdBlockM : 0;
    return min(max(steps - first, 0), kSchedMaxCost);
  };
  for (int b = threadIdx.x; b < batch; b += blockDim.x) {
    const int lk = cu_k[b + 1] - cu_k[b];
    const int nb = (lk + kBwdBlockN - 1) / kBwdBlockN;
    for (int j = 0; j < nb; ++j) atomicAdd(&hist[cost_of(b, j)], 1);
    atomicAdd(&total, nb);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int c = kSchedMaxCost; c >= 0; --c) {
      const int n = hist[c];
      hist[c] = run;
      run += n;
    }
    out[0] = total;
  }
  __syncthreads();
  for (int b = threadIdx.x; b < batch; b += blockDim.x) {
    const int lk = cu_k[b + 1] - cu_k[b];
    const int nb = (lk + kBwdBlockN - 1) / kBwdBlockN;
    for (int j = 0; j < nb; ++j) {
      const int pos = atomicAdd(&hist[cost_of(b, j)], 1);
      out[1 + 2 * pos] = b;
      out[2 + 2 * pos] = j;
    }
  }
}

template <int D>
static hipError_t launch_bwd_d(const BwdParams& p, int phases, hipStream_t stream) {
  const bool atomic = !p.deterministic;
  const int64_t rows = (int64_t)p.total_q * p.heads;
  if (phases & 1) {
    int64_t work = rows * (D / 8);
    int grid = (int)std::min<int64_t>((work + 255) / 256, 2048 * 4);
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3(grid), dim3(256), 0, stream, p, atomic ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
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
#define FA_KV(C, V, A) hipLaunchKernelGGL((bwd_kv_kernel<D, C, V, A>), dim3(grid), dim3(256), 0, stream, p)
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
  if (atomic) {
    if (!(phases & 4)) return hipSuccess;
    int64_t work = rows * (D / 4);
    int grid = (int)std::min<int64_t>((work + 255) / 256, 2048 * 4);
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(bwd_post_kernel<D>, dim3(grid), dim3(256), 0, stream, p);
    return hipGetLastError();
  }
  // deterministic: query-major dQ kernel; its list reuses the forward's query-tile order
  if (!(phases & 2)) return hipSuccess;
  unsigned grid;
  int32_t* qsched = p.sched + 1 + 2 * ((p.total_k + kBwdBlockN - 1) / kBwdBlockN + p.batch);
  if (p.varlen) {
    hipError_t e = launch_fwd_schedule(p.cu_q, p.cu_k, p.batch, kFwdTileRows, kFwdBlockN, p.causal, qsched, stream);
    if (e != hipSuccess) return e;
    grid = (unsigned)((p.total_q + kFwdTileRows - 1) / kFwdTileRows + p.batch) * (unsigned)p.heads;
  } else {
    grid = (unsigned)((p.seqlen_q + kFwdTileRows - 1) / kFwdTileRows) * (unsigned)(p.batch * p.heads);
  }
  if (grid == 0) return hipSuccess;
  BwdParams pq = p;
  pq.sched = qsched;
#define FA_DQ(C, V) hipLaunchKernelGGL((bwd_dq_kernel<D, C, V>), dim3(grid), dim3(256), 0, stream, pq)
  if (p.causal) { if (p.varlen) FA_DQ(true, true); else FA_DQ(true, false); }
  else { if (p.varlen) FA_DQ(false, true); else FA_DQ(false, false); }
#undef FA_DQ
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdParams& p, int phases, hipStream_t stream) {
  return p.head_dim == 128 ? launch_bwd_d<128>(p, phases, stream) : launch_bwd_d<64>(p, phases, stream);
}

}  // namespace fa
