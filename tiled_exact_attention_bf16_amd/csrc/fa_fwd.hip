// Forward pass of exact tiled attention for gfx950.
//
// Method (FlashAttention-4 pages): Q is tiled against K/V; each key tile's scores
// S = Q K^T are turned into weights by an online softmax that keeps every row's
// running maximum and running sum on chip, the output O = P V is accumulated tile
// by tile, and O plus the log-sum-exp are written at the end, so the score matrix
// never reaches device memory (fdeinterviews.com FA4 summary, opening paragraph;
// lecompute.fr FA4 article, section "Between the matrix products the kernel must
// produce weights").  The output is rescaled only when a row maximum grows by more
// than 8 in log2 units ("Lazy rescaling" bullet), part of the exponentials may run
// on the FMA units ("Software exponentials" bullet), two query tiles share each
// workgroup so one tile's softmax overlaps the other's matrix products ("Pipeline
// for asynchronous tensor cores" bullet), and work items are dispatched longest
// first (features paragraph).
//
// gfx950 mapping:
//   * a workgroup owns 128*NQT query rows of one (sequence, head); each wave owns
//     32 rows and keeps Q in registers as the B operand of S^T = K Q^T, so every
//     lane holds one query row: row max/sum are lane-local plus one
//     v_permlane32_swap between the two halves of the wave;
//   * K and V tiles of 64 keys are staged into LDS by buffer->LDS DMA loads into a
//     double buffer (the next tile streams in while the current one is used), with
//     an XOR swizzle that keeps the operand reads bank-conflict free;
//   * P goes from the S^T accumulators straight into the B operand of
//     O^T = V^T P^T; V^T comes from ds_read_b64_tr_b16 transpose reads;
//   * the O^T accumulators also hold one query row per lane, so the rescale factor
//     is a per-lane scalar.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

template <int D, int NQT, bool CAUSAL, bool VARLEN, int POLY, int TAU>
__global__ __launch_bounds__(256 * NQT) void fwd_kernel(FwdParams p) {
  constexpr int BN = kFwdBlockN;
  constexpr int NW = 4 * NQT;
  constexpr int WG_ROWS = kFwdTileRows * NQT;
  constexpr int ROWB = D * 2;                 // bytes of one K/V row
  constexpr int TILE_BYTES = BN * ROWB;       // one K or V tile
  constexpr int STAGE_BYTES = 2 * TILE_BYTES; // K + V
  constexpr int SLOTS = D / 8;                // 16-byte slots per row
  constexpr int NKB = BN / 32;                // 32-key blocks per tile
  constexpr int NDS = D / 16;                 // k-steps of the QK product
  constexpr int NDB = D / 32;                 // 32-wide blocks of head_dim
  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * STAGE_BYTES];
  FA_LDS char* smem = (FA_LDS char*)smem_raw;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane >> 5;

  // ---- work item ----
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
    qtile = CAUSAL ? (p.n_qtiles - 1 - t) : t;  // longest first under the causal mask
    b = bh / p.heads;
    h = bh - b * p.heads;
  }
  int Lq = p.seqlen_q, Lk = p.seqlen_k;
  int64_t qoff, koff, voff, ooff, lseoff;
  if constexpr (VARLEN) {
    const int sq = p.cu_q[b], sk = p.cu_k[b];
    Lq = p.cu_q[b + 1] - sq;
    Lk = p.cu_k[b + 1] - sk;
    qoff = sq * p.q_ss + h * p.q_sh;
    koff = sk * p.k_ss + h * p.k_sh;
    voff = sk * p.v_ss + h * p.v_sh;
    ooff = sq * p.o_ss + h * p.o_sh;
    lseoff = (int64_t)h * p.total_q + sq;
  } else {
    qoff = b * p.q_sb + h * p.q_sh;
    koff = b * p.k_sb + h * p.k_sh;
    voff = b * p.v_sb + h * p.v_sh;
    ooff = b * p.o_sb + h * p.o_sh;
    lseoff = ((int64_t)b * p.heads + h) * Lq;
  }
  const int wg_q0 = qtile * WG_ROWS;
  if (wg_q0 >= Lq) return;

  const uint32_t q_ss2 = (uint32_t)(p.q_ss * 2), k_ss2 = (uint32_t)(p.k_ss * 2);
  const uint32_t v_ss2 = (uint32_t)(p.v_ss * 2), o_ss2 = (uint32_t)(p.o_ss * 2);
  const rsrc_t rq = make_rsrc((const char*)p.q + qoff * 2, (uint32_t)(Lq - 1) * q_ss2 + ROWB);
  const rsrc_t rk = make_rsrc((const char*)p.k + koff * 2, Lk > 0 ? (uint32_t)(Lk - 1) * k_ss2 + ROWB : 0u);
  const rsrc_t rv = make_rsrc((const char*)p.v + voff * 2, Lk > 0 ? (uint32_t)(Lk - 1) * v_ss2 + ROWB : 0u);
  const rsrc_t ro = make_rsrc((char*)p.o + ooff * 2, (uint32_t)(Lq - 1) * o_ss2 + ROWB);

  // ---- rows of this wave; Q as B operand (lane: row, 8 consecutive d) ----
  const int q0 = wg_q0 + (wave >> 2) * kFwdTileRows + (wave & 3) * 32;
  const int my_row = q0 + (lane & 31);
  u32x4 qreg[NDS];
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) qreg[ds] = buf_load16(rq, (uint32_t)my_row * q_ss2 + (2 * ds + hl) * 16);

  int kv_end = Lk;
  if constexpr (CAUSAL) kv_end = min(Lk, min(Lq, wg_q0 + WG_ROWS));
  const int n_tiles = (kv_end + BN - 1) / BN;

  // ---- K/V stage loader: every wave issues its share of 1 KiB DMA packets ----
  auto issue_tile = [&](int t, int stage) {
    const int k0 = t * BN;
    FA_LDS char* kd = smem + stage * STAGE_BYTES;
    FA_LDS char* vd = kd + TILE_BYTES;
#pragma unroll
    for (int i = wave; i < TILE_BYTES / 1024; i += NW) {
      const int idx = i * 64 + lane;
      const int r = idx / SLOTS;
      const int c = (idx % SLOTS) ^ slot_swizzle<D>(r);
      buf_load_lds16(rk, kd + i * 1024, (uint32_t)(k0 + r) * k_ss2 + c * 16);
      buf_load_lds16(rv, vd + i * 1024, (uint32_t)(k0 + r) * v_ss2 + c * 16);
    }
  };

  // lane-constant parts of the LDS operand addresses
  const int sw_k = slot_swizzle<D>(lane & 15);                    // K rows 32kb + (lane&31)
  const int i16 = lane & 15;
  const int vr1 = 4 * hl + (i16 >> 2);                             // V rows (mod 16) of the tr reads
  const int sw_v1 = slot_swizzle<D>(vr1), sw_v2 = slot_swizzle<D>(vr1 + 8);
  const int vc_lo = 2 * ((lane >> 4) & 1) + ((i16 & 3) >> 1);      // chunk within a 32-d block
  const int vhalf = (i16 & 1) * 8;

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_used = -INFINITY;
  float lsum = 0.0f;    // sum of fp32 weights
  float lsum_r = 0.0f;  // sum of bf16-rounded weights
  const float c = p.scale_log2;

  // Under the causal mask a wave's rows stop seeing keys before the workgroup's
  // last tile; it then only helps stage K/V (second loop) and keeps the barriers.
  int n_mine = n_tiles;
  if constexpr (CAUSAL) n_mine = min(n_tiles, (q0 + 31) / BN + 1);
  if (n_tiles > 0) issue_tile(0, 0);
  int t = 0;
  for (; t < n_mine; ++t) {
    const int stage = t & 1;
    wait_vmem();
    __syncthreads();
    if (t + 1 < n_tiles) issue_tile(t + 1, stage ^ 1);
    const int k0 = t * BN;

    const FA_LDS char* kt = smem + stage * STAGE_BYTES;
    const FA_LDS char* vt = kt + TILE_BYTES;

    // S^T = K Q^T : lane holds query my_row, keys k0 + 32kb + 8(r/4) + 4hl + (r&3)
    f32x16 sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const int coff = ((2 * ds + hl) ^ sw_k) << 4;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const u32x4 a = lds_read16(kt + (32 * kb + (lane & 31)) * ROWB + coff);
        sacc[kb] = mfma_bf16(a, qreg[ds], sacc[kb]);
      }
    }

    // mask: causal diagonal tiles and the ragged last tile only
    bool need_mask = (k0 + BN > Lk);
    if constexpr (CAUSAL) need_mask = need_mask || (k0 + BN - 1 > q0);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * hl + (r & 3);
          bool hide = key >= Lk;
          if constexpr (CAUSAL) hide = hide || key > my_row;
          if (hide) sacc[kb][r] = -INFINITY;
        }
    }

    // row maximum of this tile (lane-local, then across the two wave halves)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = half_swap_max(mx);

    // lazy rescale: move the reference only when the maximum grew by more than TAU
    const float m_new = fmaxf(m_used, mx);
    bool need = m_new > m_used;
    if constexpr (TAU > 0) need = need && (m_used == -INFINITY || (m_new - m_used) * c > (float)TAU);
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float alpha = need ? (m_used == -INFINITY ? 0.0f : exp2_hw((m_used - m_new) * c)) : 1.0f;
      m_used = need ? m_new : m_used;
      lsum *= alpha;
      lsum_r *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }

    // P = 2^(s*c - m*c) -> bf16 operands.  Two row sums: of the fp32 weights (for
    // the LSE) and of the bf16-rounded weights the PV product actually uses (for
    // normalising O, so a dominant weight's rounding cancels between numerator and
    // denominator; with a stale reference that weight is up to 2^8, not 1).
    const float mref = (m_used == -INFINITY) ? 0.0f : m_used * c;
    float rs = 0.0f, rsr = 0.0f;
    u32x4 pb[2 * NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      float pv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = __builtin_fmaf(sacc[kb][r], c, -mref);
        pv[r] = (r < POLY) ? exp2_poly(x) : exp2_hw(x);
        rs += pv[r];
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w[e] = pack_bf16(pv[8 * half + 2 * e], pv[8 * half + 2 * e + 1]);
          rsr = add_bf16_pair(w[e], rsr);
        }
        pb[2 * kb + half] = u32x4{w[0], w[1], w[2], w[3]};
      }
    }
    lsum += rs;
    lsum_r += rsr;

    // O^T += V^T P^T : A operand = V^T through the transpose reads
#pragma unroll
    for (int g = 0; g < BN / 16; ++g) {
      const int r1 = 16 * g + vr1;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int cc = 4 * db + vc_lo;
        const u32x2 lo = lds_read_tr16(vt + r1 * ROWB + ((cc ^ sw_v1) << 4) + vhalf);
        const u32x2 hi = lds_read_tr16(vt + (r1 + 8) * ROWB + ((cc ^ sw_v2) << 4) + vhalf);
        oacc[db] = mfma_bf16(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb[g], oacc[db]);
      }
    }
  }
  for (; t < n_tiles; ++t) {
    wait_vmem();
    __syncthreads();
    if (t + 1 < n_tiles) issue_tile(t + 1, (t & 1) ^ 1);
  }

  // ---- epilogue: O = O_acc / l, LSE = m*scale + ln l ----
  const float lt = half_swap_sum(lsum);
  const float ltr = half_swap_sum(lsum_r);
  const float inv = ltr > 0.0f ? 1.0f / ltr : 0.0f;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = 32 * db + 8 * q4 + 4 * hl;
      const u32x2 w = {pack_bf16(oacc[db][4 * q4 + 0] * inv, oacc[db][4 * q4 + 1] * inv),
                       pack_bf16(oacc[db][4 * q4 + 2] * inv, oacc[db][4 * q4 + 3] * inv)};
      buf_store8(ro, (uint32_t)my_row * o_ss2 + d * 2, w);
    }
  if (hl == 0 && my_row < Lq) {
    float lse = -INFINITY;
    if (lt > 0.0f) lse = (m_used * c + __builtin_amdgcn_logf(lt)) * 0.69314718055994531f;
    p.lse[lseoff + my_row] = lse;
  }
}

// ---- longest-first work list for packed variable-length batches ----
// One workgroup: histogram of item costs (key tiles visited), exclusive scan from
// the most expensive bin down, scatter.  Items of equal cost may land in any order.
__global__ __launch_bounds__(1024) void sched_kernel(const int32_t* cu_q, const int32_t* cu_k, int batch,
                                                     int tile_rows, int block_n, int causal, int32_t* out) {
  __shared__ int hist[kSchedMaxCost + 1];
  __shared__ int total;
  for (int i = threadIdx.x; i <= kSchedMaxCost; i += blockDim.x) hist[i] = 0;
  if (threadIdx.x == 0) total = 0;
  __syncthreads();
  auto cost_of = [&](int b, int t) {
    const int lq = cu_q[b + 1] - cu_q[b];
    const int lk = cu_k[b + 1] - cu_k[b];
    int kv = lk;
    if (causal) kv = min(lk, min(lq, (t + 1) * tile_rows));
    return min((kv + block_n - 1) / block_n, kSchedMaxCost);
  };
  for (int b = threadIdx.x; b < batch; b += blockDim.x) {
    const int lq = cu_q[b + 1] - cu_q[b];
    const int nt = (lq + tile_rows - 1) / tile_rows;
    for (int t = 0; t < nt; ++t) atomicAdd(&hist[cost_of(b, t)], 1);
    atomicAdd(&total, nt);
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
    const int lq = cu_q[b + 1] - cu_q[b];
    const int nt = (lq + tile_rows - 1) / tile_rows;
    for (int t = 0; t < nt; ++t) {
      const int pos = atomicAdd(&hist[cost_of(b, t)], 1);
      out[1 + 2 * pos] = b;
      out[2 + 2 * pos] = t;
    }
  }
}

hipError_t launch_fwd_schedule(const int32_t* cu_q, const int32_t* cu_k, int batch, int tile_rows,
                               int block_n, bool causal, int32_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(1024), 0, stream, cu_q, cu_k, batch, tile_rows, block_n,
                     causal ? 1 : 0, out);
  return hipGetLastError();
}

template <int D, int NQT, bool CAUSAL, bool VARLEN, int POLY, int TAU>
static hipError_t launch_one(const FwdParams& p, hipStream_t stream, int max_items) {
  const int items = VARLEN ? max_items : p.n_qtiles * p.batch;
  const unsigned grid = (unsigned)items * (unsigned)p.heads;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_kernel<D, NQT, CAUSAL, VARLEN, POLY, TAU>), dim3(grid), dim3(256 * NQT), 0, stream, p);
  return hipGetLastError();
}

template <int D, int NQT, bool CAUSAL, bool VARLEN>
static hipError_t dispatch_poly_tau(const FwdParams& p, const FwdConfig& cfg, hipStream_t s, int mi) {
  if (cfg.tau == 8) {
    switch (cfg.poly_per16) {
      case 0: return launch_one<D, NQT, CAUSAL, VARLEN, 0, 8>(p, s, mi);
      case 2: return launch_one<D, NQT, CAUSAL, VARLEN, 2, 8>(p, s, mi);
      case 4: return launch_one<D, NQT, CAUSAL, VARLEN, 4, 8>(p, s, mi);
    }
  } else if (cfg.tau == 0 && cfg.poly_per16 == 0) {
    return launch_one<D, NQT, CAUSAL, VARLEN, 0, 0>(p, s, mi);
  }
  return hipErrorInvalidValue;
}

template <int D, int NQT>
static hipError_t dispatch_mask(const FwdParams& p, const FwdConfig& cfg, hipStream_t s, int mi) {
  if (cfg.varlen) {
    return cfg.causal ? dispatch_poly_tau<D, NQT, true, true>(p, cfg, s, mi)
                      : dispatch_poly_tau<D, NQT, false, true>(p, cfg, s, mi);
  }
  return cfg.causal ? dispatch_poly_tau<D, NQT, true, false>(p, cfg, s, mi)
                    : dispatch_poly_tau<D, NQT, false, false>(p, cfg, s, mi);
}

hipError_t launch_fwd(const FwdParams& p, const FwdConfig& cfg, hipStream_t stream) {
  const int wg_rows = kFwdTileRows * cfg.q_tiles;
  const int max_items = (p.total_q + wg_rows - 1) / wg_rows + p.batch;
  if (cfg.head_dim == 128) {
    return cfg.q_tiles == 2 ? dispatch_mask<128, 2>(p, cfg, stream, max_items)
                            : dispatch_mask<128, 1>(p, cfg, stream, max_items);
  }
  return cfg.q_tiles == 2 ? dispatch_mask<64, 2>(p, cfg, stream, max_items)
                          : dispatch_mask<64, 1>(p, cfg, stream, max_items);
}

}  // namespace fa
