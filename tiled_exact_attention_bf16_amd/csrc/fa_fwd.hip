// Forward pass of exact tiled attention for gfx950.
//
// Method (FlashAttention-4 pages): Q is tiled against K/V; each key tile's scores
// S = Q K^T are turned into weights by an online softmax that keeps every row's
// running maximum and running sum on chip, the output O = P V is accumulated tile
// by tile, and O plus the log-sum-exp are written at the end, so the score matrix
// never reaches device memory (fdeinterviews.com FA4 summary, opening paragraph;
// lecompute.fr FA4 article, section "Between the matrix products the kernel must
// produce weights").  A row's reference maximum -- and with it the accumulated
// output -- is moved only once the true maximum exceeds it by over 8 in base-2
// exponent units ("Lazy rescaling" bullet), part of the exponentials may run
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
//     O^T = V^T P^T, rounded to fp16: with the lazy reference a row's largest
//     weights sit up to 2^8 above it, and bf16's 8 significant bits then leave an
//     error near 1e-2 on outputs of magnitude 2-4, where fp16's 11 bits do not.  V is
//     read from an fp16 copy made by vprep_kernel, each 64-key tile scaled by a
//     power of two 2^-e so that the copy is exact; the tile's weights carry the
//     factor 2^e back (it is folded into the exponent argument), so P'V' = PV;
//     V^T comes from ds_read_b64_tr_b16 transpose reads;
//   * the O^T accumulators also hold one query row per lane, so the rescale factor
//     is a per-lane scalar;
//   * with two query tiles per workgroup (the default) the tiles run in ping-pong:
//     wave w (first tile) and wave w+4 (second tile) share a SIMD, and in each half
//     step one of them issues the step's 32 MFMAs while the other forms its weights,
//     so that the vector work runs beside matrix products of the other wave.  The
//     row sum there is a plain fp32 sum: v_dot2 executes on the matrix pipeline and
//     would wait behind the other wave's MFMAs.
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

template <int D, int NQT, bool CAUSAL, bool VARLEN, int POLY, int TAU, bool SPLIT = false>
__global__ __launch_bounds__(256 * NQT, 2) void fwd_kernel(FwdParams p) {
  constexpr int BN = kFwdBlockN;
  constexpr int NW = 4 * NQT;
  constexpr int WG_ROWS = kFwdTileRows * NQT;
  constexpr int ROWB = D * 2;                 // bytes of one K/V row
  constexpr int TILE_BYTES = BN * ROWB;       // one K or V tile
  constexpr int SLOTS = D / 8;                // 16-byte slots per row
  constexpr int NKB = BN / 32;                // 32-key blocks per tile
  constexpr int NDS = D / 16;                 // k-steps of the QK product
  constexpr int NDB = D / 32;                 // 32-wide blocks of head_dim
  // The main path forms fp16 weights against the fp16 copy of V (the lazy reference
  // leaves weights up to 2^8, which bf16 would round too coarsely).  The key-split path
  // serves short query blocks against long keys, where reading K and V bounds the time
  // and an fp16 copy of V would double V's traffic: it reads V itself, with bf16
  // weights and eager rescaling (every row's largest weight stays exactly 1, and a
  // rescale costs nothing there).  With the largest weight exactly 1 the others'
  // bf16 rounding stays small against the sum, so it normalises O and forms the LSE
  // from the fp32 weights' sum.
  constexpr bool F16 = !SPLIT;
  // two query tiles per workgroup run in ping-pong (one tile's matrix products beside
  // the other's weights); one tile per workgroup and the key split pipeline each
  // wave's own step instead
  constexpr bool PP = NQT == 2 && !SPLIT;
  // Two K buffers and two V buffers (K runs one tile ahead of V), declared as
  // separate objects: the compiler can then tell that the buffers a step reads are
  // not the ones its DMA loads are filling, and does not make the reads wait for
  // those loads.
  __shared__ __attribute__((aligned(1024))) char k_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char k_lds1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds1[TILE_BYTES];
  auto kbuf = [&](int par) { return (FA_LDS char*)(par ? k_lds1 : k_lds0); };
  auto vbuf = [&](int par) { return (FA_LDS char*)(par ? v_lds1 : v_lds0); };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane >> 5;

  // ---- work item (and key chunk when the keys are split) ----
  const int chunk = SPLIT ? (int)(blockIdx.x % (unsigned)p.n_split) : 0;
  const int wid = SPLIT ? (int)(blockIdx.x / (unsigned)p.n_split) : (int)blockIdx.x;
  int b, h, qtile;
  if constexpr (VARLEN) {
    const int item = wid / p.heads;
    h = wid - item * p.heads;
    if (item >= p.sched[0]) return;
    b = p.sched[1 + 2 * item];
    qtile = p.sched[2 + 2 * item];
  } else {
    const int bh_count = p.batch * p.heads;
    const int t = wid / bh_count;
    const int bh = wid - t * bh_count;
    qtile = CAUSAL ? (p.n_qtiles - 1 - t) : t;  // longest first under the causal mask
    b = bh / p.heads;
    h = bh - b * p.heads;
  }
  int Lq = p.seqlen_q, Lk = p.seqlen_k;
  int64_t qoff, koff, voff, ooff, lseoff;
  int64_t krow0;  // first key row of the sequence among all key rows (the fp16 V copy's rows)
  if constexpr (VARLEN) {
    const int sq = p.cu_q[b], sk = p.cu_k[b];
    Lq = p.cu_q[b + 1] - sq;
    Lk = p.cu_k[b + 1] - sk;
    qoff = sq * p.q_ss + h * p.q_sh;
    koff = sk * p.k_ss + h * p.k_sh;
    voff = sk * p.v_ss + h * p.v_sh;
    ooff = sq * p.o_ss + h * p.o_sh;
    lseoff = (int64_t)h * p.total_q + sq;
    krow0 = sk;
  } else {
    qoff = b * p.q_sb + h * p.q_sh;
    koff = b * p.k_sb + h * p.k_sh;
    voff = b * p.v_sb + h * p.v_sh;
    ooff = b * p.o_sb + h * p.o_sh;
    lseoff = ((int64_t)b * p.heads + h) * Lq;
    krow0 = (int64_t)b * Lk;
  }
  const int wg_q0 = qtile * WG_ROWS;
  if (wg_q0 >= Lq) return;
  // causal: row i sees keys j <= i + coff (the mask's diagonal ends at the last query
  // and the last key; coff = 0 for equal lengths)
  int coff = Lk - Lq;
  int64_t row_base = 0;  // this sequence's first row among all query rows (split output)
  if constexpr (SPLIT) {
    // chunk `chunk` of the key tiles: shift K/V to its first key and shrink Lk
    row_base = VARLEN ? (int64_t)p.cu_q[b] : (int64_t)b * Lq;
    const int tiles = (Lk + kFwdBlockN - 1) / kFwdBlockN;
    const int per = (tiles + p.n_split - 1) / p.n_split;
    const int kbase = min(chunk * per, tiles) * kFwdBlockN;
    koff += (int64_t)kbase * p.k_ss;
    voff += (int64_t)kbase * p.v_ss;
    krow0 += kbase;
    Lk = max(0, min(Lk - kbase, per * kFwdBlockN));
    coff -= kbase;
  }

  const uint32_t q_ss2 = (uint32_t)(p.q_ss * 2), k_ss2 = (uint32_t)(p.k_ss * 2);
  const uint32_t v_ss2 = F16 ? (uint32_t)ROWB : (uint32_t)(p.v_ss * 2), o_ss2 = (uint32_t)(p.o_ss * 2);
  const rsrc_t rq = make_rsrc((const char*)p.q + qoff * 2, (uint32_t)(Lq - 1) * q_ss2 + ROWB);
  const rsrc_t rk = make_rsrc((const char*)p.k + koff * 2, Lk > 0 ? (uint32_t)(Lk - 1) * k_ss2 + ROWB : 0u);
  // the fp16 copy of V: rows of this (sequence, head) are contiguous, ROWB bytes apart
  const int64_t vrow = (int64_t)h * p.total_k + krow0;
  const rsrc_t rv = F16 ? make_rsrc(p.v16 + vrow * D, Lk > 0 ? (uint32_t)Lk * ROWB : 0u)
                        : make_rsrc((const char*)p.v + voff * 2, Lk > 0 ? (uint32_t)(Lk - 1) * v_ss2 + ROWB : 0u);
  // tile j's exponent at v_exp[j * BN], read through the constant address space so that
  // it is a scalar load: a vector load would share vmcnt with the K/V DMA loads, and
  // waiting for it would wait for them
  const FA_CONST int32_t* v_exp = (const FA_CONST int32_t*)(p.v_exp + vrow);
  const rsrc_t ro = make_rsrc((char*)p.o + ooff * 2, (uint32_t)(Lq - 1) * o_ss2 + ROWB);

  // ---- rows of this wave; Q as B operand (lane: row, 8 consecutive d) ----
  const int q0 = wg_q0 + (wave >> 2) * kFwdTileRows + (wave & 3) * 32;
  const int my_row = q0 + (lane & 31);
  u32x4 qreg[NDS];
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) qreg[ds] = buf_load16(rq, (uint32_t)my_row * q_ss2 + (2 * ds + hl) * 16);

  int kv_end = Lk;
  if constexpr (CAUSAL) kv_end = max(0, min(Lk, min(Lq, wg_q0 + WG_ROWS) + coff));
  const int n_tiles = (kv_end + BN - 1) / BN;

  // ---- tile loaders: every wave issues its share of 1 KiB DMA packets ----
  auto issue = [&](const rsrc_t& rsrc, uint32_t ss2, int t, FA_LDS char* dst) {
    const int k0 = t * BN;
#pragma unroll
    for (int i = wave; i < TILE_BYTES / 1024; i += NW) {
      const int idx = i * 64 + lane;
      const int r = idx / SLOTS;
      const int cs = (idx % SLOTS) ^ slot_swizzle<D>(r);
      buf_load_lds16(rsrc, dst + i * 1024, (uint32_t)(k0 + r) * ss2 + cs * 16);
    }
    dma_issued();
  };

  // lane-constant LDS offsets within a tile buffer: with the buffer index a
  // compile-time constant every K/V read is one register plus an immediate
  const int sw_k = slot_swizzle<D>(lane & 15);                    // K rows 32kb + (lane&31)
  const int i16 = lane & 15;
  const int vr1 = 4 * hl + (i16 >> 2);                             // V rows (mod 16) of the tr reads
  const int sw_v1 = slot_swizzle<D>(vr1), sw_v2 = slot_swizzle<D>(vr1 + 8);
  const int vc_lo = 2 * ((lane >> 4) & 1) + ((i16 & 3) >> 1);      // chunk within a 32-d block
  const int vhalf = (i16 & 1) * 8;
  int off_k[NDS], off_v1[NDB], off_v2[NDB];
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) off_k[ds] = (lane & 31) * ROWB + (((2 * ds + hl) ^ sw_k) << 4);
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int cc = 4 * db + vc_lo;
    off_v1[db] = vr1 * ROWB + ((cc ^ sw_v1) << 4) + vhalf;
    off_v2[db] = (vr1 + 8) * ROWB + ((cc ^ sw_v2) << 4) + vhalf;
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_used = -INFINITY;
  float mref = 0.0f;    // m_used * c once a row has seen a key
  float mref_x = 0.0f;  // mref - e of the tile whose weights are formed next (weights carry 2^e)
  float esc = 1.0f;     // 2^-e of that tile: its weight sums back in true units
  // One row sum serves both O and LSE.  The ping-pong path and the key-split path
  // sum the fp32 weights.  The one-tile path sums the fp16-rounded weights the PV
  // products used: O normalised by it has a dominant weight's rounding cancel between
  // numerator and denominator, and since every weight rounds with relative error
  // <= 2^-11, ln of it is within 4.9e-4 of ln of the exact sum.
  float lsum_r = 0.0f;
  const float c = p.scale_log2;

  // Under the causal mask a wave's rows stop seeing keys before the workgroup's
  // last tile; it then only helps stage K/V and keeps the barriers.
  int n_mine = q0 < Lq ? n_tiles : 0;  // a wave whose rows are all past the end only helps stage K/V
  if constexpr (CAUSAL) n_mine = (q0 >= Lq || q0 + 31 + coff < 0) ? 0 : min(n_tiles, (q0 + 31 + coff) / BN + 1);

  // ---- (one query tile per workgroup, and the key split) one pipelined step j of a
  // wave: S(j) = K(j) Q^T runs on the matrix cores while the
  // weights of tile j-1 are exponentiated; then O^T += V(j-1)^T P(j-1)^T runs
  // while the row maxima of S(j) are reduced.  Each wave's instruction stream thus
  // alternates matrix and vector work: a few vector instructions issued after an
  // MFMA run while it executes, and the other wave on the SIMD fills the rest.
  // K(j) sits in K buffer j&1, V(j-1) in V buffer (j-1)&1; the loads of K(j+1) and
  // V(j) are issued between the MFMAs of phase 1 of step j and waited for at the
  // barrier that opens step j+1.
  auto step = [&](const int j, auto par_c, auto prev_c, auto next_c, auto mask_c, f32x16(&s_prev)[NKB],
                  f32x16(&s_next)[NKB]) {
    constexpr int PAR = decltype(par_c)::value;
    constexpr bool PREV = decltype(prev_c)::value;  // tile j-1 exists: softmax + PV
    constexpr bool NEXT = decltype(next_c)::value;  // tile j exists for this wave: S + max
    constexpr bool MASK = decltype(mask_c)::value;  // tile j may hold keys this wave must not see
    wait_vmem();
    __syncthreads();
    // this wave's packets of K(j+1) and V(j) (the last tile again past the end, into
    // the buffer no product reads any more): part u is packet wave + NW (u % PW) of K
    // (u < PW) or of V, one after every second MFMA of phase 1
    constexpr int PW = TILE_BYTES / 1024 / NW;
    static_assert(PW * NW * 1024 == TILE_BYTES && (NW * 64 / SLOTS) % 16 == 0, "packet layout");
    auto part = [&](const int u) __attribute__((always_inline)) {
      const int l_row = (wave * 64 + lane) / SLOTS;
      const int l_cs = ((wave * 64 + lane) % SLOTS) ^ slot_swizzle<D>(l_row);
      const int k = u % PW;
      if (u < PW) {
        const int t = max(0, min(j + 1, n_tiles - 1));
        buf_load_lds16(rk, kbuf(PAR ^ 1) + (wave + NW * k) * 1024,
                       (uint32_t)(t * BN + k * (NW * 64 / SLOTS) + l_row) * k_ss2 + l_cs * 16);
      } else {
        const int t = max(0, min(j, n_tiles - 1));
        buf_load_lds16(rv, vbuf(PAR) + (wave + NW * k) * 1024,
                       (uint32_t)(t * BN + k * (NW * 64 / SLOTS) + l_row) * v_ss2 + l_cs * 16);
      }
      dma_issued();
    };
    if constexpr (!NEXT) {
#pragma unroll
      for (int u = 0; u < 2 * PW; ++u) part(u);
    }
    const FA_LDS char* kt = kbuf(PAR);
    const FA_LDS char* vt = vbuf(PAR ^ 1);
    const int k0 = j * BN;
    int e_cur = 0;  // power-of-two exponent of tile j's fp16 V copy (wave-uniform)
    if constexpr (NEXT && F16) e_cur = v_exp[k0];

    // -- phase 1: S(j)'s MFMAs, with the exponentials of tile j-1's first 32-key
    // block (with their fp16 packing) between them.  The second block's
    // exponentials run beside the first half of phase 2, whose PV products only need
    // the first block's weights: the vector work (an exponential costs four FMA
    // issue slots) is then spread over 24 of the step's 32 MFMAs instead of 16 --
    u32x4 pb[2 * NKB];
    float rs[2] = {0.0f, 0.0f};  // key-split path: fp32 sums
    auto exp_pair = [&](const int q) {  // scores 2u, 2u+1 of block kb = q / 8 of tile j-1
      const int kb = q >> 3, u = q & 7, e = 2 * u;
      // P' = 2^(s*c - m*c + e) = P 2^e -> fp16 operands
      const float x0 = __builtin_fmaf(s_prev[kb][e], c, -mref_x);
      const float x1 = __builtin_fmaf(s_prev[kb][e + 1], c, -mref_x);
      const float p0 = (e < POLY) ? exp2_poly(x0) : exp2_hw(x0);
      const float p1 = (e + 1 < POLY) ? exp2_poly(x1) : exp2_hw(x1);
      if constexpr (F16) {
        pb[2 * kb + (u >> 2)][u & 3] = pack_f16(p0, p1);
      } else {
        pb[2 * kb + (u >> 2)][u & 3] = pack_bf16(p0, p1);
        rs[u & 1] += p0 + p1;
      }
    };
    constexpr int NPAIR = 8 * NKB;   // pairs of scores per lane and tile
    constexpr int P1 = 8;            // pairs of phase 1: the first block
    constexpr int NM1 = NKB * NDS;   // MFMAs of phase 1
    static_assert(NKB == 2, "two 32-key blocks per tile");
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      if constexpr (NEXT) s_next[kb] = f32x16{};
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const int i = kb * NDS + ds;
        if constexpr (NEXT) {
          const u32x4 a = lds_read16(kt + 32 * kb * ROWB + off_k[ds]);
          s_next[kb] = mfma_bf16(a, qreg[ds], s_next[kb]);
          if ((kb * NDS + ds) % (NKB * NDS / (2 * PW)) == 0) part((kb * NDS + ds) / (NKB * NDS / (2 * PW)));
        }
        if constexpr (PREV) {
#pragma unroll
          for (int q = i * P1 / NM1; q < (i + 1) * P1 / NM1; ++q) exp_pair(q);
        }
      }
    }
    if constexpr (NEXT && PREV) {
      // K reads run three MFMAs ahead
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
      for (int i = 0; i < NM1; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i % (NM1 / (2 * PW)) == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
        if (i < NM1 - 3) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    // mask S(j) (the diagonal tiles under the causal mask and the ragged last tile)
    if constexpr (NEXT && MASK) {
      // key k0 + 4hl + rel is hidden when rel >= lim (one register; rel is a constant)
      int lim = Lk;
      if constexpr (CAUSAL) lim = min(lim, my_row + 1 + coff);
      lim -= k0 + 4 * hl;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rel = 32 * kb + 8 * (r >> 2) + (r & 3);
          s_next[kb][r] = rel >= lim ? -INFINITY : s_next[kb][r];
        }
    }

    // -- phase 2: O^T += V^T P^T; the first half's MFMAs (keys of the first block)
    // carry the second block's exponentials, every MFMA a step of the row maximum of
    // S(j), and the second half the row sum of the rounded weights --
    float mx = -INFINITY;
    if constexpr (PREV) {
      float rsr[2] = {0.0f, 0.0f};
      constexpr int NM2 = BN / 16 * NDB;  // MFMAs of phase 2
#pragma unroll
      for (int g = 0; g < BN / 16; ++g) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int i = g * NDB + db;
#pragma unroll
          for (int q = P1 + i * (NPAIR - P1) / (NM2 / 2); q < P1 + (i + 1) * (NPAIR - P1) / (NM2 / 2) && q < NPAIR; ++q)
            exp_pair(q);
          const u32x2 lo = lds_read_tr16(vt + 16 * g * ROWB + off_v1[db]);
          const u32x2 hi = lds_read_tr16(vt + 16 * g * ROWB + off_v2[db]);
          if constexpr (F16) oacc[db] = mfma_f16(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb[g], oacc[db]);
          else oacc[db] = mfma_bf16(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb[g], oacc[db]);
          if constexpr (NEXT) {
            // two scores of S(j) per MFMA, 32 in all
#pragma unroll
            for (int q = i * 32 / NM2; q < (i + 1) * 32 / NM2; q += 2)
              mx = max3(mx, s_next[q >> 4][q & 15], s_next[q >> 4][(q & 15) + 1]);
          }
        }
      }
      // sum of the fp16-rounded weights the products used: O is normalised by it, so
      // a dominant weight's rounding cancels between numerator and denominator (with a
      // stale reference that weight is up to 2^8, not 1)
#pragma unroll
      for (int g = 0; g < BN / 16; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (F16) rsr[e & 1] = add_f16_pair(pb[g][e], rsr[e & 1]);
        }
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
      for (int i = 0; i < NM2 / 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
#pragma unroll
      for (int i = NM2 / 2; i < NM2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        if (i < NM2 - 3) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      // the empty asm makes the sums exist here, so their adds are scheduled among
      // this phase's MFMAs instead of being sunk past the rescale branch
      if constexpr (F16) lsum_r += (rsr[0] + rsr[1]) * esc;
      else lsum_r += rs[0] + rs[1];
      asm volatile("" : "+v"(lsum_r));
      __builtin_amdgcn_sched_barrier(0);
    } else if constexpr (NEXT) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) mx = max3(mx, s_next[kb][r], s_next[kb][r + 1]);
    }

    if constexpr (NEXT) {
      // row maximum across the two wave halves; lazy rescale: move the reference
      // only when the maximum grew by more than TAU.  O and the sums then hold
      // everything up to tile j-1 and are scaled before tile j's weights are added.
      // A tile whose V copy needed e > 7 (|V| >= 2^15) moves every reference that
      // grew, so that its weights stay <= 1 and P 2^e <= 2^15 fits fp16.
      mx = half_swap_max(mx);
      const float m_new = fmaxf(m_used, mx);
      bool need = m_new > m_used;
      if constexpr (TAU > 0 && F16) {
        const float tau = e_cur > 7 ? 0.0f : (float)TAU;
        need = need && (m_used == -INFINITY || (m_new - m_used) * c > tau);
      }
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float alpha = need ? (m_used == -INFINITY ? 0.0f : exp2_hw((m_used - m_new) * c)) : 1.0f;
        m_used = need ? m_new : m_used;
        mref = (m_used == -INFINITY) ? 0.0f : m_used * c;
        lsum_r *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      }
      mref_x = mref - (float)e_cur;
      esc = __int_as_float((127 - e_cur) << 23);
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using BF = std::false_type;
  using BT = std::true_type;
  using MF = std::false_type;
  using MT = std::true_type;
  // tiles before j_plain need no mask for this wave's rows
  int j_plain = Lk / BN;
  if constexpr (CAUSAL) j_plain = min(j_plain, max(0, q0 + 1 + coff) / BN);
  const int j_lim = min(n_mine, j_plain);
  if constexpr (PP) {
    // ---- two query tiles in ping-pong.  The workgroup's two 128-row tiles run half a
    // step apart: a step is two slots between workgroup barriers, and in each slot
    // one tile's waves issue the matrix products while the other tile's waves, on the
    // same SIMDs (wave w and wave w+4 share one), form the weights of their last
    // scores.  The lead tile (waves 0-3) runs M(m) in slot 2m and V(m) in slot 2m+1;
    // the lag tile runs V(m-1) in slot 2m and M(m) in slot 2m+1.  K(m+1) and V(m) are
    // loaded by the lead tile's waves during slot 2m and waited for at the barrier
    // that opens slot 2m+2; K(j) sits in K buffer j&1, V(j) in V buffer j&1. ----
    const bool lead = (wave >> 2) == 0;
    f32x16 s[NKB];      // S(j) of the tile in hand
    u32x4 pb[2 * NKB];  // its fp16 weights, the B operand of the next PV product
    static_assert(NKB * NDS == (BN / 16) * NDB, "S and PV products pair up");
    // matrix slot of tile j: S(j) = K(j) Q^T (DS) and O^T += V(j-1)^T P(j-1)^T (DPV).
    // The wave's priority is raised so that its MFMAs issue as soon as the matrix
    // core is free.
    // Step m's loads (K(m+1), V(m)) are issued by the lead tile's waves, one 1 KiB
    // packet after every second MFMA of their matrix slot.  Issued by all eight waves
    // at the step's opening, the 32 packets would queue at the CU's address unit (~15
    // cycles each) and the waves issuing last would start their slot ~480 cycles late.
    // Part u of a lead wave's share is packet wave + 4 (u % PPL) of K (u < PPL) or of
    // V.  Past the last tile the last tile is loaded again, into the buffer that no
    // product reads any more, so that the issue needs no branch.
    constexpr int PPL = TILE_BYTES / 1024 / 4;  // packets of a tile per lead wave
    constexpr int NPART = 2 * PPL;
    static_assert(PPL * 4 * 1024 == TILE_BYTES, "whole packets per lead wave");
    // A wave's packets wave + 4k start 256k / SLOTS rows apart, a multiple of 16, and
    // the slot swizzle depends on the row mod 16 only: each lane's offset is one
    // register per tensor plus a wave-uniform row term.
    static_assert((256 / SLOTS) % 16 == 0, "the packets of a wave share the swizzle");
    const int l_row = (wave * 64 + lane) / SLOTS;
    const int l_cs = ((wave * 64 + lane) % SLOTS) ^ slot_swizzle<D>(l_row);
    const uint32_t k_lane = (uint32_t)l_row * k_ss2 + l_cs * 16, v_lane = (uint32_t)l_row * v_ss2 + l_cs * 16;
    auto dma_part = [&](const int m, auto par_c, const int u) __attribute__((always_inline)) {
      constexpr int P = decltype(par_c)::value;
      const int k = u % PPL;
      if (u < PPL) {
        const int t = max(0, min(m + 1, n_tiles - 1));
        buf_load_lds16(rk, kbuf(P ^ 1) + (wave + 4 * k) * 1024, k_lane + (uint32_t)(t * BN + k * (256 / SLOTS)) * k_ss2);
      } else {
        const int t = max(0, min(m, n_tiles - 1));
        buf_load_lds16(rv, vbuf(P) + (wave + 4 * k) * 1024, v_lane + (uint32_t)(t * BN + k * (256 / SLOTS)) * v_ss2);
      }
      dma_issued();
    };
    auto mphase = [&](auto par_c, auto ds_c, auto dpv_c, auto dma_c, const int m) __attribute__((always_inline)) {
      constexpr int P = decltype(par_c)::value;  // j & 1
      constexpr bool DS = decltype(ds_c)::value, DPV = decltype(dpv_c)::value;
      constexpr bool DMA = decltype(dma_c)::value;  // this wave issues step m's loads
      if constexpr (DMA && !(DS || DPV)) {
#pragma unroll
        for (int u = 0; u < NPART; ++u) dma_part(m, par_c, u);
      }
      const FA_LDS char* kt = kbuf(P);
      const FA_LDS char* vt = vbuf(P ^ 1);
      if constexpr (DS || DPV) __builtin_amdgcn_s_setprio(1);
      if constexpr (DS) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
      }
      // S and PV products alternate, so that no MFMA waits for the one before it
#pragma unroll
      for (int i = 0; i < NKB * NDS; ++i) {
        if constexpr (DS) {
          const int kb = i & 1, ds = i >> 1;
          const u32x4 a = lds_read16(kt + 32 * kb * ROWB + off_k[ds]);
          s[kb] = mfma_bf16(a, qreg[ds], s[kb]);
        }
        if constexpr (DPV) {
          const int g = i / NDB, db = i % NDB;
          const u32x2 lo = lds_read_tr16(vt + 16 * g * ROWB + off_v1[db]);
          const u32x2 hi = lds_read_tr16(vt + 16 * g * ROWB + off_v2[db]);
          oacc[db] = mfma_f16(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb[g], oacc[db]);
        }
        if constexpr (DMA && (DS || DPV)) {
          if (i < NPART) dma_part(m, par_c, i);
        }
      }
      if constexpr (DS || DPV) {
        // operand reads run a few MFMAs ahead; the loads go out one per loop step
        constexpr int NMF = (DS ? NKB * NDS : 0) + (DPV ? (BN / 16) * NDB : 0);
        constexpr int PER = NMF / (NKB * NDS);  // MFMAs per loop step
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < NMF; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (DMA && i % PER == PER - 1 && i / PER < NPART) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_s_setprio(0);
      }
    };
    // fp16 weights P' = 2^(s c - mx_ref) of the tile in hand, and the fp32 sum of the
    // unrounded weights (plain adds: v_dot2 runs on the matrix pipeline and would wait
    // behind the other wave's MFMAs)
    float wsum[2];
    // hidden keys (the causal diagonal, the ragged last tile): key k0 + 4hl + rel(kb, r)
    // is hidden when rel >= lim; their weights are 0 and they take no part in the row
    // maximum (the scores themselves stay as they are: masking them in place keeps
    // both the raw and the masked scores live, and the masked steps spill more)
    auto rel_of = [](const int kb, const int r) { return 32 * kb + 8 * (r >> 2) + (r & 3); };
    auto weights = [&](const float mx_ref, auto mask_c, const int lim) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_c)::value;
      wsum[0] = wsum[1] = 0.0f;
#pragma unroll
      for (int q = 0; q < 8 * NKB; ++q) {
        const int kb = q >> 3, u = q & 7, e = 2 * u;
        const float x0 = __builtin_fmaf(s[kb][e], c, -mx_ref);
        const float x1 = __builtin_fmaf(s[kb][e + 1], c, -mx_ref);
        float p0 = (e < POLY) ? exp2_poly(x0) : exp2_hw(x0);
        float p1 = (e + 1 < POLY) ? exp2_poly(x1) : exp2_hw(x1);
        if constexpr (MASK) {
          p0 = rel_of(kb, e) >= lim ? 0.0f : p0;
          p1 = rel_of(kb, e + 1) >= lim ? 0.0f : p1;
        }
        pb[2 * kb + (u >> 2)][u & 3] = pack_f16(p0, p1);
        wsum[q & 1] += p0 + p1;
      }
    };
    // vector slot of tile j: mask; weights against the current reference, formed
    // before the row maximum is known (they stand unless the maximum moves the
    // reference, which the lazy threshold makes rare, and are redone then); row
    // maximum as four independent chains; lazy rescale; row sum
    auto vphase = [&](const int j, auto mask_c) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_c)::value;
      const int k0 = j * BN;
      const int e_cur = v_exp[k0];  // tile j's V-copy exponent: weights carry 2^e_cur
      int lim = 0;
      if constexpr (MASK) {
        lim = Lk;
        if constexpr (CAUSAL) lim = min(lim, my_row + 1 + coff);
        lim -= k0 + 4 * hl;
      }
      auto sv = [&](const int kb, const int r) {  // score as the row maximum sees it
        if constexpr (MASK) return rel_of(kb, r) >= lim ? -INFINITY : s[kb][r];
        else return s[kb][r];
      };
      weights(mref - (float)e_cur, mask_c, lim);
      float mp[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int kb = t >> 1, r0 = 8 * (t & 1);
        mp[t] = max3(sv(kb, r0), sv(kb, r0 + 1), sv(kb, r0 + 2));
        mp[t] = max3(mp[t], sv(kb, r0 + 3), sv(kb, r0 + 4));
        mp[t] = max3(mp[t], sv(kb, r0 + 5), sv(kb, r0 + 6));
        mp[t] = fmaxf(mp[t], sv(kb, r0 + 7));
      }
      float mx = max3(mp[0], mp[1], fmaxf(mp[2], mp[3]));
      mx = half_swap_max(mx);
      // lazy rescale: move the reference only when the maximum grew by more than TAU
      // (every growth on a tile whose V copy needed e > 7, so that P 2^e fits fp16)
      const float m_new = fmaxf(m_used, mx);
      bool need = m_new > m_used;
      if constexpr (TAU > 0) {
        const float tau = e_cur > 7 ? 0.0f : (float)TAU;
        need = need && (m_used == -INFINITY || (m_new - m_used) * c > tau);
      }
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float alpha = need ? (m_used == -INFINITY ? 0.0f : exp2_hw((m_used - m_new) * c)) : 1.0f;
        m_used = need ? m_new : m_used;
        mref = (m_used == -INFINITY) ? 0.0f : m_used * c;
        lsum_r *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        weights(mref - (float)e_cur, mask_c, lim);
      }
      lsum_r += (wsum[0] + wsum[1]) * __int_as_float((127 - e_cur) << 23);
    };
    // opening of step m (slot 2m): wait for the loads issued in slot 2m-2, barrier.
    // The barrier between the two slots of a step orders no memory (the loads in
    // flight fill buffers that neither slot reads): a bare s_barrier, at which no wave
    // waits for its loads.
    auto open_step = [&]() __attribute__((always_inline)) {
      wait_vmem();
      __syncthreads();
    };
    // Steps come in kinds fixed at compile time (which products and weights a wave
    // has in them, whether the tile needs the mask), run from straight-line
    // sequences: branching on the kind inside one loop makes the register allocator
    // copy the accumulators between the paths.
    auto lead_step = [&](const int m, auto par_c, auto ds_c, auto dpv_c, auto v_c, auto mask_c)
                         __attribute__((always_inline)) {
      open_step();
      mphase(par_c, ds_c, dpv_c, std::true_type{}, m);
      __builtin_amdgcn_s_barrier();
      if constexpr (decltype(v_c)::value) vphase(m, mask_c);
    };
    auto lag_step = [&](const int m, auto par_c, auto v_c, auto mask_c, auto ds_c, auto dpv_c)
                        __attribute__((always_inline)) {
      open_step();
      if constexpr (decltype(v_c)::value) vphase(m - 1, mask_c);
      __builtin_amdgcn_s_barrier();
      mphase(par_c, ds_c, dpv_c, std::false_type{}, m);
    };
    // A wave with n = n_mine tiles: step 0 has S(0) and (lead) its weights; steps
    // 1..n-1 have everything; step n has PV(n-1) (and, lag, the weights of n-1);
    // steps past n only load and keep the barriers.  Weights of tile j are masked
    // from j_plain on.  Every wave runs steps 0..n_tiles, two barriers each.
    const int n = n_mine, jl = min(n_mine, j_plain);
    if (n_tiles > 0) issue(rk, k_ss2, 0, kbuf(0));
    int m = 0;
    if (lead) {
      if (n > 0) {
        lead_step(0, I0{}, BT{}, BF{}, BT{}, MT{});
        m = 1;
        for (; m + 1 < jl; m += 2) {  // m odd
          lead_step(m, I1{}, BT{}, BT{}, BT{}, MF{});
          lead_step(m + 1, I0{}, BT{}, BT{}, BT{}, MF{});
        }
        for (; m + 1 < n; m += 2) {
          lead_step(m, I1{}, BT{}, BT{}, BT{}, MT{});
          lead_step(m + 1, I0{}, BT{}, BT{}, BT{}, MT{});
        }
        if (m < n) {  // m = n - 1: tile m, then PV(m) alone
          lead_step(m, I1{}, BT{}, BT{}, BT{}, MT{});
          lead_step(m + 1, I0{}, BF{}, BT{}, BF{}, MF{});
          m += 2;
        } else {      // m = n
          lead_step(m, I1{}, BF{}, BT{}, BF{}, MF{});
          m += 1;
        }
      }
      for (; m <= n_tiles; ++m) {
        if (m & 1) lead_step(m, I1{}, BF{}, BF{}, BF{}, MF{});
        else lead_step(m, I0{}, BF{}, BF{}, BF{}, MF{});
      }
    } else {
      if (n > 0) {
        lag_step(0, I0{}, BF{}, MF{}, BT{}, BF{});
        m = 1;
        for (; m < jl && m + 1 < n; m += 2) {  // m odd; V(m-1), V(m) unmasked
          lag_step(m, I1{}, BT{}, MF{}, BT{}, BT{});
          lag_step(m + 1, I0{}, BT{}, MF{}, BT{}, BT{});
        }
        for (; m + 1 < n; m += 2) {
          lag_step(m, I1{}, BT{}, MT{}, BT{}, BT{});
          lag_step(m + 1, I0{}, BT{}, MT{}, BT{}, BT{});
        }
        if (m < n) {  // m = n - 1
          lag_step(m, I1{}, BT{}, MT{}, BT{}, BT{});
          lag_step(m + 1, I0{}, BT{}, MT{}, BF{}, BT{});
          m += 2;
        } else {      // m = n
          lag_step(m, I1{}, BT{}, MT{}, BF{}, BT{});
          m += 1;
        }
      }
      for (; m <= n_tiles; ++m) {
        if (m & 1) lag_step(m, I1{}, BF{}, MF{}, BF{}, BF{});
        else lag_step(m, I0{}, BF{}, MF{}, BF{}, BF{});
      }
    }
    // the last steps' loads (the last tile again) land before the workgroup's LDS is
    // released
    wait_vmem();
  } else {
  f32x16 sa[NKB], sb[NKB];
  if (n_tiles > 0) issue(rk, k_ss2, 0, kbuf(0));
  int j = 0;
  if (n_mine > 0) {
    step(0, I0{}, BF{}, BT{}, MT{}, sb, sa);
    j = 1;
    for (; j + 1 < j_lim; j += 2) {  // j odd
      step(j, I1{}, BT{}, BT{}, MF{}, sa, sb);
      step(j + 1, I0{}, BT{}, BT{}, MF{}, sb, sa);
    }
    // the remaining tiles (masked when needed), then the last step
    for (; j + 1 < n_mine; j += 2) {  // j odd
      step(j, I1{}, BT{}, BT{}, MT{}, sa, sb);
      step(j + 1, I0{}, BT{}, BT{}, MT{}, sb, sa);
    }
    if (j < n_mine) {
      step(j, I1{}, BT{}, BT{}, MT{}, sa, sb);
      step(j + 1, I0{}, BT{}, BF{}, MF{}, sb, sa);
      j += 2;
    } else {
      step(j, I1{}, BT{}, BF{}, MF{}, sa, sb);
      j += 1;
    }
  }
  // steps past this wave's last tile: barriers and loads only
  for (; j <= n_tiles; ++j) {
    wait_vmem();
    __syncthreads();
    const int par = j & 1;
    if (j + 1 < n_tiles) issue(rk, k_ss2, j + 1, kbuf(par ^ 1));
    if (j < n_tiles) issue(rv, v_ss2, j, vbuf(par));
  }
  wait_vmem();  // the last steps' repeated loads land before the LDS is released
  }

  // ---- epilogue: O = O_acc / l, LSE = m*scale + ln l (O_acc and the sums are in
  // true units: each tile's 2^e on the weights cancels the 2^-e on its V copy) ----
  const float ltr = half_swap_sum(lsum_r);
  const float inv = ltr > 0.0f ? 1.0f / ltr : 0.0f;
  float lse = -INFINITY;
  if (ltr > 0.0f) lse = (m_used * c + __builtin_amdgcn_logf(ltr)) * 0.69314718055994531f;
  if constexpr (SPLIT) {
    // this chunk's normalised partial O (fp32) and LSE; rows past the end are dropped
    const int64_t slot = ((int64_t)chunk * p.heads + h) * p.total_q + row_base;
    const rsrc_t rpo = make_rsrc(p.part_o + slot * D, (uint32_t)Lq * D * 4);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * db + 8 * q4 + 4 * hl;
        buf_store16(rpo, ((uint32_t)my_row * D + d) * 4,
                    u32x4{__float_as_uint(oacc[db][4 * q4 + 0] * inv), __float_as_uint(oacc[db][4 * q4 + 1] * inv),
                          __float_as_uint(oacc[db][4 * q4 + 2] * inv), __float_as_uint(oacc[db][4 * q4 + 3] * inv)});
      }
    if (hl == 0 && my_row < Lq) p.part_lse[slot + my_row] = lse;
  } else if (p.o_f32) {
    // fp32 O (a diagnostic): four consecutive columns per 16-byte write
    const rsrc_t ro32 = make_rsrc((char*)p.o + ooff * 4, (uint32_t)(Lq - 1) * (uint32_t)(p.o_ss * 4) + D * 4);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * db + 8 * q4 + 4 * hl;
        buf_store16(ro32, (uint32_t)my_row * (uint32_t)(p.o_ss * 4) + d * 4,
                    u32x4{__float_as_uint(oacc[db][4 * q4 + 0] * inv), __float_as_uint(oacc[db][4 * q4 + 1] * inv),
                          __float_as_uint(oacc[db][4 * q4 + 2] * inv), __float_as_uint(oacc[db][4 * q4 + 3] * inv)});
      }
    if (hl == 0 && my_row < Lq) p.lse[lseoff + my_row] = lse;
  } else {
    // lane l and lane l+32 hold the same row's columns 32db+8q4+0..3 and +4..7: one
    // swap of the halves per pair of q4 gives every lane 8 consecutive columns (lane l
    // those of q4 = 2k, lane l+32 those of 2k+1), stored with one 16-byte write
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        uint32_t a[2], b[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          a[e] = pack_bf16(oacc[db][8 * k + 2 * e] * inv, oacc[db][8 * k + 2 * e + 1] * inv);
          b[e] = pack_bf16(oacc[db][8 * k + 4 + 2 * e] * inv, oacc[db][8 * k + 4 + 2 * e + 1] * inv);
          const auto r = __builtin_amdgcn_permlane32_swap(a[e], b[e], false, false);
          a[e] = r[0];
          b[e] = r[1];
        }
        const int d = 32 * db + 16 * k + 8 * hl;
        buf_store16(ro, (uint32_t)my_row * o_ss2 + d * 2, u32x4{a[0], a[1], b[0], b[1]});
      }
    if (hl == 0 && my_row < Lq) p.lse[lseoff + my_row] = lse;
  }
}

// ---- fp16 copy of V with one power-of-two scale per 64-key tile ----
// One workgroup per (tile, sequence, head).  The weights P' = P 2^e go to fp16 with
// P <= 2^8 (the lazy bound), so e <= 7 keeps them finite; the largest e keeps the most
// weights in fp16's normal range (a row's many small weights carry much of its mass,
// and a subnormal weight has few bits).  So e = 7, and the copy is V 2^-7: a bf16
// value (8 significant bits) then converts exactly unless it falls below 2^-7 in
// magnitude, where the fp16 subnormal it becomes is off by less than 2^-18.  With
// E the exponent of the tile's largest |v| (a bf16 value widens exactly):
//   E < -4:       e = max(E + 11, -10), so that a tile of tiny values keeps its
//                 largest elements normal in the copy;
//   -4 <= E <= 22: e = 7 (the copy stays below 2^16);
//   E > 22:       e = E - 15 (at most 15); the forward then moves every growing row
//                 reference on that tile, so that its weights stay <= 1 and P 2^e fits;
//                 |v| must stay below 2^31.
template <int D, bool VARLEN>
__global__ __launch_bounds__(256) void vprep_kernel(FwdParams p) {
  constexpr int BN = kFwdBlockN;
  constexpr int CPR = D / 8;               // 16-byte chunks per row
  constexpr int PER = BN * CPR / 256;      // chunks per thread
  __shared__ uint32_t wmax[4];
  // heads fastest: neighbouring workgroups read the same rows of V (all heads of a row
  // are adjacent in memory)
  const int h = blockIdx.x, t = blockIdx.y, b = blockIdx.z;
  int Lk = p.seqlen_k;
  int64_t voff, krow0;
  if constexpr (VARLEN) {
    const int sk = p.cu_k[b];
    Lk = p.cu_k[b + 1] - sk;
    voff = (int64_t)sk * p.v_ss + (int64_t)h * p.v_sh;
    krow0 = sk;
  } else {
    voff = (int64_t)b * p.v_sb + (int64_t)h * p.v_sh;
    krow0 = (int64_t)b * Lk;
  }
  const int r_first = t * BN;
  if (r_first >= Lk) return;
  const uint16_t* src = (const uint16_t*)p.v + voff;
  u32x4 v[PER];
  uint32_t mx = 0;  // largest |v| as a bf16 magnitude pattern (ordered like the values)
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = i * 256 + threadIdx.x;
    const int r = r_first + idx / CPR, cc = idx % CPR;
    v[i] = r < Lk ? *(const u32x4*)(src + (int64_t)r * p.v_ss + cc * 8) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int w = 0; w < 4; ++w) mx = max(mx, max(v[i][w] & 0x7FFFu, (v[i][w] >> 16) & 0x7FFFu));
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, m, 64));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const int E = (int)(mx >> 7) - 127;  // -127 for an all-zero tile
  const int e = E > 22 ? min(E - 15, 15) : min(max(E + 11, -10), 7);
  const float sc = __int_as_float((127 - e) << 23);  // 2^-e, exact
  uint16_t* dst = p.v16 + ((int64_t)h * p.total_k + krow0) * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = i * 256 + threadIdx.x;
    const int r = r_first + idx / CPR, cc = idx % CPR;
    if (r < Lk) {
      u32x4 o;
#pragma unroll
      for (int w = 0; w < 4; ++w) o[w] = pack_f16(bf16_lo(v[i][w]) * sc, bf16_hi(v[i][w]) * sc);
      *(u32x4*)(dst + (int64_t)r * D + cc * 8) = o;
    }
  }
  if (threadIdx.x == 0) p.v_exp[(int64_t)h * p.total_k + krow0 + r_first] = e;
}

hipError_t launch_fwd_vprep(const FwdParams& p, int head_dim, bool varlen, hipStream_t stream) {
  const int tiles = (p.seqlen_k + kFwdBlockN - 1) / kFwdBlockN;  // seqlen_k: the longest key sequence
  if (tiles == 0 || p.batch == 0) return hipSuccess;
  const dim3 grid((unsigned)p.heads, (unsigned)tiles, (unsigned)p.batch);
  if (head_dim == 128) {
    if (varlen) hipLaunchKernelGGL((vprep_kernel<128, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((vprep_kernel<128, false>), grid, dim3(256), 0, stream, p);
  } else {
    if (varlen) hipLaunchKernelGGL((vprep_kernel<64, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((vprep_kernel<64, false>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

// ---- merge of the key chunks' partial results ----
// One thread per (head, query row, 4 columns of O): LSE = m + ln sum_c e^(LSE_c - m)
// with m = max_c LSE_c, and O = sum_c e^(LSE_c - LSE) O_c, in chunk order.  Chunks
// where the row saw no key carry LSE_c = -inf and weigh nothing; a row that saw no
// key at all gets O = 0, LSE = -inf.
template <int D, bool VARLEN>
__global__ __launch_bounds__(256) void fwd_merge_kernel(FwdParams p) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rows = (int64_t)p.heads * p.total_q;
  if (idx >= rows * (D / 4)) return;
  const int64_t r = idx / (D / 4);
  const int d = (int)(idx - r * (D / 4)) * 4;
  const int h = (int)(r / p.total_q);
  const int rowg = (int)(r - (int64_t)h * p.total_q);
  const int64_t stride = (int64_t)p.heads * p.total_q;  // between chunks
  float m = -INFINITY;
  for (int c = 0; c < p.n_split; ++c) m = fmaxf(m, p.part_lse[c * stride + r]);
  float o0 = 0.0f, o1 = 0.0f, o2 = 0.0f, o3 = 0.0f, wsum = 0.0f;
  if (m != -INFINITY) {
    for (int c = 0; c < p.n_split; ++c) {
      const float lc = p.part_lse[c * stride + r];
      const float w = __expf(lc - m);  // 0 for an empty chunk
      const f32x4 oc = *(const f32x4*)(p.part_o + (c * stride + r) * D + d);
      o0 = __builtin_fmaf(w, oc[0], o0);
      o1 = __builtin_fmaf(w, oc[1], o1);
      o2 = __builtin_fmaf(w, oc[2], o2);
      o3 = __builtin_fmaf(w, oc[3], o3);
      wsum += w;
    }
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  int64_t ooff, lidx;
  if constexpr (VARLEN) {
    ooff = (int64_t)rowg * p.o_ss + (int64_t)h * p.o_sh;
    lidx = (int64_t)h * p.total_q + rowg;
  } else {
    const int b = rowg / p.seqlen_q, i = rowg - b * p.seqlen_q;
    ooff = (int64_t)b * p.o_sb + (int64_t)i * p.o_ss + (int64_t)h * p.o_sh;
    lidx = ((int64_t)b * p.heads + h) * p.seqlen_q + i;
  }
  if (p.o_f32) *(f32x4*)((float*)p.o + ooff + d) = f32x4{o0 * inv, o1 * inv, o2 * inv, o3 * inv};
  else *(u32x2*)((uint16_t*)p.o + ooff + d) = u32x2{pack_bf16(o0 * inv, o1 * inv), pack_bf16(o2 * inv, o3 * inv)};
  if (d == 0) p.lse[lidx] = wsum > 0.0f ? m + __logf(wsum) : -INFINITY;
}

// ---- longest-first work list for packed variable-length batches ----
// One workgroup: histogram of item costs (key tiles visited), exclusive scan from
// the most expensive bin down, scatter.  Items of equal cost may land in any order.
__global__ __launch_bounds__(1024) void sched_kernel(const int32_t* cu_q, const int32_t* cu_k, int batch,
                                                     int tile_rows, int block_n, int causal, int32_t* out) {
  __shared__ int hist[kSchedMaxCost + 1];
  __shared__ int wsum[16];
  __shared__ int total;
  for (int i = threadIdx.x; i <= kSchedMaxCost; i += blockDim.x) hist[i] = 0;
  if (threadIdx.x == 0) total = 0;
  __syncthreads();
  auto cost_of = [&](int b, int t) {
    const int lq = cu_q[b + 1] - cu_q[b];
    const int lk = cu_k[b + 1] - cu_k[b];
    int kv = lk;
    if (causal) kv = max(0, min(lk, min(lq, (t + 1) * tile_rows) + lk - lq));
    return min((kv + block_n - 1) / block_n, kSchedMaxCost);
  };
  // Longest first by cost bucket: a bucket spans the cost growth of 16 consecutive
  // causal tiles (16 * tile_rows keys), and within a bucket each sequence's tiles stay
  // together, longest first, so that the workgroups running at one time read the same
  // sequences' K/V and find it in L2
  const int bw = max(1, 16 * tile_rows / block_n);
  for (int b = threadIdx.x; b < batch; b += blockDim.x) {
    const int lq = cu_q[b + 1] - cu_q[b];
    const int nt = (lq + tile_rows - 1) / tile_rows;
    for (int t = 0; t < nt;) {
      const int bk = cost_of(b, t) / bw;
      int t1 = t + 1;
      while (t1 < nt && cost_of(b, t1) / bw == bk) ++t1;
      atomicAdd(&hist[bk], t1 - t);
      t = t1;
    }
    atomicAdd(&total, nt);
  }
  __syncthreads();
  scan_bins_descending<kSchedMaxCost + 1>(hist, wsum);
  if (threadIdx.x == 0) out[0] = total;
  for (int b = threadIdx.x; b < batch; b += blockDim.x) {
    const int lq = cu_q[b + 1] - cu_q[b];
    const int nt = (lq + tile_rows - 1) / tile_rows;
    for (int t = 0; t < nt;) {
      const int bk = cost_of(b, t) / bw;
      int t1 = t + 1;
      while (t1 < nt && cost_of(b, t1) / bw == bk) ++t1;
      int pos = atomicAdd(&hist[bk], t1 - t);
      for (int u = t1 - 1; u >= t; --u, ++pos) {
        out[1 + 2 * pos] = b;
        out[2 + 2 * pos] = u;
      }
      t = t1;
    }
  }
}

// ---- probe of the two exponentials the forward uses ----
// y_poly[i] = the software 2^x (integer/fraction split and cubic on the multiply-add
// units) and y_hw[i] = v_exp_f32, both exactly as the forward evaluates them.
__global__ __launch_bounds__(256) void exp2_probe_kernel(const float* x, float* y_poly, float* y_hw, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float v = x[i];
    y_poly[i] = exp2_poly(v);
    y_hw[i] = exp2_hw(v);
  }
}

hipError_t launch_exp2_probe(const float* x, float* y_poly, float* y_hw, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(exp2_probe_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, stream, x,
                     y_poly, y_hw, n);
  return hipGetLastError();
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
  if constexpr (NQT == 1) {
    if (p.n_split > 1) {
      // the key-split kernel rescales eagerly (tau = 0; see F16 in fwd_kernel)
      hipLaunchKernelGGL((fwd_kernel<D, 1, CAUSAL, VARLEN, POLY, 0, true>), dim3(grid * (unsigned)p.n_split),
                         dim3(256), 0, stream, p);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const int64_t threads = (int64_t)p.heads * p.total_q * (D / 4);
      hipLaunchKernelGGL((fwd_merge_kernel<D, VARLEN>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                         stream, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((fwd_kernel<D, NQT, CAUSAL, VARLEN, POLY, TAU>), dim3(grid), dim3(256 * NQT), 0, stream, p);
  return hipGetLastError();
}

// The exp2 split shares 2 and 4 and the eager threshold (tau = 0) are measurement
// variants: compiled for head_dim 128 and fixed-length batches only.
template <int D, int NQT, bool CAUSAL, bool VARLEN>
static hipError_t dispatch_poly_tau(const FwdParams& p, const FwdConfig& cfg, hipStream_t s, int mi) {
  if (cfg.tau == 8 && cfg.poly_per16 == 0) return launch_one<D, NQT, CAUSAL, VARLEN, 0, 8>(p, s, mi);
  if constexpr (D == 128 && !VARLEN) {
    if (cfg.tau == 8 && cfg.poly_per16 == 2) return launch_one<D, NQT, CAUSAL, VARLEN, 2, 8>(p, s, mi);
    if (cfg.tau == 8 && cfg.poly_per16 == 4) return launch_one<D, NQT, CAUSAL, VARLEN, 4, 8>(p, s, mi);
    if (cfg.tau == 0 && cfg.poly_per16 == 0) return launch_one<D, NQT, CAUSAL, VARLEN, 0, 0>(p, s, mi);
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
