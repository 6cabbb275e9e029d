// Device-side building blocks for the gfx950 (CDNA4) attention kernels.
//
// Matrix-core conventions used throughout (32x32x16 BF16 MFMA, wave64):
//   A operand (32 x 16): lane l holds row (l & 31), k = 8*(l >> 5) + e, e = 0..7
//   B operand (16 x 32): lane l holds column (l & 31), same k mapping
//   C/D (32 x 32 fp32):  register r of lane l holds row 8*(r/4) + 4*(l>>5) + (r&3),
//                        column (l & 31)
// Because A and B share one k mapping, any consistent relabelling of the k index
// is a valid contraction; the kernels use that freedom to feed an accumulator
// tile straight back as the next product's operand.
//
// ds_read_b64_tr_b16 (LDS transpose read): within each 16-lane group, lane s
// supplies an address of four consecutive 16-bit values M[s][0..3]; lane i of the
// group receives M[4e + i/4][i%4] in element e.  With source lane s pointing at
// row (s/4) and column 4*(s%4) of a row-major tile, lane i receives column i of
// four consecutive rows: a 4 x 16 transpose, used to feed V (and Q, dO, K in the
// backward) as the k-major operand without an extra pass.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))
#define FA_CONST __attribute__((address_space(4)))

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer resource over [base, base + bytes): loads past the end return zero
// and stores past the end are dropped, which handles ragged tails.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           (int)0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ __forceinline__ void buf_store8(rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}

__device__ __forceinline__ void buf_store16(rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}

// 16 bytes per lane straight from global memory into LDS: lane l's bytes land at
// lds_wave_base + 16*l (lds_wave_base must be wave-uniform).
__device__ __forceinline__ void buf_load_lds16(rsrc_t r, FA_LDS void* lds_wave_base, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_wave_base, 16, off, 0, 0, 0);
}

__device__ __forceinline__ void wait_vmem() {
  // s_waitcnt vmcnt(0), other counters left at their maxima
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Called after every batch of buffer->LDS loads.  A check build (FA_SERIAL_LOADS)
// waits for the batch right there, so that no load overlaps the computation; its
// results must equal the normal build's bit for bit, which they do only if no
// computation reads LDS that a load in flight is still filling.
__device__ __forceinline__ void dma_issued() {
#ifdef FA_SERIAL_LOADS
  wait_vmem();
#endif
}

// s_waitcnt vmcnt(16): vector memory operations retire in issue order, so this
// waits for everything but the 16 most recent ones (e.g. fire-and-forget atomics
// issued after a stage's loads).
__device__ __forceinline__ void wait_vmem_keep16() { __builtin_amdgcn_s_waitcnt(0x4F70); }

__device__ __forceinline__ f32x16 mfma_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Same tile shapes and k mapping with fp16 operands (v_mfma_f32_32x32x16_f16).
__device__ __forceinline__ f32x16 mfma_f16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                0, 0);
}

__device__ __forceinline__ u32x2 lds_read_tr16(const FA_LDS char* p) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)p);
  return __builtin_bit_cast(u32x2, r);
}

__device__ __forceinline__ u32x4 lds_read16(const FA_LDS char* p) {
  return *(const FA_LDS u32x4*)p;
}

__device__ __forceinline__ void lds_write16(FA_LDS char* p, u32x4 v) { *(FA_LDS u32x4*)p = v; }

// Round-to-nearest-even narrowing of two floats into one packed bf16 pair.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Round-to-nearest-even narrowing of two floats into one packed fp16 pair.
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  f16x2 v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// acc + lo + hi of a packed fp16 pair, in one v_dot2 instruction (products by 1.0 are exact).
__device__ __forceinline__ float add_f16_pair(uint32_t w, float acc) {
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), one, acc, false);
}

// acc + lo + hi of a packed bf16 pair, in one v_dot2 instruction (products by 1.0 are exact).
__device__ __forceinline__ float add_bf16_pair(uint32_t w, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// max(a, b, c) as one v_maximum3_f32.  NaN-propagating (IEEE maximum), so unlike
// fmaxf it needs no canonicalising copies of operands that come out of an MFMA.
__device__ __forceinline__ float max3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// Combine a value with the same lane's value in the other half of the wave
// (lane l and lane l ^ 32) using v_permlane32_swap.
__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// In-place exclusive prefix sum of hist[0..NB) taken from the last bin down (bin NB-1
// receives 0, bin c the sum of bins c+1..NB-1), by a whole 1024-thread workgroup:
// each thread sums a run of bins, the 64-wide waves scan their runs with shuffles,
// wave 0 scans the 16 wave totals, and each thread writes its run.  Returns the total.
template <int NB>
__device__ int scan_bins_descending(int* hist, int* wsum /* 16 ints of LDS */) {
  constexpr int PER = (NB + 1023) / 1024;
  const int t = threadIdx.x;
  int local = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int d = t * PER + i;
    if (d < NB) local += hist[NB - 1 - d];
  }
  int x = local;  // inclusive scan within the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if ((t & 63) >= o) x += y;
  }
  if ((t & 63) == 63) wsum[t >> 6] = x;
  __syncthreads();
  if (t < 64) {
    int w = t < 16 ? wsum[t] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int y = __shfl_up(w, o, 64);
      if (t >= o) w += y;
    }
    if (t < 16) wsum[t] = w;
  }
  __syncthreads();
  int run = x - local + ((t >> 6) > 0 ? wsum[(t >> 6) - 1] : 0);
  const int total = wsum[15];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int d = t * PER + i;
    if (d < NB) {
      const int c = NB - 1 - d;
      const int n = hist[c];
      hist[c] = run;
      run += n;
    }
  }
  __syncthreads();
  return total;
}

// XOR swizzle of the 16-byte slots of a K/V row held in LDS.  Chosen so that (a)
// 16 consecutive rows read at one column hit 16 different slots (row-major MFMA
// operand reads) and (b) 4-row groups read through the transpose unit hit
// disjoint slot quartets.  D = 128: 16 slots per 256-byte row.  D = 64: 8 slots
// per 128-byte row (two rows share one 256-byte bank window).
template <int D>
__device__ __forceinline__ int slot_swizzle(int row) {
  if constexpr (D == 128) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else {
    return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  }
}

// 2^x on the multiply-add units (the software exponential): split x into an
// integer j and a fraction f in [0,1), evaluate a cubic in f, and add j to the
// exponent field.  Valid for x <= 8 (the lazy-rescale bound); x < -126 and -inf
// return 0.  Coefficients: least-squares fit of 2^f on 4,097 Chebyshev nodes in
// relative error with p(0) = 1 held fixed (see exp2_poly_coeffs.py next to this
// file); maximum relative error 8.7e-5.
constexpr float kExp2P1 = 0.695122898f;
constexpr float kExp2P2 = 0.227645576f;
constexpr float kExp2P3 = 0.0770580471f;

__device__ __forceinline__ float exp2_poly(float x) {
  const float xc = fmaxf(x, -127.0f);
  const float j = __builtin_floorf(xc);
  const float f = xc - j;
  const float p = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(kExp2P3, f, kExp2P2), f, kExp2P1), f, 1.0f);
  const int bits = __float_as_int(p) + ((int)j << 23);
  return xc < -126.0f ? 0.0f : __int_as_float(bits);
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace fa
