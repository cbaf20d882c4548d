// Device-side helpers shared by the LRM kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <stdint.h>

#include "platform.h"

namespace lrm {

constexpr int kWave = 64;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- bf16 bits
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// fp32 -> bf16, round to nearest even (inputs are finite by precondition)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// ------------------------------------------------------- wave reductions
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Inclusive scan across a wave with DPP moves (no LDS round trips):
// Hillis-Steele inside each 16-lane row (row_shr 1, 2, 4, 8; lanes whose
// source falls before the row keep the 0 passed as "old"), then row 0's total
// into row 1 and row 2's into row 3 (row_bcast:15 on rows 1, 3), then rows
// 0-1's total into rows 2, 3 (row_bcast:31).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);
  return v;
}

// Row addressing of a pair: the row a matrix holds for pair p.
__device__ __forceinline__ int64_t pair_row(int rows_is_pair, const int32_t* token, int64_t p) {
  return rows_is_pair ? p : (int64_t)token[p];
}

// SiLU pieces in fp32 (accurate expf).
__device__ __forceinline__ float sigmoidf_acc(float a) { return 1.0f / (1.0f + expf(-a)); }

// Device error bits (written into the first word of a workspace).
enum : uint32_t {
  kErrExpertRange = 1u,
  kErrTokenRange = 2u,
  kErrTokenOrder = 4u,
  // more kept rows than the packed buffers were sized for (only a captured
  // call replayed with host quotas other than those it was sized with)
  kErrCapacity = 8u,
  // a replica assignment that does not match the kept counts
  kErrAssign = 16u,
};

// Exclusive scan of one int per thread over an NT-thread block.  lds must hold
// NT/64 + 1 ints.  Returns the exclusive prefix; *total gets the block sum.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* lds, int* total) {
  constexpr int NW = NT / kWave;
  const int incl = wave_incl_scan(v);
  const int w = threadIdx.x >> 6, l = lane_id();
  if (l == kWave - 1) lds[w] = incl;
  __syncthreads();
  if (threadIdx.x < kWave) {
    const int t = (l < NW) ? lds[l] : 0;
    const int ti = wave_incl_scan(t);
    if (l < NW) lds[l] = ti - t;
    if (l == NW - 1) lds[NW] = ti;
  }
  __syncthreads();
  const int res = lds[w] + incl - v;
  *total = lds[NW];
  __syncthreads();
  return res;
}

// Exclusive scan of n values (n <= 4 * NT) given by get(i) into out[0..n],
// out[n] = total.  Values are handled in contiguous runs of 4 per thread.
template <int NT, typename F>
__device__ void block_scan_array(int n, F get, int32_t* out, int* lds) {
  const int per = 4;
  const int i0 = threadIdx.x * per;
  int v[per];
  int local = 0;
#pragma unroll
  for (int j = 0; j < per; ++j) {
    v[j] = (i0 + j < n) ? get(i0 + j) : 0;
    local += v[j];
  }
  int total;
  int run = block_excl_scan<NT>(local, lds, &total);
#pragma unroll
  for (int j = 0; j < per; ++j) {
    if (i0 + j < n) out[i0 + j] = run;
    run += v[j];
  }
  if (threadIdx.x == 0) out[n] = total;
}

}  // namespace lrm
