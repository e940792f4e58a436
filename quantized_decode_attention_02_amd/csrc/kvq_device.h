// Device helpers shared by the kvq kernels: plane addressing, fp16 bit
// conversions and the fixed-order Hadamard butterflies.
//
// Sources cited here:
//   [troisinh] "KV Cache Quantization — Nén cache INT4/INT3, mở khóa
//              ultra-long context" (troisinh.com).
//   [trefon]   "Matematyka cache KV: ile kosztuje długi kontekst i co daje
//              4-bitowy cache" (trefon.com).
#pragma once

#include "kvq_internal.h"

namespace kvq {

// fp32(1/sqrt(128)), bits 0x3DB504F3: the final scaling of the normalized
// Hadamard transform.
__device__ __forceinline__ float c32() { return __uint_as_float(0x3DB504F3u); }

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
  return __half2float(__ushort_as_half(b));
}

// fp32 -> fp16 round-to-nearest-even, returned as bits.
__device__ __forceinline__ uint16_t float_to_half_bits(float x) {
  return __half_as_ushort(__float2half_rn(x));
}

// fp16(x) + (+0.0): turns -0 into +0 so that a degenerate group's parameters
// do not depend on which signed zero min/max returned.
__device__ __forceinline__ uint16_t canonical_half_bits(float x) {
  uint16_t b = float_to_half_bits(x);
  return b == 0x8000u ? (uint16_t)0 : b;
}

__device__ __forceinline__ int64_t pair_index(const Geom& g, int b, int h) {
  return (int64_t)b * g.Hkv + h;
}

// Bytes of a 32-token x 128-channel tile at `bits` per code.
__host__ __device__ __forceinline__ int64_t tile_bytes(int bits) { return 512 * bits; }

// Tile of group `grp` for (pair), tier chosen by the group's first token.
__device__ __forceinline__ const uint8_t* tile_ptr(const Geom& g, const Planes& p, int plane_hi,
                                                   int plane_lo, int64_t pair, int64_t grp,
                                                   int* bits_out) {
  if (g.scheme == KVQ_BLOCK128_SYM || grp * kGroup >= g.hi_start) {
    *bits_out = g.hi_bits;
    return p.p[plane_hi] + (pair * g.hi_slots + grp % g.hi_slots) * tile_bytes(g.hi_bits);
  }
  *bits_out = g.lo_bits;
  return p.p[plane_lo] + (pair * g.gmax + grp) * tile_bytes(g.lo_bits);
}

// Byte offset inside a key tile of canonical byte `cb` of token `t`
// (16-byte chunks of all 32 rows are contiguous 512-byte runs).
__host__ __device__ __forceinline__ int ktile_offset(int t, int cb) {
  return (cb >> 4) * 512 + t * 16 + (cb & 15);
}

// Work-group barrier for data exchanged through LDS only: each wave waits for
// its own LDS operations, then all waves meet.  Unlike __syncthreads() it
// does not wait for outstanding global loads (a tile still in flight to LDS
// or registers stays in flight across it).  The "memory" clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Orders the LDS accesses of one wave before and after it.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Normalized FWHT-128 of `nvec` vectors stored as float rows of 128 in LDS,
// in the fixed fp32 schedule: for h = 1, 2, ..., 64 in that order every pair
// (x[i], x[i+h]) with bit log2(h) of i clear becomes (a + b, a - b), each one
// fp32 operation; then every element is multiplied by fp32(1/sqrt(128)).
// H in Sylvester order is orthonormal after the scaling, so nothing is lost
// and dot products are kept ([troisinh] "Tại sao nó hoạt động", item 2;
// [trefon] "Jak 4-bitowemu cache to uchodzi: najpierw obrót").
// All threads of the block must call it; it synchronizes internally, on LDS
// only (the vectors are exchanged through LDS and nothing else).
__device__ __forceinline__ void fwht128_lds(float* x, int nvec, int tid, int nthreads) {
  for (int h = 1; h < kD; h <<= 1) {
    for (int i = tid; i < nvec * 64; i += nthreads) {
      const int v = i >> 6, pr = i & 63;
      const int i0 = (pr / h) * 2 * h + (pr % h);
      float* row = x + v * kD;
      const float a = row[i0], b = row[i0 + h];
      row[i0] = a + b;
      row[i0 + h] = a - b;
    }
    lds_barrier();
  }
  const float c = c32();
  for (int i = tid; i < nvec * kD; i += nthreads) x[i] = x[i] * c;
  lds_barrier();
}

// fwht128_lds for one wave (64 lanes, one butterfly each per stage), same
// schedule and arithmetic.
__device__ __forceinline__ void fwht128_wave(float* x, int nvec, int lane) {
  for (int h = 1; h < kD; h <<= 1) {
    for (int i = lane; i < nvec * 64; i += 64) {
      const int v = i >> 6, pr = i & 63;
      const int i0 = (pr / h) * 2 * h + (pr % h);
      float* row = x + v * kD;
      const float a = row[i0], b = row[i0 + h];
      row[i0] = a + b;
      row[i0 + h] = a - b;
    }
    wave_sync();
  }
  const float c = c32();
  for (int i = lane; i < nvec * kD; i += 64) x[i] = x[i] * c;
  wave_sync();
}

// Cross-lane reductions without LDS round trips.
// DPP lane permutations within a 16-lane row (full rows, so every lane has a
// source): xor 1, xor 2, reverse 8, reverse 16.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// ds_swizzle bitmask mode within 32 lanes: partner = lane ^ 16
__device__ __forceinline__ float swz16(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
}
__device__ __forceinline__ float half_sum(float v) {   // over the 32 lanes of a half-wave
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  return v + swz16(v);
}
__device__ __forceinline__ float half_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  return fmaxf(v, swz16(v));
}
__device__ __forceinline__ float wave_sum64(float v) {
  v = half_sum(v);
  return v + __shfl_xor(v, 32, 64);
}
__device__ __forceinline__ float wave_max64(float v) {
  v = half_max(v);
  return fmaxf(v, __shfl_xor(v, 32, 64));
}

}  // namespace kvq
