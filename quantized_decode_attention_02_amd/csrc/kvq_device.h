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
  if (block_scheme(g.scheme) || grp * kGroup >= g.hi_start) {
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

// Value of lane (lane ^ M) of the wave: M = 1, 2 by DPP quad permutes, 4, 8, 16
// by ds_swizzle in bitmask mode (within 32 lanes), 32 by ds_bpermute.
template <int M>
__device__ __forceinline__ float lane_xor(float v, int lane) {
  if (M == 1) return dpp<0xB1>(v);
  if (M == 2) return dpp<0x4E>(v);
  if (M == 4) return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x101F));
  if (M == 8) return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x201F));
  if (M == 16) return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __float_as_int(v)));
}

// One butterfly stage h = 2M of fwht128_reg: this lane's elements pair with
// lane (lane ^ M)'s; the lane holding the lower index keeps a + b, the other
// a - b, a being the lower element.  Both are computed as p + (+-e) (x + y
// and y + x, and a + (-b) and a - b, are the same IEEE operation), the sign
// flip an exact xor.
template <int M>
__device__ __forceinline__ void fwht_stage(float& e0, float& e1, int lane) {
  const float p0 = lane_xor<M>(e0, lane), p1 = lane_xor<M>(e1, lane);
  const uint32_t flip = (lane & M) ? 0x80000000u : 0u;
  e0 = p0 + __uint_as_float(__float_as_uint(e0) ^ flip);
  e1 = p1 + __uint_as_float(__float_as_uint(e1) ^ flip);
}

// Normalized FWHT-128 of one vector held in the registers of a wave, lane l
// holding elements 2l (e0) and 2l + 1 (e1), in the fixed fp32 schedule: for
// h = 1, 2, ..., 64 in that order every pair (x[i], x[i+h]) with bit log2(h)
// of i clear becomes (a + b, a - b), each one fp32 operation; then every
// element is multiplied by fp32(1/sqrt(128)).  H in Sylvester order is
// orthonormal after the scaling, so nothing is lost and dot products are kept
// ([troisinh] "Tại sao nó hoạt động", item 2; [trefon] "Jak 4-bitowemu cache
// to uchodzi: najpierw obrót").  Stage h = 1 stays in the lane; stage h = 2M
// exchanges with lane l ^ M through DPP / ds_swizzle / ds_bpermute: no LDS
// memory, no barrier.
__device__ __forceinline__ void fwht128_reg(float& e0, float& e1, int lane) {
  {
    const float a = e0, b = e1;
    e0 = a + b;
    e1 = a - b;
  }
  fwht_stage<1>(e0, e1, lane);
  fwht_stage<2>(e0, e1, lane);
  fwht_stage<4>(e0, e1, lane);
  fwht_stage<8>(e0, e1, lane);
  fwht_stage<16>(e0, e1, lane);
  fwht_stage<32>(e0, e1, lane);
  const float c = c32();
  e0 = e0 * c;
  e1 = e1 * c;
}

// Value of lane (lane ^ M) within a 16-lane row: M = 1, 2 by DPP quad
// permutes, 4, 8 by ds_swizzle in bitmask mode.
template <int M>
__device__ __forceinline__ uint32_t row_xor(uint32_t v) {
  if (M == 1) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
  if (M == 2) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
  if (M == 4) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x101F);
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x201F);
}

// Cross-lane butterfly stage h = 8M of fwht128_row16: with p the partner's
// element, the lower lane keeps e + p and the upper one p - e, both as one
// exactly rounded fma(e, +-1, p).
template <int M>
__device__ __forceinline__ void fwht_row_stage(float* x, int i) {
  const float sgn = (i & M) ? -1.0f : 1.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float p = __uint_as_float(row_xor<M>(__float_as_uint(x[j])));
    x[j] = fmaf(x[j], sgn, p);
  }
}

// fwht128_reg for a vector spread over a 16-lane row, lane i of the row
// holding elements 8i .. 8i + 7 in x[0..7] (four vectors per wave).  Same
// schedule and fp32 operations: stages h = 1, 2, 4 inside the lane, h = 8,
// 16, 32, 64 with lanes i ^ 1, i ^ 2, i ^ 4, i ^ 8; then the scaling.
__device__ __forceinline__ void fwht128_row16(float* x, int i) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j & h) continue;
      const float a = x[j], b = x[j + h];
      x[j] = a + b;
      x[j + h] = a - b;
    }
  }
  fwht_row_stage<1>(x, i);
  fwht_row_stage<2>(x, i);
  fwht_row_stage<4>(x, i);
  fwht_row_stage<8>(x, i);
  const float c = c32();
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = x[j] * c;
}

// Sign flips of the randomized rotation D_post H D_pre / sqrt(128) ([trefon]
// "Jak 4-bitowemu cache to uchodzi: najpierw obrót": signs, transform,
// signs): coordinate i is negated when bit i of the mask (word i / 32) is
// set, by an exact xor of its sign bit, so the fp32 schedule is unchanged.
__device__ __forceinline__ uint32_t mask_word(const Mask128& m, int word) {
  const uint32_t a = (word & 1) ? m.w[1] : m.w[0];
  const uint32_t b = (word & 1) ? m.w[3] : m.w[2];
  return (word & 2) ? b : a;
}
__device__ __forceinline__ float flip_by(float v, uint32_t bits, int bit) {
  return __uint_as_float(__float_as_uint(v) ^ (((bits >> bit) & 1u) << 31));
}

// fwht128_reg between the flips of `pre` and `post` (elements 2 lane and
// 2 lane + 1: word lane / 16, bits 2 lane mod 32 and the next).
__device__ __forceinline__ void fwht128_reg_signed(float& e0, float& e1, int lane, const Mask128& pre,
                                                   const Mask128& post) {
  const int word = lane >> 4, bit = (2 * lane) & 31;
  uint32_t m = mask_word(pre, word);
  e0 = flip_by(e0, m, bit);
  e1 = flip_by(e1, m, bit + 1);
  fwht128_reg(e0, e1, lane);
  m = mask_word(post, word);
  e0 = flip_by(e0, m, bit);
  e1 = flip_by(e1, m, bit + 1);
}

// fwht128_row16 between the flips of `pre` and `post` (row lane i holds
// elements 8i .. 8i + 7: word i / 4, bits 8 (i mod 4) ..).
__device__ __forceinline__ void fwht128_row16_signed(float* x, int i, const Mask128& pre,
                                                     const Mask128& post) {
  const int word = i >> 2, b0 = 8 * (i & 3);
  uint32_t m = mask_word(pre, word);
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = flip_by(x[j], m, b0 + j);
  fwht128_row16(x, i);
  m = mask_word(post, word);
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = flip_by(x[j], m, b0 + j);
}

// Maximum of a non-negative float over a quad of lanes (4q .. 4q + 3), on
// its bit pattern.
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
  v = max(v, row_xor<1>(v));
  return max(v, row_xor<2>(v));
}

// Maximum of a non-negative float over a 16-lane row, on its bit pattern
// (for non-negative floats the integer order is the numeric order).
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
  v = max(v, row_xor<1>(v));
  v = max(v, row_xor<2>(v));
  v = max(v, row_xor<4>(v));
  return max(v, row_xor<8>(v));
}

// fwht128_reg over `nvec` float rows of 128 in LDS by a whole work-group:
// wave w transforms rows w, w + nthreads / 64, ... in its registers and
// writes them back.  With `sgn`, each row goes through D_post H D_pre /
// sqrt(128) instead.  The rows must be complete when it is called; it ends
// with a barrier on LDS.
__device__ __forceinline__ void fwht128_rows(float* x, int nvec, int tid, int nthreads,
                                             const Mask128& pre, const Mask128& post, bool sgn) {
  const int lane = tid & 63;
  for (int v = tid >> 6; v < nvec; v += nthreads >> 6) {
    float2* r = reinterpret_cast<float2*>(x + v * kD) + lane;
    float2 e = *r;
    if (sgn) fwht128_reg_signed(e.x, e.y, lane, pre, post);
    else fwht128_reg(e.x, e.y, lane);
    *r = e;
  }
  lds_barrier();
}

// The same for rows of one wave's own (wave barriers only).
__device__ __forceinline__ void fwht128_rows_wave(float* x, int nvec, int lane, const Mask128& pre,
                                                  const Mask128& post, bool sgn) {
  wave_sync();
  for (int v = 0; v < nvec; ++v) {
    float2* r = reinterpret_cast<float2*>(x + v * kD) + lane;
    float2 e = *r;
    if (sgn) fwht128_reg_signed(e.x, e.y, lane, pre, post);
    else fwht128_reg(e.x, e.y, lane);
    *r = e;
  }
  wave_sync();
}

}  // namespace kvq
