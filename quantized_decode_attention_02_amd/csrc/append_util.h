// Helpers of the quantize-on-append kernels that work on a vector per lane
// pair (append_block.hip, append_kivi.hip): source rows staged through LDS,
// the fp32 FWHT of half a vector per lane, code packing and the transposes
// from token rows to the value tiles' channel rows.
#pragma once

#include "kvq_device.h"

namespace kvq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTr = 36;   // dwords per row of the code transpose: 32 tokens + 4 (rows 36 dwords
                          // apart: 16 rows read at one offset hit 16 different bank quads)

// fp32 2^23: for |v| < 2^22, fma(x, r, 2^23 + o) is x r + o rounded to an
// integer (ulp 1 in [2^23, 2^24)), which lands in the low mantissa bits.
constexpr float kTwo23 = 8388608.0f;

// One launch: the tokens [T0, T0 + n) of an append whose source rows are
// (b, t - src_t0, h) of a [batch, src_tokens, Hkv, 128] fp16 array.
struct SegArgs {
  const __half* k_new;
  const __half* v_new;
  int64_t src_tokens, src_t0;
  int64_t T0, n;
  int64_t tile0, n_tiles, n_items;
};

// Pack the low `B`-bit fields of eight words f[0..7] (each a code in its low
// bits, zero above up to bit 23, anything from bit 24 on) as f[j] << (B j).
// Shifts of 8 or more push the high garbage out; the low fields go through
// one masked merge.
template <int B>
__device__ __forceinline__ uint32_t pack8(const uint32_t* f) {
  if (B == 4) {   // nibble pairs as bytes, then the four bytes by byte permutes
    const uint32_t b01 = (f[1] << 4) | f[0], b23 = (f[3] << 4) | f[2];
    const uint32_t b45 = (f[5] << 4) | f[4], b67 = (f[7] << 4) | f[6];
    const uint32_t lo = __builtin_amdgcn_perm(b23, b01, 0x0C0C0400u);
    const uint32_t hi = __builtin_amdgcn_perm(b67, b45, 0x0C0C0400u);
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
  } else {        // B == 3: 24 bits
    uint32_t acc = f[7] << 21;
    acc |= f[6] << 18;
    acc |= f[5] << 15;
    acc |= f[4] << 12;
    acc |= f[3] << 9;
    const uint32_t lo = (((f[2] << 6) | (f[1] << 3)) | f[0]);
    return ((lo & 0x1FFu) | acc) & 0xFFFFFFu;
  }
}
__device__ __forceinline__ uint32_t pack4x8(const uint32_t* f) {
  const uint32_t lo = __builtin_amdgcn_perm(f[1], f[0], 0x0C0C0400u);
  const uint32_t hi = __builtin_amdgcn_perm(f[3], f[2], 0x0C0C0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// (a ^ b) + c in one instruction; opaque to the compiler, which would
// otherwise split the accumulation of a bracket's disagreement into a
// compare and select per element.
__device__ __forceinline__ uint32_t xor_add(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t d;
  asm("v_xad_u32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// fp32 of the low (sel 0) or high (sel 1) fp16 half of w, plus or minus the
// other half, rounded once: v_fma_mix_f32 with the fp16 operands converted
// exactly inside the instruction (a + b and a - b are the same IEEE
// operations as fma(a, 1, b) and fma(b, -1, a)).
__device__ __forceinline__ float mix_sum(uint32_t w) {
  float d;
  asm("v_fma_mix_f32 %0, %1, 1.0, %1 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "=v"(d) : "v"(w));
  return d;
}
__device__ __forceinline__ float mix_diff(uint32_t w) {
  float d;
  asm("v_fma_mix_f32 %0, %1, -1.0, %1 op_sel:[1,0,0] op_sel_hi:[1,0,1]" : "=v"(d) : "v"(w));
  return d;
}

// 8 x 8 transpose of 4-bit fields: in[i] holds row i (field j at bits 4j);
// out[j] holds column j (field i at bits 4i).
__device__ __forceinline__ void transpose_nib8(const uint32_t* in, uint32_t* out) {
  uint32_t a[8], b[8];
  // 4 x 4 blocks of fields: the halves of rows i and i + 4
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = __builtin_amdgcn_perm(in[i + 4], in[i], 0x05040100u);       // lo(i), lo(i + 4)
    a[i + 4] = __builtin_amdgcn_perm(in[i + 4], in[i], 0x07060302u);   // hi(i), hi(i + 4)
  }
  // 2 x 2 blocks: bytes of rows r and r + 2
#pragma unroll
  for (int q = 0; q < 2; ++q) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = 4 * q + r;
      b[i] = __builtin_amdgcn_perm(a[i + 2], a[i], 0x06020400u);       // bytes 0, 2 of each
      b[i + 2] = __builtin_amdgcn_perm(a[i + 2], a[i], 0x07030501u);   // bytes 1, 3 of each
    }
  }
  // single fields: rows r and r + 1
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const uint32_t x = b[i], y = b[i + 1];
    b[i] = (x & 0x0F0F0F0Fu) | ((y << 4) & 0xF0F0F0F0u);
    b[i + 1] = ((x >> 4) & 0x0F0F0F0Fu) | (y & 0xF0F0F0F0u);
  }
  // b[k] now holds column j(k) with its fields in row order
  out[0] = b[0]; out[1] = b[1]; out[2] = b[2]; out[3] = b[3];
  out[4] = b[4]; out[5] = b[5]; out[6] = b[6]; out[7] = b[7];
}

// 4 x 4 transpose of bytes.
__device__ __forceinline__ void transpose_byte4(const uint32_t* in, uint32_t* out) {
  const uint32_t t0 = __builtin_amdgcn_perm(in[1], in[0], 0x05010400u);
  const uint32_t t1 = __builtin_amdgcn_perm(in[1], in[0], 0x07030602u);
  const uint32_t t2 = __builtin_amdgcn_perm(in[3], in[2], 0x05010400u);
  const uint32_t t3 = __builtin_amdgcn_perm(in[3], in[2], 0x07030602u);
  out[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
  out[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  out[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// Mask of the fields [lo, hi) of width W in a word whose fields start at
// bit `first` (fields outside the word ignored).
__device__ __forceinline__ uint32_t field_mask(int lo, int hi, int first, int W) {
  const int b0 = min(max(lo * W - first, 0), 32), b1 = min(max(hi * W - first, 0), 32);
  const uint32_t upto1 = b1 >= 32 ? 0xFFFFFFFFu : ((1u << b1) - 1u);
  const uint32_t upto0 = b0 >= 32 ? 0xFFFFFFFFu : ((1u << b0) - 1u);
  return upto1 & ~upto0;
}

// Value of `v` in the lane 32 apart (the other half of the lane's vector).
__device__ __forceinline__ uint32_t other_half(uint32_t v, int half) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return half ? r[0] : r[1];
}

// 16 x 16 transpose of 2-bit fields: in[i] holds row i (field j at bits
// 2j); out[j] holds column j (field i at bits 2i).  Four rounds of swapping
// the off-diagonal quarters of ever smaller blocks.
__device__ __forceinline__ void transpose_crumb16(const uint32_t* in, uint32_t* out) {
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) w[i] = in[i];
  // 8 x 8 blocks: 16-bit halves of rows i and i + 8
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t a = w[i], b = w[i + 8];
    w[i] = __builtin_amdgcn_perm(b, a, 0x05040100u);
    w[i + 8] = __builtin_amdgcn_perm(b, a, 0x07060302u);
  }
  // 4 x 4 blocks: bytes of rows i and i + 4
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i & 4) continue;
    const uint32_t a = w[i], b = w[i + 4];
    w[i] = __builtin_amdgcn_perm(b, a, 0x06020400u);
    w[i + 4] = __builtin_amdgcn_perm(b, a, 0x07030501u);
  }
  // 2 x 2 blocks: nibbles of rows i and i + 2
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i & 2) continue;
    const uint32_t a = w[i], b = w[i + 2];
    w[i] = (a & 0x0F0F0F0Fu) | ((b << 4) & 0xF0F0F0F0u);
    w[i + 2] = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
  }
  // single fields: rows i and i + 1
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    const uint32_t a = w[i], b = w[i + 1];
    w[i] = (a & 0x33333333u) | ((b << 2) & 0xCCCCCCCCu);
    w[i + 1] = ((a >> 2) & 0x33333333u) | (b & 0xCCCCCCCCu);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) out[i] = w[i];
}

// The 32 fp16 rows of a tile, 16-byte chunk (lane & 15) of rows 4 i +
// (lane >> 4) in raw[i], into a wave's LDS area: row v at 256 v, its chunk c
// at slot c ^ (v & 15).
__device__ __forceinline__ void stage_rows(uint8_t* reg, const u32x4* raw, int lane) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 4 * i + (lane >> 4), c = lane & 15;
    *reinterpret_cast<u32x4*>(reg + row * 256 + 16 * (c ^ (row & 15))) = raw[i];
  }
}

// Half a vector per lane: lane v + 32 half gets elements 64 half + k of row
// v in r[k] as fp32.  HAD: the unnormalized FWHT instead, in its fixed fp32
// stage order -- stage h = 1 folded into the conversion, stages 2 .. 32 in
// the lane, stage 64 with the other half through v_permlane32_swap, after
// which r[k] (k < 32) is transform output k + 32 half and r[32 + k] output
// 64 + 32 half + k.  HAD == 2: the input signs (sgn_in: per fp16 pair, bits
// 15 and 31) are flipped first.
template <int HAD>
__device__ __forceinline__ void read_half(const uint8_t* reg, const uint32_t* sgn_in, int lane, float* r) {
  const int half = lane >> 5, v = lane & 31;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int chunk = 8 * half + c;
    const u32x4 q = *reinterpret_cast<const u32x4*>(reg + v * 256 + 16 * (chunk ^ (v & 15)));
    u32x4 sg = {0u, 0u, 0u, 0u};
    if (HAD == 2) sg = *reinterpret_cast<const u32x4*>(sgn_in + 4 * chunk);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t w = q[k] ^ sg[k];
      if (HAD) {
        r[8 * c + 2 * k] = mix_sum(w);
        r[8 * c + 2 * k + 1] = mix_diff(w);
      } else {
        r[8 * c + 2 * k] = __half2float(__ushort_as_half((uint16_t)(w & 0xFFFFu)));
        r[8 * c + 2 * k + 1] = __half2float(__ushort_as_half((uint16_t)(w >> 16)));
      }
    }
  }
  if (HAD) {
#pragma unroll
    for (int hs = 2; hs < 64; hs <<= 1) {
#pragma unroll
      for (int j = 0; j < 64; ++j) {
        if (j & hs) continue;
        const float a = r[j], b = r[j + hs];
        r[j] = a + b;
        r[j + hs] = a - b;
      }
    }
    // stage 64: the halves trade r[32 ..] of the lower and r[.. 31] of the
    // upper, so each lane holds pairs (x_e, x_{e+64}) as (r[i], r[32 + i])
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(r[i]), __float_as_uint(r[32 + i]),
                                                       false, false);
      const float a = __uint_as_float(sw[0]), b = __uint_as_float(sw[1]);
      r[i] = a + b;
      r[32 + i] = a - b;
    }
  }
}

// Channel of r[k] after read_half (see there).
template <int HAD>
__device__ __forceinline__ int half_chan(int k, int half) {
  return HAD ? k + 32 * half + (k >= 32 ? 32 : 0) : 64 * half + k;
}

}  // namespace kvq
