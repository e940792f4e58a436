// Quantize-on-append of whole KIVI groups that come entirely from the new
// tokens (the bulk of a prefill or of a long append), at 4, 3 or 2 bits.
//
// Sources cited here:
//   [troisinh] "KV Cache Quantization — Nén cache INT4/INT3, mở khóa
//              ultra-long context" (troisinh.com): "Tại sao nó hoạt động",
//              items 1 and 2 (per-channel keys, per-token values, the
//              rotation), "Mixed Precision" (the tiers).
//   [nalar]    "Kuantisasi KV Cache dengan Error Budget yang Eksplisit"
//              (nalar.dev): "Granularitas kuantisasi mengendalikan rentang
//              yang harus dicakup setiap scale".
//
// What is stored is the asymmetric group quantizer of append.hip, bit for
// bit: over a group x (keys: one channel over the group's 32 tokens; values:
// one token over a 32-channel slice), s_h = fp16(fl32(fl32(max - min) / Q))
// + 0, z_h = fp16(min) + 0, code = clamp(rint(fl32(fl32(x - z_h) / s_h)), 0,
// Q), 0 when s_h == 0; x is the fp16 input, or fl32(FWHT(x) c) when the
// cache is rotated.
//
// Work: a wave item is the keys or the values of one 32-token group of one
// (sequence, kv head) pair; each wave takes a contiguous run of items.  The
// 32 fp16 rows come through the wave's LDS area as in the block appends
// (append_util.h).  Values are per token: lanes v and v + 32 hold token v's
// two halves (two 32-channel slices each) and quantize in the lane; their
// codes leave through the LDS area, transposed into the value tile's
// channel rows.  Keys are per channel: lane l takes channels 2l and 2l + 1
// over the 32 tokens, read as columns of the staged rows (or, rotated, of
// the fp32 transform written back to LDS); their codes leave transposed into
// the key tile's token rows.  Codes come from the bracket of append_block.hip
// (fma(d, r (1 -+ 2^-21), 2^23) at both ends, r within 1 ulp of 1/s_h, then
// clamped to [0, Q]):
// the exact quotient lies strictly inside, so where the ends agree it rounds
// and clamps the same way; elsewhere the wave redoes those codes with the
// division.  The bracket's ends are compared before the clamp (equal
// inputs clamp equally), and fl32(1/s_h) may be v_rcp_f32's (1 ulp): the
// 2^-21 margin covers it.  3-bit codes take the 4-bit path as nibbles (top bit clear) up
// to the transposed rows, whose 4-bit dwords then shrink to 24 bits each
// (nib_to_3) and join their neighbours' into the 3-bit bit strings.
#pragma clang fp contract(off)

#include "append_util.h"

namespace kvq {
namespace {

struct KiviArgs {
  const __half* k_new;
  const __half* v_new;
  int64_t n_new, T0;       // the append: tokens [T0, T0 + n_new)
  int64_t g0, n_grp;       // groups [g0, g0 + n_grp) of every pair
  int64_t hi_start;        // first token of the high-bit tier
  int64_t n_items;
};

struct KItem {
  int64_t pair, grp;
  int b, h, tensor;
};

__device__ __forceinline__ KItem kitem_at(const Geom& g, const KiviArgs& a, int64_t it) {
  KItem r;
  r.tensor = (int)(it & 1);
  const int64_t rest = it >> 1;
  r.pair = rest / a.n_grp;
  r.grp = a.g0 + rest % a.n_grp;
  r.b = (int)(r.pair / g.Hkv);
  r.h = (int)(r.pair % g.Hkv);
  return r;
}

// fl32(x - z) of the fp16 in the low (HI = false) or high half of w and the
// fp16 z: one v_fma_mix (x and z converted exactly, one rounding).
template <bool HI>
__device__ __forceinline__ float mix_sub(uint32_t w, uint32_t z) {
  float d;
  if (HI)
    asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel:[1,0,0] op_sel_hi:[1,0,1]" : "=v"(d) : "v"(w), "v"(z));
  else
    asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel:[0,0,0] op_sel_hi:[1,0,1]" : "=v"(d) : "v"(w), "v"(z));
  return d;
}

// (s_h, z_h) of a group with extremes mn, mx; rs = fl32(1 / s_h) (0 when
// s_h == 0) and the bracket around it.
struct Grp {
  uint32_t sz;        // s_h | z_h << 16
  float s, z, lo, hi;
};
__device__ __forceinline__ Grp grp_params(float mn, float mx, float Q) {
  Grp r;
  uint16_t sb = float_to_half_bits((mx - mn) / Q);
  uint16_t zb = float_to_half_bits(mn);
  if (sb == 0x8000u) sb = 0;
  if (zb == 0x8000u) zb = 0;
  r.sz = (uint32_t)sb | ((uint32_t)zb << 16);
  r.s = half_bits_to_float(sb);
  r.z = half_bits_to_float(zb);
  // v_rcp_f32 (within 1 ulp of 1 / s_h): the ends r (1 -+ 2^-21), rounded,
  // still lie strictly below and above 1 / s_h
  const float rs = r.s != 0.0f ? __builtin_amdgcn_rcpf(r.s) : 0.0f;
  r.lo = rs * (1.0f - 0x1p-21f);
  r.hi = rs * (1.0f + 0x1p-21f);
  return r;
}

// 2^23 + rint(d r) for d = fl32(x - z_h) at one end r of the bracket
// (unclamped: where the two ends agree unclamped, they agree clamped).
__device__ __forceinline__ float code_end(float d, float r) { return fmaf(d, r, kTwo23); }
// The code word from an end: 2^23 + code, clamped to [0, Q].
__device__ __forceinline__ uint32_t code_clamp(float e, float Q) {
  return __float_as_uint(__builtin_amdgcn_fmed3f(e, kTwo23, kTwo23 + Q));
}
// The exact code, 2^23 + code as a word like code_clamp().
__device__ __forceinline__ uint32_t code_exact(float d, const Grp& gp, float Q) {
  const float c = gp.s != 0.0f ? rintf(d / gp.s) : 0.0f;
  return __float_as_uint(kTwo23 + fminf(fmaxf(c, 0.0f), Q));
}

// Eight nibbles n_k (bits 4k, each < 8) as eight 3-bit fields (bits 3k):
// nibble pairs into 6-bit bytes, byte pairs into 12-bit halves, then the
// halves into 24 bits.
__device__ __forceinline__ uint32_t nib_to_3(uint32_t x) {
  const uint32_t y = (x & 0x07070707u) | ((x >> 1) & 0x38383838u);
  const uint32_t y2 = (y & 0x003F003Fu) | ((y >> 2) & 0x0FC00FC0u);
  return (y2 & 0xFFFu) | ((y2 >> 4) & 0xFFF000u);
}

// Dword k (0..2) of a 96-bit run made of four 24-bit pieces, from piece k
// (own) and piece k + 1 (next).
__device__ __forceinline__ uint32_t join3(uint32_t own, uint32_t next, int k) {
  return k == 0 ? (own | (next << 24)) : k == 1 ? ((own >> 8) | (next << 16)) : ((own >> 16) | (next << 8));
}

// Waves per SIMD: the unrotated kernels' 32 KiB of LDS per work-group leave
// room for three work-groups per compute unit, the rotated ones' for two.
template <int HB, int LB, int HAD>
__global__ __launch_bounds__(256, HAD ? 2 : 3) void kivi_group_kernel(Geom g, Planes p, KiviArgs a) {
  // LDS of one wave: the group's 32 fp16 rows; rotated keys: then their
  // fp32 transform, rows of 132 floats (4 of pad: the 16 row writes of one
  // pass hit 16 different bank quads)
  constexpr int kF32Row = 132;
  constexpr int kWaveLds = HAD ? kGroup * kF32Row * 4 : kGroup * kD * 2;
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kWaveLds];
  __shared__ __attribute__((aligned(16))) uint32_t sgn_in[64];   // fp16 pair sign masks
  __shared__ __attribute__((aligned(16))) uint32_t sgn_f[kD];    // fp32 output sign masks
  if (HAD == 2) {
    const int t = threadIdx.x;
    if (t < 64) {
      const uint32_t w = mask_word(g.sign_in, t >> 4);
      const int bit = (2 * t) & 31;
      sgn_in[t] = (((w >> bit) & 1u) << 15) | (((w >> (bit + 1)) & 1u) << 31);
    } else if (t >= 128) {
      const int c = t - 128;
      sgn_f[c] = ((mask_word(g.sign_out, c >> 5) >> (c & 31)) & 1u) << 31;
    }
    __syncthreads();
  }

  // the wave index is uniform: a scalar register keeps the item walk and its
  // addresses on the scalar unit
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, v = lane & 31;
  const int64_t nwaves = (int64_t)gridDim.x * 4, gw = (int64_t)blockIdx.x * 4 + wv;
  const int64_t i0 = gw * a.n_items / nwaves, i1 = (gw + 1) * a.n_items / nwaves;
  if (i0 >= i1) return;
  uint8_t* reg = lds + wv * kWaveLds;
  const uint32_t rowbytes = (uint32_t)g.Hkv * kD * 2;

  // 16-byte chunk (lane & 15) of the group's rows 4 i + (lane >> 4); the row
  // offset from the pair's first new row fits 32 bits (checked by the host)
#define KVQ_ISSUE_GROUP(it)                                                                     \
  {                                                                                             \
    const uint8_t* base_ = reinterpret_cast<const uint8_t*>(                                    \
        ((it).tensor ? a.v_new : a.k_new) + ((int64_t)(it).b * a.n_new * g.Hkv + (it).h) * kD); \
    const uint32_t r0_ = (uint32_t)((it).grp * kGroup - a.T0) + (uint32_t)(lane >> 4);          \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) raw[i] = *reinterpret_cast<const u32x4*>(     \
        base_ + ((r0_ + 4u * i) * rowbytes + 16u * (uint32_t)(lane & 15)));                     \
  }

  KItem cur = kitem_at(g, a, i0);
  u32x4 raw[8];
  KVQ_ISSUE_GROUP(cur)
  for (int64_t item = i0;; ++item) {
    stage_rows(reg, raw, lane);
    // the next item's rows (past the last item: this item's again, from L2)
    KItem nit = cur;
    if (item + 1 < i1) {
      nit.tensor ^= 1;
      if (nit.tensor == 0) {
        if (++nit.grp == a.g0 + a.n_grp) {
          nit.grp = a.g0;
          ++nit.pair;
          if (++nit.h == g.Hkv) {
            nit.h = 0;
            ++nit.b;
          }
        }
      }
    }
    KVQ_ISSUE_GROUP(nit)

    const bool hi_tier = cur.grp * kGroup >= a.hi_start;
    auto body = [&](auto bits_tag) {
    constexpr int bits = decltype(bits_tag)::value;
    const float Q = (float)((1 << bits) - 1);
    const int64_t tb = 512 * (int64_t)bits;
    uint8_t* kt = hi_tier ? p.p[KVQ_PLANE_K_HI] + (cur.pair * g.hi_slots + cur.grp % g.hi_slots) * tb
                          : p.p[KVQ_PLANE_K_LO] + (cur.pair * g.gmax + cur.grp) * tb;
    uint8_t* vt = hi_tier ? p.p[KVQ_PLANE_V_HI] + (cur.pair * g.hi_slots + cur.grp % g.hi_slots) * tb
                          : p.p[KVQ_PLANE_V_LO] + (cur.pair * g.gmax + cur.grp) * tb;
    uint32_t* tr = reinterpret_cast<uint32_t*>(reg);

    if (cur.tensor == 1) {
      // ================= values: token v, two 32-channel slices per lane
      float r[64];
      read_half<HAD>(reg, sgn_in, lane, r);
      if (HAD) {
#pragma unroll
        for (int j = 0; j < 64; ++j) {
          float y = r[j] * c32();
          if (HAD == 2) y = __uint_as_float(__float_as_uint(y) ^ sgn_f[half_chan<HAD>(j, half)]);
          r[j] = y;
        }
      }
      uint32_t U[8];   // 4 and 3 bits: eight 8-channel nibble words; 2 bits: four 16-channel words
      uint32_t szw[2];
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        float mn = r[32 * sl], mx = r[32 * sl];
#pragma unroll
        for (int j = 1; j < 32; ++j) {
          mn = fminf(mn, r[32 * sl + j]);
          mx = fmaxf(mx, r[32 * sl + j]);
        }
        const Grp gp = grp_params(mn, mx, Q);
        szw[sl] = gp.sz;
        // 8 codes a unit at 4 and 3 bits, 16 at 2
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (bits == 2 && u >= 2) break;
          const int n = bits == 2 ? 16 : 8;
          const int j0 = 32 * sl + n * u;
          uint32_t f[16];
          uint32_t diff = 0;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            if (j >= n) break;
            const float d = r[j0 + j] - gp.z;
            const float lo = code_end(d, gp.lo), hi = code_end(d, gp.hi);
            diff = xor_add(__float_as_uint(lo), __float_as_uint(hi), diff);
            f[j] = code_clamp(lo, Q);
          }
          if (__builtin_expect(__any(diff != 0u), 0)) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              if (j >= n) break;
              f[j] = code_exact(r[j0 + j] - gp.z, gp, Q);
            }
          }
          if (bits != 2) {
            U[4 * sl + u] = pack8<4>(f);
          } else {   // crumb pairs as nibbles, then the nibbles as pack8<4>
            uint32_t nb[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) nb[k] = (f[2 * k + 1] << 2) | f[2 * k];
            U[2 * sl + u] = pack8<4>(nb);
          }
        }
      }
      // metadata: token v, slice of r[32 sl ..]
      {
        uint32_t* vm = reinterpret_cast<uint32_t*>(p.p[KVQ_PLANE_V_META] + (cur.pair * g.gmax + cur.grp) * 512);
        const int s0 = half_chan<HAD>(0, half) / 32, s1 = half_chan<HAD>(32, half) / 32;
        vm[4 * v + s0] = szw[0];
        vm[4 * v + s1] = szw[1];
      }
      // token rows -> channel rows (the rows were read above; this wave's
      // LDS operations run in order)
      if (bits != 2) {
#pragma unroll
        for (int u = 0; u < 8; ++u) tr[(half_chan<HAD>(8 * u, half) / 8) * kTr + v] = U[u];
        const int cg = lane & 15, tg = lane >> 4;
        const uint32_t* src = tr + cg * kTr + 8 * tg;
        uint32_t in[8], o[8];
        const uint4 q0 = *reinterpret_cast<const uint4*>(src), q1 = *reinterpret_cast<const uint4*>(src + 4);
        in[0] = q0.x; in[1] = q0.y; in[2] = q0.z; in[3] = q0.w;
        in[4] = q1.x; in[5] = q1.y; in[6] = q1.z; in[7] = q1.w;
        transpose_nib8(in, o);
        if (bits == 4) {
#pragma unroll
          for (int j = 0; j < 8; ++j) *reinterpret_cast<uint32_t*>(vt + 16 * (8 * cg + j) + 4 * tg) = o[j];
        } else {
          // o[j]: tokens 8 tg .. 8 tg + 7 of channel 8 cg + j, bits 24 tg .. of
          // its 12-byte row; lane + 16 holds the next 8 tokens
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t c = nib_to_3(o[j]);
            const uint32_t nx = __shfl_down(c, 16);
            if (tg < 3) *reinterpret_cast<uint32_t*>(vt + 12 * (8 * cg + j) + 4 * tg) = join3(c, nx, tg);
          }
        }
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) tr[(half_chan<HAD>(16 * u, half) / 16) * kTr + v] = U[u];
        if (lane < 16) {
          const int cg = lane & 7, tg = lane >> 3;
          const uint32_t* src = tr + cg * kTr + 16 * tg;
          uint32_t in[16], o[16];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint4 q = *reinterpret_cast<const uint4*>(src + 4 * k);
            in[4 * k] = q.x; in[4 * k + 1] = q.y; in[4 * k + 2] = q.z; in[4 * k + 3] = q.w;
          }
          transpose_crumb16(in, o);
#pragma unroll
          for (int j = 0; j < 16; ++j) *reinterpret_cast<uint32_t*>(vt + 8 * (16 * cg + j) + 4 * tg) = o[j];
        }
      }
    } else {
      // ================= keys: channels 2 lane, 2 lane + 1 over the 32 tokens
      float mn0, mx0, mn1, mx1;
      uint32_t xh[kGroup];   // plain: the fp16 pair of each token
      float y0[HAD ? kGroup : 1], y1[HAD ? kGroup : 1];
      if (HAD) {
        float r[64];
        read_half<HAD>(reg, sgn_in, lane, r);
        // y = fl32(x c), signed, back to LDS as fp32 rows [token][channel]
        float* rows = reinterpret_cast<float*>(reg);
#pragma unroll
        for (int j = 0; j < 64; ++j) {
          float y = r[j] * c32();
          if (HAD == 2) y = __uint_as_float(__float_as_uint(y) ^ sgn_f[half_chan<HAD>(j, half)]);
          r[j] = y;
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int j = 4 * k;
          *reinterpret_cast<float4*>(rows + v * kF32Row + half_chan<HAD>(j, half)) =
              make_float4(r[j], r[j + 1], r[j + 2], r[j + 3]);
        }
#pragma unroll
        for (int t = 0; t < kGroup; ++t) {
          const float2 yy = *reinterpret_cast<const float2*>(rows + t * kF32Row + 2 * lane);
          y0[t] = yy.x;
          y1[t] = yy.y;
        }
        mn0 = mx0 = y0[0];
        mn1 = mx1 = y1[0];
#pragma unroll
        for (int t = 1; t < kGroup; ++t) {
          mn0 = fminf(mn0, y0[t]); mx0 = fmaxf(mx0, y0[t]);
          mn1 = fminf(mn1, y1[t]); mx1 = fmaxf(mx1, y1[t]);
        }
      } else {
#pragma unroll
        for (int t = 0; t < kGroup; ++t)
          xh[t] = *reinterpret_cast<const uint32_t*>(reg + t * 256 + 16 * ((lane >> 2) ^ (t & 15)) + 4 * (lane & 3));
        // extremes of both channels at once on the fp16 pairs
        typedef _Float16 hh2 __attribute__((ext_vector_type(2)));
        hh2 mn = __builtin_bit_cast(hh2, xh[0]), mx = mn;
#pragma unroll
        for (int t = 1; t < kGroup; ++t) {
          const hh2 x = __builtin_bit_cast(hh2, xh[t]);
          mn = __builtin_elementwise_min(mn, x);
          mx = __builtin_elementwise_max(mx, x);
        }
        mn0 = (float)mn[0]; mn1 = (float)mn[1];
        mx0 = (float)mx[0]; mx1 = (float)mx[1];
      }
      const Grp g0p = grp_params(mn0, mx0, Q), g1p = grp_params(mn1, mx1, Q);
      {
        uint2* km = reinterpret_cast<uint2*>(p.p[KVQ_PLANE_K_META] + (cur.pair * g.gmax + cur.grp) * 512);
        km[lane] = make_uint2(g0p.sz, g1p.sz);
      }
      // codes per token: 4 and 3 bits: byte c0 | c1 << 4; 2 bits: nibble c0 | c1 << 2
      uint32_t tw[8];   // 4 and 3 bits: tokens 4j .. 4j + 3 a word; 2 bits: 8j .. 8j + 7
      const uint32_t z0h = g0p.sz >> 16, z1h = g1p.sz >> 16;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int n = bits == 2 ? 8 : 4;
        if (bits == 2 && q >= 4) break;
        uint32_t f0[8], f1[8], diff = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          if (k >= n) break;
          const int t = n * q + k;
          const float d0 = HAD ? y0[t] - g0p.z : mix_sub<false>(xh[t], z0h);
          const float d1 = HAD ? y1[t] - g1p.z : mix_sub<true>(xh[t], z1h);
          const float a0 = code_end(d0, g0p.lo), b0 = code_end(d0, g0p.hi);
          const float a1 = code_end(d1, g1p.lo), b1 = code_end(d1, g1p.hi);
          diff = xor_add(__float_as_uint(a0), __float_as_uint(b0), diff);
          diff = xor_add(__float_as_uint(a1), __float_as_uint(b1), diff);
          f0[k] = code_clamp(a0, Q);
          f1[k] = code_clamp(a1, Q);
        }
        if (__builtin_expect(__any(diff != 0u), 0)) {
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            if (k >= n) break;
            const int t = n * q + k;
            const float d0 = HAD ? y0[t] - g0p.z : mix_sub<false>(xh[t], z0h);
            const float d1 = HAD ? y1[t] - g1p.z : mix_sub<true>(xh[t], z1h);
            f0[k] = code_exact(d0, g0p, Q);
            f1[k] = code_exact(d1, g1p, Q);
          }
        }
        if (bits != 2) {
          uint32_t by[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) by[k] = (f1[k] << 4) | f0[k];
          tw[q] = pack4x8(by);
        } else {
          uint32_t nb[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) nb[k] = (f1[k] << 2) | f0[k];
          tw[q] = pack8<4>(nb);
        }
      }
      // lane words -> token rows: word q of lane l is column l of tokens
      // (4 or 8) q ..; a token row's word w gathers lanes 4w .. 4w + 3 (4
      // bits, a byte each) or 8w .. 8w + 7 (2 bits, a nibble each).  The
      // column reads above are done (in-order LDS), so the area is free.
      if (bits != 2) {
#pragma unroll
        for (int q = 0; q < 8; ++q) tr[q * 64 + lane] = tw[q];
        const int w = lane & 15, q0 = lane >> 4;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int q = q0 + 4 * e;
          const uint4 in4 = *reinterpret_cast<const uint4*>(tr + q * 64 + 4 * w);
          const uint32_t in[4] = {in4.x, in4.y, in4.z, in4.w};
          uint32_t o[4];
          transpose_byte4(in, o);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (bits == 4) {
              *reinterpret_cast<uint32_t*>(kt + ktile_offset(4 * q + i, 4 * w)) = o[i];
            } else {
              // o[i]: channels 8 w .. 8 w + 7 of token 4 q + i, bits 24 w .. of
              // its 48-byte row; lane + 1 holds channels 8 w + 8 ..
              const uint32_t c = nib_to_3(o[i]);
              const uint32_t nx = __shfl_down(c, 1);
              const int k = w & 3;
              if (k < 3)
                *reinterpret_cast<uint32_t*>(kt + ktile_offset(4 * q + i, 4 * (3 * (w >> 2) + k))) = join3(c, nx, k);
            }
          }
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) tr[q * 64 + lane] = tw[q];
        if (lane < 32) {
          const int w = lane & 7, q = lane >> 3;
          const uint4 a4 = *reinterpret_cast<const uint4*>(tr + q * 64 + 8 * w);
          const uint4 b4 = *reinterpret_cast<const uint4*>(tr + q * 64 + 8 * w + 4);
          const uint32_t in[8] = {a4.x, a4.y, a4.z, a4.w, b4.x, b4.y, b4.z, b4.w};
          uint32_t o[8];
          transpose_nib8(in, o);
#pragma unroll
          for (int i = 0; i < 8; ++i)
            *reinterpret_cast<uint32_t*>(kt + ktile_offset(8 * q + i, 4 * w)) = o[i];
        }
      }
    }
    };
    if (HB == LB || hi_tier) body(std::integral_constant<int, HB>{});
    else body(std::integral_constant<int, LB>{});
    if (item + 1 >= i1) break;
    cur = nit;
  }
#undef KVQ_ISSUE_GROUP
}

template <int HB, int LB, int HAD>
hipError_t launch_kg(const Geom& g, const Planes& p, const KiviArgs& a, hipStream_t s) {
  const void* fn = reinterpret_cast<const void*>(&kivi_group_kernel<HB, LB, HAD>);
  const int64_t resident = (int64_t)occupancy_wgs_per_cu(fn) * device_compute_units();
  int64_t wgs = (a.n_items + 3) / 4;
  if (wgs > resident) wgs = resident;
  hipLaunchKernelGGL((kivi_group_kernel<HB, LB, HAD>), dim3((unsigned)wgs), dim3(256), 0, s, g, p, a);
  return hipGetLastError();
}

template <int HB, int LB>
hipError_t launch_kg_had(const Geom& g, const Planes& p, const KiviArgs& a, hipStream_t s) {
  if (g.hadamard && g.hsigned) return launch_kg<HB, LB, 2>(g, p, a, s);
  if (g.hadamard) return launch_kg<HB, LB, 1>(g, p, a, s);
  return launch_kg<HB, LB, 0>(g, p, a, s);
}

}  // namespace

bool kivi_groups_supported(const Geom& g, int64_t n_new) {
  // one bit width, or an INT4 window over an INT3 or INT2 tier
  const bool bits_ok = (g.hi_bits == g.lo_bits && g.hi_bits >= 2 && g.hi_bits <= 4) ||
                       (g.hi_bits == 4 && (g.lo_bits == 3 || g.lo_bits == 2));
  // row offsets from a pair's first new row must fit 32 bits
  const bool offs_ok = n_new * (int64_t)g.Hkv * kD * 2 < ((int64_t)1 << 32);
  return bits_ok && offs_ok;
}

hipError_t launch_kivi_groups(const Geom& g, const Planes& p, const __half* k_new, const __half* v_new,
                              int64_t n_new, int64_t T0, int64_t g0, int64_t g1, int64_t hi_start_new,
                              hipStream_t s) {
  if (g1 <= g0) return hipSuccess;
  KiviArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.n_new = n_new;
  a.T0 = T0;
  a.g0 = g0;
  a.n_grp = g1 - g0;
  a.hi_start = hi_start_new;
  a.n_items = (int64_t)g.B * g.Hkv * a.n_grp * 2;
  if (g.hi_bits == 4 && g.lo_bits == 4) return launch_kg_had<4, 4>(g, p, a, s);
  if (g.hi_bits == 4 && g.lo_bits == 3) return launch_kg_had<4, 3>(g, p, a, s);
  if (g.hi_bits == 4) return launch_kg_had<4, 2>(g, p, a, s);
  if (g.hi_bits == 3) return launch_kg_had<3, 3>(g, p, a, s);
  return launch_kg_had<2, 2>(g, p, a, s);
}

}  // namespace kvq
