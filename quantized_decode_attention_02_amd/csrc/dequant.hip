// Dequantize a token range to fp32 in the stored domain: the
// dequantize-before-arithmetic path of [nalar] "Kuantisasi KV Cache dengan
// Error Budget yang Eksplisit", section "Biaya dequantization harus masuk ke
// model latency" — here only for tests and inspection; decode never uses it.
//   KIVI:     x = fl32(c * s_h + z_h)   (the product is exact, so fused or not
//                                        gives the same bits)
//   BLOCK128: y = fl32((n - 8) * s_h)  (exact; n - 4 at 3 bits)
//   TBQ4:     y = fl32(norm * level[n])
//   Q4_0:     y = fl32((n - 8) * s_h of the value's 32-value slice)  (exact)
//   Q8_0:     y = fl32((n - 128) * s_h of the value's 32-value slice)  (exact)
//   window:   the fp16 value.
#pragma clang fp contract(off)

#include "kvq_device.h"

namespace kvq {
namespace {

// 3-bit tiles: a row's codes are one little-endian bit string, code c at bits
// 3c .. 3c + 2, so a code may straddle two bytes.  Key rows are 48 bytes of
// the token-major key tile, value rows 12 bytes per channel.
__device__ __forceinline__ int key_code3(const uint8_t* kt, int row, int d) {
  const int kb = (3 * d) >> 3, sh = (3 * d) & 7;
  const uint32_t w = kt[ktile_offset(row, kb)] | (kb + 1 < 48 ? (uint32_t)kt[ktile_offset(row, kb + 1)] << 8 : 0u);
  return (int)((w >> sh) & 7u);
}
__device__ __forceinline__ int value_code3(const uint8_t* vt, int d, int t) {
  const int vb = (3 * t) >> 3, sh = (3 * t) & 7;
  const uint32_t w = vt[d * 12 + vb] | (vb + 1 < 12 ? (uint32_t)vt[d * 12 + vb + 1] << 8 : 0u);
  return (int)((w >> sh) & 7u);
}

__global__ __launch_bounds__(256) void dequant_kernel(Geom g, Planes p, int64_t t0, int64_t nt,
                                                      float* k_out, float* v_out) {
  const int64_t items = (int64_t)g.B * nt * g.Hkv * kD;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < items;
       i += (int64_t)gridDim.x * blockDim.x) {
    int64_t r = i;
    const int d = r % kD;
    r /= kD;
    const int h = r % g.Hkv;
    r /= g.Hkv;
    const int64_t t = t0 + r % nt;
    const int b = (int)(r / nt);
    const int64_t pair = pair_index(g, b, h);
    float kv, vv;
    if (block_scheme(g.scheme)) {
      const int64_t grp = t / kGroup;
      const int row = (int)(t % kGroup);
      const int bits = g.hi_bits;
      const uint8_t* kt = p.p[KVQ_PLANE_K_HI] + (pair * g.gmax + grp) * 512 * bits;
      const uint8_t* vt = p.p[KVQ_PLANE_V_HI] + (pair * g.gmax + grp) * 512 * bits;
      int kn, vn;
      if (bits == 3) {
        kn = key_code3(kt, row, d);
        vn = value_code3(vt, d, row);
      } else if (bits == 8) {   // one byte per code
        kn = kt[ktile_offset(row, d)];
        vn = vt[d * 32 + row];
      } else {
        kn = (kt[ktile_offset(row, d >> 1)] >> (4 * (d & 1))) & 15;
        vn = (vt[d * 16 + (row >> 1)] >> (4 * (row & 1))) & 15;
      }
      const int per = g.q40 ? 4 : 1;   // fp16 scales per token
      const uint16_t* ks = reinterpret_cast<const uint16_t*>(p.p[KVQ_PLANE_K_META]) + pair * g.gmax * kGroup * per;
      const uint16_t* vs = reinterpret_cast<const uint16_t*>(p.p[KVQ_PLANE_V_META]) + pair * g.gmax * kGroup * per;
      if (g.tbq4) {
        float kl = g.cb_level[0], vl = g.cb_level[0];
#pragma unroll
        for (int k = 1; k < 16; ++k) {
          kl = kn == k ? g.cb_level[k] : kl;
          vl = vn == k ? g.cb_level[k] : vl;
        }
        kv = half_bits_to_float(ks[t]) * kl;
        vv = half_bits_to_float(vs[t]) * vl;
      } else if (g.q40) {
        const int off = bits == 8 ? 128 : 8;
        kv = (float)(kn - off) * half_bits_to_float(ks[4 * t + (d >> 5)]);
        vv = (float)(vn - off) * half_bits_to_float(vs[4 * t + (d >> 5)]);
      } else {
        const int off = bits == 3 ? 4 : 8;
        kv = (float)(kn - off) * half_bits_to_float(ks[t]);
        vv = (float)(vn - off) * half_bits_to_float(vs[t]);
      }
    } else if (t < g.Tq) {
      const int64_t grp = t / kGroup;
      const int row = (int)(t % kGroup);
      int bits;
      const uint8_t* kt = tile_ptr(g, p, KVQ_PLANE_K_HI, KVQ_PLANE_K_LO, pair, grp, &bits);
      const uint8_t* vt = tile_ptr(g, p, KVQ_PLANE_V_HI, KVQ_PLANE_V_LO, pair, grp, &bits);
      int kc, vc;
      if (bits == 3) {
        kc = key_code3(kt, row, d);
        vc = value_code3(vt, d, row);
      } else {
        const int per = 8 / bits, mask = (1 << bits) - 1;
        kc = (kt[ktile_offset(row, d / per)] >> (bits * (d % per))) & mask;
        vc = (vt[d * 4 * bits + row / per] >> (bits * (row % per))) & mask;
      }
      const uint16_t* km = reinterpret_cast<const uint16_t*>(p.p[KVQ_PLANE_K_META] + (pair * g.gmax + grp) * 512);
      const uint16_t* vm = reinterpret_cast<const uint16_t*>(p.p[KVQ_PLANE_V_META] + (pair * g.gmax + grp) * 512);
      const int dg = d >> 5;
      kv = (float)kc * half_bits_to_float(km[2 * d]) + half_bits_to_float(km[2 * d + 1]);
      vv = (float)vc * half_bits_to_float(vm[2 * (row * 4 + dg)]) +
           half_bits_to_float(vm[2 * (row * 4 + dg) + 1]);
    } else {
      const __half* kr = reinterpret_cast<const __half*>(p.p[KVQ_PLANE_K_WIN]) + (pair * kRing + t % kRing) * kD;
      const __half* vr = reinterpret_cast<const __half*>(p.p[KVQ_PLANE_V_WIN]) + pair * kD * kRing;
      kv = __half2float(kr[d]);
      vv = __half2float(vr[d * kRing + t % kRing]);
    }
    k_out[i] = kv;
    v_out[i] = vv;
  }
}

}  // namespace

hipError_t launch_dequant(const Geom& g, const Planes& p, int64_t t0, int64_t t1, float* k_out,
                          float* v_out, hipStream_t s) {
  const int64_t items = (int64_t)g.B * (t1 - t0) * g.Hkv * kD;
  if (items > 0) {
    int64_t blocks = (items + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)blocks), dim3(256), 0, s, g, p, t0, t1 - t0, k_out,
                       v_out);
  }
  return hipGetLastError();
}

}  // namespace kvq
