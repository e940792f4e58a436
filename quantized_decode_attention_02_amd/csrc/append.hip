// Quantize-on-append kernels.
//
// Sources cited here:
//   [troisinh] "KV Cache Quantization — Nén cache INT4/INT3, mở khóa
//              ultra-long context" (troisinh.com).
//   [nalar]    "Kuantisasi KV Cache dengan Error Budget yang Eksplisit"
//              (nalar.dev).
//   [trefon]   "Matematyka cache KV: ile kosztuje długi kontekst i co daje
//              4-bitowy cache" (trefon.com).
//
// Everything that produces stored bytes is bit-exact with the documented
// float32 round-to-nearest-even arithmetic: one IEEE operation per step,
// correctly rounded division, rintf, RNE fp32->fp16.  No fused multiply-add
// contraction in this file (the only products are exact anyway).
#pragma clang fp contract(off)

#include "kvq_device.h"

namespace kvq {
namespace {

// ---------------------------------------------------------------------------
// Asymmetric group quantizer ([troisinh] "Tại sao nó hoạt động", item 1;
// [nalar] "Granularitas kuantisasi mengendalikan rentang yang harus dicakup
// setiap scale"): over a group x, Q = 2^bits - 1,
//   s = fl32(fl32(max - min) / Q), s_h = fp16(s) + 0, z_h = fp16(min) + 0,
//   c = clamp(rint(fl32(fl32(x - z_h) / s_h)), 0, Q), c = 0 when s_h == 0.
// The full [min, max] range is used (no clipping).
struct GroupParams {
  uint16_t s_bits, z_bits;
  float s, z;
  float rs;   // fl32(1 / s) (0 when s == 0)
};

// rint(fl32(d / s)) without a full IEEE division per element, for
// quotients a caller clamps to a code range.  q0 = fl32(d * rs) with
// rs = fl32(1 / s) is within 2^-23 |d / s| + 2^-24 |d / s| <= 2^-19
// (|q| <= 16) of d / s, and the correctly rounded quotient fl32(d / s) is
// within 2^-20 of it, so both round to the same integer unless q0 lies within
// 2^-18 of a half integer (`margin`; for |q| <= 128, 8-bit codes, the same
// argument gives 1.5 * 2^-16 and 2^-17, and the margin is 2^-14).  Such a
// quotient inside (lo, hi) -- the half integers that can move a clamped code
// lie there -- sets `risky`, and the caller redoes the group with the
// division; outside, q0 stands.
__device__ __forceinline__ float quot_fast(float d, float rs, float lo, float hi, bool& risky,
                                           float margin = 0x1p-18f) {
  const float q0 = d * rs;
  const float r = rintf(q0);
  risky |= (q0 > lo) & (q0 < hi) & (fabsf(q0 - r) >= 0.5f - margin);
  return r;
}

__device__ __forceinline__ GroupParams group_params(float mn, float mx, int bits) {
  const float Q = (float)((1 << bits) - 1);
  GroupParams gp;
  gp.s_bits = canonical_half_bits((mx - mn) / Q);
  gp.z_bits = canonical_half_bits(mn);
  gp.s = half_bits_to_float(gp.s_bits);
  gp.z = half_bits_to_float(gp.z_bits);
  gp.rs = gp.s == 0.0f ? 0.0f : 1.0f / gp.s;
  return gp;
}

// Code of x: clamp(rint(fl32(fl32(x - z) / s)), 0, Q), 0 when s == 0, by the
// reciprocal unless EXACT (see quot_fast; `risky` reports a quotient that
// needs the division).
// Branch-free: with s == 0, rs is 0 and the fast path gives 0; the exact
// path's quotient (inf or NaN) is discarded by the select.
template <bool EXACT>
__device__ __forceinline__ uint8_t quantize_code(float x, const GroupParams& gp, int bits, bool& risky) {
  const float Q = (float)((1 << bits) - 1);
  const float d = x - gp.z;
  float r;
  if (EXACT) {
    const float e = rintf(d / gp.s);
    r = gp.s == 0.0f ? 0.0f : e;
  } else {
    r = quot_fast(d, gp.rs, 0.25f, Q - 0.25f, risky);
  }
  return (uint8_t)fminf(fmaxf(r, 0.0f), Q);
}

// One 32-token group in LDS: xk[32][128], xv[32][128] float (the values the
// quantizer sees: fp16 inputs, or their rotation) -> codes ck, cv and the
// metadata records (key: (s, z) per channel; value: (s, z) per token and
// 32-dim slice, token-major).
// Keys use one range per channel over the 32 tokens, values one range per
// token over each 32-dim slice ([trefon] "Dlaczego cache trudniej
// skwantyzować niż wagi").  Needs 256 threads.
__device__ void quantize_group(const float (*xk)[kD], const float (*xv)[kD], uint8_t (*ck)[kD],
                               uint8_t (*cv)[kD], uint16_t* kmeta, uint16_t* vmeta, int bits,
                               int tid) {
  // each thread reads its 32 elements from LDS once, into registers
  float x[kGroup];
  if (tid < kD) {
    const int c = tid;
#pragma unroll
    for (int t = 0; t < kGroup; ++t) x[t] = xk[t][c];
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int t = 1; t < kGroup; ++t) {
      mn = fminf(mn, x[t]);
      mx = fmaxf(mx, x[t]);
    }
    const GroupParams gp = group_params(mn, mx, bits);
    bool risky = false;
#pragma unroll
    for (int t = 0; t < kGroup; ++t) ck[t][c] = quantize_code<false>(x[t], gp, bits, risky);
    if (risky)
      for (int t = 0; t < kGroup; ++t) ck[t][c] = quantize_code<true>(x[t], gp, bits, risky);
    kmeta[2 * c] = gp.s_bits;
    kmeta[2 * c + 1] = gp.z_bits;
  } else {
    // lane t of a wave walks its slice starting at element t: the 32 lanes
    // of one slice index hit 32 different LDS banks (min and max do not
    // depend on the order, and each code depends on its element only)
    const int u = tid - kD;
    const int t = u & 31, dg = u >> 5;
    const float* row = xv[t] + dg * 32;
    // x[i] = element (i + t) mod 32 of the slice: the 32 lanes of one slice
    // index hit 32 different LDS banks on every read
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = row[(i + t) & 31];
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) {
      mn = fminf(mn, x[i]);
      mx = fmaxf(mx, x[i]);
    }
    const GroupParams gp = group_params(mn, mx, bits);
    bool risky = false;
#pragma unroll
    for (int i = 0; i < 32; ++i) cv[t][dg * 32 + ((i + t) & 31)] = quantize_code<false>(x[i], gp, bits, risky);
    if (risky)
      for (int i = 0; i < 32; ++i) cv[t][dg * 32 + ((i + t) & 31)] = quantize_code<true>(x[i], gp, bits, risky);
    vmeta[2 * (t * 4 + dg)] = gp.s_bits;
    vmeta[2 * (t * 4 + dg) + 1] = gp.z_bits;
  }
}

// Byte cb of a 3-bit row of n codes: bits 8 cb .. 8 cb + 7 of the row read as
// one little-endian bit string, code i at bits 3i .. 3i + 2.
template <class Code>
__device__ __forceinline__ uint8_t row3_byte(Code code, int cb, int n) {
  const int i0 = (8 * cb) / 3, sh = 8 * cb - 3 * i0;
  uint32_t w = 0;
  for (int k = 0; k < 4; ++k)
    if (i0 + k < n) w |= (uint32_t)code(i0 + k) << (3 * k);
  return (uint8_t)(w >> sh);
}

// Pack codes into the tile byte images (canonical nibble/crumb order: element
// 2k in the low nibble of byte k; element 4k+j in bits 2j..2j+1; at 3 bits a
// row is one bit string, row3_byte).
//   key tile:   token-major rows, byte cb of token t at ktile_offset(t, cb)
//   value tile: channel-major rows of 32 tokens, row d at d * (4 * bits)
// Each of the 256 threads builds 2 * bits consecutive bytes of the tile image
// in registers (the loops unroll with constant indices) and stores them.
template <int BITS>
__device__ __forceinline__ void store_packed(uint8_t* dst, int o0, const uint32_t* w) {
  if (BITS == 4) {
    *reinterpret_cast<uint2*>(dst + o0) = make_uint2(w[0], w[1]);
  } else if (BITS == 2) {
    *reinterpret_cast<uint32_t*>(dst + o0) = w[0];
  } else {   // six bytes at an even offset: three 16-bit stores
    uint16_t* d16 = reinterpret_cast<uint16_t*>(dst + o0);
    d16[0] = (uint16_t)w[0];
    d16[1] = (uint16_t)(w[0] >> 16);
    d16[2] = (uint16_t)w[1];
  }
}

template <int BITS>
__device__ __forceinline__ void pack_key_tile_t(const uint8_t (*ck)[kD], uint8_t* dst, int tid) {
  constexpr int PT = 2 * BITS;   // 2048, 1536 or 1024 bytes over 256 threads
  const int o0 = tid * PT;
  uint32_t w[2] = {0, 0};
#pragma unroll
  for (int k = 0; k < PT; ++k) {
    const int o = o0 + k;
    const int t = (o & 511) >> 4;
    const int cb = (o >> 9) * 16 + (o & 15);
    uint32_t v = 0;
    if (BITS == 4) {
      v = ck[t][2 * cb] | (ck[t][2 * cb + 1] << 4);
    } else if (BITS == 2) {
      for (int j = 0; j < 4; ++j) v |= (uint32_t)ck[t][4 * cb + j] << (2 * j);
    } else {
      v = row3_byte([&](int i) { return ck[t][i]; }, cb, kD);
    }
    w[k >> 2] |= v << (8 * (k & 3));
  }
  store_packed<BITS>(dst, o0, w);
}

template <int BITS>
__device__ __forceinline__ void pack_value_tile_t(const uint8_t (*cv)[kD], uint8_t* dst, int tid) {
  constexpr int PT = 2 * BITS;
  constexpr int RB = 4 * BITS;   // bytes per channel row
  const int o0 = tid * PT;
  uint32_t w[2] = {0, 0};
#pragma unroll
  for (int k = 0; k < PT; ++k) {
    const int o = o0 + k;
    const int d = o / RB, kb = o % RB;
    uint32_t v = 0;
    if (BITS == 4) {
      v = cv[2 * kb][d] | (cv[2 * kb + 1][d] << 4);
    } else if (BITS == 2) {
      for (int j = 0; j < 4; ++j) v |= (uint32_t)cv[4 * kb + j][d] << (2 * j);
    } else {
      v = row3_byte([&](int i) { return cv[i][d]; }, kb, kGroup);
    }
    w[k >> 2] |= v << (8 * (k & 3));
  }
  store_packed<BITS>(dst, o0, w);
}

__device__ void pack_key_tile(const uint8_t (*ck)[kD], uint8_t* dst, int bits, int tid) {
  if (bits == 4) pack_key_tile_t<4>(ck, dst, tid);
  else if (bits == 3) pack_key_tile_t<3>(ck, dst, tid);
  else pack_key_tile_t<2>(ck, dst, tid);
}

__device__ void pack_value_tile(const uint8_t (*cv)[kD], uint8_t* dst, int bits, int tid) {
  if (bits == 4) pack_value_tile_t<4>(cv, dst, tid);
  else if (bits == 3) pack_value_tile_t<3>(cv, dst, tid);
  else pack_value_tile_t<2>(cv, dst, tid);
}

__device__ __forceinline__ uint8_t* hi_tile(const Geom& g, const Planes& p, int plane,
                                            int64_t pair, int64_t grp, int bits) {
  return p.p[plane] + (pair * g.hi_slots + grp % g.hi_slots) * tile_bytes(bits);
}
__device__ __forceinline__ uint8_t* lo_tile(const Geom& g, const Planes& p, int plane,
                                            int64_t pair, int64_t grp, int bits) {
  return p.p[plane] + (pair * g.gmax + grp) * tile_bytes(bits);
}

__device__ void store_group(const Geom& g, const Planes& p, int64_t pair, int64_t grp, int bits,
                            bool hi, const uint8_t (*ck)[kD], const uint8_t (*cv)[kD],
                            const uint16_t* kmeta, const uint16_t* vmeta, int tid) {
  uint8_t* kt = hi ? hi_tile(g, p, KVQ_PLANE_K_HI, pair, grp, bits)
                   : lo_tile(g, p, KVQ_PLANE_K_LO, pair, grp, bits);
  uint8_t* vt = hi ? hi_tile(g, p, KVQ_PLANE_V_HI, pair, grp, bits)
                   : lo_tile(g, p, KVQ_PLANE_V_LO, pair, grp, bits);
  pack_key_tile(ck, kt, bits, tid);
  pack_value_tile(cv, vt, bits, tid);
  uint16_t* km = reinterpret_cast<uint16_t*>(p.p[KVQ_PLANE_K_META] + (pair * g.gmax + grp) * 512);
  uint16_t* vm = reinterpret_cast<uint16_t*>(p.p[KVQ_PLANE_V_META] + (pair * g.gmax + grp) * 512);
  km[tid] = kmeta[tid];
  vm[tid] = vmeta[tid];
}

// ---------------------------------------------------------------------------
// KIVI group sources.
//
// load_group: the fp16 keys and values of group grp of (b, h) as floats in
// xk / xv.  A token before T0 is read from the fp16 window rings (keys: row
// t mod 160, token-major; values: slot t mod 160 of each channel row), a
// token from T0 on from the new input.  A group never wraps around the ring
// (160 = 5 * 32), so a group that lies wholly before T0 is 32 consecutive
// ring rows and 128 runs of 32 consecutive value slots: those are read as
// 16-byte vectors.
__device__ void load_group(const Geom& g, const Planes& p, float (*xk)[kD], float (*xv)[kD],
                           const __half* k_new, const __half* v_new, int64_t n_new, int64_t T0,
                           int b, int h, int64_t grp, int tid) {
  const int64_t pair = pair_index(g, b, h);
  const __half* kring = reinterpret_cast<const __half*>(p.p[KVQ_PLANE_K_WIN]) + pair * kRing * kD;
  const __half* vring = reinterpret_cast<const __half*>(p.p[KVQ_PLANE_V_WIN]) + pair * kD * kRing;
  if ((grp + 1) * kGroup <= T0) {
    const int slot0 = (int)(grp % 5) * kGroup;
    for (int e = tid; e < kGroup * 16; e += 256) {
      const int tok = e >> 4, c8 = e & 15;
      const uint4 raw = *reinterpret_cast<const uint4*>(kring + (slot0 + tok) * kD + 8 * c8);
      const __half* hv = reinterpret_cast<const __half*>(&raw);
      for (int i = 0; i < 8; ++i) xk[tok][8 * c8 + i] = __half2float(hv[i]);
    }
    for (int e = tid; e < kD * 4; e += 256) {
      const int d = e & 127, c4 = e >> 7;
      const uint4 raw = *reinterpret_cast<const uint4*>(vring + d * kRing + slot0 + 8 * c4);
      const __half* hv = reinterpret_cast<const __half*>(&raw);
      for (int i = 0; i < 8; ++i) xv[8 * c4 + i][d] = __half2float(hv[i]);
    }
    return;
  }
  for (int e = tid; e < kGroup * 16; e += 256) {
    const int tok = e >> 4, c8 = e & 15;
    const int64_t t = grp * kGroup + tok;
    const __half* src = t < T0 ? kring + (t % kRing) * kD
                               : k_new + (((int64_t)b * n_new + (t - T0)) * g.Hkv + h) * kD;
    const uint4 raw = *reinterpret_cast<const uint4*>(src + 8 * c8);
    const __half* hv = reinterpret_cast<const __half*>(&raw);
    for (int i = 0; i < 8; ++i) xk[tok][8 * c8 + i] = __half2float(hv[i]);
  }
  if (grp * kGroup >= T0) {
    // wholly new: token-major rows like the keys, 16-byte pieces
    for (int e = tid; e < kGroup * 16; e += 256) {
      const int tok = e >> 4, c8 = e & 15;
      const int64_t t = grp * kGroup + tok;
      const uint4 raw =
          *reinterpret_cast<const uint4*>(v_new + (((int64_t)b * n_new + (t - T0)) * g.Hkv + h) * kD + 8 * c8);
      const __half* hv = reinterpret_cast<const __half*>(&raw);
      for (int i = 0; i < 8; ++i) xv[tok][8 * c8 + i] = __half2float(hv[i]);
    }
    return;
  }
  for (int e = tid; e < kGroup * kD; e += 256) {
    const int tok = e >> 7, d = e & 127;
    const int64_t t = grp * kGroup + tok;
    const __half v = t < T0 ? vring[d * kRing + t % kRing]
                            : v_new[(((int64_t)b * n_new + (t - T0)) * g.Hkv + h) * kD + d];
    xv[tok][d] = __half2float(v);
  }
}

// load_demoted: group grp leaves the high-bit tier; its fp16 source is gone,
// so the values it is requantized from are its dequantized high-bit values
// x = fl32(c * s_h + z_h) (the product is exact).
__device__ void load_demoted(const Geom& g, const Planes& p, float (*xk)[kD], float (*xv)[kD],
                             int64_t pair, int64_t grp, int tid) {
  const int hb = g.hi_bits;
  const uint8_t* kt = hi_tile(g, p, KVQ_PLANE_K_HI, pair, grp, hb);
  const uint8_t* vt = hi_tile(g, p, KVQ_PLANE_V_HI, pair, grp, hb);
  const uint16_t* km =
      reinterpret_cast<const uint16_t*>(p.p[KVQ_PLANE_K_META] + (pair * g.gmax + grp) * 512);
  const uint16_t* vm =
      reinterpret_cast<const uint16_t*>(p.p[KVQ_PLANE_V_META] + (pair * g.gmax + grp) * 512);
  const int per = 8 / hb, mask = (1 << hb) - 1;
  for (int e = tid; e < kGroup * kD; e += 256) {
    const int t = e >> 7, d = e & 127;
    const int kcode = (kt[ktile_offset(t, d / per)] >> (hb * (d % per))) & mask;
    const int vcode = (vt[d * 4 * hb + t / per] >> (hb * (t % per))) & mask;
    const float ks = half_bits_to_float(km[2 * d]), kz = half_bits_to_float(km[2 * d + 1]);
    const int dg = d >> 5;
    const float vs = half_bits_to_float(vm[2 * (t * 4 + dg)]);
    const float vz = half_bits_to_float(vm[2 * (t * 4 + dg) + 1]);
    xk[t][d] = (float)kcode * ks + kz;
    xv[t][d] = (float)vcode * vs + vz;
  }
}

// LDS of one group in flight.
struct GroupLds {
  float xs[2][kGroup][kD];
  uint8_t cs[2][kGroup][kD];
  uint16_t meta[2][256];
};

// Quantize the group held in gl.xs (already rotated if it is to be) at
// `bits` and store it in its tier.  Synchronizes before returning, so gl can
// be reloaded right after.
__device__ void quantize_store(const Geom& g, const Planes& p, GroupLds& gl, int64_t pair,
                               int64_t grp, int bits, bool hi, int tid) {
  quantize_group(gl.xs[0], gl.xs[1], gl.cs[0], gl.cs[1], gl.meta[0], gl.meta[1], bits, tid);
  lds_barrier();
  store_group(g, p, pair, grp, bits, hi, gl.cs[0], gl.cs[1], gl.meta[0], gl.meta[1], tid);
  // LDS only: the group's global stores need not land before gl is reused
  lds_barrier();
}

// KIVI: quantize the groups [g0, g1) of every (sequence, kv head), one
// work-group per group.  A group goes to the high-bit tier if it starts at or
// after hi_start_new, else straight to the low-bit tier.
__global__ __launch_bounds__(256) void kivi_quantize_kernel(Geom g, Planes p, const __half* k_new,
                                                            const __half* v_new, int64_t n_new,
                                                            int64_t T0, int64_t g0,
                                                            int64_t hi_start_new) {
  __shared__ GroupLds gl;
  const int tid = threadIdx.x;
  const int64_t grp = g0 + blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  load_group(g, p, gl.xs[0], gl.xs[1], k_new, v_new, n_new, T0, b, h, grp, tid);
  __syncthreads();
  if (g.hadamard) fwht128_rows(&gl.xs[0][0][0], 2 * kGroup, tid, 256, g.sign_in, g.sign_out, g.hsigned);
  const bool hi = grp * kGroup >= hi_start_new;
  quantize_store(g, p, gl, pair_index(g, b, h), grp, hi ? g.hi_bits : g.lo_bits, hi, tid);
}

// KIVI: groups [g0, g1) leave the high-bit tier and are requantized at
// low_bits.  Must run before new groups reuse their ring slots.
__global__ __launch_bounds__(256) void kivi_demote_kernel(Geom g, Planes p, int64_t g0) {
  __shared__ GroupLds gl;
  const int tid = threadIdx.x;
  const int64_t grp = g0 + blockIdx.x;
  const int64_t pair = pair_index(g, blockIdx.z, blockIdx.y);
  load_demoted(g, p, gl.xs[0], gl.xs[1], pair, grp, tid);
  __syncthreads();
  quantize_store(g, p, gl, pair, grp, g.lo_bits, false, tid);
}

// KIVI appends of at most kSmallAppendMax tokens (decode steps): one work-group
// per (sequence, kv head) does the whole append of its pair in order: demote
// the groups [d0, d1) leaving the high-bit tier, quantize the groups [q0, q1)
// leaving the fp16 window at their tier, copy the new tokens [T0, T0 + n_new)
// into the rings.  With fewer than 128 new tokens, a group leaving the window
// lies wholly in the ring; a new token may overwrite the ring slot of a token
// of such a group, which is why the copies come last, after a barrier that
// follows every group load.  The new tokens are read into registers first so
// their latency overlaps the group work.
__global__ __launch_bounds__(256) void kivi_small_append_kernel(Geom g, Planes p,
                                                                const __half* k_new,
                                                                const __half* v_new, int64_t n_new,
                                                                int64_t T0, int64_t d0, int64_t d1,
                                                                int64_t q0, int64_t q1,
                                                                int64_t hi_start_new) {
  __shared__ GroupLds gl;
  const int tid = threadIdx.x;
  const int h = blockIdx.x, b = blockIdx.y;
  const int64_t pair = pair_index(g, b, h);
  // 16-byte pieces per tensor: at most 512, two per thread.  Two named
  // registers each, not an indexed array, which the compiler could move to LDS.
  const int items = (int)n_new * 16;
  const int e0 = tid, e1 = tid + 256;
  auto piece = [&](int e) { return (((int64_t)b * n_new + (e >> 4)) * g.Hkv + h) * kD + 8 * (e & 15); };
  uint4 k0 = {}, v0 = {}, k1 = {}, v1 = {};
  if (e0 < items) {
    k0 = *reinterpret_cast<const uint4*>(k_new + piece(e0));
    v0 = *reinterpret_cast<const uint4*>(v_new + piece(e0));
  }
  if (e1 < items) {
    k1 = *reinterpret_cast<const uint4*>(k_new + piece(e1));
    v1 = *reinterpret_cast<const uint4*>(v_new + piece(e1));
  }
  // demotions first, then the groups leaving the window: one quantize_store
  // for both (the group quantizer is large; a single copy of it keeps the
  // kernel's code small)
  const int64_t nd = d1 - d0, nq = q1 - q0;
  for (int64_t i = 0; i < nd + nq; ++i) {
    const bool demote = i < nd;
    const int64_t grp = demote ? d0 + i : q0 + (i - nd);
    if (demote) {
      load_demoted(g, p, gl.xs[0], gl.xs[1], pair, grp, tid);
    } else {
      load_group(g, p, gl.xs[0], gl.xs[1], k_new, v_new, n_new, T0, b, h, grp, tid);
    }
    __syncthreads();
    if (!demote && g.hadamard)
      fwht128_rows(&gl.xs[0][0][0], 2 * kGroup, tid, 256, g.sign_in, g.sign_out, g.hsigned);
    const bool hi = !demote && grp * kGroup >= hi_start_new;
    quantize_store(g, p, gl, pair, grp, hi ? g.hi_bits : g.lo_bits, hi, tid);
  }
  __half* kring = reinterpret_cast<__half*>(p.p[KVQ_PLANE_K_WIN]) + pair * kRing * kD;
  __half* vring = reinterpret_cast<__half*>(p.p[KVQ_PLANE_V_WIN]) + pair * kD * kRing;
  auto put = [&](int e, const uint4& kv, const uint4& vv) {
    const int c8 = e & 15;
    const int slot = (int)((T0 + (e >> 4)) % kRing);
    *reinterpret_cast<uint4*>(kring + slot * kD + 8 * c8) = kv;
    const __half* hv = reinterpret_cast<const __half*>(&vv);
    for (int i = 0; i < 8; ++i) vring[(8 * c8 + i) * kRing + slot] = hv[i];
  };
  if (e0 < items) put(e0, k0, v0);
  if (e1 < items) put(e1, k1, v1);
}

// KIVI: copy new tokens [w0, w1) (absolute positions, all >= T0) into the fp16
// window rings: keys to row t mod 160 (one thread per 16-byte chunk), values
// to slot t mod 160 of each channel row (one thread per 8 channels).
__global__ __launch_bounds__(256) void window_write_kernel(Geom g, Planes p, const __half* k_new,
                                                           const __half* v_new, int64_t n_new,
                                                           int64_t T0, int64_t w0, int64_t nw) {
  const int64_t items = (int64_t)g.B * nw * g.Hkv * 16;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < 2 * items;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int tensor = i >= items;
    int64_t r = tensor ? i - items : i;
    const int c8 = r % 16;
    r /= 16;
    const int h = r % g.Hkv;
    r /= g.Hkv;
    const int64_t t = w0 + r % nw;
    const int b = (int)(r / nw);
    const __half* src = (tensor ? v_new : k_new) + (((int64_t)b * n_new + (t - T0)) * g.Hkv + h) * kD;
    const int64_t pair = pair_index(g, b, h);
    const uint4 raw = *reinterpret_cast<const uint4*>(src + 8 * c8);
    if (tensor == 0) {
      __half* dst = reinterpret_cast<__half*>(p.p[KVQ_PLANE_K_WIN]) + (pair * kRing + t % kRing) * kD;
      *reinterpret_cast<uint4*>(dst + 8 * c8) = raw;
    } else {
      __half* dst = reinterpret_cast<__half*>(p.p[KVQ_PLANE_V_WIN]) + pair * kD * kRing + t % kRing;
      const __half* hv = reinterpret_cast<const __half*>(&raw);
      for (int k = 0; k < 8; ++k) dst[(8 * c8 + k) * kRing] = hv[k];
    }
  }
}

// ---------------------------------------------------------------------------
// Split-half RoPE table for pre-RoPE keys ([troisinh] "Tại sao nó hoạt
// động", item 3): row t holds (cos, sin) of t * theta_j, theta_j =
// base^(-2j/128), computed in fp64 and rounded to fp32.
__global__ __launch_bounds__(256) void rope_table_kernel(Geom g, Planes p, int64_t t0, int64_t n) {
  float* tab = reinterpret_cast<float*>(p.p[KVQ_PLANE_ROPE]);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n * 64;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = t0 + i / 64;
    const int j = (int)(i % 64);
    const double theta = pow((double)g.rope_theta, -2.0 * (double)j / 128.0);
    const double ang = (double)t * theta;
    tab[t * 128 + 2 * j] = (float)cos(ang);
    tab[t * 128 + 2 * j + 1] = (float)sin(ang);
  }
}

int grid_for(int64_t items) {
  int64_t blocks = (items + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  return (int)(blocks < 1 ? 1 : blocks);
}

}  // namespace

hipError_t launch_rope_table(const Geom& g, const Planes& p, int64_t t0, int64_t t1, hipStream_t s) {
  if (t1 > t0) {
    hipLaunchKernelGGL(rope_table_kernel, dim3(grid_for((t1 - t0) * 64)), dim3(256), 0, s, g, p, t0,
                       t1 - t0);
  }
  return hipGetLastError();
}

hipError_t launch_kivi_demote(const Geom& g, const Planes& p, int64_t g0, int64_t g1, hipStream_t s) {
  if (g1 > g0) {
    hipLaunchKernelGGL(kivi_demote_kernel, dim3((unsigned)(g1 - g0), g.Hkv, g.B), dim3(256), 0, s, g, p,
                       g0);
  }
  return hipGetLastError();
}

hipError_t launch_kivi_quantize(const Geom& g, const Planes& p, const __half* k_new,
                                const __half* v_new, int64_t n_new, int64_t T0, int64_t g0,
                                int64_t g1, int64_t hi_start_new, hipStream_t s) {
  // groups wholly from the new tokens go to the group kernel of
  // append_kivi.hip where it covers the code widths; the others (a group
  // that starts in the fp16 window, 3-bit codes) come here
  int64_t gm = g0;
  if (kivi_groups_supported(g, n_new)) {
    gm = (T0 + kGroup - 1) / kGroup;
    gm = gm < g0 ? g0 : (gm > g1 ? g1 : gm);
    const hipError_t e = launch_kivi_groups(g, p, k_new, v_new, n_new, T0, gm, g1, hi_start_new, s);
    if (e != hipSuccess) return e;
  } else {
    gm = g1;
  }
  if (gm > g0) {
    hipLaunchKernelGGL(kivi_quantize_kernel, dim3((unsigned)(gm - g0), g.Hkv, g.B), dim3(256), 0, s, g,
                       p, k_new, v_new, n_new, T0, g0, hi_start_new);
  }
  return hipGetLastError();
}

hipError_t launch_kivi_small_append(const Geom& g, const Planes& p, const __half* k_new,
                                    const __half* v_new, int64_t n_new, int64_t T0, int64_t d0,
                                    int64_t d1, int64_t q0, int64_t q1, int64_t hi_start_new,
                                    hipStream_t s) {
  if (n_new < 1 || n_new > kSmallAppendMax) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kivi_small_append_kernel, dim3(g.Hkv, g.B), dim3(256), 0, s, g, p, k_new, v_new,
                     n_new, T0, d0, d1, q0, q1, hi_start_new);
  return hipGetLastError();
}

hipError_t launch_window_write(const Geom& g, const Planes& p, const __half* k_new,
                               const __half* v_new, int64_t n_new, int64_t T0, int64_t w0,
                               int64_t w1, hipStream_t s) {
  if (w1 > w0) {
    const int64_t items = 2 * (int64_t)g.B * (w1 - w0) * g.Hkv * 16;
    hipLaunchKernelGGL(window_write_kernel, dim3(grid_for(items)), dim3(256), 0, s, g, p, k_new, v_new,
                       n_new, T0, w0, w1 - w0);
  }
  return hipGetLastError();
}

}  // namespace kvq
