// Quantize-on-append for the block formats: symmetric 128-value blocks at 4
// or 3 bits, TBQ4, Q4_0 and Q8_0, each optionally after the (randomized)
// normalized Hadamard rotation.
//
// Sources cited here:
//   [trefon] "Matematyka cache KV: ile kosztuje długi kontekst i co daje
//            4-bitowy cache" (trefon.com): "Przykład: model 27B przy 262K"
//            (the block formats and their sizes), "Jak 4-bitowemu cache to
//            uchodzi: najpierw obrót" (the rotation, TBQ4).
//
// Every stored byte is bit-exact with the float32 definitions: the FWHT in
// its fixed stage order h = 1, 2, ..., 64, one IEEE operation per step, then
// fl32(1/sqrt(128)) scaling; s_h = fp16(fl32(a / top)) with a the absmax of
// the (scaled) block; code = clamp(rint(fl32(y / s_h)), -top, top) + top + 1
// (0 when s_h == 0); TBQ4: n_h = fp16(min(fl32(sqrt(sum y^2) in fp64),
// 65504)), index = number of fp32 boundaries strictly below fl32(y / n_h).
//
// Layout of the work: a wave item is one tensor (keys or values) of one
// 32-token tile of one (sequence, kv head) pair; each wave takes a
// contiguous run of items, and lanes v and v + 32 own token v's vector,
// elements 0..63 and 64..127.  Every FWHT stage but the last stays inside
// the lane; the last trades half a register set between the two lanes with
// v_permlane32_swap, after which each lane holds whole (x_e, x_{e+64}) pairs
// (7.5 fp32 operations an element for the transform, the fp16 -> fp32
// conversion folded into stage h = 1 by v_fma_mix).  The vectors enter
// through LDS: the wave reads them with 16-byte loads, four tokens' rows a
// load, and writes them to its LDS area with the 16-byte chunks of row v
// rotated by v mod 16 (chunk c at slot c ^ (v & 15)), so that the
// lane-per-half-row reads hit 16 different bank quads.  The next item's
// loads are in flight while the current one is computed.  Value codes leave
// through the same area, transposed from token rows to the channel rows of
// the value tile.  No work-group barrier after the set-up: waves are
// independent.
//
// Codes come from one fma per end of a bracket: with crs = fl32(c / s_h)
// (c the scaling, or 1), fma(x, crs (1 -+ 2^-21), 2^23 + top + 1) rounds
// the bracket's ends to integers, code + offset in the low bits.  The
// exact quotient fl32(fl32(x c) / s_h) lies strictly inside the bracket
// (its distance from x crs is below 2^-22 relative), so where both ends
// round alike it rounds the same way; otherwise -- near a half integer,
// about one unit of eight codes in 2^14 -- the wave redoes those codes
// with the division.  A subnormal fp16 scale (the only case where a code
// can leave [-top, top] before the clamp) always takes the division.
#pragma clang fp contract(off)

#include "append_util.h"

namespace kvq {
namespace {

// TBQ4 index lookup: |u| is bucketed by its exponent and top two mantissa
// bits (buckets 25% wide or less) from 2^-8 up; bucket 0 is [0, 1.25 2^-8),
// the last everything from 2^-2.  Consecutive decision boundaries of the
// codebook are more than 25% apart above 0.02, so a bucket holds at most one
// (checked when the table is built).
constexpr int kTbqBuckets = 25;
constexpr int kTbqT0 = (127 - 8) << 2;   // (exponent, 2 mantissa bits) of 2^-8

template <int BITS>
struct Sym {
  static constexpr int kTop = BITS == 3 ? 3 : (BITS == 8 ? 127 : 7);
  static constexpr int kRowWords = 4 * BITS;        // dwords of a key row: 12, 16, 32
  static constexpr int kPer = BITS == 8 ? 4 : 8;    // codes per packed unit
  static constexpr int kUnits = kD / kPer;          // units: a dword (8 bits: 4 codes, 4 bits:
                                                    // 8 codes) or a 24-bit group (3 bits: 8 codes)
};

// Item coordinates (wave-uniform).
struct Item {
  int64_t pair, tb;    // tb: first token of the item's tile
  int b, h, tensor;    // tensor 0: keys, 1: values
};

__device__ __forceinline__ Item item_at(const Geom& g, int64_t it, int64_t tile0, int64_t n_tiles) {
  Item r;
  r.tensor = (int)(it & 1);
  const int64_t rest = it >> 1;
  r.pair = rest / n_tiles;
  r.b = (int)(r.pair / g.Hkv);
  r.h = (int)(r.pair % g.Hkv);
  r.tb = (tile0 + rest % n_tiles) * kGroup;
  return r;
}

template <int BITS, bool Q40, int HAD, bool TBQ>
__global__ __launch_bounds__(256, 2) void block_append_kernel(Geom g, Planes p, SegArgs a) {
  constexpr int kTop = Sym<BITS>::kTop;
  constexpr int kPer = Sym<BITS>::kPer;
  constexpr int kUnits = Sym<BITS>::kUnits;
  constexpr int kLU = kUnits / 2;            // units of one lane (half a vector)
  constexpr int64_t kTileBytes = 512 * BITS;
  // LDS of one wave: the tile's 32 fp16 vectors, later its value-code transpose
  constexpr int kWaveLds = (kGroup * kD * 2 > kUnits * kTr * 4) ? kGroup * kD * 2 : kUnits * kTr * 4;
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kWaveLds];
  __shared__ __attribute__((aligned(16))) uint32_t sgn_in[64];    // randomized rotation: fp16 pair
                                                                   // sign masks (bits 15, 31)
  __shared__ __attribute__((aligned(16))) uint32_t sgn_out[32];   // negation masks of packed codes
  __shared__ __attribute__((aligned(16))) uint32_t sgn_f[kD];     // TBQ4: fp32 output sign masks
  // TBQ4: per (sign, bucket) of u: (the boundary inside, or +inf; the number
  // of boundaries below the bucket); tbq_exact: the table cannot be used
  __shared__ __attribute__((aligned(8))) uint2 tbq_tab[2 * kTbqBuckets];
  __shared__ int tbq_exact;
  if (TBQ) {
    const int t = threadIdx.x;
    if (t == 0) tbq_exact = 0;
    __syncthreads();
    if (t < 2 * kTbqBuckets) {
      const int j = t % kTbqBuckets;
      const bool neg = t >= kTbqBuckets;
      // |u| in [lo, hi)
      const float lo = j == 0 ? 0.0f : ldexpf(1.0f + 0.25f * ((kTbqT0 + j) & 3), ((kTbqT0 + j) >> 2) - 127);
      const float hi = j == kTbqBuckets - 1 ? INFINITY
                                            : ldexpf(1.0f + 0.25f * ((kTbqT0 + j + 1) & 3), ((kTbqT0 + j + 1) >> 2) - 127);
      uint32_t below = 0, inside = 0;
      float bin = INFINITY;
      bool near_edge = false;
      for (int k = 0; k < 15; ++k) {
        const float b = g.cb_bound[k];
        // u in [lo, hi) (positive) or (-hi, -lo] (negative)
        const bool bel = neg ? b <= -hi : b < lo;
        const bool ins = neg ? (b > -hi && b <= -lo) : (b >= lo && b < hi);
        below += bel ? 1u : 0u;
        if (ins) {
          ++inside;
          bin = b;
        } else {
          // a boundary next to the bucket but outside it: the rounding of
          // u could cross it without the risk test (on this bucket's
          // boundary) seeing it.  Zero is no such edge: q and u have the
          // sign of y.
          if (j > 0) near_edge |= fabsf(fabsf(b) - lo) < 0x1p-20f;
          if (j < kTbqBuckets - 1) near_edge |= fabsf(fabsf(b) - hi) < 0x1p-20f;
        }
      }
      tbq_tab[t] = make_uint2(__float_as_uint(bin), below);
      if (inside > 1 || near_edge) tbq_exact = 1;
    }
    __syncthreads();
  }
  if (HAD == 2) {
    const int t = threadIdx.x;
    if (t < 64) {
      const uint32_t w = mask_word(g.sign_in, t >> 4);
      const int bit = (2 * t) & 31;
      sgn_in[t] = (((w >> bit) & 1u) << 15) | (((w >> (bit + 1)) & 1u) << 31);
    } else if (t < 64 + kUnits && !TBQ) {
      const int m = t - 64;
      uint32_t mk = 0;
      for (int j = 0; j < kPer; ++j) {
        const int c = kPer * m + j;
        if ((mask_word(g.sign_out, c >> 5) >> (c & 31)) & 1u) mk |= ((1u << BITS) - 1u) << (BITS * j);
      }
      sgn_out[m] = mk;
    } else if (t >= 128 && TBQ) {
      const int c = t - 128;
      sgn_f[c] = ((mask_word(g.sign_out, c >> 5) >> (c & 31)) & 1u) << 31;
    }
    __syncthreads();
  }

  // the wave index is uniform: a scalar register keeps the item walk and its
  // addresses on the scalar unit
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, v = lane & 31;   // vector v of the tile, elements 64 half ..
  // this wave's items: a contiguous run [i0, i1) of (pair, tile, tensor)
  // in that order, tensor fastest
  const int64_t nwaves = (int64_t)gridDim.x * 4, gw = (int64_t)blockIdx.x * 4 + wv;
  const int64_t i0 = gw * a.n_items / nwaves, i1 = (gw + 1) * a.n_items / nwaves;
  if (i0 >= i1) return;
  uint8_t* reg = lds + wv * kWaveLds;
  const int64_t T0 = a.T0, T1 = a.T0 + a.n;
  const uint32_t rowbytes = (uint32_t)g.Hkv * kD * 2;

  // 16-byte chunk (lane & 15) of the rows of tokens tb + 4 i + (lane >> 4);
  // rows outside the segment are replaced by the nearest row inside (never
  // used).  The row offset from the pair's first segment row fits 32 bits.
#define KVQ_ISSUE_ROWS(it)                                                                      \
  {                                                                                             \
    const uint8_t* base_ = reinterpret_cast<const uint8_t*>(                                    \
        ((it).tensor ? a.v_new : a.k_new) +                                                     \
        (((int64_t)(it).b * a.src_tokens + (T0 - a.src_t0)) * g.Hkv + (it).h) * kD);             \
    const int r0_ = (int)((it).tb - T0) + (lane >> 4);                                         \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                             \
      const int tr_ = min(max(r0_ + 4 * i, 0), (int)a.n - 1);                                   \
      raw[i] = *reinterpret_cast<const u32x4*>(base_ + ((uint32_t)tr_ * rowbytes +              \
                                                        16u * (uint32_t)(lane & 15)));          \
    }                                                                                           \
  }

  Item cur = item_at(g, i0, a.tile0, a.n_tiles);
  u32x4 raw[8];
  KVQ_ISSUE_ROWS(cur)
  for (int64_t item = i0;; ++item) {
    stage_rows(reg, raw, lane);
    // the next item's rows (past the last item: this item's again, from L2)
    Item nit = cur;
    if (item + 1 < i1) {
      nit.tensor ^= 1;
      if (nit.tensor == 0) {
        nit.tb += kGroup;
        if (nit.tb == (a.tile0 + a.n_tiles) * kGroup) {
          nit.tb = a.tile0 * kGroup;
          ++nit.pair;
          if (++nit.h == g.Hkv) {
            nit.h = 0;
            ++nit.b;
          }
        }
      }
    }
    KVQ_ISSUE_ROWS(nit)

    // ---- half a vector: elements 64 half + k in r[k], or half the
    // unnormalized transform (see read_half)
    float r[64];
    read_half<HAD>(reg, sgn_in, lane, r);
    auto chan = [&](int k) { return half_chan<HAD>(k, half); };

    // ---- codes (r holds the unscaled transform when rotated: y = fl32(r c))
    const int64_t t = cur.tb + v;
    const bool valid = t >= T0 && t < T1;
    uint32_t U[kLU];       // packed codes: lane unit u = r[kPer u .. kPer u + kPer - 1]
    uint32_t sbw = 0;      // this lane's fp16 scales (Q4_0 / Q8_0: its two slices)
    if (TBQ) {
      double ss = 0.0;
#pragma unroll
      for (int j = 0; j < 64; ++j) {
        float y = r[j] * c32();
        if (HAD == 2) y = __uint_as_float(__float_as_uint(y) ^ sgn_f[chan(j)]);
        r[j] = y;
        ss = fma((double)y, (double)y, ss);
      }
      const uint64_t sbits = (uint64_t)__double_as_longlong(ss);
      const uint32_t olo = other_half((uint32_t)sbits, half), ohi = other_half((uint32_t)(sbits >> 32), half);
      ss = ss + __longlong_as_double((long long)(((uint64_t)ohi << 32) | olo));
      const uint16_t nb = float_to_half_bits(fminf((float)sqrt(ss), 65504.0f));
      sbw = nb;
      const float nrm = half_bits_to_float(nb);
      const float rn = nrm != 0.0f ? 1.0f / nrm : 0.0f;
      const bool exact_all = tbq_exact != 0;
#pragma unroll
      for (int u = 0; u < kLU; ++u) {
        uint32_t f[8];
        float near = INFINITY;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          // q = fl32(y fl32(1/n)) is within 3 2^-24 |u| < 2^-22 of
          // u = fl32(y / n) (|u| <= 1.01); both count the same boundaries
          // below them unless one lies within 2^-22 of q: that can only be
          // the boundary of q's bucket (none lies that close to a bucket edge)
          const float q = r[8 * u + j] * rn;
          const uint32_t qb = __float_as_uint(q);
          const int bk = min(max((int)((qb >> 21) & 0x3FFu) - kTbqT0, 0), kTbqBuckets - 1);
          const uint2 e = tbq_tab[bk + kTbqBuckets * (int)(qb >> 31)];
          const float bin = __uint_as_float(e.x);
          f[j] = e.y + (q > bin ? 1u : 0u);
          near = fminf(near, fabsf(q - bin));
        }
        if (__builtin_expect(__any(near < 0x1p-22f || exact_all), 0)) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float uq = nrm != 0.0f ? r[8 * u + j] / nrm : 0.0f;
            uint32_t idx = 0;
#pragma unroll
            for (int k = 0; k < 15; ++k) idx += uq > g.cb_bound[k] ? 1u : 0u;
            f[j] = idx;
          }
        }
        U[u] = pack8<4>(f);
      }
    } else {
      // per slice: a, s_h, 1/s_h folded with the scaling, and a bracket
      // clo <= c / s_h <= chi around it (relative 2^-21 each way)
      constexpr int kLS = Q40 ? 2 : 1;   // slices of this lane: r[0..31], r[32..63]
      float s[kLS], clo[kLS], chi[kLS];
      bool exact_lane = false;
#pragma unroll
      for (int sl = 0; sl < kLS; ++sl) {
        float am = 0.0f;
#pragma unroll
        for (int j = 0; j < 64 / kLS; ++j) am = fmaxf(am, fabsf(r[sl * (64 / kLS) + j]));
        if (!Q40) am = fmaxf(am, __uint_as_float(other_half(__float_as_uint(am), half)));
        const float a = HAD ? am * c32() : am;
        const uint16_t sb = float_to_half_bits(a / (float)kTop);
        sbw |= (uint32_t)sb << (16 * sl);
        s[sl] = half_bits_to_float(sb);
        // v_rcp_f32 is within 1 ulp of 1 / s_h; with the scaling's rounding
        // the ends below still bracket c / s_h
        const float rs = s[sl] != 0.0f ? __builtin_amdgcn_rcpf(s[sl]) : 0.0f;
        const float crs = HAD ? rs * c32() : rs;
        clo[sl] = crs * (1.0f - 0x1p-21f);
        chi[sl] = crs * (1.0f + 0x1p-21f);
        // a subnormal fp16 scale can push quotients past the code range
        exact_lane |= s[sl] != 0.0f && s[sl] < 0x1p-14f;
      }
      const float magic = kTwo23 + (float)(kTop + 1);
#pragma unroll
      for (int u = 0; u < kLU; ++u) {
        const int sl = Q40 ? (kPer * u) / 32 : 0;
        uint32_t f[8];
        uint32_t diff = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const float xv = r[kPer * u + j];
          const uint32_t lo = __float_as_uint(fmaf(xv, clo[sl], magic));
          const uint32_t hi = __float_as_uint(fmaf(xv, chi[sl], magic));
          diff = xor_add(lo, hi, diff);
          f[j] = lo;
        }
        // the bracket's ends round alike, so does the exact quotient in
        // between; otherwise (rare) the wave redoes the unit by division
        if (__builtin_expect(__any(diff != 0u || exact_lane), 0)) {
#pragma unroll
          for (int j = 0; j < kPer; ++j) {
            const float y = HAD ? r[kPer * u + j] * c32() : r[kPer * u + j];
            const float q = s[sl] != 0.0f ? rintf(y / s[sl]) : 0.0f;
            const int c = (int)fminf(fmaxf(q, (float)-kTop), (float)kTop);
            f[j] = (uint32_t)(c + kTop + 1);
          }
        }
        uint32_t packed = BITS == 8 ? pack4x8(f) : pack8<BITS>(f);
        if (HAD == 2) {   // negated coordinates: code 2 (top + 1) - code, fieldwise
          const uint32_t mk = sgn_out[chan(kPer * u) / kPer];
          const uint32_t ones = BITS == 8 ? 0x01010101u : (BITS == 4 ? 0x11111111u : 0x249249u);
          packed = (packed ^ mk) + (mk & ones);
        }
        U[u] = packed;
      }
    }

    // ---- store: scales, then key rows or value tiles
    const int64_t tile = cur.tb / kGroup;
    if (Q40) {   // four slices, two in each half
      const uint32_t o = other_half(sbw, half);
      if (valid && half == 0) {   // transformed: slices 0, 2 here, 1, 3 there; plain: 0, 1 | 2, 3
        uint16_t* sp = reinterpret_cast<uint16_t*>(p.p[cur.tensor ? KVQ_PLANE_V_META : KVQ_PLANE_K_META]);
        *reinterpret_cast<uint2*>(sp + (cur.pair * g.gmax * kGroup + t) * 4) =
            HAD ? make_uint2((sbw & 0xFFFFu) | (o << 16), (sbw >> 16) | (o & 0xFFFF0000u)) : make_uint2(sbw, o);
      }
    } else if (valid && half == 0) {
      uint16_t* sp = reinterpret_cast<uint16_t*>(p.p[cur.tensor ? KVQ_PLANE_V_META : KVQ_PLANE_K_META]);
      sp[cur.pair * g.gmax * kGroup + t] = (uint16_t)sbw;
    }
    if (cur.tensor == 0) {
      uint8_t* kt = p.p[KVQ_PLANE_K_HI] + (cur.pair * g.gmax + tile) * kTileBytes + v * 16;
      if (BITS == 3) {
        // 384-bit row, channel c at bit 3c: this lane's two 96-bit runs
        // (channels chan(0) .., chan(32) ..) are words 3 chan(0) / 32 ..;
        // the 16-byte chunks straddle the halves: the lower half writes
        // chunks 0 and 1, the upper chunk 2, each with words of the other
        uint32_t A[6];
        A[0] = U[0] | (U[1] << 24);
        A[1] = (U[1] >> 8) | (U[2] << 16);
        A[2] = (U[2] >> 16) | (U[3] << 8);
        A[3] = U[4] | (U[5] << 24);
        A[4] = (U[5] >> 8) | (U[6] << 16);
        A[5] = (U[6] >> 16) | (U[7] << 8);
        // transformed: lower half = words 0-2, 6-8, upper = 3-5, 9-11;
        // plain: lower = words 0-5, upper = 6-11
        if (HAD) {
          const uint32_t x0 = other_half(A[0], half), x1 = other_half(A[1], half),
                         x2 = other_half(A[2], half), x5 = other_half(A[5], half);
          if (valid) {
            if (half == 0) {
              *reinterpret_cast<uint4*>(kt) = make_uint4(A[0], A[1], A[2], x0);
              *reinterpret_cast<uint4*>(kt + 512) = make_uint4(x1, x2, A[3], A[4]);
            } else {
              *reinterpret_cast<uint4*>(kt + 1024) = make_uint4(x5, A[3], A[4], A[5]);
            }
          }
        } else {
          const uint32_t x0 = other_half(A[0], half), x1 = other_half(A[1], half);
          if (valid) {
            if (half == 0) {
              *reinterpret_cast<uint4*>(kt) = make_uint4(A[0], A[1], A[2], A[3]);
              *reinterpret_cast<uint4*>(kt + 512) = make_uint4(A[4], A[5], x0, x1);
            } else {
              *reinterpret_cast<uint4*>(kt + 1024) = make_uint4(A[2], A[3], A[4], A[5]);
            }
          }
        }
      } else if (valid) {
        // each run of four units is one 16-byte chunk of the row
#pragma unroll
        for (int q = 0; q < kLU / 4; ++q) {
          const int chunk = chan(4 * kPer * q) * BITS / 128;
          *reinterpret_cast<uint4*>(kt + chunk * 512) =
              make_uint4(U[4 * q], U[4 * q + 1], U[4 * q + 2], U[4 * q + 3]);
        }
      }
    } else {
      // token rows -> channel rows through the LDS area (the row reads above
      // are complete: their values are in registers; one wave's LDS
      // operations run in order)
      uint32_t* tr = reinterpret_cast<uint32_t*>(reg);
#pragma unroll
      for (int u = 0; u < kLU; ++u) tr[(chan(kPer * u) / kPer) * kTr + v] = U[u];
      const int64_t rlo = T0 - cur.tb, rhi = T1 - cur.tb;
      const int vlo = rlo < 0 ? 0 : (rlo > kGroup ? kGroup : (int)rlo);
      const int vhi = rhi < 0 ? 0 : (rhi > kGroup ? kGroup : (int)rhi);
      uint8_t* vt = p.p[KVQ_PLANE_V_HI] + (cur.pair * g.gmax + tile) * kTileBytes;
      if (BITS == 4) {
        // lane: channels 8 cg .. 8 cg + 7, tokens 8 tg .. 8 tg + 7
        const int cg = lane & 15, tg = lane >> 4;
        const uint32_t* src = tr + cg * kTr + 8 * tg;
        uint32_t a[8], o[8];
        const uint4 q0 = *reinterpret_cast<const uint4*>(src), q1 = *reinterpret_cast<const uint4*>(src + 4);
        a[0] = q0.x; a[1] = q0.y; a[2] = q0.z; a[3] = q0.w;
        a[4] = q1.x; a[5] = q1.y; a[6] = q1.z; a[7] = q1.w;
        transpose_nib8(a, o);
        const int lo = vlo - 8 * tg < 0 ? 0 : vlo - 8 * tg, hi = vhi - 8 * tg > 8 ? 8 : vhi - 8 * tg;
        if (hi > lo) {
          const uint32_t mk = field_mask(lo, hi, 0, 4);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            uint32_t* dst = reinterpret_cast<uint32_t*>(vt + 16 * (8 * cg + j) + 4 * tg);
            uint32_t w = o[j];
            if (mk != 0xFFFFFFFFu) w = (w & mk) | (*dst & ~mk);
            *dst = w;
          }
        }
      } else if (BITS == 8) {
        // lane: channels 4 cg .. 4 cg + 3, tokens 16 tq .. 16 tq + 15
        const int cg = lane & 31, tq = lane >> 5;
        const uint32_t* src = tr + cg * kTr + 16 * tq;
        uint32_t o[4][4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint4 q = *reinterpret_cast<const uint4*>(src + 4 * k);
          const uint32_t in[4] = {q.x, q.y, q.z, q.w};
          uint32_t out[4];
          transpose_byte4(in, out);
#pragma unroll
          for (int j = 0; j < 4; ++j) o[j][k] = out[j];
        }
        if (vhi > 16 * tq && vlo < 16 * tq + 16) {
          const bool whole = vlo <= 16 * tq && vhi >= 16 * tq + 16;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint4* dst = reinterpret_cast<uint4*>(vt + 32 * (4 * cg + j) + 16 * tq);
            uint32_t w[4] = {o[j][0], o[j][1], o[j][2], o[j][3]};
            if (!whole) {
              const uint4 old = *dst;
              const uint32_t ol[4] = {old.x, old.y, old.z, old.w};
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                const uint32_t mk = field_mask(vlo, vhi, 8 * (16 * tq + 4 * k), 8);
                w[k] = (w[k] & mk) | (ol[k] & ~mk);
              }
            }
            *dst = make_uint4(w[0], w[1], w[2], w[3]);
          }
        }
      } else {   // BITS == 3
        // lane: channels 8 cg + 2 jq, + 1, all 32 tokens; row d is one
        // 96-bit string, token k at bits 3k
        const int cg = lane & 15, jq = lane >> 4;
        const uint32_t* src = tr + cg * kTr;
        uint32_t a[32];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint4 q = *reinterpret_cast<const uint4*>(src + 4 * k);
          a[4 * k] = q.x; a[4 * k + 1] = q.y; a[4 * k + 2] = q.z; a[4 * k + 3] = q.w;
        }
        if (vhi > vlo) {
          const bool whole = vlo == 0 && vhi == kGroup;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int j = 2 * jq + e;
            uint32_t o[3] = {0u, 0u, 0u};
#pragma unroll
            for (int k = 0; k < kGroup; ++k) {
              const uint32_t code = (a[k] >> (3 * j)) & 7u;
              const int bit = 3 * k;
              o[bit >> 5] |= code << (bit & 31);
              if ((bit & 31) > 29) o[(bit >> 5) + 1] |= code >> (32 - (bit & 31));
            }
            uint32_t* dst = reinterpret_cast<uint32_t*>(vt + 12 * (8 * cg + j));
#pragma unroll
            for (int w = 0; w < 3; ++w) {
              uint32_t val = o[w];
              if (!whole) {
                const uint32_t mk = field_mask(vlo, vhi, 32 * w, 3);
                val = (val & mk) | (dst[w] & ~mk);
              }
              dst[w] = val;
            }
          }
        }
      }
    }
    if (item + 1 >= i1) break;
    cur = nit;
  }
#undef KVQ_ISSUE_ROWS
}

template <int BITS, bool Q40, int HAD, bool TBQ>
hipError_t launch_one(const Geom& g, const Planes& p, const SegArgs& a, hipStream_t s) {
  const void* fn = reinterpret_cast<const void*>(&block_append_kernel<BITS, Q40, HAD, TBQ>);
  const int64_t resident = (int64_t)occupancy_wgs_per_cu(fn) * device_compute_units();
  int64_t wgs = (a.n_items + 3) / 4;
  if (wgs > resident) wgs = resident;
  hipLaunchKernelGGL((block_append_kernel<BITS, Q40, HAD, TBQ>), dim3((unsigned)wgs), dim3(256), 0, s, g, p, a);
  return hipGetLastError();
}

template <int BITS, bool Q40, bool TBQ>
hipError_t launch_had(const Geom& g, const Planes& p, const SegArgs& a, hipStream_t s) {
  if (g.hadamard && g.hsigned) return launch_one<BITS, Q40, 2, TBQ>(g, p, a, s);
  if (g.hadamard) return launch_one<BITS, Q40, 1, TBQ>(g, p, a, s);
  if (TBQ) return hipErrorInvalidValue;
  return launch_one<BITS, Q40, 0, false>(g, p, a, s);
}

}  // namespace

hipError_t launch_block128_append(const Geom& g, const Planes& p, const __half* k_new,
                                  const __half* v_new, int64_t n_new, int64_t T0, hipStream_t s) {
  if (n_new <= 0) return hipSuccess;
  // segments of whole tiles whose rows lie within 4 GiB of their first row
  const int64_t row_bytes = (int64_t)g.Hkv * kD * 2;
  const int64_t seg_tokens = ((((int64_t)1 << 32) - 1) / row_bytes) / kGroup * kGroup;
  const int64_t T1 = T0 + n_new;
  for (int64_t ts = T0; ts < T1;) {
    int64_t te = (ts / kGroup) * kGroup + seg_tokens;
    if (te > T1) te = T1;
    SegArgs a;
    a.k_new = k_new;
    a.v_new = v_new;
    a.src_tokens = n_new;
    a.src_t0 = T0;
    a.T0 = ts;
    a.n = te - ts;
    a.tile0 = ts / kGroup;
    a.n_tiles = (te + kGroup - 1) / kGroup - a.tile0;
    a.n_items = (int64_t)g.B * g.Hkv * a.n_tiles * 2;
    hipError_t e;
    if (g.tbq4) e = launch_had<4, false, true>(g, p, a, s);
    else if (g.hi_bits == 8) e = launch_had<8, true, false>(g, p, a, s);
    else if (g.hi_bits == 3) e = launch_had<3, false, false>(g, p, a, s);
    else if (g.q40) e = launch_had<4, true, false>(g, p, a, s);
    else e = launch_had<4, false, false>(g, p, a, s);
    if (e != hipSuccess) return e;
    ts = te;
  }
  return hipSuccess;
}

}  // namespace kvq
