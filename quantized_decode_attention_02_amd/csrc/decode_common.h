// Pieces shared by the split-K decode kernels on the 4x4x4 fp16 MFMA and,
// for four query heads' values, the 16x16x32 one (decode_mfma.hip: keys
// stored after RoPE or rotated; decode_rope.hip: keys stored before RoPE).
//
// Sources cited here:
//   [nalar]  "Kuantisasi KV Cache dengan Error Budget yang Eksplisit"
//            (nalar.dev).
//
// MFMA 4x4x4 with 16 blocks: block b is lanes 4b..4b+3; A lane 4b+m holds
// row m, B lane 4b+n holds column n, D lane 4b+n register r holds row r of
// column n.  A wave streams 64-token tiles; lane l owns token l for the scores
// and channels l and 64 + l for the output; rows are query heads.
//
// Values (both kernels): per-token scales fold into the probabilities,
// p'_t = p_t s_t, written to LDS in A order as hi + lo fp16 halves (a single
// fp16 would put a 2^-12 relative error on c * s, i.e. on the group's whole
// range rather than on the value); zero points add sum_t p_t z_t.  B is the
// codes of 4 tokens of one channel (value tiles are channel-major): a nibble
// masked into an fp16 (w & 0x000F000F, ...) is the exact subnormal n * 2^-24,
// which the epilogue scales back by 2^24 ([nalar] "Error pada value masuk
// setelah attention probability").  The 16x16x32 value side (value_mfma16)
// keeps these rules with another operand layout.
#pragma once

#include "kvq_device.h"

namespace kvq {
namespace {

typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef float f4_t __attribute__((ext_vector_type(4)));

// One launch of a partials kernel: one token range of one code width.  The
// range's tiles (64 tokens each) of pair p = (sequence, kv head) form
// n_chunks chunks of `chunk` tiles, worked by a team of `team` waves that
// claim them dynamically, so that a wave which runs faster (older waves win
// issue priority on a SIMD; some XCDs see more fabric traffic) takes more of
// them instead of finishing early:
//   - assignment a in [0, pairs * team) is member k = a / pairs of the team
//     of pair (a + k) mod pairs; the wave of rank r = w * pwgs + blockIdx.x
//     - wins takes assignments r, r + 4 pwgs, ...  The skew spreads every team over
//     all XCDs (blockIdx.x mod 8) and all dispatch rounds.
//   - member k starts on chunk k; a claim on ctr[pair] returning c then
//     hands out chunk team + c, if that is below n_chunks.  A member claims
//     one chunk at a time and stops at its first failed claim, so a pair
//     sees exactly n_chunks claims (n_chunks - team that succeed, team that
//     fail); the one returning n_chunks - 1 is the last, and its wave puts
//     the counter back to zero for the next call.
//   - member k writes one partial, in slot slot_base + k.
// The first `wins` work-groups attend the fp16 window, one per pair; they go
// first so that they run beside the start of the tile work, not after it.
struct MfmaArgs {
  Geom g;
  Planes p;
  const __half* q;
  float* ws;            // partial records
  uint32_t* ctr;        // chunk counters of this launch: pair p at p * kCounterStride (zero on entry and exit)
  float scale_log2;
  int64_t q_pos;        // query position (keys stored before RoPE)
  int64_t t_lo, t_hi;   // token range of this launch; t_lo is 32-aligned
  int hi_tier;          // KIVI: tiles in the high-bit planes (ring) or low-bit
  int64_t tiles_pp;     // tiles per (sequence, kv head)
  int64_t pairs;        // sequences * kv heads
  int64_t team;         // waves per pair; also the range's partial slots per query head
  int64_t chunk;        // tiles per chunk
  int64_t n_chunks;     // chunks per pair, >= team
  int64_t n_big;        // chunks [0, n_big) have `chunk` tiles, later ones one tile
  int64_t pwgs;         // work-groups of the quantized tiles
  int64_t slot_base;    // first partial slot of this range
  int64_t wins;         // work-groups of the fp16 window (0 or pairs), launched first
  int64_t win_slot;     // first of the window's 4 slots
  int64_t n_slots;      // partial slots per (sequence, query head)
};

// (pair, member) of assignment asg (asg < pairs * team).
__device__ __forceinline__ void team_member(const MfmaArgs& a, int64_t asg, int64_t* pair,
                                            int64_t* k) {
  *k = asg / a.pairs;
  *pair = (asg + *k) % a.pairs;
}

// Claims of chunks: lane 0 issues the atomic; the result stays in its
// register until claim_value() (so the wave does not wait for it earlier).
__device__ __forceinline__ uint32_t claim_issue(uint32_t* ctr, int lane) {
  uint32_t v = 0;
  if (lane == 0) v = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return v;
}
__device__ __forceinline__ int64_t claim_value(uint32_t v) {
  return (int64_t)__builtin_amdgcn_readfirstlane(v);
}
// After a failed claim that returned `got` (the counter's old value): the
// last claim of the pair puts its counter back to zero.
__device__ __forceinline__ void claim_done(const MfmaArgs& a, uint32_t* ctr, int64_t got, int lane) {
  if (got == a.n_chunks - 1 && lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ h4_t as_h4(uint32_t x, uint32_t y) {
  typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
  u2_t v = {x, y};
  return __builtin_bit_cast(h4_t, v);
}

// Four 3-bit codes of a bit string (codes 4q .. 4q + 3, code k at bits 3k of
// the little-endian words w) as the fp16 B operand of one k-step: each code
// masked into the low bits of a 16-bit half is the exact subnormal n 2^-24.
__device__ __forceinline__ h4_t codes3_b(const uint32_t* w, int q) {
  const int bit = 12 * q, d = bit >> 5, sh = bit & 31;
  const uint32_t x = sh <= 20 ? (w[d] >> sh) : ((w[d] >> sh) | (w[d + 1] << (32 - sh)));
  const uint32_t a = (x & 7u) | ((x << 13) & 0x00070000u);          // codes 0, 1
  const uint32_t b = ((x >> 6) & 7u) | ((x << 7) & 0x00070000u);    // codes 2, 3
  return as_h4(a, b);
}

// TBQ4 levels of the eight 4-bit codes of a dword, as fp16 pairs in the
// order the code masks take them: out[0] = (code 0, code 4), out[1] =
// (1, 5), out[2] = (2, 6), out[3] = (3, 7) (code k = bits 4k .. 4k + 3).
// A level is carried as hi + lo, two fp16 values (hi = fp16(level), lo =
// fp16(level - hi)): a single fp16 would put a 2^-12 relative error on every
// key and value, systematic per level, which the tolerance does not absorb
// on large norms.  The 16 levels are symmetric (level[15 - k] = -level[k],
// ascending), so a code n is the magnitude level[8 + m] with m = n - 8
// (n >= 8) or 7 - n, negated for n < 8.  Byte lookups by v_perm: lut[0..1]
// hold the low bytes of the eight magnitudes' hi halves, lut[2..3] their high
// bytes, lut[4..7] the same for the lo halves; the magnitude nibbles
// themselves are the selectors.  No memory is read.
__device__ __forceinline__ void tbq4_levels(uint32_t w, const uint32_t* lut, uint32_t* hi, uint32_t* lo) {
  const uint32_t neg = (~w >> 3) & 0x11111111u;                 // code < 8
  // 7 neg, the nibbles of the codes below 8 set to 7: neg | neg << 1 |
  // neg << 2 (the bits lie apart), written as asm so that it stays two
  // full-rate shifts-and-ors rather than becoming an integer multiply
  uint32_t neg7;
  asm("v_lshl_or_b32 %0, %1, 1, %1\n\tv_lshl_or_b32 %0, %1, 2, %0" : "=&v"(neg7) : "v"(neg));
  const uint32_t mag = (w & 0x77777777u) ^ neg7;                // m per nibble
  const uint32_t s_even = mag & 0x0F0F0F0Fu;                    // m of codes 0, 2, 4, 6
  const uint32_t s_odd = (mag >> 4) & 0x0F0F0F0Fu;              // m of codes 1, 3, 5, 7
  // the sign of code k moves from bit 4k to bit 15 or 31 of its pair
  const uint32_t sg[4] = {(neg & 0x00010001u) << 15, (neg & 0x00100010u) << 11,
                          (neg & 0x01000100u) << 7, (neg & 0x10001000u) << 3};
#pragma unroll
  for (int part = 0; part < 2; ++part) {
    const uint32_t* t = lut + 4 * part;
    uint32_t* out = part ? lo : hi;
    const uint32_t lb_e = __builtin_amdgcn_perm(t[1], t[0], s_even);
    const uint32_t hb_e = __builtin_amdgcn_perm(t[3], t[2], s_even);
    const uint32_t lb_o = __builtin_amdgcn_perm(t[1], t[0], s_odd);
    const uint32_t hb_o = __builtin_amdgcn_perm(t[3], t[2], s_odd);
    // [low, high] byte of selector bytes 0 and 2 (codes 0, 4 / 1, 5), 1 and
    // 3 (codes 2, 6 / 3, 7); xor for the sign, as a lo half may be negative
    out[0] = __builtin_amdgcn_perm(hb_e, lb_e, 0x06020400u) ^ sg[0];
    out[1] = __builtin_amdgcn_perm(hb_o, lb_o, 0x06020400u) ^ sg[1];
    out[2] = __builtin_amdgcn_perm(hb_e, lb_e, 0x07030501u) ^ sg[2];
    out[3] = __builtin_amdgcn_perm(hb_o, lb_o, 0x07030501u) ^ sg[3];
  }
}

__device__ __forceinline__ f4_t mfma4(h4_t x, h4_t y, f4_t c) {
  return __builtin_amdgcn_mfma_f32_4x4x4f16(x, y, c, 0, 0, 0);
}

// A wave's fp16 A-operand tables of the 4x4x4 MFMA (query or probabilities):
// tables of NKS k-steps, a k-step being HL blocks of 4 rows x 4 halves.  With
// KPAD each k-step takes 8 bytes more, with TPAD each table 32 bytes more, so
// that the k-steps one instruction writes (one per group of lanes) and the
// tables one instruction reads (one per half wave) fall in different LDS
// banks: for four query heads, 64-byte k-steps put the 16 k-steps a
// probability write spans into 4 banks.  Tables that are written rarely go
// without.
template <int HL, int NKS, bool KPAD = false, bool TPAD = false>
struct ATab {
  static constexpr int KS = HL * 16 + (KPAD ? 4 : 0);   // halves per k-step
  static constexpr int T = NKS * KS + (TPAD ? 16 : 0);  // halves per table
  _Float16* p;
  __device__ __forceinline__ _Float16& at(int t, int ks, int hl, int m, int slot) const {
    return p[t * T + ks * KS + hl * 16 + m * 4 + slot];
  }
  __device__ __forceinline__ h4_t& h4(int t, int ks, int hl, int m) const {
    return *reinterpret_cast<h4_t*>(&p[t * T + ks * KS + hl * 16 + m * 4]);
  }
};

// Value token tl (0..31 in its group) -> (k-step within the group, slot).
template <int BITS>
__device__ __forceinline__ void value_slot(int tl, int* kk, int* slot) {
  if (BITS == 3) {   // natural order: k-step tl / 4, slot tl % 4
    *kk = tl >> 2;
    *slot = tl & 3;
  } else if (BITS == 8) {   // a dword's bytes 0, 2 then 1, 3: tokens 4k, 4k + 2, 4k + 1, 4k + 3
    const int j = tl & 3;
    *kk = tl >> 2;
    *slot = ((j & 1) << 1) | (j >> 1);
  } else if (BITS == 4) {
    const int i = tl >> 3, r = tl & 7, j = r & 3, hp = r >> 2;
    *kk = 2 * i + (j >> 1);
    *slot = (j & 1) * 2 + hp;
  } else {
    const int i = tl >> 4, e = tl & 15, j = e & 7, hp = e >> 3;
    *kk = 4 * i + (j >> 1);
    *slot = (j & 1) * 2 + hp;
  }
}

// hi + lo fp16 split of x (x - hi is exact in fp32)
__device__ __forceinline__ void split_half(float x, _Float16* hi, _Float16* lo) {
  *hi = (_Float16)x;
  *lo = (_Float16)(x - (float)*hi);
}

// ---------------------------------------------------------------------------
// Value side of four query heads on the 16x16x32 f16 MFMA (4- and 2-bit
// codes).  Per value scale group dg (NDG of them: 32 channels each, or one
// for the whole row) and key group gg, the A operand is p' = p s of the
// group's 32 tokens as a 16 x 32 matrix: row 4 hl + m holds the hi (hl = 0)
// or lo (hl = 1) fp16 half of head m's p'; rows 8..15 repeat rows 0..7 and
// their sums are never read.  Column k = 8 kc + j: lane group kc = lane / 16
// covers the 8 tokens whose codes one dword of a channel row holds (at 2
// bits half of one), j orders them as the masked words do.  B is the codes
// of 16 channels, one per column (channel 16 cb + lane % 16).  Lane l then
// holds rows 4 (l / 16) + i of column l % 16: lanes 0..15 the hi sums of
// heads i = 0..3, lanes 16..31 the lo sums.  One tile is 16 MFMAs (2 groups
// x 8 channel blocks) where the 4x4x4 shape needs 64 (hi and lo each
// 4 heads x 4 tokens x 4 channels a block).
typedef uint32_t u2v_t __attribute__((ext_vector_type(2)));
typedef uint32_t u4v_t __attribute__((ext_vector_type(4)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)(p);
}

__device__ __forceinline__ f4_t mfma16(h8_t a, h8_t b, f4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Lane group kc, position j and the inverse place factor of value token tl
// (0..31 in its group).  4 bits: dword tl / 8 of the row, nibble o = tl % 8,
// masked word o % 4 (x16 when odd), half o / 4.  3 bits: the 24 bits of
// tokens 8 kc .. 8 kc + 7 of the row's 96-bit string, token o = tl % 8 in
// masked word o % 4, half o / 4, with the factor its bits keep there
// (codes16_b): 1, 16, 64, 64 in the low halves, 1, 1, 4, 4 in the high ones.
// 2 bits: dword tl / 16, crumb e = tl % 16: lane group 2 (tl / 16) +
// (e / 4) % 2, masked word e % 4 (x4^(e % 4)), half e / 8.
template <int BITS>
__device__ __forceinline__ void v16_slot(int tl, int* kc, int* j, float* inv_f) {
  if (BITS == 4 || BITS == 3) {
    const int o = tl & 7;
    *kc = tl >> 3;
    *j = 2 * (o & 3) + (o >> 2);
    if (BITS == 4) {
      *inv_f = (o & 1) ? 1.0f / 16 : 1.0f;
    } else {
      const int e = (o < 4) ? (o == 0 ? 0 : o == 1 ? 4 : 6) : (o < 6 ? 0 : 2);   // log2 of the factor
      *inv_f = __int_as_float((127 - e) << 23);
    }
  } else {
    const int e = tl & 15, w = e & 3;
    *kc = 2 * (tl >> 4) + ((e >> 2) & 1);
    *j = 2 * w + (e >> 3);
    *inv_f = __int_as_float((127 - 2 * w) << 23);   // 4^-w
  }
}

// Table half offset of (dg, gg, row, column); a table is NDG x 2 blocks of
// 8 rows of 32 halves, each block padded by 32 halves, so that the two key
// groups' columns (written by the wave's two halves in one store) fall in
// different LDS banks.  Byte strides: row 64, block 576, scale group 1152.
constexpr int kV16Blk = 8 * 32 + 32;
__device__ __forceinline__ int v16_at(int dg, int gg, int row, int col) {
  return (dg * 2 + gg) * kV16Blk + row * 32 + col;
}
constexpr int v16_halves(int ndg) { return ndg * 2 * kV16Blk; }

// One token's p' of one scale group: hi halves into rows 0..3, lo halves
// into rows 4..7 (64 bytes a row) of the column at LDS byte address sb.
// Written as asm, so that the compiler does not first wait for global-to-LDS
// copies in flight (it cannot tell that they go elsewhere).
__device__ __forceinline__ void store_p16(uint32_t sb, const _Float16* hi, const _Float16* lo) {
  asm volatile(
      "ds_write_b16 %0, %1\n\t"
      "ds_write_b16 %0, %2 offset:64\n\t"
      "ds_write_b16 %0, %3 offset:128\n\t"
      "ds_write_b16 %0, %4 offset:192\n\t"
      "ds_write_b16 %0, %5 offset:256\n\t"
      "ds_write_b16 %0, %6 offset:320\n\t"
      "ds_write_b16 %0, %7 offset:384\n\t"
      "ds_write_b16 %0, %8 offset:448"
      ::"v"(sb), "v"(hi[0]), "v"(hi[1]), "v"(hi[2]), "v"(hi[3]), "v"(lo[0]), "v"(lo[1]), "v"(lo[2]), "v"(lo[3])
      : "memory");
}

// The lane's A operands of key group gg, av[dg], in one asm block with its
// own LDS wait.  pvb: the lane's address for (dg, gg) = (0, 0) (row
// lane % 8, columns 8 (lane / 16) ..); (dg, gg) lies 1152 dg + 576 gg bytes
// further.
template <int NDG>
__device__ __forceinline__ void read_a16(uint32_t pvb, int gg, u4v_t* av) {
  if (NDG == 1) {
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(av[0]) : "v"(pvb + 576 * gg) : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %4 offset:1152\n\t"
        "ds_read_b128 %2, %4 offset:2304\n\t"
        "ds_read_b128 %3, %4 offset:3456\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=v"(av[0]), "=v"(av[1]), "=v"(av[2]), "=v"(av[3])
        : "v"(pvb + 576 * gg)
        : "memory");
  }
}

// The B operand of one code dword: four masked words, two codes each (at 2
// bits from the dword's half the lane group takes; at 3 bits x is the lane
// group's 24-bit window, code o at bits 3o, each masked word keeps two codes
// inside the 10 mantissa bits of their halves).
template <int BITS>
__device__ __forceinline__ h8_t codes16_b(uint32_t x, int lane) {
  u4v_t v;
  if (BITS == 3) {
    v = u4v_t{(x & 7u) | ((x << 4) & 0x00070000u),   // codes 0, 4 (x1, x1)
              (x << 1) & 0x00070070u,                 // codes 1, 5 (x16, x1)
              x & 0x001C01C0u,                        // codes 2, 6 (x64, x4)
              (x >> 3) & 0x001C01C0u};                // codes 3, 7 (x64, x4)
  } else if (BITS == 4) {
    const uint32_t x8 = x >> 8;
    v = u4v_t{x & 0x000F000Fu, x & 0x00F000F0u, x8 & 0x000F000Fu, x8 & 0x00F000F0u};
  } else {
    const uint32_t y = x >> (8 * ((lane >> 4) & 1));
    v = u4v_t{y & 0x00030003u, y & 0x000C000Cu, y & 0x00300030u, y & 0x00C000C0u};
  }
  return __builtin_bit_cast(h8_t, v);
}

// p' = p s of this lane's token into the table (LDS byte address pv), and
// the zero-point sums (blocks: the sums of p' for the code offset).  TBQ:
// the B operands are levels, without place factors.
template <int G, int BITS, bool BLOCK, int NDG, bool TBQ = false>
__device__ __forceinline__ void stage_probs16(const float* p, const float* vs, const float* vz, uint32_t pv,
                                              float (*zacc)[NDG], int tl, int gh) {
  int kc, j;
  float inv_f;
  v16_slot<BITS>(tl, &kc, &j, &inv_f);
  if (TBQ) inv_f = 1.0f;
  const uint32_t sb = pv + 2 * v16_at(0, gh, 0, 8 * kc + j);
  for (int d = 0; d < NDG; ++d) {
    _Float16 hi[4], lo[4];
    const float vsi = vs[d] * inv_f;   // a power of two: p (s / f) = (p s) / f exactly
    for (int m = 0; m < G; ++m) {
      split_half(p[m] * vsi, &hi[m], &lo[m]);
      zacc[m][d] += BLOCK ? p[m] * vs[d] : p[m] * vz[d];
    }
    store_p16(sb + 1152 * d, hi, lo);
  }
}

// O += p' . codes over a tile whose code dwords are in registers,
// vd[gg][cb] (channel 16 cb + lane % 16, lane group lane / 16).  TBQ: the
// codes' levels as hi + lo fp16 (tbq4_levels, same order as the masked
// words), one MFMA for each against both halves of p'.
template <int BITS, int NDG, bool TBQ = false>
__device__ __forceinline__ void value_mfma16(const uint32_t (*vd)[8], uint32_t pv, int lane, f4_t* acc,
                                             const uint32_t* lut = nullptr) {
  const uint32_t pvb = pv + 2 * v16_at(0, 0, lane & 7, 8 * (lane >> 4));
  for (int gg = 0; gg < 2; ++gg) {
    u4v_t av[NDG];
    read_a16<NDG>(pvb, gg, av);
    for (int cb = 0; cb < 8; ++cb) {
      const h8_t a8 = __builtin_bit_cast(h8_t, av[NDG == 1 ? 0 : cb >> 1]);
      if (TBQ) {
        uint32_t hi[4], lo[4];
        tbq4_levels(vd[gg][cb], lut, hi, lo);
        acc[cb] = mfma16(a8, __builtin_bit_cast(h8_t, u4v_t{hi[0], hi[1], hi[2], hi[3]}), acc[cb]);
        acc[cb] = mfma16(a8, __builtin_bit_cast(h8_t, u4v_t{lo[0], lo[1], lo[2], lo[3]}), acc[cb]);
      } else {
        acc[cb] = mfma16(a8, codes16_b<BITS>(vd[gg][cb], lane), acc[cb]);
      }
    }
  }
}

// Online-softmax step of head m on the 16x16x32 accumulators (as
// softmax_step: rescale when the running maximum moves).
template <int G, int NDG>
__device__ __forceinline__ float softmax_step16(int m, float s, bool tok_ok, float* m_run, float* l_acc,
                                                f4_t* acc, float (*zacc)[NDG]) {
  if (__any(s > m_run[m])) {
    const float mnew = fmaxf(m_run[m], wave_max64(s));
    const float alpha = (m_run[m] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run[m] - mnew);
    m_run[m] = mnew;
    l_acc[m] *= alpha;
    for (int c = 0; c < 8; ++c) acc[c][m] *= alpha;
    for (int d = 0; d < NDG; ++d) zacc[m][d] *= alpha;
  }
  const float p = tok_ok ? __builtin_amdgcn_exp2f(s - m_run[m]) : 0.0f;
  l_acc[m] += p;
  return p;
}

// Online-softmax update of one head for one tile; returns p for this lane.
template <int G, int HL, int NDG>
__device__ __forceinline__ float softmax_step(int m, float s, bool tok_ok, float* m_run, float* l_acc,
                                              f4_t& o0, f4_t& o1, f4_t& o2, f4_t& o3,
                                              float (*zacc)[NDG]) {
  if (__any(s > m_run[m])) {
    const float mnew = fmaxf(m_run[m], wave_max64(s));
    const float alpha = (m_run[m] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run[m] - mnew);
    m_run[m] = mnew;
    l_acc[m] *= alpha;
    o0[m] *= alpha; o1[m] *= alpha; o2[m] *= alpha; o3[m] *= alpha;
    if (HL == 1) {
      o0[G + m] *= alpha; o1[G + m] *= alpha; o2[G + m] *= alpha; o3[G + m] *= alpha;
    }
    for (int d = 0; d < NDG; ++d) zacc[m][d] *= alpha;
  }
  // the hardware exp2 (v_exp_f32, about 1 ulp): it flushes results below
  // 2^-126 to zero, a probability mass the fp32 sums could not hold anyway;
  // exp2f would add a denormal-preserving range reduction around it
  const float p = tok_ok ? __builtin_amdgcn_exp2f(s - m_run[m]) : 0.0f;
  l_acc[m] += p;
  return p;
}

// Raw bytes of one 64-token tile for this lane: its token's key row, the
// value rows of channels lane and 64 + lane for both groups, the metadata of
// its token / group.
template <int BITS, bool BLOCK>
struct TileRaw {
  uint4 kc[BITS];
  uint32_t vc[2][2][BITS];
  uint32_t vd[2][8];   // 16x16x32 value side: dword lane / 16 (2 bits: lane / 32) of channel 16 cb + lane % 16
  uint2 km0, km1;   // KIVI, keys after RoPE: (s, z) of the key channels of this lane's k-step
  uint4 kmr;        // KIVI, keys before RoPE: (s, z) of channels 4 (lane % 32) .. + 3
  uint4 vm;         // KIVI: (s, z) x 4 of this lane's token
  uint16_t ks16, vs16;   // BLOCK: per-token scales
  uint2 kq4, vq4;        // BLOCK, Q4_0 / Q8_0: the four 32-value slice scales of the token
};

struct TilePos {
  int64_t base;
  int nvalid;
  uint32_t s0, s1;  // tile slots of the two groups
  uint32_t grp0;
};

// Position of tile t (0 .. tiles_pp - 1) of a pair in the range.
__device__ __forceinline__ void tile_at(const MfmaArgs& a, int64_t t, int64_t slots, bool ring,
                                       TilePos& tp) {
  tp.base = a.t_lo + t * 64;
  tp.nvalid = (int)min((int64_t)64, a.t_hi - tp.base);
  tp.grp0 = (uint32_t)(tp.base >> 5);
  tp.s0 = tp.grp0;
  tp.s1 = tp.grp0 + 1;
  if (ring) {
    tp.s0 = tp.grp0 % (uint32_t)slots;
    tp.s1 = (tp.s0 + 1 == (uint32_t)slots) ? 0 : tp.s0 + 1;
  }
}

// A wave's walk over the tiles of its assignments (see MfmaArgs).
struct TileCursor {
  int64_t asg;        // assignment
  int64_t pair, k;    // its pair and member index
  int64_t t, t_stop;  // tile, end of its chunk
  uint32_t pend;      // the claim in flight
};

// Tiles [t, t_stop) of chunk ch: chunks of `chunk` tiles, then single tiles,
// so that the last claims of a pair are short and its members finish close
// together.
__device__ __forceinline__ void chunk_range(const MfmaArgs& a, int64_t ch, int64_t* t, int64_t* t_stop) {
  if (ch < a.n_big) {
    *t = ch * a.chunk;
    *t_stop = min(*t + a.chunk, a.tiles_pp);
  } else {
    *t = a.n_big * a.chunk + (ch - a.n_big);
    *t_stop = *t + 1;
  }
}

// First tile of assignment asg: the member's own chunk; its first claim
// goes out at once.
__device__ __forceinline__ void cursor_start(const MfmaArgs& a, int64_t asg, TileCursor& c, int lane) {
  c.asg = asg;
  team_member(a, asg, &c.pair, &c.k);
  chunk_range(a, c.k, &c.t, &c.t_stop);
  c.pend = claim_issue(a.ctr + c.pair * kCounterStride, lane);
}

// Moves c to the tile after the current one.  *ends: the current tile was
// the last of its assignment (its partial is due).  Returns false when the
// wave has no tile left.
__device__ __forceinline__ bool cursor_next(const MfmaArgs& a, TileCursor& c, int lane, bool* ends) {
  *ends = false;
  if (c.t + 1 < c.t_stop) {
    ++c.t;
    return true;
  }
  const int64_t got = claim_value(c.pend);
  const int64_t ch = a.team + got;
  if (ch < a.n_chunks) {
    chunk_range(a, ch, &c.t, &c.t_stop);
    c.pend = claim_issue(a.ctr + c.pair * kCounterStride, lane);
    return true;
  }
  claim_done(a, a.ctr + c.pair * kCounterStride, got, lane);
  *ends = true;
  const int64_t nxt = c.asg + 4 * a.pwgs;
  if (nxt >= a.pairs * a.team) return false;
  cursor_start(a, nxt, c, lane);
  return true;
}

// cursor_next that leaves the claim of a new chunk to the
// caller (*claim set), so that the claim has one issue site in the tile loop:
// the atomic's result then goes straight into the cursor's register, and no
// register copy (which would wait for the atomic at once) is needed.
__device__ __forceinline__ bool cursor_next_deferred(const MfmaArgs& a, TileCursor& c, int lane, bool* ends,
                                                     bool* claim) {
  *ends = false;
  *claim = false;
  if (c.t + 1 < c.t_stop) {
    ++c.t;
    return true;
  }
  const int64_t got = claim_value(c.pend);
  const int64_t ch = a.team + got;
  if (ch < a.n_chunks) {
    chunk_range(a, ch, &c.t, &c.t_stop);
    *claim = true;
    return true;
  }
  claim_done(a, a.ctr + c.pair * kCounterStride, got, lane);
  *ends = true;
  const int64_t nxt = c.asg + 4 * a.pwgs;
  if (nxt >= a.pairs * a.team) return false;
  c.asg = nxt;
  team_member(a, nxt, &c.pair, &c.k);
  chunk_range(a, c.k, &c.t, &c.t_stop);
  *claim = true;
  return true;
}

template <int BITS, bool BLOCK, bool ROPE, bool Q40 = false>
__device__ __forceinline__ void load_tile(TileRaw<BITS, BLOCK>& r, const TilePos& tp, int lane,
                                          const uint8_t* kpair, const uint8_t* vpair,
                                          const uint8_t* kmpair, const uint8_t* vmpair,
                                          const uint16_t* ksc, const uint16_t* vsc, int kch0,
                                          int kch1) {
  constexpr int TB = 512 * BITS;
  constexpr int VROW = 4 * BITS;
  const int gh = lane >> 5, tl = lane & 31;
  const bool tok_ok = lane < tp.nvalid;
  const bool grp1_ok = tp.nvalid > 32;
  const uint32_t my_slot = gh ? tp.s1 : tp.s0;
  const uint8_t* kt = kpair + (int64_t)my_slot * TB + tl * 16;
  for (int j = 0; j < BITS; ++j)
    r.kc[j] = tok_ok ? *reinterpret_cast<const uint4*>(kt + j * 512) : make_uint4(0, 0, 0, 0);
  for (int gg = 0; gg < 2; ++gg) {
    const bool ok = gg == 0 || grp1_ok;
    const uint8_t* vt = vpair + (int64_t)(gg ? tp.s1 : tp.s0) * TB;
    for (int hf = 0; hf < 2; ++hf) {
      const uint8_t* src = vt + (lane + 64 * hf) * VROW;
      if constexpr (BITS == 8) {
        for (int hv = 0; hv < 2; ++hv) {
          const uint4 x = ok ? *reinterpret_cast<const uint4*>(src + 16 * hv) : make_uint4(0, 0, 0, 0);
          r.vc[gg][hf][4 * hv] = x.x; r.vc[gg][hf][4 * hv + 1] = x.y;
          r.vc[gg][hf][4 * hv + 2] = x.z; r.vc[gg][hf][4 * hv + 3] = x.w;
        }
      } else if constexpr (BITS == 3) {
        const uint32_t* s32 = reinterpret_cast<const uint32_t*>(src);
        r.vc[gg][hf][0] = ok ? s32[0] : 0u; r.vc[gg][hf][1] = ok ? s32[1] : 0u; r.vc[gg][hf][2] = ok ? s32[2] : 0u;
      } else if (BITS == 4) {
        const uint4 x = ok ? *reinterpret_cast<const uint4*>(src) : make_uint4(0, 0, 0, 0);
        r.vc[gg][hf][0] = x.x; r.vc[gg][hf][1] = x.y; r.vc[gg][hf][2] = x.z; r.vc[gg][hf][3] = x.w;
      } else {
        const uint2 x = ok ? *reinterpret_cast<const uint2*>(src) : make_uint2(0, 0);
        r.vc[gg][hf][0] = x.x; r.vc[gg][hf][1] = x.y;
      }
    }
  }
  if (BLOCK && Q40) {
    const int64_t t = tp.base + lane;
    r.kq4 = tok_ok ? reinterpret_cast<const uint2*>(ksc)[t] : make_uint2(0, 0);
    r.vq4 = tok_ok ? reinterpret_cast<const uint2*>(vsc)[t] : make_uint2(0, 0);
  } else if (BLOCK) {
    const int64_t t = tp.base + lane;
    r.ks16 = tok_ok ? ksc[t] : (uint16_t)0;
    r.vs16 = tok_ok ? vsc[t] : (uint16_t)0;
  } else {
    const bool my_grp_ok = gh == 0 || grp1_ok;
    const uint32_t my_grp = tp.grp0 + gh;
    const uint8_t* kmeta = kmpair + (int64_t)my_grp * 512;
    const uint8_t* vmeta = vmpair + (int64_t)my_grp * 512;
    if (ROPE) {
      r.kmr = my_grp_ok ? *reinterpret_cast<const uint4*>(kmeta + 16 * tl) : make_uint4(0, 0, 0, 0);
    } else {
      r.km0 = my_grp_ok ? *reinterpret_cast<const uint2*>(kmeta + 4 * kch0) : make_uint2(0, 0);
      r.km1 = my_grp_ok ? *reinterpret_cast<const uint2*>(kmeta + 4 * kch1) : make_uint2(0, 0);
    }
    r.vm = tok_ok ? *reinterpret_cast<const uint4*>(vmeta + 16 * tl) : make_uint4(0, 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// Tile staging.  A wave copies the code bytes of its next tile straight from
// HBM into its own LDS stage with 16-byte global-to-LDS loads (lane l of one
// load writes bytes [16 l, 16 l + 16) of a 1 KiB run), and the few metadata
// bytes into registers, while it computes the current tile: a whole tile is
// in flight during the compute.  Stage layout (TB = tile bytes of one group):
//   [0, 2 TB)    key tiles of the two groups
//   [2 TB, 4 TB) value tiles of the two groups
// A second group past the tile's tokens is read from the first group's slot
// (what it brings is never used), and block scales past the end of the
// pair's region from inside it: every source lies inside the data.
template <int BITS>
constexpr int stage_bytes() {
  return 4 * 512 * BITS;
}

__device__ __forceinline__ void lds_dma16(const void* src, void* lds_run) {
  __builtin_amdgcn_global_load_lds(src, lds_run, 16, 0, 0);
}

template <int BITS>
__device__ __forceinline__ void stage_issue(uint8_t* st, const TilePos& tp, int lane,
                                            const uint8_t* kpair, const uint8_t* vpair) {
  constexpr int TB = 512 * BITS;
  const bool g1 = tp.nvalid > 32;
  for (int gg = 0; gg < 2; ++gg) {
    const int64_t slot = (gg && g1) ? tp.s1 : tp.s0;
    for (int k = 0; k * 1024 < TB; ++k) {
      if (k * 1024 + 16 * lane < TB) {   // a 3-bit tile ends half way through a kilobyte
        lds_dma16(kpair + slot * TB + k * 1024 + 16 * lane, st + gg * TB + k * 1024);
        lds_dma16(vpair + slot * TB + k * 1024 + 16 * lane, st + 2 * TB + gg * TB + k * 1024);
      }
    }
  }
}

// Metadata of the lane's token / group into registers (plain loads).
template <int BITS, bool BLOCK, bool ROPE, bool Q40 = false>
__device__ __forceinline__ void meta_issue(TileRaw<BITS, BLOCK>& r, const TilePos& tp, int lane,
                                           const uint8_t* kmpair, const uint8_t* vmpair,
                                           const uint16_t* ksc, const uint16_t* vsc, int64_t scale_end,
                                           int kch0, int kch1) {
  const int gh = lane >> 5, tl = lane & 31;
  if (BLOCK) {
    int64_t t = tp.base + lane;
    if (t >= scale_end) t = scale_end - 1;
    if (Q40) {
      r.kq4 = reinterpret_cast<const uint2*>(ksc)[t];
      r.vq4 = reinterpret_cast<const uint2*>(vsc)[t];
    } else {
      r.ks16 = ksc[t];
      r.vs16 = vsc[t];
    }
  } else {
    const int64_t grp = tp.grp0 + ((gh && tp.nvalid > 32) ? 1 : 0);
    const uint8_t* kmeta = kmpair + grp * 512;
    if (ROPE) {
      r.kmr = *reinterpret_cast<const uint4*>(kmeta + 16 * tl);
    } else {
      r.km0 = *reinterpret_cast<const uint2*>(kmeta + 4 * kch0);
      r.km1 = *reinterpret_cast<const uint2*>(kmeta + 4 * kch1);
    }
    r.vm = *reinterpret_cast<const uint4*>(vmpair + grp * 512 + 16 * tl);
  }
}

// This lane's codes from the staged tile (same contents as load_tile).
template <int BITS, bool BLOCK>
__device__ __forceinline__ void stage_read(TileRaw<BITS, BLOCK>& r, const uint8_t* st, int lane) {
  constexpr int TB = 512 * BITS;
  constexpr int VROW = 4 * BITS;
  const int gh = lane >> 5, tl = lane & 31;
  for (int j = 0; j < BITS; ++j) r.kc[j] = *reinterpret_cast<const uint4*>(st + gh * TB + j * 512 + tl * 16);
  for (int gg = 0; gg < 2; ++gg)
    for (int hf = 0; hf < 2; ++hf) {
      const uint8_t* src = st + 2 * TB + gg * TB + (lane + 64 * hf) * VROW;
      if constexpr (BITS == 8) {
        for (int hv = 0; hv < 2; ++hv) {
          const uint4 x = *reinterpret_cast<const uint4*>(src + 16 * hv);
          r.vc[gg][hf][4 * hv] = x.x; r.vc[gg][hf][4 * hv + 1] = x.y;
          r.vc[gg][hf][4 * hv + 2] = x.z; r.vc[gg][hf][4 * hv + 3] = x.w;
        }
      } else if constexpr (BITS == 3) {
        const uint32_t* s32 = reinterpret_cast<const uint32_t*>(src);
        r.vc[gg][hf][0] = s32[0]; r.vc[gg][hf][1] = s32[1]; r.vc[gg][hf][2] = s32[2];
      } else if (BITS == 4) {
        const uint4 x = *reinterpret_cast<const uint4*>(src);
        r.vc[gg][hf][0] = x.x; r.vc[gg][hf][1] = x.y; r.vc[gg][hf][2] = x.z; r.vc[gg][hf][3] = x.w;
      } else {
        const uint2 x = *reinterpret_cast<const uint2*>(src);
        r.vc[gg][hf][0] = x.x; r.vc[gg][hf][1] = x.y;
      }
    }
}

// stage_read for the 16x16x32 value side: the key rows as stage_read, the
// value code dwords as value_mfma16 takes them (4 or 2 bits: whole dwords;
// 3 bits: each lane group's 24-bit window of the row).
template <int BITS, bool BLOCK>
__device__ __forceinline__ void stage_read16(TileRaw<BITS, BLOCK>& r, const uint8_t* st, int lane) {
  constexpr int TB = 512 * BITS;
  constexpr int VROW = 4 * BITS;
  const int gh = lane >> 5, tl = lane & 31;
  for (int j = 0; j < BITS; ++j) r.kc[j] = *reinterpret_cast<const uint4*>(st + gh * TB + j * 512 + tl * 16);
  if (BITS == 3) {
    // the lane group's 24 bits of the 96-bit row: bits 24 kc .. 24 kc + 23,
    // from dwords lo and (lo + 1, at most 2)
    const int kc = lane >> 4, bit = 24 * kc, lo = bit >> 5, sh = bit & 31, hi = lo < 2 ? lo + 1 : 2;
    const uint8_t* src = st + 2 * TB + (lane & 15) * VROW;
    for (int gg = 0; gg < 2; ++gg)
      for (int cb = 0; cb < 8; ++cb) {
        const uint8_t* row = src + gg * TB + cb * 16 * VROW;
        const uint32_t a = *reinterpret_cast<const uint32_t*>(row + 4 * lo);
        const uint32_t b = *reinterpret_cast<const uint32_t*>(row + 4 * hi);
        r.vd[gg][cb] = sh ? ((a >> sh) | (b << (32 - sh))) : a;
      }
    return;
  }
  const uint8_t* src = st + 2 * TB + (lane & 15) * VROW + 4 * (lane >> (BITS == 4 ? 4 : 5));
  for (int gg = 0; gg < 2; ++gg)
    for (int cb = 0; cb < 8; ++cb)
      r.vd[gg][cb] = *reinterpret_cast<const uint32_t*>(src + gg * TB + cb * 16 * VROW);
}

__device__ __forceinline__ void wait_stage_landed() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_stage_read() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Per-token value scales / zeros of this lane's token from the raw tile.
// Tokens past the tile get 0 (their probability is 0, and 0 * anything
// non-finite would not be).
template <int BITS, bool BLOCK, int NDG, bool Q40 = false>
__device__ __forceinline__ void value_meta(const TileRaw<BITS, BLOCK>& r, bool tok_ok, float* vs,
                                           float* vz) {
  if (BLOCK && Q40) {   // a scale per 32-dim slice; the code offset (8 or 128) comes back in the flush
    const uint32_t vw[2] = {r.vq4.x, r.vq4.y};
    for (int d = 0; d < NDG; ++d) {
      const uint16_t h = (uint16_t)((vw[d >> 1] >> (16 * (d & 1))) & 0xFFFF);
      vs[d] = tok_ok ? half_bits_to_float(h) : 0.0f;
      vz[d] = 0.0f;
    }
  } else if (BLOCK) {
    vs[0] = tok_ok ? half_bits_to_float(r.vs16) : 0.0f;
    vz[0] = 0.0f;
  } else {
    const uint32_t vw[4] = {r.vm.x, r.vm.y, r.vm.z, r.vm.w};
    for (int d = 0; d < 4; ++d) {
      vs[d] = tok_ok ? half_bits_to_float((uint16_t)(vw[d] & 0xFFFF)) : 0.0f;
      vz[d] = tok_ok ? half_bits_to_float((uint16_t)(vw[d] >> 16)) : 0.0f;
    }
  }
}

// p' = p s into this wave's value A tables (PLw, one per value scale group);
// zero-point sums.
template <int G, int BITS, bool BLOCK, int HL, int NDG, bool TBQ = false, class PT>
__device__ __forceinline__ void stage_probs(const float* p, const float* vs, const float* vz,
                                            const PT& PLw, float (*zacc)[NDG],
                                            int tl, int gh) {
  int kk, slot;
  value_slot<BITS>(tl, &kk, &slot);
  const int ks = 8 * gh + kk;
  // value_mfma masks codes in place, so this token's code carries the factor
  // 16^(j & 1) (4-bit) or 4^(j & 3) (2-bit), j its nibble / crumb position
  // within a 16-bit half of its word; its probability takes the inverse (a
  // power of two: exact)
  const float inv_f = (TBQ || BITS == 3 || BITS == 8) ? 1.0f
                      : BITS == 4 ? ((tl & 1) ? 1.0f / 16 : 1.0f) : 1.0f / (float)(1 << (2 * (tl & 3)));
  for (int d = 0; d < NDG; ++d)
    for (int m = 0; m < G; ++m) {
      const float x = p[m] * vs[d];
      _Float16 hi, lo;
      split_half(x * inv_f, &hi, &lo);
      PLw.at(d, ks, 0, m, slot) = hi;
      if (HL == 1) PLw.at(d, ks, 0, G + m, slot) = lo;
      else PLw.at(d, ks, 1, m, slot) = lo;
      zacc[m][d] += BLOCK ? x : p[m] * vz[d];
    }
}

// O += p' . codes over the tile's value rows: 16 k-steps x 2 halves.
template <int G, int BITS, bool BLOCK, int HL, int NDG, bool TBQ = false, class PT>
__device__ __forceinline__ void value_mfma(const uint32_t (*vc)[2][BITS],
                                           const PT& PLw, int row, int gh,
                                           f4_t& o0, f4_t& o1, f4_t& o2, f4_t& o3,
                                           const uint32_t* lut = nullptr) {
  if constexpr (BITS == 4 || BITS == 2) {
    // one dword: 8 tokens (4-bit) or 16 tokens (2-bit), two per pr[] (one per
    // 16-bit half), masked in place in the low byte of each half: the code of
    // position j enters as n * 2^-24 times 16^(j & 1) or 4^(j & 3), which
    // stage_probs divided out of its probability.  Both channel halves of a
    // dword position are unpacked first; their MFMAs then alternate between
    // the four accumulators, so that no MFMA waits on the one issued just
    // before it (each accumulator still sums its terms in the same order).
    constexpr int NP = (BITS == 4) ? 4 : 8;
    constexpr int NL = HL + (TBQ ? 1 : 0);
    for (int gg = 0; gg < 2; ++gg) {
      for (int u = 0; u < BITS; ++u) {
        uint32_t pr[2][NP];
        uint32_t prl[2][4] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
        for (int hf = 0; hf < 2; ++hf) {
          const uint32_t x = vc[gg][hf][u];
          const uint32_t x8 = x >> 8;
          if (TBQ) {
            tbq4_levels(x, lut, pr[hf], prl[hf]);   // the levels themselves, no factors
          } else if (BITS == 4) {
            pr[hf][0] = x & 0x000F000Fu;
            pr[hf][1] = x & 0x00F000F0u;
            pr[hf][2] = x8 & 0x000F000Fu;
            pr[hf][3] = x8 & 0x00F000F0u;
          } else {
            for (int j = 0; j < 4; ++j) {
              pr[hf][j] = x & (0x00030003u << (2 * j));
              pr[hf][4 + j] = x8 & (0x00030003u << (2 * j));
            }
          }
        }
        for (int qp = 0; qp < NP / 4; ++qp)
          for (int hl = 0; hl < NL; ++hl)
            for (int q2 = 2 * qp; q2 < 2 * qp + 2; ++q2)
              for (int hf = 0; hf < 2; ++hf) {
                const int dg = NDG == 1 ? 0 : (gh + 2 * hf);   // the 32-dim slice of channel lane + 64 hf
                const int ks = 8 * gg + (NP / 2) * u + q2;    // k-step of pairs (2 q2, 2 q2 + 1)
                // TBQ: one more pass for the levels' lo halves against the hi
                // half of p' (rows G.. of a HL = 1 table carry p's lo half:
                // included)
                const bool lo_lv = TBQ && hl == HL;
                const h4_t av = PLw.h4(dg, ks, lo_lv ? 0 : hl, row);
                const h4_t b = lo_lv ? as_h4(prl[hf][2 * q2], prl[hf][2 * q2 + 1])
                                     : as_h4(pr[hf][2 * q2], pr[hf][2 * q2 + 1]);
                if (hf == 0) {
                  if (q2 & 1) o2 = mfma4(av, b, o2); else o0 = mfma4(av, b, o0);
                } else {
                  if (q2 & 1) o3 = mfma4(av, b, o3); else o1 = mfma4(av, b, o1);
                }
              }
      }
    }
    return;
  }
  // 8 bits: a dword holds tokens 4u .. 4u + 3 of the channel row, one byte
  // each: bytes 0 and 2 masked in place, bytes 1 and 3 shifted down (codes n
  // enter as n * 2^-24, no factors).  3 bits: the channel row's 32 tokens as
  // one 96-bit string, token t at bits 3t: k-step q takes tokens
  // 4q .. 4q + 3 in natural order.  As above, the MFMAs of two k-steps and
  // both channel halves alternate between the four accumulators.
  for (int gg = 0; gg < 2; ++gg) {
#pragma unroll
    for (int qp = 0; qp < 4; ++qp) {
      h4_t bv[2][2];
      for (int hf = 0; hf < 2; ++hf)
        for (int j = 0; j < 2; ++j) {
          const int q = 2 * qp + j;
          if constexpr (BITS == 8) {
            const uint32_t x = vc[gg][hf][q];
            bv[hf][j] = as_h4(x & 0x00FF00FFu, (x >> 8) & 0x00FF00FFu);
          } else {
            const uint32_t w[3] = {vc[gg][hf][0], vc[gg][hf][1], vc[gg][hf][2]};
            bv[hf][j] = codes3_b(w, q);
          }
        }
      for (int hl = 0; hl < HL; ++hl)
        for (int j = 0; j < 2; ++j)
          for (int hf = 0; hf < 2; ++hf) {
            const int dg = NDG == 1 ? 0 : (gh + 2 * hf);
            const h4_t av = PLw.h4(dg, 8 * gg + 2 * qp + j, hl, row);
            if (hf == 0) {
              if (j) o2 = mfma4(av, bv[hf][j], o2); else o0 = mfma4(av, bv[hf][j], o0);
            } else {
              if (j) o3 = mfma4(av, bv[hf][j], o3); else o1 = mfma4(av, bv[hf][j], o1);
            }
          }
    }
  }
}

// fp16 window values: O += p . V over tokens [base, base + nvalid) of the
// channel-major value ring, with p in natural token order in table 0 of PLw (k-step
// lane/4, slot lane%4).  Halves of tokens past the window are zeroed (stale
// ring slots may hold anything).
template <int HL, class PT>
__device__ __forceinline__ void window_value_mfma(const __half* vring, int64_t base, int nvalid,
                                                  const PT& PLw, int lane, int row,
                                                  f4_t& o0, f4_t& o1, f4_t& o2, f4_t& o3) {
  for (int kp = 0; kp < 8; ++kp) {    // 8 tokens (two k-steps) per load
    const int64_t t0 = base + 8 * kp;
    const int slot = (int)(t0 % kRing);
    for (int hf = 0; hf < 2; ++hf) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (8 * kp < nvalid) {
        x = *reinterpret_cast<const uint4*>(vring + (lane + 64 * hf) * kRing + slot);
        const int left = nvalid - 8 * kp;
        if (left < 8) {
          uint32_t xw[4] = {x.x, x.y, x.z, x.w};
          for (int k = 0; k < 4; ++k) {
            if (2 * k >= left) xw[k] = 0;
            else if (2 * k + 1 >= left) xw[k] &= 0xFFFFu;
          }
          x = make_uint4(xw[0], xw[1], xw[2], xw[3]);
        }
      }
      for (int hl = 0; hl < HL; ++hl) {
        const h4_t a0 = PLw.h4(0, 2 * kp, hl, row);
        const h4_t a1 = PLw.h4(0, 2 * kp + 1, hl, row);
        if (hf == 0) {
          o0 = mfma4(a0, as_h4(x.x, x.y), o0);
          o2 = mfma4(a1, as_h4(x.z, x.w), o2);
        } else {
          o1 = mfma4(a0, as_h4(x.x, x.y), o1);
          o3 = mfma4(a1, as_h4(x.z, x.w), o3);
        }
      }
    }
  }
}

// fp16 window probabilities in natural token order (k-step lane/4, slot lane%4).
template <int G, int HL, class PT>
__device__ __forceinline__ void stage_window_probs(const float* p, const PT& PLw,
                                                   int lane) {
  for (int m = 0; m < G; ++m) {
    _Float16 hi, lo;
    split_half(p[m], &hi, &lo);
    PLw.at(0, lane >> 2, 0, m, lane & 3) = hi;
    if (HL == 1) PLw.at(0, lane >> 2, 0, G + m, lane & 3) = lo;
    else PLw.at(0, lane >> 2, 1, m, lane & 3) = lo;
  }
}

// The wave's partial (m, l, o[128]) of each head into workspace slot `slot`.
// `scale` multiplies the MFMA sums (2^24 for code B operands, 1 for fp16),
// `add0` / `add1` are added to channels lane / 64 + lane of head m.
template <int G, int HL>
__device__ __forceinline__ void write_partial(const MfmaArgs& a, int b, int h, int64_t slot, int lane,
                                              const float* m_run, const float* l_acc,
                                              const f4_t& o0, const f4_t& o1, const f4_t& o2,
                                              const f4_t& o3, float scale, const float* add0,
                                              const float* add1) {
  for (int m = 0; m < G; ++m) {
    const float lsum = wave_sum64(l_acc[m]);
    float* rec = a.ws + (((int64_t)b * a.g.Hq + h * G + m) * a.n_slots + slot) * kPartial;
    const float a0 = (HL == 1) ? o0[m] + o0[G + m] + o2[m] + o2[G + m] : o0[m] + o2[m];
    const float a1 = (HL == 1) ? o1[m] + o1[G + m] + o3[m] + o3[G + m] : o1[m] + o3[m];
    rec[2 + lane] = a0 * scale + add0[m];
    rec[2 + 64 + lane] = a1 * scale + add1[m];
    if (lane == 0) {
      rec[0] = m_run[m];
      rec[1] = lsum;
    }
  }
}

// The partial of the 16x16x32 accumulators: hi + lo rows (lanes l and
// l + 16) times `scale`, plus add[m][cb / 2] (add[m][0] for every channel
// when NDG is 1).
template <int G, int NDG>
__device__ __forceinline__ void write_partial16(const MfmaArgs& a, int b, int h, int64_t slot, int lane,
                                                const float* m_run, const float* l_acc, const f4_t* acc,
                                                float scale, const float (*add)[NDG]) {
  for (int m = 0; m < G; ++m) {
    const float lsum = wave_sum64(l_acc[m]);
    float* rec = a.ws + (((int64_t)b * a.g.Hq + h * G + m) * a.n_slots + slot) * kPartial;
    for (int c = 0; c < 8; ++c) {
      const float v = acc[c][m] + __shfl_xor(acc[c][m], 16);
      if (lane < 16) rec[2 + 16 * c + lane] = v * scale + add[m][NDG == 1 ? 0 : c >> 1];
    }
    if (lane == 0) {
      rec[0] = m_run[m];
      rec[1] = lsum;
    }
  }
}

// An empty partial (m = -inf, l = 0, o = 0) for every head in `slot`.
template <int G>
__device__ __forceinline__ void write_empty(const MfmaArgs& a, int b, int h, int64_t slot, int lane) {
  for (int m = 0; m < G; ++m) {
    float* rec = a.ws + (((int64_t)b * a.g.Hq + h * G + m) * a.n_slots + slot) * kPartial;
    rec[2 + lane] = 0.0f;
    rec[2 + 64 + lane] = 0.0f;
    if (lane == 0) {
      rec[0] = -INFINITY;
      rec[1] = 0.0f;
    }
  }
}

// The query of (sequence b, kv head h) for one wave: qsw[m][c] = fp32 q of
// head h G + m, rotated by the normalized Hadamard transform if asked, times
// scale_log2.  Returns max |qsw| over the wave's heads.
template <int G>
__device__ __forceinline__ float wave_query(const MfmaArgs& a, int b, int h, bool rotate,
                                            float (*qsw)[kD], int lane) {
  for (int e = lane; e < G * kD; e += 64)
    qsw[e / kD][e % kD] = __half2float(a.q[((int64_t)b * a.g.Hq + h * G + e / kD) * kD + e % kD]);
  wave_sync();
  if (rotate) fwht128_rows_wave(&qsw[0][0], G, lane, a.g.sign_in, a.g.sign_out, a.g.hsigned);
  float mx = 0.0f;
  for (int e = lane; e < G * kD; e += 64) {
    const float v = qsw[e / kD][e % kD] * a.scale_log2;
    qsw[e / kD][e % kD] = v;
    mx = fmaxf(mx, fabsf(v));
  }
  wave_sync();
  return wave_max64(mx);
}

}  // namespace
}  // namespace kvq
