// Split-K decode for KIVI caches whose keys are stored before RoPE.
//
// Sources cited here:
//   [troisinh] "KV Cache Quantization — Nén cache INT4/INT3, mở khóa
//              ultra-long context" (troisinh.com).
//   [nalar]    "Kuantisasi KV Cache dengan Error Budget yang Eksplisit"
//              (nalar.dev).
//
// Keys are quantized per channel before the rotary embedding and rotated at
// attention time ([troisinh] "Ý tưởng cốt lõi", "RoPE — Cái bẫy tinh vi";
// "Tại sao nó hoạt động", item 3).  Split-half RoPE rotates each channel pair
// (j, j + 64) of the key at position t by t * theta_j.  With the query at
// q_pos rotated the same way, the score of token t is
//     s_t = (R(q_pos) q) . (R(t) k_t) = (R(-t0) R(q_pos) q) . (R(t - t0) k_t)
// for any t0.  Here t0 is the first token of the key's 32-token group: the
// query is rotated once per group, every key by its offset d = t - t0 < 32,
// with cos / sin from rows 0..31 of the cache's RoPE table (fp64-derived).
//
// Precision decides the arithmetic.  Per-channel outliers (the reason keys
// are quantized per channel) make single terms of the score large, so the
// rotated key and the query enter the contraction in fp32: the key is
// dequantized and rotated in fp32 on the VALU (x = n s + z, then the 2 x 2
// rotation of each pair) and contracted on the fp32 4x4x1 MFMA (16 blocks;
// lane 4b + n of block b is token column n, rows are query heads, one
// channel per instruction).  An fp16 key or query would put a 2^-11 relative
// error on an outlier channel's term ([nalar] "Error pada key mengubah input
// softmax").
//
// Work of a wave on one 64-token tile (two groups).  For the key side lane L
// is block b = L / 4, column n = L % 4 of the MFMA; it owns the channel-pair
// quarter kq = b % 4 (pairs [16 kq, 16 kq + 16), i.e. channels
// 16 kq .. 16 kq + 15 and 64 + 16 kq ..) and the token offsets tau and
// tau + 16 of each group, tau = 4 (L / 16) + L % 4.  Its offsets never
// change, so the cos / sin it needs (2 offsets x 16 pairs) stay in registers
// for the whole kernel.  As the MFMA's A operand it supplies query head
// L % 4.  Each group's scores come out split by quarter and are summed over
// the four quarters inside 16-lane rows (DPP); the four (group, offset)
// results of a lane then collapse to one token, t(L) = 16 kq + tau, which is
// the lane's token for the softmax and the value side (decode_common.h).
// Codes enter the dequantization unconverted: a nibble or crumb masked into
// a 16-bit half is the fp16 subnormal n 2^-24 (times 16^k or 4^k for its
// place), and v_fma_mix forms n s + z from it, the per-channel scale
// pre-multiplied by 2^24 / 16^k (or 4^k), with one rounding of an exact
// product: the same value the dequantizer stores.
#include "decode_common.h"

namespace kvq {
namespace {

__device__ __forceinline__ f4_t mfma1(float x, float y, f4_t c) {
  return __builtin_amdgcn_mfma_f32_4x4x1f32(x, y, c, 0, 0, 0);
}

// Sum over the four channel quarters of a 16-lane row (lanes 4 kq + n).
__device__ __forceinline__ float quarter_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, true));   // row_ror:4
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, true));   // row_ror:8
  return v;
}

// Per-wave LDS tables of one tile (floats):
//   QB  the group-anchored query u = R(-t0) R(q_pos) q of both groups:
//       [group][head][quarter][pair in quarter](u_j, u_{j+64}); heads 144
//       floats apart and quarters 36, so that the sixteen (head, quarter)
//       runs one read instruction gathers fall in different LDS banks.
//   SZ  the key (scale, zero) of both groups as (s', z) fp32 per channel, s'
//       pre-multiplied by the code's place factor: [group][quarter][pair in
//       quarter](s'_j, z_j, s'_{j+64}, z_{j+64}); quarters 68 floats apart.
constexpr int kQbQuarter = 36, kQbHead = 4 * kQbQuarter, kQbGroup = 4 * kQbHead;
constexpr int kSzQuarter = 68, kSzGroup = 4 * kSzQuarter;

// Place factor of channel ch's code in the masked 16-bit half (2^24 for the
// subnormal, divided by the code's position weight within its half).
template <int BITS>
__device__ __forceinline__ float code_place_scale(int ch) {
  if (BITS == 4) return (ch & 1) ? 1048576.0f : 16777216.0f;
  return 16777216.0f / (float)(1 << (2 * (ch & 3)));
}

// Masked word k of a code dword: two codes in the low bits of its 16-bit
// halves.  4 bits (w covers channels c0 .. c0 + 7, nibble p at bits 4p):
// k = 0: (c0, c0 + 4), 1: (c0 + 1, c0 + 5) x16, 2: (c0 + 2, c0 + 6),
// 3: (c0 + 3, c0 + 7) x16, as (lo half, hi half).  2 bits (w covers
// c0 .. c0 + 15, crumb p at bits 2p): k < 4: (c0 + k, c0 + 8 + k) x4^k,
// k >= 4: (c0 + k, c0 + 8 + k) x4^(k - 4).
template <int BITS>
__device__ __forceinline__ uint32_t mask_code(uint32_t w, int k) {
  if (BITS == 4) return ((k & 2) ? (w >> 8) : w) & ((k & 1) ? 0x00F000F0u : 0x000F000Fu);
  return ((k & 4) ? (w >> 8) : w) & (0x00030003u << (2 * (k & 3)));
}

__device__ __forceinline__ float half_lo(uint32_t m) {
  return (float)__builtin_bit_cast(h2_t, m).x;
}
__device__ __forceinline__ float half_hi(uint32_t m) {
  return (float)__builtin_bit_cast(h2_t, m).y;
}


// A 64-bit LDS store of (x, y) written as asm.  The stores that build the
// per-tile tables run while the stage's global-to-LDS copies are in flight;
// the compiler loses track of which LDS array such a store's address points
// into and would wait for every copy before it.  The asm carries no memory
// operand for that wait to key on; its "memory" clobber keeps it ordered
// with the table's later reads (one wave's LDS operations execute in order).
__device__ __forceinline__ void lds_store2(float* p, float x, float y) {
  const u2v_t v = {__float_as_uint(x), __float_as_uint(y)};
  asm volatile("ds_write_b64 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}

// The lane's key codes from the key half of the stage, read in one asm block
// that ends with its own LDS wait.  Plain reads would make the compiler wait
// first for every global-to-LDS copy in flight (it cannot tell the two stage
// halves apart), the next tile's value copies included.  kc[gg][s][...]:
// token tau + 16 s of group gg, the quarter's low then high channels.
//   4 bits: byte 8 kq .. of the row (chunk kq / 2 at 8 (kq % 2)) and 32 + 8 kq ..
//   2 bits: byte 4 kq .. (chunk 0) and 16 + 4 kq .. (chunk 1)
template <int BITS>
__device__ __forceinline__ void read_key_codes(const uint8_t* stk, int kq, int tau, uint32_t (*kc)[2][4]) {
  if (BITS == 4) {
    const uint32_t base = lds_addr(stk) + (kq >> 1) * 512 + 16 * tau + 8 * (kq & 1);
    u2v_t r[8];
    asm volatile(
        "ds_read_b64 %0, %8\n\t"
        "ds_read_b64 %1, %8 offset:1024\n\t"
        "ds_read_b64 %2, %8 offset:256\n\t"
        "ds_read_b64 %3, %8 offset:1280\n\t"
        "ds_read_b64 %4, %8 offset:2048\n\t"
        "ds_read_b64 %5, %8 offset:3072\n\t"
        "ds_read_b64 %6, %8 offset:2304\n\t"
        "ds_read_b64 %7, %8 offset:3328\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=v"(r[0]), "=v"(r[1]), "=v"(r[2]), "=v"(r[3]), "=v"(r[4]), "=v"(r[5]), "=v"(r[6]), "=v"(r[7])
        : "v"(base)
        : "memory");
    // r[4 gg + 2 s + hf]: group gg (+2048), token offset s (+256), half hf (+1024)
    for (int gg = 0; gg < 2; ++gg)
      for (int ss = 0; ss < 2; ++ss)
        for (int hf = 0; hf < 2; ++hf) {
          kc[gg][ss][2 * hf] = r[4 * gg + 2 * ss + hf].x;
          kc[gg][ss][2 * hf + 1] = r[4 * gg + 2 * ss + hf].y;
        }
  } else {
    const uint32_t base = lds_addr(stk) + 16 * tau + 4 * kq;
    uint32_t r[8];
    asm volatile(
        "ds_read_b32 %0, %8\n\t"
        "ds_read_b32 %1, %8 offset:512\n\t"
        "ds_read_b32 %2, %8 offset:256\n\t"
        "ds_read_b32 %3, %8 offset:768\n\t"
        "ds_read_b32 %4, %8 offset:1024\n\t"
        "ds_read_b32 %5, %8 offset:1536\n\t"
        "ds_read_b32 %6, %8 offset:1280\n\t"
        "ds_read_b32 %7, %8 offset:1792\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=v"(r[0]), "=v"(r[1]), "=v"(r[2]), "=v"(r[3]), "=v"(r[4]), "=v"(r[5]), "=v"(r[6]), "=v"(r[7])
        : "v"(base)
        : "memory");
    // r[4 gg + 2 s + hf]: group gg (+1024), token offset s (+256), half hf (+512)
    for (int gg = 0; gg < 2; ++gg)
      for (int ss = 0; ss < 2; ++ss)
        for (int hf = 0; hf < 2; ++hf) kc[gg][ss][hf] = r[4 * gg + 2 * ss + hf];
  }
}

// The lane's value rows (channels lane and 64 + lane of both groups) from the
// value half of the stage, in one asm block with its own LDS wait (as above).
// Value tiles are channel-major, 4 BITS bytes a row.
template <int BITS>
__device__ __forceinline__ void read_value_codes(const uint8_t* stv, int lane, uint32_t (*vc)[2][BITS]) {
  if (BITS == 4) {
    const uint32_t base = lds_addr(stv) + 16 * lane;
    u4v_t r[4];
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %4 offset:1024\n\t"
        "ds_read_b128 %2, %4 offset:2048\n\t"
        "ds_read_b128 %3, %4 offset:3072\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=v"(r[0]), "=v"(r[1]), "=v"(r[2]), "=v"(r[3])
        : "v"(base)
        : "memory");
    // r[2 gg + hf]: group gg (+2048), channel half hf (+1024)
    for (int gg = 0; gg < 2; ++gg)
      for (int hf = 0; hf < 2; ++hf)
        for (int u = 0; u < 4; ++u) vc[gg][hf][u] = r[2 * gg + hf][u];
  } else {
    const uint32_t base = lds_addr(stv) + 8 * lane;
    u2v_t r[4];
    asm volatile(
        "ds_read_b64 %0, %4\n\t"
        "ds_read_b64 %1, %4 offset:512\n\t"
        "ds_read_b64 %2, %4 offset:1024\n\t"
        "ds_read_b64 %3, %4 offset:1536\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=v"(r[0]), "=v"(r[1]), "=v"(r[2]), "=v"(r[3])
        : "v"(base)
        : "memory");
    // r[2 gg + hf]: group gg (+1024), channel half hf (+512)
    for (int gg = 0; gg < 2; ++gg)
      for (int hf = 0; hf < 2; ++hf) {
        vc[gg][hf][0] = r[2 * gg + hf].x;
        vc[gg][hf][1] = r[2 * gg + hf].y;
      }
  }
}

// The lane's code dwords for the B operands, vd[gg][cb] (channel 16 cb +
// lane % 16, lane group lane / 16), and the A operands of key group 0,
// a0[dg], in one asm block with its own LDS wait (as read_value_codes).
// 4 bits: 16-byte rows, dword lane / 16; 2 bits: 8-byte rows, dword
// lane / 32.  pvb: the lane's A address for (dg, gg) = (0, 0); (dg, gg) is
// 1152 dg + 576 gg bytes further.
template <int BITS>
__device__ __forceinline__ void read_value_codes16(const uint8_t* stv, uint32_t pvb, int lane, uint32_t (*vd)[8],
                                                   u4v_t* a0) {
  u2v_t r[8];
  if (BITS == 4) {
    const uint32_t base = lds_addr(stv) + 16 * (lane & 15) + 4 * (lane >> 4);
    asm volatile(
        "ds_read2st64_b32 %0, %12 offset1:1\n\t"
        "ds_read2st64_b32 %1, %12 offset0:2 offset1:3\n\t"
        "ds_read2st64_b32 %2, %12 offset0:4 offset1:5\n\t"
        "ds_read2st64_b32 %3, %12 offset0:6 offset1:7\n\t"
        "ds_read2st64_b32 %4, %12 offset0:8 offset1:9\n\t"
        "ds_read2st64_b32 %5, %12 offset0:10 offset1:11\n\t"
        "ds_read2st64_b32 %6, %12 offset0:12 offset1:13\n\t"
        "ds_read2st64_b32 %7, %12 offset0:14 offset1:15\n\t"
        "ds_read_b128 %8, %13\n\t"
        "ds_read_b128 %9, %13 offset:1152\n\t"
        "ds_read_b128 %10, %13 offset:2304\n\t"
        "ds_read_b128 %11, %13 offset:3456\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=v"(r[0]), "=v"(r[1]), "=v"(r[2]), "=v"(r[3]), "=v"(r[4]), "=v"(r[5]), "=v"(r[6]), "=v"(r[7]),
          "=v"(a0[0]), "=v"(a0[1]), "=v"(a0[2]), "=v"(a0[3])
        : "v"(base), "v"(pvb)
        : "memory");
  } else {
    const uint32_t b0 = lds_addr(stv) + 8 * (lane & 15) + 4 * (lane >> 5), b1 = b0 + 1024;
    asm volatile(
        "ds_read2_b32 %0, %12 offset1:32\n\t"
        "ds_read2_b32 %1, %12 offset0:64 offset1:96\n\t"
        "ds_read2_b32 %2, %12 offset0:128 offset1:160\n\t"
        "ds_read2_b32 %3, %12 offset0:192 offset1:224\n\t"
        "ds_read2_b32 %4, %13 offset1:32\n\t"
        "ds_read2_b32 %5, %13 offset0:64 offset1:96\n\t"
        "ds_read2_b32 %6, %13 offset0:128 offset1:160\n\t"
        "ds_read2_b32 %7, %13 offset0:192 offset1:224\n\t"
        "ds_read_b128 %8, %14\n\t"
        "ds_read_b128 %9, %14 offset:1152\n\t"
        "ds_read_b128 %10, %14 offset:2304\n\t"
        "ds_read_b128 %11, %14 offset:3456\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=v"(r[0]), "=v"(r[1]), "=v"(r[2]), "=v"(r[3]), "=v"(r[4]), "=v"(r[5]), "=v"(r[6]), "=v"(r[7]),
          "=v"(a0[0]), "=v"(a0[1]), "=v"(a0[2]), "=v"(a0[3])
        : "v"(b0), "v"(b1), "v"(pvb)
        : "memory");
  }
  // r[4 gg + c]: channel blocks 2c (.x) and 2c + 1 (.y)
  for (int gg = 0; gg < 2; ++gg)
    for (int c = 0; c < 4; ++c) {
      vd[gg][2 * c] = r[4 * gg + c].x;
      vd[gg][2 * c + 1] = r[4 * gg + c].y;
    }
}

template <int G, int BITS>
__global__ __launch_bounds__(256, 2) void decode_rope_kernel(MfmaArgs a) {
  constexpr int HL = (G <= 2) ? 1 : 2;   // value-side MFMAs per k-step (hi/lo of p')
  constexpr int NDG = 4;                 // value scale groups per token
  constexpr int TB = 512 * BITS;         // tile bytes
  constexpr int NW = BITS == 4 ? 2 : 1;  // code dwords per quarter-half of a key row
  constexpr bool V16 = G == 4;           // value side on the 16x16x32 MFMA
  const Geom& g = a.g;
  __shared__ __attribute__((aligned(16))) float QB[4][2 * kQbGroup];
  __shared__ __attribute__((aligned(16))) float SZ[4][2 * kSzGroup];
  using PTab = ATab<HL, 16, G == 4, G == 4>;
  // p' tables: NDG ATab tables, or (four heads) the 16x16x32 A operands of
  // 4 scale groups x 2 key groups (the window's table 0 overlays them)
  __shared__ __attribute__((aligned(16))) _Float16 PL[4][V16 ? v16_halves(NDG) : NDG * PTab::T];
  // the tile stage, keys and values apart: the value half of tile N is still
  // read while the key half of tile N + 1 is in flight into the other array
  __shared__ __attribute__((aligned(16))) uint8_t STK[4][2 * TB];
  __shared__ __attribute__((aligned(16))) uint8_t STV[4][2 * TB];

  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index is uniform: read it into a scalar register, so that the
  // tile walk and its addresses stay on the scalar unit
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kq = (lane >> 2) & 3;                    // channel-pair quarter (key side)
  const int tau = 4 * (lane >> 4) + (lane & 3);      // token offset slot (key side)
  const int hq_a = lane & 3;                         // query head this lane feeds to the MFMA
  const int tok = 16 * kq + tau;                     // the lane's tile token after the scores
  const int tl = tok & 31, gh = tok >> 5;
  const float* rope_tab = reinterpret_cast<const float*>(a.p.p[KVQ_PLANE_ROPE]);
  float* QBw = QB[w];
  float* SZw = SZ[w];
  const PTab PLw{PL[w]};
  uint8_t* stk = STK[w];
  uint8_t* stv = STV[w];

  // cos / sin of offsets tau (A) and tau + 16 (B) for the quarter's pairs
  // (rows 0..31 of the RoPE table: the plane always holds at least 32 rows)
  float cA[16], sA[16], cB[16], sB[16];
  for (int i = 0; i < 16; i += 2) {
    const float4 ra = *reinterpret_cast<const float4*>(rope_tab + tau * 128 + 2 * (16 * kq + i));
    const float4 rb = *reinterpret_cast<const float4*>(rope_tab + (tau + 16) * 128 + 2 * (16 * kq + i));
    cA[i] = ra.x; sA[i] = ra.y; cA[i + 1] = ra.z; sA[i + 1] = ra.w;
    cB[i] = rb.x; sB[i] = rb.y; cB[i + 1] = rb.z; sB[i + 1] = rb.w;
  }
  for (int e = lane; e < (int)(sizeof(PL[0]) / 2); e += 64) PL[w][e] = (_Float16)0.0f;
  for (int e = lane; e < 2 * kQbGroup; e += 64) QBw[e] = 0.0f;   // heads >= G stay zero
  wave_sync();

  float qx[G], qy[G];   // R(q_pos) q, scaled: pair `lane` (channels lane, lane + 64) of every head
  // the query of (b, h) at q_pos (fp64 angles); lane j takes channel pair j
  auto load_query = [&](int b, int h) {
    const double theta = pow((double)g.rope_theta, -2.0 * (double)lane / 128.0);
    const double ang = (double)a.q_pos * theta;
    const float c = (float)cos(ang), s = (float)sin(ang);
    for (int m = 0; m < G; ++m) {
      const int64_t qb = ((int64_t)b * g.Hq + h * G + m) * kD;
      const float x = __half2float(a.q[qb + lane]), y = __half2float(a.q[qb + lane + 64]);
      qx[m] = (x * c - y * s) * a.scale_log2;
      qy[m] = (x * s + y * c) * a.scale_log2;
    }
  };
  // QB of both groups from the RoPE rows of their first tokens (lane j holds
  // the (cos, sin) of pair j): u_j = x c + y s, u_{j+64} = y c - x s
  auto build_query = [&](const float2* rows) {
    const int q4 = lane >> 4, pi = lane & 15;
    for (int gg = 0; gg < 2; ++gg) {
      const float2 cs = rows[gg];
      for (int m = 0; m < G; ++m) {
        const float x = qx[m], y = qy[m];
        lds_store2(&QBw[gg * kQbGroup + m * kQbHead + q4 * kQbQuarter + 2 * pi], x * cs.x + y * cs.y,
                   y * cs.x - x * cs.y);
      }
    }
  };
  // this lane's query values for the key side: head hq_a, the quarter's
  // pairs (read pair by pair)
  auto query_of = [&](int gg) -> const float* { return &QBw[gg * kQbGroup + hq_a * kQbHead + kq * kQbQuarter]; };

  float m_run[G], l_acc[G];
  float zacc[G][NDG];
  f4_t o0, o1, o2, o3;
  f4_t acc16[8];   // V16: channel blocks 0..7
  auto reset = [&]() {
    for (int m = 0; m < G; ++m) {
      m_run[m] = -INFINITY;
      l_acc[m] = 0.0f;
      for (int d = 0; d < NDG; ++d) zacc[m][d] = 0.0f;
    }
    o0 = f4_t{0, 0, 0, 0}; o1 = o0; o2 = o0; o3 = o0;
    if (V16)
      for (int c = 0; c < 8; ++c) acc16[c] = f4_t{0, 0, 0, 0};
  };

  reset();

  // Scores of one group: the quarter's rotated keys of tokens tau (xa, ya:
  // channels j and j + 64 of pair i) and tau + 16 (xb, yb) against u, four
  // MFMA chains; returns the quarter-summed scores of both tokens.
  auto rotate_contract = [&](int i, float xa, float ya, float xb, float yb, const float* uq, f4_t* acc) {
    const float2 u = *reinterpret_cast<const float2*>(uq + 2 * i);
    const float rla = xa * cA[i] - ya * sA[i], rha = xa * sA[i] + ya * cA[i];
    const float rlb = xb * cB[i] - yb * sB[i], rhb = xb * sB[i] + yb * cB[i];
    acc[0] = mfma1(u.x, rla, acc[0]);
    acc[1] = mfma1(u.y, rha, acc[1]);
    acc[2] = mfma1(u.x, rlb, acc[2]);
    acc[3] = mfma1(u.y, rhb, acc[3]);
  };
  // The quarter-summed scores of the group's two tokens, folded into this
  // lane's token: group gg holds the lane's token when kq / 2 == gg, offset
  // tau + 16 (kq odd) or tau (kq even).  Named values, not an array indexed
  // by the lane, so that the selection stays in registers.
  const bool odd_kq = (kq & 1) != 0;
  auto finish_scores = [&](const f4_t* acc, int gg, float* sel) {
    for (int m = 0; m < G; ++m) {
      const float sa = quarter_sum(acc[0][m] + acc[1][m]);
      const float sb = quarter_sum(acc[2][m] + acc[3][m]);
      const float v = odd_kq ? sb : sa;
      if (gg == 0) sel[m] = v;
      else if (kq >= 2) sel[m] = v;
    }
  };

  if (blockIdx.x < a.wins) {
    // ================= fp16 window of one pair: tokens [Tq, length), wave w takes tile w
    const int64_t pair = blockIdx.x;
    const int b = (int)(pair / g.Hkv), h = (int)(pair % g.Hkv);
    load_query(b, h);
    const int64_t base = g.Tq + 64 * (int64_t)w;
    if (base < g.length) {
      const int nvalid = (int)min((int64_t)64, g.length - base);
      float2 rows[2];
      rows[0] = *reinterpret_cast<const float2*>(rope_tab + base * 128 + 2 * lane);
      rows[1] = *reinterpret_cast<const float2*>(rope_tab + (nvalid > 32 ? base + 32 : base) * 128 + 2 * lane);
      build_query(rows);
      wave_sync();
      const __half* kring = reinterpret_cast<const __half*>(a.p.p[KVQ_PLANE_K_WIN]) + pair * kRing * kD;
      float sel[4];
      for (int gg = 0; gg < 2; ++gg) {
        const float* uq = query_of(gg);
        // rows of tokens tau and tau + 16 of this group; tokens past the
        // window read as zero
        const int ta = 32 * gg + tau, tb = ta + 16;
        uint4 ka[4], kb[4];
        for (int k = 0; k < 4; ++k) {
          const int off = (k >> 1) * 64 + 16 * kq + 8 * (k & 1);   // channels 16 kq + 8 (k & 1) (+64)
          ka[k] = ta < nvalid ? *reinterpret_cast<const uint4*>(kring + ((base + ta) % kRing) * kD + off)
                              : make_uint4(0, 0, 0, 0);
          kb[k] = tb < nvalid ? *reinterpret_cast<const uint4*>(kring + ((base + tb) % kRing) * kD + off)
                              : make_uint4(0, 0, 0, 0);
        }
        f4_t acc[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
        for (int i = 0; i < 16; ++i) {
          const __half* la = reinterpret_cast<const __half*>(&ka[i >> 3]);
          const __half* ha = reinterpret_cast<const __half*>(&ka[2 + (i >> 3)]);
          const __half* lb = reinterpret_cast<const __half*>(&kb[i >> 3]);
          const __half* hb = reinterpret_cast<const __half*>(&kb[2 + (i >> 3)]);
          rotate_contract(i, __half2float(la[i & 7]), __half2float(ha[i & 7]), __half2float(lb[i & 7]),
                          __half2float(hb[i & 7]), uq, acc);
        }
        finish_scores(acc, gg, sel);
      }
      const bool tok_ok = tok < nvalid;
      float p[G];
      for (int m = 0; m < G; ++m) {
        const float s = tok_ok ? sel[m] : -INFINITY;
        p[m] = softmax_step<G, HL, NDG>(m, s, tok_ok, m_run, l_acc, o0, o1, o2, o3, zacc);
      }
      // probabilities in natural token order (k-step tok / 4, slot tok % 4)
      for (int m = 0; m < G; ++m) {
        _Float16 hi, lo;
        split_half(p[m], &hi, &lo);
        PLw.at(0, tok >> 2, 0, m, tok & 3) = hi;
        if (HL == 1) PLw.at(0, tok >> 2, 0, G + m, tok & 3) = lo;
        else PLw.at(0, tok >> 2, 1, m, tok & 3) = lo;
      }
      wave_sync();
      const __half* vring = reinterpret_cast<const __half*>(a.p.p[KVQ_PLANE_V_WIN]) + pair * kD * kRing;
      window_value_mfma<HL>(vring, base, nvalid, PLw, lane, lane & 3, o0, o1, o2, o3);
    }
    const float zero[G] = {};
    write_partial<G, HL>(a, b, h, a.win_slot + w, lane, m_run, l_acc, o0, o1, o2, o3, 1.0f, zero, zero);
    return;
  }

  // ================= quantized tiles: this wave's assignments (see MfmaArgs)
  const int64_t rank = (int64_t)w * a.pwgs + (blockIdx.x - a.wins);
  if (rank >= a.pairs * a.team) return;

  const uint8_t* kplane = a.p.p[a.hi_tier ? KVQ_PLANE_K_HI : KVQ_PLANE_K_LO];
  const uint8_t* vplane = a.p.p[a.hi_tier ? KVQ_PLANE_V_HI : KVQ_PLANE_V_LO];
  const int64_t slots = a.hi_tier ? g.hi_slots : g.gmax;
  const bool ring = slots != g.gmax;

  // Metadata of a tile into registers: this lane's four key channels
  // 4 (lane % 32) .. of group lane / 32 (as stored: fp16 (s, z) words), the
  // value (s, z) of its token t(lane), and the RoPE rows of the two groups'
  // first tokens (pair `lane`).  A second group past the tile's tokens reads
  // the first group's (never used, always inside the data).
  struct Meta {
    uint4 km;
    uint4 vm;
    float2 rows[2];
  };
  auto meta_fetch = [&](Meta& mt, const TilePos& tp, int64_t pr) {
    const bool g1 = tp.nvalid > 32;
    const int64_t kg = tp.grp0 + ((lane >> 5) && g1 ? 1 : 0);
    const int64_t vg = tp.grp0 + (gh && g1 ? 1 : 0);
    mt.km = *reinterpret_cast<const uint4*>(a.p.p[KVQ_PLANE_K_META] + (pr * g.gmax + kg) * 512 + 16 * (lane & 31));
    mt.vm = *reinterpret_cast<const uint4*>(a.p.p[KVQ_PLANE_V_META] + (pr * g.gmax + vg) * 512 + 16 * tl);
    mt.rows[0] = *reinterpret_cast<const float2*>(rope_tab + tp.base * 128 + 2 * lane);
    mt.rows[1] = *reinterpret_cast<const float2*>(rope_tab + (g1 ? tp.base + 32 : tp.base) * 128 + 2 * lane);
  };
  // global-to-LDS copies of a tile's key tiles (or value tiles) into the
  // wave's stage: BITS 16-byte loads per lane (two groups, TB / 1024 runs of
  // 1 KiB each)
  auto stage_half = [&](uint8_t* dst, const uint8_t* plane, const TilePos& tp, int64_t pr) {
    const bool g1 = tp.nvalid > 32;
    const uint8_t* src = plane + pr * slots * TB;
    for (int gg = 0; gg < 2; ++gg) {
      const int64_t slot = (gg && g1) ? tp.s1 : tp.s0;
      for (int k = 0; k * 1024 < TB; ++k)
        lds_dma16(src + slot * TB + k * 1024 + 16 * lane, dst + gg * TB + k * 1024);
    }
  };

  TileCursor cs;
  cursor_start(a, rank, cs, lane);
  int64_t cur_pair = cs.pair, cur_k = cs.k;
  TilePos cur_pos, nxt_pos;
  tile_at(a, cs.t, slots, ring, cur_pos);
  Meta nxt;
  stage_half(stk, kplane, cur_pos, cur_pair);
  meta_fetch(nxt, cur_pos, cur_pair);

  int64_t pair = -1, pk = 0;
  int pb = 0, ph = 0;
  // this member's partial of `pair`
  auto flush = [&]() {
    if constexpr (V16) {
      // codes entered as n 2^-24; the zero-point sum of each scale group
      float zsum[G][NDG];
      for (int m = 0; m < G; ++m)
        for (int d = 0; d < NDG; ++d) zsum[m][d] = wave_sum64(zacc[m][d]);
      write_partial16<G, NDG>(a, pb, ph, a.slot_base + pk, lane, m_run, l_acc, acc16, 16777216.0f, zsum);
      reset();
      return;
    }
    float add0[G], add1[G];
    for (int m = 0; m < G; ++m) {
      float zsum[NDG];
      for (int d = 0; d < NDG; ++d) zsum[d] = wave_sum64(zacc[m][d]);
      add0[m] = zsum[lane >> 5];
      add1[m] = zsum[(lane >> 5) + 2];
    }
    write_partial<G, HL>(a, pb, ph, a.slot_base + pk, lane, m_run, l_acc, o0, o1, o2, o3, 16777216.0f,
                         add0, add1);
    reset();
  };

  // Memory pipeline of a tile N (tile codes go to the wave's stage, the
  // metadata to registers):
  //   top:         wait for everything in flight (tile N's key copies and
  //                metadata, a chunk claim); issue a chunk claim if one is
  //                due, then N's value copies; read the key codes; issue
  //                tile N + 1's key copies and metadata
  //   value phase: wait for everything again (the claim and N's value
  //                copies, issued a key phase ago, then N + 1's key copies
  //                and metadata), read the value codes
  // The value copies thus have the key phase to land, the key copies a whole
  // tile, and every wait the compiler adds by itself (for the metadata
  // registers, the query, the claim's result) falls where it has nothing
  // younger to drain.
  bool fresh = true;   // the current tile opens an assignment
  for (;;) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (fresh) {
      pair = cur_pair;
      pk = cur_k;
      pb = (int)(pair / g.Hkv);
      ph = (int)(pair % g.Hkv);
      load_query(pb, ph);
    }
    const Meta cur = nxt;
    // the copy of the metadata registers is made here, before the value
    // copies go out (the compiler waits for the metadata loads to make it)
    asm volatile("" ::"v"(cur.km.x), "v"(cur.km.y), "v"(cur.km.z), "v"(cur.km.w), "v"(cur.vm.x), "v"(cur.vm.y),
                 "v"(cur.vm.z), "v"(cur.vm.w), "v"(cur.rows[0].x), "v"(cur.rows[0].y), "v"(cur.rows[1].x),
                 "v"(cur.rows[1].y));
    bool ends = false;
    bool need_claim = false;
    const bool more = cursor_next_deferred(a, cs, lane, &ends, &need_claim);
    if (more) tile_at(a, cs.t, slots, ring, nxt_pos);
    // the chunk claim the cursor asked for goes out first: its result is
    // read at the top of a later tile, and the waits before then (the value
    // phase's) come a key phase after it
    if (need_claim) cs.pend = claim_issue(a.ctr + cs.pair * kCounterStride, lane);
    if (more) meta_fetch(nxt, nxt_pos, cs.pair);
    stage_half(stv, vplane, cur_pos, cur_pair);
    // key codes: tokens tau (a) and tau + 16 (b) of both groups, the
    // quarter's low channels then its high channels (NW dwords each)
    uint32_t kc[2][2][4];
    read_key_codes<BITS>(stk, kq, tau, kc);
    if (more) stage_half(stk, kplane, nxt_pos, cs.pair);

    // SZ of both groups: this lane's four channels (group lane / 32)
    {
      const uint32_t mw[4] = {cur.km.x, cur.km.y, cur.km.z, cur.km.w};
      const int kg = lane >> 5;
      for (int e = 0; e < 4; ++e) {
        const int ch = 4 * (lane & 31) + e, j = ch & 63;
        // the place factor depends on ch % 4 = e only
        const float s = half_bits_to_float((uint16_t)(mw[e] & 0xFFFF)) * code_place_scale<BITS>(e);
        const float z = half_bits_to_float((uint16_t)(mw[e] >> 16));
        lds_store2(&SZw[kg * kSzGroup + (j >> 4) * kSzQuarter + 4 * (j & 15) + 2 * (ch >> 6)], s, z);
      }
    }
    build_query(cur.rows);
    const uint4 cur_vm = cur.vm;
    wave_sync();

    // ---------------- scores
    float sel[4];
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      const float* uq = query_of(gg);
      f4_t acc[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
      const float* szq = &SZw[gg * kSzGroup + kq * kSzQuarter];
      // the two pairs whose codes share a masked word (lo / hi halves) back to back
      auto two_pairs = [&](int i0, int i1, uint32_t la, uint32_t ha, uint32_t lb, uint32_t hb) {
        const float4 s0 = *reinterpret_cast<const float4*>(szq + 4 * i0);
        const float4 s1 = *reinterpret_cast<const float4*>(szq + 4 * i1);
        // x = n s + z with one rounding (the product is exact)
        rotate_contract(i0, __builtin_fmaf(half_lo(la), s0.x, s0.y), __builtin_fmaf(half_lo(ha), s0.z, s0.w),
                        __builtin_fmaf(half_lo(lb), s0.x, s0.y), __builtin_fmaf(half_lo(hb), s0.z, s0.w), uq, acc);
        rotate_contract(i1, __builtin_fmaf(half_hi(la), s1.x, s1.y), __builtin_fmaf(half_hi(ha), s1.z, s1.w),
                        __builtin_fmaf(half_hi(lb), s1.x, s1.y), __builtin_fmaf(half_hi(hb), s1.z, s1.w), uq, acc);
      };
#pragma unroll
      for (int d = 0; d < NW; ++d) {
        const uint32_t wa = kc[gg][0][d], wha = kc[gg][0][NW + d];   // token a: low / high channels
        const uint32_t wb = kc[gg][1][d], whb = kc[gg][1][NW + d];   // token b
#pragma unroll
        for (int k = 0; k < (BITS == 4 ? 4 : 8); ++k) {
          // 4 bits: masked word k of dword d holds pairs 8d + k and 8d + k + 4
          // (mask_codes); 2 bits: word k holds pairs k and k + 8, word 4 + k
          // pairs 4 + k and 12 + k
          const int i0 = BITS == 4 ? 8 * d + k : k;
          const int i1 = BITS == 4 ? 8 * d + k + 4 : k + 8;
          two_pairs(i0, i1, mask_code<BITS>(wa, k), mask_code<BITS>(wha, k), mask_code<BITS>(wb, k),
                    mask_code<BITS>(whb, k));
        }
      }
      finish_scores(acc, gg, sel);
    }
    const int nvalid = cur_pos.nvalid;
    const bool tok_ok = tok < nvalid;
    float p[G];
    for (int m = 0; m < G; ++m) {
      const float s = tok_ok ? sel[m] : -INFINITY;
      if constexpr (V16) p[m] = softmax_step16<G, NDG>(m, s, tok_ok, m_run, l_acc, acc16, zacc);
      else p[m] = softmax_step<G, HL, NDG>(m, s, tok_ok, m_run, l_acc, o0, o1, o2, o3, zacc);
    }

    // ---------------- values
    {
      TileRaw<BITS, false> meta;
      meta.vm = cur_vm;
      float vs[NDG], vz[NDG];
      value_meta<BITS, false, NDG>(meta, tok_ok, vs, vz);
      if constexpr (V16) {
        stage_probs16<G, BITS, false, NDG>(p, vs, vz, lds_addr(PL[w]), zacc, tl, gh);
      } else {
        stage_probs<G, BITS, false, HL, NDG>(p, vs, vz, PLw, zacc, tl, gh);
      }
    }
    // this tile's value copies have landed: all but the next tile's key
    // copies, the last vector memory operations issued (loads return in
    // order), when there is a next tile
    if (more) {
      if constexpr (BITS == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    wave_sync();
    if constexpr (V16) {
      // rows 8..15 of A repeat rows 0..7 (lane & 7)
      const uint32_t pvb = lds_addr(PL[w]) + 2 * v16_at(0, 0, lane & 7, 8 * (lane >> 4));
      uint32_t vd[2][8];
      u4v_t av[2][4];
      read_value_codes16<BITS>(stv, pvb, lane, vd, av[0]);
      for (int gg = 0; gg < 2; ++gg) {
        if (gg == 1) read_a16<4>(pvb, 1, av[1]);
        for (int d = 0; d < 4; ++d) {
          const h8_t a8 = __builtin_bit_cast(h8_t, av[gg][d]);
          acc16[2 * d] = mfma16(a8, codes16_b<BITS>(vd[gg][2 * d], lane), acc16[2 * d]);
          acc16[2 * d + 1] = mfma16(a8, codes16_b<BITS>(vd[gg][2 * d + 1], lane), acc16[2 * d + 1]);
        }
      }
    } else {
      uint32_t vc[2][2][BITS];
      read_value_codes<BITS>(stv, lane, vc);
      value_mfma<G, BITS, false, HL, NDG>(vc, PLw, lane & 3, lane >> 5, o0, o1, o2, o3);
    }
    wave_sync();

    if (ends) flush();
    if (!more) break;
    cur_pos = nxt_pos;
    cur_pair = cs.pair;
    cur_k = cs.k;
    fresh = ends;
  }
}

}  // namespace

int decode_rope_wgs_per_cu(const Geom& g, int bits) {
  const void* fn = nullptr;
#define KVQ_FN(GG, BB) fn = reinterpret_cast<const void*>(&decode_rope_kernel<GG, BB>)
  if (bits == 4) {
    if (g.G == 1) KVQ_FN(1, 4); else if (g.G == 2) KVQ_FN(2, 4); else KVQ_FN(4, 4);
  } else {
    if (g.G == 1) KVQ_FN(1, 2); else if (g.G == 2) KVQ_FN(2, 2); else KVQ_FN(4, 2);
  }
#undef KVQ_FN
  return occupancy_wgs_per_cu(fn);
}

hipError_t launch_decode_rope(const Geom& g, const Planes& p, const ChunkPlan& cp, const __half* q,
                              int64_t q_pos, float sm_scale, float* ws, hipStream_t s) {
  for (int r = 0; r < cp.nr; ++r) {
    const RangePlan& rp = cp.r[r];
    const int64_t wins = rp.window ? (int64_t)g.B * g.Hkv : 0;
    if (rp.pwgs == 0 && wins == 0) continue;
    MfmaArgs a;
    a.g = g;
    a.p = p;
    a.q = q;
    a.ws = ws + cp.ctr_floats;
    a.scale_log2 = sm_scale * 1.4426950408889634f;
    a.q_pos = q_pos;
    a.t_lo = rp.t_lo;
    a.t_hi = rp.t_hi;
    a.hi_tier = rp.hi_tier;
    a.ctr = reinterpret_cast<uint32_t*>(ws) + r * (int64_t)g.B * g.Hkv * kCounterStride;
    a.tiles_pp = rp.tiles_pp;
    a.pairs = (int64_t)g.B * g.Hkv;
    a.team = rp.team;
    a.chunk = rp.chunk;
    a.n_chunks = rp.n_chunks;
    a.n_big = rp.n_big;
    a.pwgs = rp.pwgs;
    a.slot_base = rp.slot_base;
    a.wins = wins;
    a.win_slot = cp.nq;
    a.n_slots = cp.n;
    const dim3 grid((unsigned)(rp.pwgs + wins)), block(256);
#define KVQ_RP(GG, BB) hipLaunchKernelGGL((decode_rope_kernel<GG, BB>), grid, block, 0, s, a)
    if (rp.bits == 4) {
      if (g.G == 1) KVQ_RP(1, 4);
      else if (g.G == 2) KVQ_RP(2, 4);
      else KVQ_RP(4, 4);
    } else {
      if (g.G == 1) KVQ_RP(1, 2);
      else if (g.G == 2) KVQ_RP(2, 2);
      else KVQ_RP(4, 2);
    }
#undef KVQ_RP
  }
  return hipGetLastError();
}

}  // namespace kvq
