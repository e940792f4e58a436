// Split-K decode over packed 4-bit / 2-bit tiles on the 4x4x4 fp16 MFMA.
//
// Sources cited here:
//   [nalar]  "Kuantisasi KV Cache dengan Error Budget yang Eksplisit"
//            (nalar.dev).
//   [trefon] "Matematyka cache KV: ile kosztuje długi kontekst i co daje
//            4-bitowy cache" (trefon.com).
//
// What is computed is the decode attention of decode.hip: s_i = q.k_i scale,
// out = sum softmax(s)_i v_i ([nalar] "Error pada key mengubah input
// softmax", "Error pada value masuk setelah attention probability"), with the
// unpacking and scaling of the codes fused into the kernel instead of a
// dequantized copy ([nalar] "Biaya dequantization harus masuk ke model
// latency").  Hadamard caches are attended in the rotated domain and the merge
// rotates the output back ([trefon] "Jak 4-bitowemu cache to uchodzi").
//
// Mapping onto gfx950.  One wave streams 64-token tiles (two 32-token key
// groups).  MFMA 4x4x4 with 16 blocks: block b is lanes 4b..4b+3; A lane 4b+m
// holds row m, B lane 4b+n holds column n, D lane 4b+n register r holds row r
// of column n.  So lane l owns token l for the scores, and channels l and
// 64 + l for the output; rows are query heads.
//   keys:   a code nibble masked into an fp16 (w & 0x000F000F, ...) is the
//           subnormal n * 2^-24, exact; odd positions carry a x16 factor
//           (x4 .. x256 for 2-bit crumbs) that the A side divides out.  The
//           per-channel scales fold into the query, q'_d = q_d s_d, stored in
//           LDS as hi + lo fp16 halves after a per-group power-of-two
//           normalization (nothing overflows, lo carries the next 11 bits);
//           zero points become one per-group bias sum_d q_d z_d.
//   values: per-token scales fold into the probabilities, p'_t = p_t s_t,
//           written to LDS in A order as hi + lo fp16 halves (a single fp16
//           would put a 2^-12 relative error on c * s, i.e. on the group's
//           whole range rather than on the value); zero points add
//           sum_t p_t z_t.  B is the codes of 4 tokens of one channel (value
//           tiles are channel-major), unpacked without factors.
//   softmax: online in the log2 domain; the running max moves only when a
//           score exceeds it (one wave vote per tile).
// Each wave writes its own (m, l, o[128]) partial per query head.
#include "kvq_device.h"

namespace kvq {
namespace {

typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef float f4_t __attribute__((ext_vector_type(4)));

struct MfmaArgs {
  Geom g;
  Planes p;
  const __half* q;
  float* ws;
  float scale_log2;
  int64_t t_lo, t_hi;   // token range of this launch; t_lo is 32-aligned
  int nt;               // 64-token tiles per wave
  int hi_tier;          // KIVI: tiles in the high-bit planes (ring) or low-bit
  int64_t slot_base;    // first partial slot of this launch
  int64_t n_slots;      // partial slots per (sequence, query head)
};

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float xor_max(float v, int width) {
  for (int o = width / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float xor_sum(float v, int width) {
  for (int o = width / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ h4_t as_h4(uint32_t x, uint32_t y) {
  typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
  u2_t v = {x, y};
  return __builtin_bit_cast(h4_t, v);
}

__device__ __forceinline__ f4_t mfma4(h4_t x, h4_t y, f4_t c) {
  return __builtin_amdgcn_mfma_f32_4x4x4f16(x, y, c, 0, 0, 0);
}

// Key k-step ks (0..31) covers four channels: slot s of the operands holds
// channel ch[s], whose B value carries the factor 1/inv_f[s] (see unpacking
// in the tile loop).
template <int BITS>
__device__ __forceinline__ void key_quad(int ks, int* ch, float* inv_f) {
  if (BITS == 4) {
    const int i = ks >> 1, par = ks & 1;
    const int base = 8 * i + 2 * par;
    ch[0] = base; ch[1] = base + 4; ch[2] = base + 1; ch[3] = base + 5;
    inv_f[0] = 1.0f; inv_f[1] = 1.0f; inv_f[2] = 1.0f / 16; inv_f[3] = 1.0f / 16;
  } else {
    const int i = ks >> 2, qq = ks & 3;
    const int p0 = 2 * qq, p1 = 2 * qq + 1;
    const float f0 = (p0 == 0 || p0 == 5) ? 1.f : (p0 == 1 || p0 == 6) ? 4.f : (p0 == 2 || p0 == 7) ? 16.f : p0 == 3 ? 64.f : 256.f;
    const float f1 = (p1 == 0 || p1 == 5) ? 1.f : (p1 == 1 || p1 == 6) ? 4.f : (p1 == 2 || p1 == 7) ? 16.f : p1 == 3 ? 64.f : 256.f;
    ch[0] = 16 * i + p0; ch[1] = 16 * i + p0 + 8; ch[2] = 16 * i + p1; ch[3] = 16 * i + p1 + 8;
    inv_f[0] = 1.0f / f0; inv_f[1] = 1.0f / f0; inv_f[2] = 1.0f / f1; inv_f[3] = 1.0f / f1;
  }
}

// Value token tl (0..31 in its group) -> (k-step within the group, slot).
template <int BITS>
__device__ __forceinline__ void value_slot(int tl, int* kk, int* slot) {
  if (BITS == 4) {
    const int i = tl >> 3, r = tl & 7, j = r & 3, hp = r >> 2;
    *kk = 2 * i + (j >> 1);
    *slot = (j & 1) * 2 + hp;
  } else {
    const int i = tl >> 4, e = tl & 15, j = e & 7, hp = e >> 3;
    *kk = 4 * i + (j >> 1);
    *slot = (j & 1) * 2 + hp;
  }
}

template <int G, int BITS, bool BLOCK>
__global__ __launch_bounds__(256) void decode_mfma_kernel(MfmaArgs a) {
  constexpr int HL = (G <= 2) ? 1 : 2;   // key MFMAs per k-step (hi/lo)
  constexpr int NKW = BITS;              // key uint4 loads per token (64 or 32 bytes)
  constexpr int NDG = BLOCK ? 1 : 4;     // value scale groups per token
  const Geom& g = a.g;
  __shared__ float qs[G][kD];
  __shared__ float qmax_s;
  __shared__ __attribute__((aligned(16))) _Float16 QL[4][2][32][HL][4][4];
  __shared__ __attribute__((aligned(16))) _Float16 PL[4][NDG][16][HL][4][4];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t pair = pair_index(g, b, h);
  const int gh = lane >> 5, tl = lane & 31, row = lane & 3;

  // ---------------- prologue: scaled (and rotated) queries, zeroed tables
  for (int e = tid; e < G * kD; e += 256)
    qs[e / kD][e % kD] = __half2float(a.q[((int64_t)b * g.Hq + h * G + e / kD) * kD + e % kD]);
  for (int e = tid; e < (int)(sizeof(QL) / 2); e += 256) (&QL[0][0][0][0][0][0])[e] = (_Float16)0.0f;
  for (int e = tid; e < (int)(sizeof(PL) / 2); e += 256) (&PL[0][0][0][0][0][0])[e] = (_Float16)0.0f;
  __syncthreads();
  if (g.hadamard) fwht128_lds(&qs[0][0], G, tid, 256);
  for (int e = tid; e < G * kD; e += 256) (&qs[0][0])[e] *= a.scale_log2;
  __syncthreads();

  // this lane writes key k-step ks = tl of the query table: four channels
  int kch[4];
  float kinv[4];
  key_quad<BITS>(tl, kch, kinv);
  float qv[G][4];
  for (int m = 0; m < G; ++m)
    for (int i = 0; i < 4; ++i) qv[m][i] = qs[m][kch[i]];

  // BLOCK: per-token key scales, so the query table is fixed for the chunk
  float qsum[G];
  float e_scale_blk = 1.0f;
  if (BLOCK) {
    if (tid < 64) {
      float mx = 0.0f;
      for (int e = lane; e < G * kD; e += 64) mx = fmaxf(mx, fabsf((&qs[0][0])[e]));
      mx = xor_max(mx, 64);
      if (lane == 0) qmax_s = mx;
    }
    __syncthreads();
    int ex = 0;
    if (qmax_s > 0.0f) frexpf(qmax_s, &ex);
    const int e_blk = 10 - ex;
    e_scale_blk = ldexpf(1.0f, 24 - e_blk);
    for (int m = 0; m < G; ++m) {
      float s = 0.0f;
      for (int d = lane; d < kD; d += 64) s += qs[m][d];
      qsum[m] = xor_sum(s, 64);
    }
    for (int m = 0; m < G; ++m)
      for (int i = 0; i < 4; ++i) {
        const float x = ldexpf(qv[m][i], e_blk) * kinv[i];
        const _Float16 hi = (_Float16)x;
        const _Float16 lo = (_Float16)(x - (float)hi);
        if (HL == 1) {
          QL[w][gh][tl][0][m][i] = hi;
          QL[w][gh][tl][0][G + m][i] = lo;
        } else {
          QL[w][gh][tl][0][m][i] = hi;
          QL[w][gh][tl][1][m][i] = lo;
        }
      }
    wave_sync();
  }

  float m_run[G], l_acc[G];
  float zacc[G][NDG];
  for (int m = 0; m < G; ++m) {
    m_run[m] = -INFINITY;
    l_acc[m] = 0.0f;
    for (int d = 0; d < NDG; ++d) zacc[m][d] = 0.0f;
  }
  f4_t o0 = {0, 0, 0, 0}, o1 = {0, 0, 0, 0};

  const int64_t chunk_tok0 = a.t_lo + (int64_t)chunk * 4 * a.nt * 64;
  constexpr int TB = 512 * BITS;   // tile bytes
  constexpr int VROW = 4 * BITS;   // value row bytes per channel
  const uint8_t* kplane = a.p.p[a.hi_tier ? KVQ_PLANE_K_HI : KVQ_PLANE_K_LO];
  const uint8_t* vplane = a.p.p[a.hi_tier ? KVQ_PLANE_V_HI : KVQ_PLANE_V_LO];
  const int64_t slots = a.hi_tier ? g.hi_slots : g.gmax;

  for (int it = 0; it < a.nt; ++it) {
    const int64_t base = chunk_tok0 + ((int64_t)it * 4 + w) * 64;
    if (base >= a.t_hi) break;   // wave-uniform
    const int nvalid = (int)min((int64_t)64, a.t_hi - base);
    const int64_t grp0 = base >> 5;
    const bool tok_ok = lane < nvalid;
    const bool my_grp_ok = 32 * gh < nvalid;

    // ---------------- loads: key row of my token, value rows of my channels,
    // metadata of my group
    const int64_t my_grp = grp0 + gh;
    uint4 kc[NKW];
    for (int j = 0; j < NKW; ++j) kc[j] = make_uint4(0, 0, 0, 0);
    if (tok_ok) {
      const uint8_t* kt = kplane + (pair * slots + my_grp % slots) * TB + tl * 16;
      for (int j = 0; j < NKW; ++j) kc[j] = *reinterpret_cast<const uint4*>(kt + j * 512);
    }
    uint32_t vc[2][2][BITS];   // [group][half][dwords of the 32-token row]
    for (int gg = 0; gg < 2; ++gg) {
      const bool ok = 32 * gg < nvalid;
      const int64_t grp = grp0 + gg;
      const uint8_t* vt = vplane + (pair * slots + grp % slots) * TB;
      for (int hf = 0; hf < 2; ++hf) {
        const uint8_t* src = vt + (lane + 64 * hf) * VROW;
        if (BITS == 4) {
          uint4 x = ok ? *reinterpret_cast<const uint4*>(src) : make_uint4(0, 0, 0, 0);
          vc[gg][hf][0] = x.x; vc[gg][hf][1] = x.y; vc[gg][hf][2] = x.z; vc[gg][hf][3] = x.w;
        } else {
          uint2 x = ok ? *reinterpret_cast<const uint2*>(src) : make_uint2(0, 0);
          vc[gg][hf][0] = x.x; vc[gg][hf][1] = x.y;
        }
      }
    }
    float vs[NDG], vz[NDG];
    float kscale = 0.0f;
    uint2 km0 = make_uint2(0, 0), km1 = make_uint2(0, 0);
    if (BLOCK) {
      const uint16_t* ks16 = reinterpret_cast<const uint16_t*>(a.p.p[KVQ_PLANE_K_META]);
      const uint16_t* vs16 = reinterpret_cast<const uint16_t*>(a.p.p[KVQ_PLANE_V_META]);
      const int64_t t = base + lane;
      kscale = tok_ok ? half_bits_to_float(ks16[pair * g.gmax * kGroup + t]) : 0.0f;
      vs[0] = tok_ok ? half_bits_to_float(vs16[pair * g.gmax * kGroup + t]) : 0.0f;
      vz[0] = 0.0f;
    } else {
      const uint8_t* kmeta = a.p.p[KVQ_PLANE_K_META] + (pair * g.gmax + my_grp) * 512;
      const uint8_t* vmeta = a.p.p[KVQ_PLANE_V_META] + (pair * g.gmax + my_grp) * 512;
      if (my_grp_ok) {
        km0 = *reinterpret_cast<const uint2*>(kmeta + 4 * kch[0]);   // channels kch[0], kch[2]
        km1 = *reinterpret_cast<const uint2*>(kmeta + 4 * kch[1]);   // channels kch[1], kch[3]
      }
      uint4 vm = tok_ok ? *reinterpret_cast<const uint4*>(vmeta + 16 * tl) : make_uint4(0, 0, 0, 0);
      const uint32_t vw[4] = {vm.x, vm.y, vm.z, vm.w};
      for (int d = 0; d < 4; ++d) {
        vs[d] = half_bits_to_float((uint16_t)(vw[d] & 0xFFFF));
        vz[d] = half_bits_to_float((uint16_t)(vw[d] >> 16));
      }
    }

    // ---------------- KIVI: query table of my group (k-step tl)
    float bias[G];
    float kscale_grp = 1.0f;
    if (!BLOCK) {
      // km0 = (s, z) of channels kch[0], kch[0] + 1 == kch[2]
      // km1 = (s, z) of channels kch[1], kch[1] + 1 == kch[3]
      const float sK[4] = {half_bits_to_float((uint16_t)(km0.x & 0xFFFF)),
                           half_bits_to_float((uint16_t)(km1.x & 0xFFFF)),
                           half_bits_to_float((uint16_t)(km0.y & 0xFFFF)),
                           half_bits_to_float((uint16_t)(km1.y & 0xFFFF))};
      const float zK[4] = {half_bits_to_float((uint16_t)(km0.x >> 16)),
                           half_bits_to_float((uint16_t)(km1.x >> 16)),
                           half_bits_to_float((uint16_t)(km0.y >> 16)),
                           half_bits_to_float((uint16_t)(km1.y >> 16))};
      float qp[G][4];
      float amax = 0.0f;
      for (int m = 0; m < G; ++m) {
        float bp = 0.0f;
        for (int i = 0; i < 4; ++i) {
          qp[m][i] = qv[m][i] * sK[i];
          bp += qv[m][i] * zK[i];
          amax = fmaxf(amax, fabsf(qp[m][i]));
        }
        bias[m] = xor_sum(bp, 32);
      }
      amax = xor_max(amax, 32);
      int ex = 0;
      if (amax > 0.0f) frexpf(amax, &ex);
      const int e_grp = 10 - ex;
      kscale_grp = ldexpf(1.0f, 24 - e_grp);
      for (int m = 0; m < G; ++m) {
        _Float16 hi4[4], lo4[4];
        for (int i = 0; i < 4; ++i) {
          const float x = ldexpf(qp[m][i], e_grp) * kinv[i];
          hi4[i] = (_Float16)x;
          lo4[i] = (_Float16)(x - (float)hi4[i]);
        }
        h4_t hv = {hi4[0], hi4[1], hi4[2], hi4[3]};
        h4_t lv = {lo4[0], lo4[1], lo4[2], lo4[3]};
        if (HL == 1) {
          *reinterpret_cast<h4_t*>(&QL[w][gh][tl][0][m][0]) = hv;
          *reinterpret_cast<h4_t*>(&QL[w][gh][tl][0][G + m][0]) = lv;
        } else {
          *reinterpret_cast<h4_t*>(&QL[w][gh][tl][0][m][0]) = hv;
          *reinterpret_cast<h4_t*>(&QL[w][gh][tl][1][m][0]) = lv;
        }
      }
      wave_sync();
    }

    // ---------------- scores: S = q' . codes over 32 k-steps
    f4_t acc = {0, 0, 0, 0};
    const int qgh = BLOCK ? 0 : gh;  // table half of my block (tokens 0-31 / 32-63)
    for (int j = 0; j < NKW; ++j) {
      const uint32_t dw[4] = {kc[j].x, kc[j].y, kc[j].z, kc[j].w};
      for (int u = 0; u < 4; ++u) {
        const uint32_t x = dw[u];
        const int i = 4 * j + u;     // canonical dword index of the row
        if (BITS == 4) {
          const uint32_t x8 = x >> 8;
          const h4_t b0 = as_h4(x & 0x000F000Fu, x & 0x00F000F0u);
          const h4_t b1 = as_h4(x8 & 0x000F000Fu, x8 & 0x00F000F0u);
          for (int hl = 0; hl < HL; ++hl) {
            acc = mfma4(*reinterpret_cast<const h4_t*>(&QL[w][qgh][2 * i][hl][row][0]), b0, acc);
            acc = mfma4(*reinterpret_cast<const h4_t*>(&QL[w][qgh][2 * i + 1][hl][row][0]), b1, acc);
          }
        } else {
          const uint32_t x10 = x >> 10;
          const h4_t b0 = as_h4(x & 0x00030003u, x & 0x000C000Cu);
          const h4_t b1 = as_h4(x & 0x00300030u, x & 0x00C000C0u);
          const h4_t b2 = as_h4(x & 0x03000300u, x10 & 0x00030003u);
          const h4_t b3 = as_h4(x10 & 0x000C000Cu, x10 & 0x00300030u);
          for (int hl = 0; hl < HL; ++hl) {
            acc = mfma4(*reinterpret_cast<const h4_t*>(&QL[w][qgh][4 * i][hl][row][0]), b0, acc);
            acc = mfma4(*reinterpret_cast<const h4_t*>(&QL[w][qgh][4 * i + 1][hl][row][0]), b1, acc);
            acc = mfma4(*reinterpret_cast<const h4_t*>(&QL[w][qgh][4 * i + 2][hl][row][0]), b2, acc);
            acc = mfma4(*reinterpret_cast<const h4_t*>(&QL[w][qgh][4 * i + 3][hl][row][0]), b3, acc);
          }
        }
      }
    }
    float s[G];
    for (int m = 0; m < G; ++m) {
      float dotv = (HL == 1) ? acc[m] + acc[G + m] : acc[m];
      if (BLOCK) s[m] = kscale * (dotv * e_scale_blk - 8.0f * qsum[m]);
      else s[m] = dotv * kscale_grp + bias[m];
      if (!tok_ok) s[m] = -INFINITY;
    }

    // ---------------- online softmax (log2 domain)
    float p[G];
    for (int m = 0; m < G; ++m) {
      const bool up = __any(s[m] > m_run[m]);
      if (up) {
        const float mnew = fmaxf(m_run[m], xor_max(s[m], 64));
        const float alpha = (m_run[m] == -INFINITY) ? 0.0f : exp2f(m_run[m] - mnew);
        m_run[m] = mnew;
        l_acc[m] *= alpha;
        o0[m] *= alpha;
        o1[m] *= alpha;
        if (HL == 1) {
          o0[G + m] *= alpha;
          o1[G + m] *= alpha;
        }
        for (int d = 0; d < NDG; ++d) zacc[m][d] *= alpha;
      }
      p[m] = tok_ok ? exp2f(s[m] - m_run[m]) : 0.0f;
      l_acc[m] += p[m];
    }

    // ---------------- p' = p s into the value A table; zero-point sums
    {
      int kk, slot;
      value_slot<BITS>(tl, &kk, &slot);
      const int ks = 8 * gh + kk;
      for (int d = 0; d < NDG; ++d)
        for (int m = 0; m < G; ++m) {
          const float x = p[m] * vs[d];
          const _Float16 hi = (_Float16)x;
          const _Float16 lo = (_Float16)(x - (float)hi);
          PL[w][d][ks][0][m][slot] = hi;
          if (HL == 1) PL[w][d][ks][0][G + m][slot] = lo;
          else PL[w][d][ks][1][m][slot] = lo;
          if (BLOCK) zacc[m][d] += x;
          else zacc[m][d] += p[m] * vz[d];
        }
    }
    wave_sync();

    // ---------------- values: O += p' . codes over 16 k-steps x 2 halves
    for (int ks = 0; ks < 16; ++ks) {
      const int gg = ks >> 3, kk = ks & 7;
      for (int hf = 0; hf < 2; ++hf) {
        uint32_t x0, x1;
        if (BITS == 4) {
          const uint32_t x = vc[gg][hf][kk >> 1];
          const int j0 = 2 * (kk & 1);
          x0 = (x >> (4 * j0)) & 0x000F000Fu;
          x1 = (x >> (4 * j0 + 4)) & 0x000F000Fu;
        } else {
          const uint32_t x = vc[gg][hf][kk >> 2];
          const int j0 = 2 * (kk & 3);
          x0 = (x >> (2 * j0)) & 0x00030003u;
          x1 = (x >> (2 * j0 + 2)) & 0x00030003u;
        }
        const int dg = BLOCK ? 0 : (gh + 2 * hf);
        const h4_t bv = as_h4(x0, x1);
        for (int hl = 0; hl < HL; ++hl) {
          const h4_t av = *reinterpret_cast<const h4_t*>(&PL[w][dg][ks][hl][row][0]);
          if (hf == 0) o0 = mfma4(av, bv, o0);
          else o1 = mfma4(av, bv, o1);
        }
      }
    }
    wave_sync();
  }

  // ---------------- epilogue: per-head partial of this wave
  const int64_t slot = a.slot_base + (int64_t)chunk * 4 + w;
  for (int m = 0; m < G; ++m) {
    const float lsum = xor_sum(l_acc[m], 64);
    float zsum[NDG];
    for (int d = 0; d < NDG; ++d) zsum[d] = xor_sum(zacc[m][d], 64);
    float* rec = a.ws + (((int64_t)b * g.Hq + h * G + m) * a.n_slots + slot) * kPartial;
    const float a0 = (HL == 1) ? o0[m] + o0[G + m] : o0[m];
    const float a1 = (HL == 1) ? o1[m] + o1[G + m] : o1[m];
    float v0, v1;
    if (BLOCK) {
      v0 = a0 * 16777216.0f - 8.0f * zsum[0];
      v1 = a1 * 16777216.0f - 8.0f * zsum[0];
    } else {
      v0 = a0 * 16777216.0f + zsum[gh];
      v1 = a1 * 16777216.0f + zsum[gh + 2];
    }
    rec[2 + lane] = v0;
    rec[2 + 64 + lane] = v1;
    if (lane == 0) {
      rec[0] = m_run[m];
      rec[1] = lsum;
    }
  }
}

}  // namespace

hipError_t launch_decode_mfma(const Geom& g, const Planes& p, const ChunkPlan& cp, const __half* q,
                              float sm_scale, float* ws, hipStream_t s) {
  for (int r = 0; r < cp.nr; ++r) {
    const RangePlan& rp = cp.r[r];
    if (rp.chunks == 0) continue;
    MfmaArgs a;
    a.g = g;
    a.p = p;
    a.q = q;
    a.ws = ws;
    a.scale_log2 = sm_scale * 1.4426950408889634f;
    a.t_lo = rp.t_lo;
    a.t_hi = rp.t_hi;
    a.nt = rp.nt;
    a.hi_tier = rp.hi_tier;
    a.slot_base = rp.slot_base;
    a.n_slots = cp.n;
    const dim3 grid((unsigned)rp.chunks, g.Hkv, g.B), block(256);
    const bool blk = g.scheme == KVQ_BLOCK128_SYM;
#define KVQ_MF(GG, BB, BL) hipLaunchKernelGGL((decode_mfma_kernel<GG, BB, BL>), grid, block, 0, s, a)
    if (blk) {
      if (g.G == 1) KVQ_MF(1, 4, true);
      else if (g.G == 2) KVQ_MF(2, 4, true);
      else KVQ_MF(4, 4, true);
    } else if (rp.bits == 4) {
      if (g.G == 1) KVQ_MF(1, 4, false);
      else if (g.G == 2) KVQ_MF(2, 4, false);
      else KVQ_MF(4, 4, false);
    } else {
      if (g.G == 1) KVQ_MF(1, 2, false);
      else if (g.G == 2) KVQ_MF(2, 2, false);
      else KVQ_MF(4, 2, false);
    }
#undef KVQ_MF
  }
  return hipGetLastError();
}

}  // namespace kvq
