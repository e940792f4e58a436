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
// The fp16 window of a KIVI cache is one more work-group of the same launch:
// keys and values are fp16 already (B operands as stored), the query
// unrotated.  Each wave writes its own (m, l, o[128]) partial per query head.
#include "kvq_device.h"

// Tuning knobs (compile-time):
//   KVQ_DECODE_PREFETCH   1: load tile i+1 into registers while tile i is
//                         processed (more bytes in flight, more VGPRs)
//   KVQ_DECODE_MIN_WAVES  minimum waves per SIMD the register allocation
//                         must allow (0: compiler's choice)
#ifndef KVQ_DECODE_PREFETCH
#define KVQ_DECODE_PREFETCH 0
#endif
#ifndef KVQ_DECODE_MIN_WAVES
#define KVQ_DECODE_MIN_WAVES 0
#endif

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
  int64_t chunks;       // work-groups over [t_lo, t_hi)
  int window;           // 1: one more work-group attends the fp16 window
  int64_t slot_base;    // first partial slot of this launch
  int64_t n_slots;      // partial slots per (sequence, query head)
};

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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
// channel ch[s], whose B value carries the factor 1/inv_f[s] (see the
// unpacking in the tile loop).
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
    const float f0 = (p0 == 0) ? 1.f : (p0 == 2) ? 16.f : (p0 == 4) ? 256.f : 4.f;   // p0 in {0,2,4,6}
    const float f1 = (p1 == 1) ? 4.f : (p1 == 3) ? 64.f : (p1 == 5) ? 1.f : 16.f;   // p1 in {1,3,5,7}
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

// hi + lo fp16 split of x (x - hi is exact in fp32)
__device__ __forceinline__ void split_half(float x, _Float16* hi, _Float16* lo) {
  *hi = (_Float16)x;
  *lo = (_Float16)(x - (float)*hi);
}

// Online-softmax update of one head for one tile; returns p for this lane.
template <int G, int HL, int NDG>
__device__ __forceinline__ float softmax_step(int m, float s, bool tok_ok, float* m_run, float* l_acc,
                                              f4_t& o0, f4_t& o1, f4_t& o2, f4_t& o3,
                                              float (*zacc)[NDG]) {
  if (__any(s > m_run[m])) {
    const float mnew = fmaxf(m_run[m], wave_max64(s));
    const float alpha = (m_run[m] == -INFINITY) ? 0.0f : exp2f(m_run[m] - mnew);
    m_run[m] = mnew;
    l_acc[m] *= alpha;
    o0[m] *= alpha; o1[m] *= alpha; o2[m] *= alpha; o3[m] *= alpha;
    if (HL == 1) {
      o0[G + m] *= alpha; o1[G + m] *= alpha; o2[G + m] *= alpha; o3[G + m] *= alpha;
    }
    for (int d = 0; d < NDG; ++d) zacc[m][d] *= alpha;
  }
  const float p = tok_ok ? exp2f(s - m_run[m]) : 0.0f;
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
  uint2 km0, km1;   // KIVI: (s, z) of the key channels of this lane's k-step
  uint4 vm;         // KIVI: (s, z) x 4 of this lane's token
  uint16_t ks16, vs16;   // BLOCK: per-token scales
};

struct TilePos {
  int64_t base;
  int nvalid;
  uint32_t s0, s1;  // tile slots of the two groups
  uint32_t grp0;
};

template <int BITS, bool BLOCK>
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
      if (BITS == 4) {
        const uint4 x = ok ? *reinterpret_cast<const uint4*>(src) : make_uint4(0, 0, 0, 0);
        r.vc[gg][hf][0] = x.x; r.vc[gg][hf][1] = x.y; r.vc[gg][hf][2] = x.z; r.vc[gg][hf][3] = x.w;
      } else {
        const uint2 x = ok ? *reinterpret_cast<const uint2*>(src) : make_uint2(0, 0);
        r.vc[gg][hf][0] = x.x; r.vc[gg][hf][1] = x.y;
      }
    }
  }
  if (BLOCK) {
    const int64_t t = tp.base + lane;
    r.ks16 = tok_ok ? ksc[t] : (uint16_t)0;
    r.vs16 = tok_ok ? vsc[t] : (uint16_t)0;
  } else {
    const bool my_grp_ok = gh == 0 || grp1_ok;
    const uint32_t my_grp = tp.grp0 + gh;
    const uint8_t* kmeta = kmpair + (int64_t)my_grp * 512;
    const uint8_t* vmeta = vmpair + (int64_t)my_grp * 512;
    r.km0 = my_grp_ok ? *reinterpret_cast<const uint2*>(kmeta + 4 * kch0) : make_uint2(0, 0);
    r.km1 = my_grp_ok ? *reinterpret_cast<const uint2*>(kmeta + 4 * kch1) : make_uint2(0, 0);
    r.vm = tok_ok ? *reinterpret_cast<const uint4*>(vmeta + 16 * tl) : make_uint4(0, 0, 0, 0);
  }
}

template <int G, int BITS, bool BLOCK>
__global__
#if KVQ_DECODE_MIN_WAVES > 0
__launch_bounds__(256, KVQ_DECODE_MIN_WAVES)
#else
__launch_bounds__(256)
#endif
void decode_mfma_kernel(MfmaArgs a) {
  constexpr int HL = (G <= 2) ? 1 : 2;   // MFMAs per k-step (hi/lo)
  constexpr int NKW = BITS;              // key uint4 loads per token (64 or 32 bytes)
  constexpr int NDG = BLOCK ? 1 : 4;     // value scale groups per token
  constexpr int TB = 512 * BITS;         // tile bytes
  constexpr int VROW = 4 * BITS;         // value row bytes per channel
  const Geom& g = a.g;
  __shared__ float qs[G][kD];
  __shared__ float qmax_s;
  __shared__ __attribute__((aligned(16))) _Float16 QL[4][2][32][HL][4][4];
  __shared__ __attribute__((aligned(16))) _Float16 PL[4][NDG][16][HL][4][4];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t chunk = blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t pair = pair_index(g, b, h);
  const int gh = lane >> 5, tl = lane & 31, row = lane & 3;
  const bool win = a.window && chunk == a.chunks;   // the fp16 window work-group

  // ---------------- prologue: scaled (rotated unless window) queries, zero tables
  for (int e = tid; e < G * kD; e += 256)
    qs[e / kD][e % kD] = __half2float(a.q[((int64_t)b * g.Hq + h * G + e / kD) * kD + e % kD]);
  for (int e = tid; e < (int)(sizeof(QL) / 2); e += 256) (&QL[0][0][0][0][0][0])[e] = (_Float16)0.0f;
  for (int e = tid; e < (int)(sizeof(PL) / 2); e += 256) (&PL[0][0][0][0][0][0])[e] = (_Float16)0.0f;
  __syncthreads();
  if (g.hadamard && !win) fwht128_lds(&qs[0][0], G, tid, 256);
  for (int e = tid; e < G * kD; e += 256) (&qs[0][0])[e] *= a.scale_log2;
  __syncthreads();
  if (tid < 64) {
    float mx = 0.0f;
    for (int e = lane; e < G * kD; e += 64) mx = fmaxf(mx, fabsf((&qs[0][0])[e]));
    mx = wave_max64(mx);
    if (lane == 0) qmax_s = mx;
  }
  __syncthreads();

  float m_run[G], l_acc[G];
  float zacc[G][NDG];
  for (int m = 0; m < G; ++m) {
    m_run[m] = -INFINITY;
    l_acc[m] = 0.0f;
    for (int d = 0; d < NDG; ++d) zacc[m][d] = 0.0f;
  }
  // output accumulators: channel lane (o0: even value k-steps, o2: odd) and
  // channel 64 + lane (o1, o3); two chains each so dependent MFMAs interleave
  f4_t o0 = {0, 0, 0, 0}, o1 = {0, 0, 0, 0}, o2 = {0, 0, 0, 0}, o3 = {0, 0, 0, 0};

  if (win) {
    // ================= fp16 window: tokens [Tq, length), wave w takes tile w
    int ex = 0;
    if (qmax_s > 0.0f) frexpf(qmax_s, &ex);
    const int e_q = 10 - ex;
    const float unscale = ldexpf(1.0f, -e_q);
    // query table in natural channel order: k-step ks = tl holds 4tl..4tl+3
    for (int m = 0; m < G; ++m) {
      _Float16 hi[4], lo[4];
      for (int i = 0; i < 4; ++i) split_half(ldexpf(qs[m][4 * tl + i], e_q), &hi[i], &lo[i]);
      const h4_t hv = {hi[0], hi[1], hi[2], hi[3]}, lv = {lo[0], lo[1], lo[2], lo[3]};
      *reinterpret_cast<h4_t*>(&QL[w][gh][tl][0][m][0]) = hv;
      if (HL == 1) *reinterpret_cast<h4_t*>(&QL[w][gh][tl][0][G + m][0]) = lv;
      else *reinterpret_cast<h4_t*>(&QL[w][gh][tl][1][m][0]) = lv;
    }
    wave_sync();
    const int64_t base = g.Tq + 64 * (int64_t)w;
    if (base < g.length) {
      const int nvalid = (int)min((int64_t)64, g.length - base);
      const bool tok_ok = lane < nvalid;
      const __half* krow = reinterpret_cast<const __half*>(a.p.p[KVQ_PLANE_K_WIN]) +
                           (pair * kRing + (base + lane) % kRing) * kD;
      f4_t acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
      for (int c = 0; c < 4; ++c) {       // 32 channels at a time
        uint4 kr[4];
        for (int j = 0; j < 4; ++j)
          kr[j] = tok_ok ? *reinterpret_cast<const uint4*>(krow + 32 * c + 8 * j) : make_uint4(0, 0, 0, 0);
        for (int j = 0; j < 4; ++j) {
          const int ks = 8 * c + 2 * j;
          for (int hl = 0; hl < HL; ++hl) {
            acc0 = mfma4(*reinterpret_cast<const h4_t*>(&QL[w][gh][ks][hl][row][0]), as_h4(kr[j].x, kr[j].y), acc0);
            acc1 = mfma4(*reinterpret_cast<const h4_t*>(&QL[w][gh][ks + 1][hl][row][0]), as_h4(kr[j].z, kr[j].w), acc1);
          }
        }
      }
      float p[G];
      for (int m = 0; m < G; ++m) {
        const float dv = (HL == 1) ? acc0[m] + acc0[G + m] + acc1[m] + acc1[G + m] : acc0[m] + acc1[m];
        const float s = tok_ok ? dv * unscale : -INFINITY;
        p[m] = softmax_step<G, HL, NDG>(m, s, tok_ok, m_run, l_acc, o0, o1, o2, o3, zacc);
      }
      // probabilities in natural token order: k-step lane/4, slot lane%4
      for (int m = 0; m < G; ++m) {
        _Float16 hi, lo;
        split_half(p[m], &hi, &lo);
        PL[w][0][lane >> 2][0][m][lane & 3] = hi;
        if (HL == 1) PL[w][0][lane >> 2][0][G + m][lane & 3] = lo;
        else PL[w][0][lane >> 2][1][m][lane & 3] = lo;
      }
      wave_sync();
      const __half* vring = reinterpret_cast<const __half*>(a.p.p[KVQ_PLANE_V_WIN]) + pair * kD * kRing;
      for (int kp = 0; kp < 8; ++kp) {    // 8 tokens (two k-steps) per load
        const int64_t t0 = base + 8 * kp;
        const int slot = (int)(t0 % kRing);
        for (int hf = 0; hf < 2; ++hf) {
          uint4 x = make_uint4(0, 0, 0, 0);
          if (8 * kp < nvalid) {
            x = *reinterpret_cast<const uint4*>(vring + (lane + 64 * hf) * kRing + slot);
            // zero the halves of tokens past the window (stale ring slots)
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
            const h4_t a0 = *reinterpret_cast<const h4_t*>(&PL[w][0][2 * kp][hl][row][0]);
            const h4_t a1 = *reinterpret_cast<const h4_t*>(&PL[w][0][2 * kp + 1][hl][row][0]);
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
    const int64_t slot = a.slot_base + a.chunks * 4 + w;
    for (int m = 0; m < G; ++m) {
      const float lsum = wave_sum64(l_acc[m]);
      float* rec = a.ws + (((int64_t)b * g.Hq + h * G + m) * a.n_slots + slot) * kPartial;
      const float v0 = (HL == 1) ? o0[m] + o0[G + m] + o2[m] + o2[G + m] : o0[m] + o2[m];
      const float v1 = (HL == 1) ? o1[m] + o1[G + m] + o3[m] + o3[G + m] : o1[m] + o3[m];
      rec[2 + lane] = v0;
      rec[2 + 64 + lane] = v1;
      if (lane == 0) {
        rec[0] = m_run[m];
        rec[1] = lsum;
      }
    }
    return;
  }

  // ================= quantized tiles
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
    int ex = 0;
    if (qmax_s > 0.0f) frexpf(qmax_s, &ex);
    const int e_blk = 10 - ex;
    e_scale_blk = ldexpf(1.0f, 24 - e_blk);
    for (int m = 0; m < G; ++m) {
      float s = 0.0f;
      for (int i = 0; i < 4; ++i) s += qv[m][i];
      qsum[m] = half_sum(s);   // the 32 lanes of a half cover all 128 channels
    }
    for (int m = 0; m < G; ++m) {
      _Float16 hi[4], lo[4];
      for (int i = 0; i < 4; ++i) split_half(ldexpf(qv[m][i], e_blk) * kinv[i], &hi[i], &lo[i]);
      const h4_t hv = {hi[0], hi[1], hi[2], hi[3]}, lv = {lo[0], lo[1], lo[2], lo[3]};
      *reinterpret_cast<h4_t*>(&QL[w][gh][tl][0][m][0]) = hv;
      if (HL == 1) *reinterpret_cast<h4_t*>(&QL[w][gh][tl][0][G + m][0]) = lv;
      else *reinterpret_cast<h4_t*>(&QL[w][gh][tl][1][m][0]) = lv;
    }
    wave_sync();
  }

  const int64_t chunk_tok0 = a.t_lo + chunk * 4 * a.nt * 64;
  const uint8_t* kplane = a.p.p[a.hi_tier ? KVQ_PLANE_K_HI : KVQ_PLANE_K_LO];
  const uint8_t* vplane = a.p.p[a.hi_tier ? KVQ_PLANE_V_HI : KVQ_PLANE_V_LO];
  const int64_t slots = a.hi_tier ? g.hi_slots : g.gmax;
  const bool ring = slots != g.gmax;
  const uint8_t* kpair = kplane + pair * slots * TB;
  const uint8_t* vpair = vplane + pair * slots * TB;
  const uint8_t* kmpair = a.p.p[KVQ_PLANE_K_META] + pair * g.gmax * 512;
  const uint8_t* vmpair = a.p.p[KVQ_PLANE_V_META] + pair * g.gmax * 512;
  const uint16_t* ksc = reinterpret_cast<const uint16_t*>(a.p.p[KVQ_PLANE_K_META]) + pair * g.gmax * kGroup;
  const uint16_t* vsc = reinterpret_cast<const uint16_t*>(a.p.p[KVQ_PLANE_V_META]) + pair * g.gmax * kGroup;

  auto tile_pos = [&](int it, TilePos& tp) -> bool {
    tp.base = chunk_tok0 + ((int64_t)it * 4 + w) * 64;
    if (it >= a.nt || tp.base >= a.t_hi) return false;
    tp.nvalid = (int)min((int64_t)64, a.t_hi - tp.base);
    tp.grp0 = (uint32_t)(tp.base >> 5);
    tp.s0 = tp.grp0;
    tp.s1 = tp.grp0 + 1;
    if (ring) {
      tp.s0 = tp.grp0 % (uint32_t)slots;
      tp.s1 = (tp.s0 + 1 == (uint32_t)slots) ? 0 : tp.s0 + 1;
    }
    return true;
  };
  TilePos cur_pos, nxt_pos;
  TileRaw<BITS, BLOCK> cur, nxt;
  bool have = tile_pos(0, cur_pos);
  if (KVQ_DECODE_PREFETCH && have)
    load_tile<BITS, BLOCK>(cur, cur_pos, lane, kpair, vpair, kmpair, vmpair, ksc, vsc, kch[0], kch[1]);
  for (int it = 0; have; ++it) {
    bool have_next;
    if (KVQ_DECODE_PREFETCH) {
      // prefetch the next tile of this wave before working on the current one
      have_next = tile_pos(it + 1, nxt_pos);
      if (have_next)
        load_tile<BITS, BLOCK>(nxt, nxt_pos, lane, kpair, vpair, kmpair, vmpair, ksc, vsc, kch[0], kch[1]);
    } else {
      load_tile<BITS, BLOCK>(cur, cur_pos, lane, kpair, vpair, kmpair, vmpair, ksc, vsc, kch[0], kch[1]);
      have_next = tile_pos(it + 1, nxt_pos);
    }
    const int64_t base = cur_pos.base;
    const int nvalid = cur_pos.nvalid;
    const bool tok_ok = lane < nvalid;
    const uint4* kc = cur.kc;
    const uint32_t (*vc)[2][BITS] = cur.vc;
    float vs[NDG], vz[NDG];
    float kscale = 0.0f;
    const uint2 km0 = cur.km0, km1 = cur.km1;
    if (BLOCK) {
      kscale = half_bits_to_float(cur.ks16);
      vs[0] = half_bits_to_float(cur.vs16);
      vz[0] = 0.0f;
    } else {
      const uint32_t vw[4] = {cur.vm.x, cur.vm.y, cur.vm.z, cur.vm.w};
      for (int d = 0; d < 4; ++d) {
        vs[d] = half_bits_to_float((uint16_t)(vw[d] & 0xFFFF));
        vz[d] = half_bits_to_float((uint16_t)(vw[d] >> 16));
      }
    }
    (void)base;

    // ---------------- KIVI: query table of my group (k-step tl)
    float bias[G];
    float kscale_grp = 1.0f;
    if (!BLOCK) {
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
        bias[m] = half_sum(bp);
      }
      amax = half_max(amax);
      int ex = 0;
      if (amax > 0.0f) frexpf(amax, &ex);
      const int e_grp = 10 - ex;
      kscale_grp = ldexpf(1.0f, 24 - e_grp);
      for (int m = 0; m < G; ++m) {
        _Float16 hi[4], lo[4];
        for (int i = 0; i < 4; ++i) split_half(ldexpf(qp[m][i], e_grp) * kinv[i], &hi[i], &lo[i]);
        const h4_t hv = {hi[0], hi[1], hi[2], hi[3]}, lv = {lo[0], lo[1], lo[2], lo[3]};
        *reinterpret_cast<h4_t*>(&QL[w][gh][tl][0][m][0]) = hv;
        if (HL == 1) *reinterpret_cast<h4_t*>(&QL[w][gh][tl][0][G + m][0]) = lv;
        else *reinterpret_cast<h4_t*>(&QL[w][gh][tl][1][m][0]) = lv;
      }
      wave_sync();
    }

    // ---------------- scores: S = q' . codes over 32 k-steps (two chains)
    f4_t acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
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
            acc0 = mfma4(*reinterpret_cast<const h4_t*>(&QL[w][qgh][2 * i][hl][row][0]), b0, acc0);
            acc1 = mfma4(*reinterpret_cast<const h4_t*>(&QL[w][qgh][2 * i + 1][hl][row][0]), b1, acc1);
          }
        } else {
          const uint32_t x10 = x >> 10;
          const h4_t b0 = as_h4(x & 0x00030003u, x & 0x000C000Cu);
          const h4_t b1 = as_h4(x & 0x00300030u, x & 0x00C000C0u);
          const h4_t b2 = as_h4(x & 0x03000300u, x10 & 0x00030003u);
          const h4_t b3 = as_h4(x10 & 0x000C000Cu, x10 & 0x00300030u);
          for (int hl = 0; hl < HL; ++hl) {
            acc0 = mfma4(*reinterpret_cast<const h4_t*>(&QL[w][qgh][4 * i][hl][row][0]), b0, acc0);
            acc1 = mfma4(*reinterpret_cast<const h4_t*>(&QL[w][qgh][4 * i + 1][hl][row][0]), b1, acc1);
            acc0 = mfma4(*reinterpret_cast<const h4_t*>(&QL[w][qgh][4 * i + 2][hl][row][0]), b2, acc0);
            acc1 = mfma4(*reinterpret_cast<const h4_t*>(&QL[w][qgh][4 * i + 3][hl][row][0]), b3, acc1);
          }
        }
      }
    }
    float p[G];
    for (int m = 0; m < G; ++m) {
      const float dotv = (HL == 1) ? acc0[m] + acc0[G + m] + acc1[m] + acc1[G + m] : acc0[m] + acc1[m];
      float s;
      if (BLOCK) s = kscale * (dotv * e_scale_blk - 8.0f * qsum[m]);
      else s = dotv * kscale_grp + bias[m];
      if (!tok_ok) s = -INFINITY;
      p[m] = softmax_step<G, HL, NDG>(m, s, tok_ok, m_run, l_acc, o0, o1, o2, o3, zacc);
    }

    // ---------------- p' = p s into the value A table; zero-point sums
    {
      int kk, slot;
      value_slot<BITS>(tl, &kk, &slot);
      const int ks = 8 * gh + kk;
      for (int d = 0; d < NDG; ++d)
        for (int m = 0; m < G; ++m) {
          const float x = p[m] * vs[d];
          _Float16 hi, lo;
          split_half(x, &hi, &lo);
          PL[w][d][ks][0][m][slot] = hi;
          if (HL == 1) PL[w][d][ks][0][G + m][slot] = lo;
          else PL[w][d][ks][1][m][slot] = lo;
          zacc[m][d] += BLOCK ? x : p[m] * vz[d];
        }
    }
    wave_sync();

    // ---------------- values: O += p' . codes, 16 k-steps x 2 halves
    for (int gg = 0; gg < 2; ++gg) {
      for (int hf = 0; hf < 2; ++hf) {
        const int dg = BLOCK ? 0 : (gh + 2 * hf);
        for (int u = 0; u < BITS; ++u) {
          const uint32_t x = vc[gg][hf][u];
          // unpack one dword: 8 tokens (4-bit) or 16 tokens (2-bit) as pairs
          constexpr int NP = (BITS == 4) ? 4 : 8;
          uint32_t pr[NP];
          if (BITS == 4) {
            pr[0] = x & 0x000F000Fu;
            pr[1] = (x >> 4) & 0x000F000Fu;
            pr[2] = (x >> 8) & 0x000F000Fu;
            pr[3] = (x >> 12) & 0x000F000Fu;
          } else {
            for (int j = 0; j < 8; ++j) pr[j] = (x >> (2 * j)) & 0x00030003u;
          }
          for (int q2 = 0; q2 < NP / 2; ++q2) {
            const int ks = 8 * gg + (NP / 2) * u + q2;   // k-step of pairs (2 q2, 2 q2 + 1)
            const h4_t bv = as_h4(pr[2 * q2], pr[2 * q2 + 1]);
            for (int hl = 0; hl < HL; ++hl) {
              const h4_t av = *reinterpret_cast<const h4_t*>(&PL[w][dg][ks][hl][row][0]);
              if (hf == 0) {
                if (q2 & 1) o2 = mfma4(av, bv, o2); else o0 = mfma4(av, bv, o0);
              } else {
                if (q2 & 1) o3 = mfma4(av, bv, o3); else o1 = mfma4(av, bv, o1);
              }
            }
          }
        }
      }
    }
    wave_sync();
    if (KVQ_DECODE_PREFETCH) cur = nxt;
    cur_pos = nxt_pos;
    have = have_next;
  }

  // ---------------- epilogue: per-head partial of this wave
  const int64_t slot = a.slot_base + chunk * 4 + w;
  for (int m = 0; m < G; ++m) {
    const float lsum = wave_sum64(l_acc[m]);
    float zsum[NDG];
    for (int d = 0; d < NDG; ++d) zsum[d] = wave_sum64(zacc[m][d]);
    float* rec = a.ws + (((int64_t)b * g.Hq + h * G + m) * a.n_slots + slot) * kPartial;
    const float a0 = (HL == 1) ? o0[m] + o0[G + m] + o2[m] + o2[G + m] : o0[m] + o2[m];
    const float a1 = (HL == 1) ? o1[m] + o1[G + m] + o3[m] + o3[G + m] : o1[m] + o3[m];
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
    const int window = rp.window;
    if (rp.chunks == 0 && !window) continue;
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
    a.chunks = rp.chunks;
    a.window = window;
    a.slot_base = rp.slot_base;
    a.n_slots = cp.n;
    const dim3 grid((unsigned)(rp.chunks + window), g.Hkv, g.B), block(256);
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
