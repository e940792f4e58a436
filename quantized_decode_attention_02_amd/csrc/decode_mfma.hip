// Split-K decode over packed 4-bit / 2-bit tiles on the 4x4x4 fp16 MFMA, for
// caches whose keys are stored after RoPE (or Hadamard-rotated).  Value side,
// softmax, window values and partials are shared with decode_rope.hip
// (decode_common.h).
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
//           tiles are channel-major), unpacked without factors.  Four query
//           heads at 4 or 2 bits (TBQ4 included) and 3-bit blocks take the
//           16x16x32 f16 MFMA instead: hi and lo rows of p' in one A operand, 16 channels
//           x 8 tokens of codes as B (decode_common.h, value_mfma16).
//   softmax: online in the log2 domain; the running max moves only when a
//           score exceeds it (one wave vote per tile).
// The fp16 window of a KIVI cache is one more work-group of the same launch:
// keys and values are fp16 already (B operands as stored), the query
// unrotated.  Each wave writes its own (m, l, o[128]) partial per query head.
#include "decode_common.h"

// Tuning knobs (compile-time):
//   KVQ_DECODE_STAGE      1: tiles reach registers through a per-wave LDS
//                         stage filled by global-to-LDS loads one tile ahead
//                         (decode_common.h); 0: plain loads of the current tile
//   KVQ_DECODE_MIN_WAVES  minimum waves per SIMD the register allocation
//                         must allow (0: 3, or 2 for the KIVI G = 4 kernels)
#ifndef KVQ_DECODE_STAGE
#define KVQ_DECODE_STAGE 1
#endif
#ifndef KVQ_DECODE_MIN_WAVES
#define KVQ_DECODE_MIN_WAVES 0
#endif

namespace kvq {
namespace {

// Key k-step ks (0..31) covers four channels: slot s of the operands holds
// channel ch[s], whose B value carries the factor 1/inv_f[s] (see the
// unpacking in the tile loop).
template <int BITS>
__device__ __forceinline__ void key_quad(int ks, int* ch, float* inv_f) {
  if (BITS == 3) {   // 3-bit codes are unpacked in channel order, no factors
    for (int s = 0; s < 4; ++s) {
      ch[s] = 4 * ks + s;
      inv_f[s] = 1.0f;
    }
  } else if (BITS == 8) {   // a dword's bytes 0, 2 then 1, 3 (odd bytes shifted down, no factors)
    ch[0] = 4 * ks; ch[1] = 4 * ks + 2; ch[2] = 4 * ks + 1; ch[3] = 4 * ks + 3;
    for (int s = 0; s < 4; ++s) inv_f[s] = 1.0f;
  } else if (BITS == 4) {
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

// The KIVI G = 4 kernels keep a wave's fp32 query in its probability table
// (the query is read only while an assignment opens, and every tile rewrites
// every entry the value MFMAs read; the pads are never read), which saves
// 8 KiB of LDS per work-group.
template <int G, bool BLOCK>
constexpr bool query_in_prob_table() {
  return G == 4 && !BLOCK;
}

// Waves per SIMD the register allocation must allow: three work-groups per
// compute unit wherever the LDS allows it, except for the KIVI G = 4 kernels
// (the 4-bit and 3-bit stages do not fit three; the 2-bit one would, but at
// 168 VGPRs it spills, and two work-groups without spills are much faster).
template <int G, int BITS, bool BLOCK>
constexpr int decode_min_waves() {
  return KVQ_DECODE_MIN_WAVES > 0 ? KVQ_DECODE_MIN_WAVES : ((G == 4 && !BLOCK) ? 2 : 3);
}

// TBQ (with BLOCK): TBQ4 blocks; codes become their fp16 levels through
// tbq4_levels() instead of entering as subnormals, and the block scale is the
// norm, so there is neither a code offset nor a position factor.
// Q40 (with BLOCK): Q4_0 (BITS = 4) or Q8_0 (BITS = 8) blocks; every token
// has a scale per 32-value slice, so key scores are summed slice by slice (a
// slice is one uint4 of the key row at 4 bits, two at 8) and values use four
// scale groups, as KIVI's per-token values do.
template <int G, int BITS, bool BLOCK, bool TBQ = false, bool Q40 = false>
__global__ __launch_bounds__(256, (decode_min_waves<G, BITS, BLOCK>())) void decode_mfma_kernel(MfmaArgs a) {
  constexpr int HL = (G <= 2) ? 1 : 2;   // MFMAs per k-step (hi/lo)
  constexpr int NKW = BITS;              // key uint4 loads per token (64 or 32 bytes)
  constexpr int NDG = (BLOCK && !Q40) ? 1 : 4;   // value scale groups per token
  // symmetric blocks: stored code offset (c + 4 at 3 bits, c + 8 at 4, c + 128 at 8)
  constexpr float COFF = BITS == 3 ? 4.0f : BITS == 8 ? 128.0f : 8.0f;
  constexpr int TB = 512 * BITS;         // tile bytes
  // four query heads at 4 or 2 bits (TBQ4 included) and 3-bit blocks: values on
  // the 16x16x32 MFMA (3-bit KIVI measured slower there and keeps the 4x4x4)
  constexpr bool V16 = G == 4 && (BITS == 4 || BITS == 2 || (BITS == 3 && BLOCK)) && KVQ_DECODE_STAGE;
  const Geom& g = a.g;
  // everything per wave: waves never wait for each other
  constexpr bool QP = query_in_prob_table<G, BLOCK>();
  __shared__ __attribute__((aligned(16))) float qs[QP ? 1 : 4][G][kD];
  // query tables: per group half (KIVI, rebuilt per group) or one (BLOCK,
  // fixed per pair)
  // padded tables where four query heads make their writes conflict (the
  // query table only where it is rebuilt per group)
  using QTab = ATab<HL, 32, (G == 4 && !BLOCK), (G == 4 && !BLOCK)>;
  using PTab = ATab<HL, 16, G == 4, (G == 4 && NDG > 1)>;
  __shared__ __attribute__((aligned(16))) _Float16 QL[4][(BLOCK ? 1 : 2) * QTab::T];
  // (16x16x32 value side: its tables; the window's table 0 overlays them)
  __shared__ __attribute__((aligned(16))) _Float16
      PL[4][V16 ? (v16_halves(NDG) > PTab::T ? v16_halves(NDG) : PTab::T) : NDG * PTab::T];
  __shared__ __attribute__((aligned(16))) uint8_t ST[KVQ_DECODE_STAGE ? 4 : 1][stage_bytes<BITS>()];

  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index is uniform: read it into a scalar register, so that the
  // tile walk and its addresses stay on the scalar unit
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gh = lane >> 5, tl = lane & 31, row = lane & 3;
  const QTab QLw{QL[w]};
  const PTab PLw{PL[w]};
  float (*qsw)[kD] = QP ? reinterpret_cast<float (*)[kD]>(&PL[w][0]) : qs[QP ? 0 : w];
  static_assert(!QP || sizeof(PL[0]) >= sizeof(qs[0]), "the query must fit the probability table");
  const int qh = BLOCK ? 0 : gh;
  for (int e = lane; e < (int)(sizeof(QL[0]) / 2); e += 64) QL[w][e] = (_Float16)0.0f;
  for (int e = lane; e < (int)(sizeof(PL[0]) / 2); e += 64) PL[w][e] = (_Float16)0.0f;
  wave_sync();

  float m_run[G], l_acc[G];
  float zacc[G][NDG];
  // output accumulators: channel lane (o0: even value k-steps, o2: odd) and
  // channel 64 + lane (o1, o3); two chains each so dependent MFMAs interleave
  f4_t o0, o1, o2, o3;
  f4_t acc16[8];   // V16: channel blocks 0..7 (value_mfma16)
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

  if (blockIdx.x < a.wins) {
    // ================= fp16 window of one pair: tokens [Tq, length), wave w takes tile w
    const int64_t pair = blockIdx.x;
    const int b = (int)(pair / g.Hkv), h = (int)(pair % g.Hkv);
    const float qmax = wave_query<G>(a, b, h, false, qsw, lane);
    int ex = 0;
    if (qmax > 0.0f) frexpf(qmax, &ex);
    const int e_q = 10 - ex;
    const float unscale = ldexpf(1.0f, -e_q);
    // query table in natural channel order: k-step ks = tl holds 4tl..4tl+3
    for (int m = 0; m < G; ++m) {
      _Float16 hi[4], lo[4];
      for (int i = 0; i < 4; ++i) split_half(ldexpf(qsw[m][4 * tl + i], e_q), &hi[i], &lo[i]);
      const h4_t hv = {hi[0], hi[1], hi[2], hi[3]}, lv = {lo[0], lo[1], lo[2], lo[3]};
      QLw.h4(qh, tl, 0, m) = hv;
      if (HL == 1) QLw.h4(qh, tl, 0, G + m) = lv;
      else QLw.h4(qh, tl, 1, m) = lv;
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
            acc0 = mfma4(QLw.h4(qh, ks, hl, row), as_h4(kr[j].x, kr[j].y), acc0);
            acc1 = mfma4(QLw.h4(qh, ks + 1, hl, row), as_h4(kr[j].z, kr[j].w), acc1);
          }
        }
      }
      float p[G];
      for (int m = 0; m < G; ++m) {
        const float dv = (HL == 1) ? acc0[m] + acc0[G + m] + acc1[m] + acc1[G + m] : acc0[m] + acc1[m];
        const float s = tok_ok ? dv * unscale : -INFINITY;
        p[m] = softmax_step<G, HL, NDG>(m, s, tok_ok, m_run, l_acc, o0, o1, o2, o3, zacc);
      }
      stage_window_probs<G, HL>(p, PLw, lane);
      wave_sync();
      const __half* vring = reinterpret_cast<const __half*>(a.p.p[KVQ_PLANE_V_WIN]) + pair * kD * kRing;
      window_value_mfma<HL>(vring, base, nvalid, PLw, lane, row, o0, o1, o2, o3);
    }
    const float zero[G] = {};
    write_partial<G, HL>(a, b, h, a.win_slot + w, lane, m_run, l_acc, o0, o1, o2, o3, 1.0f, zero, zero);
    return;
  }

  // ================= quantized tiles: this wave's assignments (see MfmaArgs)
  const int64_t rank = (int64_t)w * a.pwgs + (blockIdx.x - a.wins);
  if (rank >= a.pairs * a.team) return;

  // this lane writes key k-step ks = tl of the query table: four channels
  int kch[4];
  float kinv[4];
  key_quad<BITS>(tl, kch, kinv);
  // KIVI key (s, z) pairs come two adjacent channels per 8-byte load: slots
  // (0, 2) and (1, 3) at 4 and 2 bits, slots (0, 1) and (2, 3) at 3 bits
  const int kmc0 = kch[0], kmc1 = BITS == 3 ? kch[2] : kch[1];
  if (TBQ)
    for (int i = 0; i < 4; ++i) kinv[i] = 1.0f;
  uint32_t lut[8];
  for (int i = 0; i < 8; ++i) lut[i] = a.g.cb_lut[i];

  const uint8_t* kplane = a.p.p[a.hi_tier ? KVQ_PLANE_K_HI : KVQ_PLANE_K_LO];
  const uint8_t* vplane = a.p.p[a.hi_tier ? KVQ_PLANE_V_HI : KVQ_PLANE_V_LO];
  const int64_t slots = a.hi_tier ? g.hi_slots : g.gmax;
  const bool ring = slots != g.gmax;
  const int64_t scale_end = g.gmax * kGroup;
  // per-pair bases of the planes
  auto kpair_of = [&](int64_t pr) { return kplane + pr * slots * TB; };
  auto vpair_of = [&](int64_t pr) { return vplane + pr * slots * TB; };
  auto kmeta_of = [&](int64_t pr) { return a.p.p[KVQ_PLANE_K_META] + pr * g.gmax * 512; };
  auto vmeta_of = [&](int64_t pr) { return a.p.p[KVQ_PLANE_V_META] + pr * g.gmax * 512; };
  constexpr int SPT = Q40 ? 4 : 1;   // fp16 scales per token (block schemes)
  auto ksc_of = [&](int64_t pr) {
    return reinterpret_cast<const uint16_t*>(a.p.p[KVQ_PLANE_K_META]) + pr * g.gmax * kGroup * SPT;
  };
  auto vsc_of = [&](int64_t pr) {
    return reinterpret_cast<const uint16_t*>(a.p.p[KVQ_PLANE_V_META]) + pr * g.gmax * kGroup * SPT;
  };

  TilePos cur_pos, nxt_pos;
  TileRaw<BITS, BLOCK> cur, nxt;
  uint8_t* stage = ST[KVQ_DECODE_STAGE ? w : 0];
  auto issue = [&](const TilePos& tp, int64_t pr) {
    stage_issue<BITS>(stage, tp, lane, kpair_of(pr), vpair_of(pr));
    meta_issue<BITS, BLOCK, false, Q40>(nxt, tp, lane, kmeta_of(pr), vmeta_of(pr), ksc_of(pr), vsc_of(pr),
                                        scale_end, kmc0, kmc1);
  };
  TileCursor cs;
  cursor_start(a, rank, cs, lane);
  int64_t cur_pair = cs.pair, cur_k = cs.k;
  tile_at(a, cs.t, slots, ring, cur_pos);
  if (KVQ_DECODE_STAGE) issue(cur_pos, cur_pair);   // in flight during the first pair's set-up

  // per-assignment state
  int64_t pair = -1, pk = 0;
  int pb = 0, ph = 0;
  float qv[G][4];
  float qabs[4];   // max over the heads of |qv|, per slot
  float qsum[G];
  float qsum4[G][4];   // Q40: sums of the query over each 32-channel slice
  float e_scale_blk = 1.0f;

  // this member's partial of `pair`
  auto flush = [&]() {
    if constexpr (V16) {
      float add[G][NDG];
      for (int m = 0; m < G; ++m)
        for (int d = 0; d < NDG; ++d) {
          const float zs = wave_sum64(zacc[m][d]);
          add[m][d] = TBQ ? 0.0f : BLOCK ? -COFF * zs : zs;
        }
      write_partial16<G, NDG>(a, pb, ph, a.slot_base + pk, lane, m_run, l_acc, acc16, TBQ ? 1.0f : 16777216.0f,
                              add);
      reset();
      return;
    }
    float add0[G], add1[G];
    for (int m = 0; m < G; ++m) {
      float zsum[NDG];
      for (int d = 0; d < NDG; ++d) zsum[d] = wave_sum64(zacc[m][d]);
      add0[m] = TBQ ? 0.0f : Q40 ? -COFF * zsum[gh] : BLOCK ? -COFF * zsum[0] : zsum[gh];
      add1[m] = TBQ ? 0.0f : Q40 ? -COFF * zsum[gh + 2] : BLOCK ? -COFF * zsum[0] : zsum[gh + 2];
    }
    write_partial<G, HL>(a, pb, ph, a.slot_base + pk, lane, m_run, l_acc, o0, o1, o2, o3, TBQ ? 1.0f : 16777216.0f,
                         add0, add1);
    reset();
  };

  bool fresh = true;   // the current tile opens an assignment
  for (;;) {
    if (fresh) {
      // ---------------- a new assignment: its pair's query (rotated for Hadamard caches)
      pair = cur_pair;
      pk = cur_k;
      pb = (int)(pair / g.Hkv);
      ph = (int)(pair % g.Hkv);
      const float qmax = wave_query<G>(a, pb, ph, g.hadamard != 0, qsw, lane);
      for (int m = 0; m < G; ++m)
        for (int i = 0; i < 4; ++i) qv[m][i] = qsw[m][kch[i]];
      for (int i = 0; i < 4; ++i) {
        qabs[i] = 0.0f;
        for (int m = 0; m < G; ++m) qabs[i] = fmaxf(qabs[i], fabsf(qv[m][i]));
      }
      wave_sync();   // the query is read before stage_probs() may overwrite it
      if (BLOCK) {
        // per-token key scales: the query table is fixed for the pair
        int ex = 0;
        if (qmax > 0.0f) frexpf(qmax, &ex);
        const int e_blk = 10 - ex;
        e_scale_blk = ldexpf(1.0f, (TBQ ? 0 : 24) - e_blk);
        for (int m = 0; m < G; ++m) {
          float s = 0.0f;
          for (int i = 0; i < 4; ++i) s += qv[m][i];
          qsum[m] = half_sum(s);   // the 32 lanes of a half cover all 128 channels
          if (Q40) {
            // k-step tl covers channels of slice tl / 8: sum over those 8 lanes
            float s8 = s;
            s8 += lane_xor<1>(s8, lane);
            s8 += lane_xor<2>(s8, lane);
            s8 += lane_xor<4>(s8, lane);
            for (int j = 0; j < 4; ++j)
              qsum4[m][j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s8), 8 * j));
          }
        }
        if (gh == 0) {
          for (int m = 0; m < G; ++m) {
            _Float16 hi[4], lo[4];
            for (int i = 0; i < 4; ++i) split_half(ldexpf(qv[m][i], e_blk) * kinv[i], &hi[i], &lo[i]);
            const h4_t hv = {hi[0], hi[1], hi[2], hi[3]}, lv = {lo[0], lo[1], lo[2], lo[3]};
            QLw.h4(0, tl, 0, m) = hv;
            if (HL == 1) QLw.h4(0, tl, 0, G + m) = lv;
            else QLw.h4(0, tl, 1, m) = lv;
          }
        }
        wave_sync();
      }
    }

    bool ends = false, more;
    if (KVQ_DECODE_STAGE) {
      // this tile has landed (and with it the claim in flight): codes from
      // the stage into registers, then the stage and the metadata registers
      // are refilled with the next tile while this one is computed
      wait_stage_landed();
      more = cursor_next(a, cs, lane, &ends);
      if (more) tile_at(a, cs.t, slots, ring, nxt_pos);
      if constexpr (V16) stage_read16<BITS, BLOCK>(cur, stage, lane);
      else stage_read<BITS, BLOCK>(cur, stage, lane);
      cur.km0 = nxt.km0; cur.km1 = nxt.km1; cur.vm = nxt.vm; cur.ks16 = nxt.ks16; cur.vs16 = nxt.vs16;
      cur.kq4 = nxt.kq4; cur.vq4 = nxt.vq4;
      wait_stage_read();
      if (more) issue(nxt_pos, cs.pair);
    } else {
      load_tile<BITS, BLOCK, false, Q40>(cur, cur_pos, lane, kpair_of(pair), vpair_of(pair), kmeta_of(pair),
                                         vmeta_of(pair), ksc_of(pair), vsc_of(pair), kmc0, kmc1);
      more = cursor_next(a, cs, lane, &ends);
      if (more) tile_at(a, cs.t, slots, ring, nxt_pos);
    }
    const int nvalid = cur_pos.nvalid;
    const bool tok_ok = lane < nvalid;
    const uint4* kc = cur.kc;
    const uint32_t (*vc)[2][BITS] = cur.vc;
    float vs[NDG], vz[NDG];
    value_meta<BITS, BLOCK, NDG, Q40>(cur, tok_ok, vs, vz);
    const float kscale = BLOCK ? half_bits_to_float(cur.ks16) : 0.0f;
    const uint2 km0 = cur.km0, km1 = cur.km1;

    // ---------------- KIVI: query table of my group (k-step tl)
    float bias[G];
    float kscale_grp = 1.0f;
    if (!BLOCK) {
      // (s, z) of slot i's channel: the words of channels kmc0, kmc0 + 1,
      // kmc1, kmc1 + 1 in slot order
      const uint32_t mw[4] = {km0.x, BITS == 3 ? km0.y : km1.x, BITS == 3 ? km1.x : km0.y, km1.y};
      float sK[4], zK[4];
      for (int i = 0; i < 4; ++i) {
        sK[i] = half_bits_to_float((uint16_t)(mw[i] & 0xFFFF));
        zK[i] = half_bits_to_float((uint16_t)(mw[i] >> 16));
      }
      float qp[G][4];
      float amax = 0.0f;
      for (int m = 0; m < G; ++m) {
        float bp = 0.0f;
        for (int i = 0; i < 4; ++i) {
          qp[m][i] = qv[m][i] * sK[i];
          bp += qv[m][i] * zK[i];
          if (G <= 2) amax = fmaxf(amax, fabsf(qp[m][i]));
        }
        bias[m] = half_sum(bp);
      }
      // four heads: max over heads of |q s| is (max over heads of |q|) |s|
      // (rounding is monotone), one product per channel
      if (G > 2)
        for (int i = 0; i < 4; ++i) amax = fmaxf(amax, qabs[i] * fabsf(sK[i]));
      amax = half_max(amax);
      int ex = 0;
      if (amax > 0.0f) frexpf(amax, &ex);
      const int e_grp = 10 - ex;
      kscale_grp = ldexpf(1.0f, 24 - e_grp);
      // 2^e_grp and the place factor (both powers of two: exact) per channel
      float fsc[4];
      for (int i = 0; i < 4; ++i) fsc[i] = ldexpf(kinv[i], e_grp);
      for (int m = 0; m < G; ++m) {
        _Float16 hi[4], lo[4];
        for (int i = 0; i < 4; ++i) split_half(qp[m][i] * fsc[i], &hi[i], &lo[i]);
        const h4_t hv = {hi[0], hi[1], hi[2], hi[3]}, lv = {lo[0], lo[1], lo[2], lo[3]};
        QLw.h4(qh, tl, 0, m) = hv;
        if (HL == 1) QLw.h4(qh, tl, 0, G + m) = lv;
        else QLw.h4(qh, tl, 1, m) = lv;
      }
      wave_sync();
    }

    // ---------------- scores: S = q' . codes over 32 k-steps (two chains)
    f4_t acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
    float sq[G];   // Q40: the score so far, slice by slice
    for (int m = 0; m < G; ++m) sq[m] = 0.0f;
    if constexpr (BITS == 3) {
      // the key row as one 384-bit string, channel c at bits 3c: k-step ks
      // takes channels 4 ks .. 4 ks + 3 in order
      uint32_t kw3[12];
      for (int j = 0; j < 3; ++j) {
        kw3[4 * j] = kc[j].x; kw3[4 * j + 1] = kc[j].y; kw3[4 * j + 2] = kc[j].z; kw3[4 * j + 3] = kc[j].w;
      }
#pragma unroll
      for (int ks = 0; ks < 32; ++ks) {
        const h4_t bk = codes3_b(kw3, ks);
        for (int hl = 0; hl < HL; ++hl) {
          if (ks & 1) acc1 = mfma4(QLw.h4(qh, ks, hl, row), bk, acc1);
          else acc0 = mfma4(QLw.h4(qh, ks, hl, row), bk, acc0);
        }
      }
    }
    for (int j = 0; j < (BITS == 3 ? 0 : NKW); ++j) {
      const uint32_t dw[4] = {kc[j].x, kc[j].y, kc[j].z, kc[j].w};
      for (int u = 0; u < 4; ++u) {
        const uint32_t xw = dw[u];
        const int i = 4 * j + u;     // canonical dword index of the row
        if (BITS == 8) {   // channels 4i .. 4i + 3, one byte each: k-step i
          const h4_t bk = as_h4(xw & 0x00FF00FFu, (xw >> 8) & 0x00FF00FFu);
          for (int hl = 0; hl < HL; ++hl) {
            if (u & 1) acc1 = mfma4(QLw.h4(qh, i, hl, row), bk, acc1);
            else acc0 = mfma4(QLw.h4(qh, i, hl, row), bk, acc0);
          }
        } else if (BITS == 4) {
          const uint32_t x8 = xw >> 8;
          uint32_t lv[4], ll[4];
          if (TBQ) tbq4_levels(xw, lut, lv, ll);
          const h4_t b0 = TBQ ? as_h4(lv[0], lv[1]) : as_h4(xw & 0x000F000Fu, xw & 0x00F000F0u);
          const h4_t b1 = TBQ ? as_h4(lv[2], lv[3]) : as_h4(x8 & 0x000F000Fu, x8 & 0x00F000F0u);
          for (int hl = 0; hl < HL; ++hl) {
            acc0 = mfma4(QLw.h4(qh, 2 * i, hl, row), b0, acc0);
            acc1 = mfma4(QLw.h4(qh, 2 * i + 1, hl, row), b1, acc1);
          }
          if (TBQ) {   // the levels' lo halves against the query's hi half
            acc0 = mfma4(QLw.h4(qh, 2 * i, 0, row), as_h4(ll[0], ll[1]), acc0);
            acc1 = mfma4(QLw.h4(qh, 2 * i + 1, 0, row), as_h4(ll[2], ll[3]), acc1);
          }
        } else {
          const uint32_t x10 = xw >> 10;
          const h4_t b0 = as_h4(xw & 0x00030003u, xw & 0x000C000Cu);
          const h4_t b1 = as_h4(xw & 0x00300030u, xw & 0x00C000C0u);
          const h4_t b2 = as_h4(xw & 0x03000300u, x10 & 0x00030003u);
          const h4_t b3 = as_h4(x10 & 0x000C000Cu, x10 & 0x00300030u);
          for (int hl = 0; hl < HL; ++hl) {
            acc0 = mfma4(QLw.h4(qh, 4 * i, hl, row), b0, acc0);
            acc1 = mfma4(QLw.h4(qh, 4 * i + 1, hl, row), b1, acc1);
            acc0 = mfma4(QLw.h4(qh, 4 * i + 2, hl, row), b2, acc0);
            acc1 = mfma4(QLw.h4(qh, 4 * i + 3, hl, row), b3, acc1);
          }
        }
      }
      // a 32-channel slice is one 16-byte piece of the row at 4 bits, two at 8
      if (Q40 && (BITS != 8 || (j & 1))) {
        // slice sl done: its scale times (q'.codes - offset sum q), then the next
        const int sl = BITS == 8 ? j >> 1 : j;
        const uint32_t kw2 = sl < 2 ? cur.kq4.x : cur.kq4.y;
        const float ksj = half_bits_to_float((uint16_t)((kw2 >> (16 * (sl & 1))) & 0xFFFF));
        for (int m = 0; m < G; ++m) {
          const float dj = (HL == 1) ? acc0[m] + acc0[G + m] + acc1[m] + acc1[G + m] : acc0[m] + acc1[m];
          sq[m] += ksj * (dj * e_scale_blk - COFF * qsum4[m][sl]);
        }
        acc0 = f4_t{0, 0, 0, 0};
        acc1 = f4_t{0, 0, 0, 0};
      }
    }
    float p[G];
    for (int m = 0; m < G; ++m) {
      const float dotv = (HL == 1) ? acc0[m] + acc0[G + m] + acc1[m] + acc1[G + m] : acc0[m] + acc1[m];
      float s;
      if (Q40) s = sq[m];
      else if (TBQ) s = kscale * (dotv * e_scale_blk);
      else if (BLOCK) s = kscale * (dotv * e_scale_blk - COFF * qsum[m]);
      else s = dotv * kscale_grp + bias[m];
      if (!tok_ok) s = -INFINITY;
      if constexpr (V16) p[m] = softmax_step16<G, NDG>(m, s, tok_ok, m_run, l_acc, acc16, zacc);
      else p[m] = softmax_step<G, HL, NDG>(m, s, tok_ok, m_run, l_acc, o0, o1, o2, o3, zacc);
    }

    // ---------------- p' = p s into the value A table; values: O += p' . codes
    if constexpr (V16) {
      stage_probs16<G, BITS, BLOCK, NDG, TBQ>(p, vs, vz, lds_addr(PL[w]), zacc, tl, gh);
      wave_sync();
      value_mfma16<BITS, NDG, TBQ>(cur.vd, lds_addr(PL[w]), lane, acc16, TBQ ? lut : nullptr);
    } else {
      stage_probs<G, BITS, BLOCK, HL, NDG, TBQ>(p, vs, vz, PLw, zacc, tl, gh);
      wave_sync();
      value_mfma<G, BITS, BLOCK, HL, NDG, TBQ>(vc, PLw, row, gh, o0, o1, o2, o3, lut);
    }
    wave_sync();

    // ---------------- the member's partial when its assignment ends
    if (ends) flush();
    if (!more) break;
    cur_pos = nxt_pos;
    cur_pair = cs.pair;
    cur_k = cs.k;
    fresh = ends;
  }
}

}  // namespace

int decode_mfma_wgs_per_cu(const Geom& g, int bits) {
  const void* fn = nullptr;
  const bool blk = g.scheme == KVQ_BLOCK128_SYM;
#define KVQ_FN(GG, BB, BL) fn = reinterpret_cast<const void*>(&decode_mfma_kernel<GG, BB, BL>)
#define KVQ_FT(GG) fn = reinterpret_cast<const void*>(&decode_mfma_kernel<GG, 4, true, true>)
#define KVQ_FQ(GG, BB) fn = reinterpret_cast<const void*>(&decode_mfma_kernel<GG, BB, true, false, true>)
  if (g.tbq4) {
    if (g.G == 1) KVQ_FT(1); else if (g.G == 2) KVQ_FT(2); else KVQ_FT(4);
  } else if (g.q40 && bits == 8) {
    if (g.G == 1) KVQ_FQ(1, 8); else if (g.G == 2) KVQ_FQ(2, 8); else KVQ_FQ(4, 8);
  } else if (g.q40) {
    if (g.G == 1) KVQ_FQ(1, 4); else if (g.G == 2) KVQ_FQ(2, 4); else KVQ_FQ(4, 4);
  } else if (blk && bits == 3) {
    if (g.G == 1) KVQ_FN(1, 3, true); else if (g.G == 2) KVQ_FN(2, 3, true); else KVQ_FN(4, 3, true);
  } else if (blk) {
    if (g.G == 1) KVQ_FN(1, 4, true); else if (g.G == 2) KVQ_FN(2, 4, true); else KVQ_FN(4, 4, true);
  } else if (bits == 4) {
    if (g.G == 1) KVQ_FN(1, 4, false); else if (g.G == 2) KVQ_FN(2, 4, false); else KVQ_FN(4, 4, false);
  } else if (bits == 3) {
    if (g.G == 1) KVQ_FN(1, 3, false); else if (g.G == 2) KVQ_FN(2, 3, false); else KVQ_FN(4, 3, false);
  } else {
    if (g.G == 1) KVQ_FN(1, 2, false); else if (g.G == 2) KVQ_FN(2, 2, false); else KVQ_FN(4, 2, false);
  }
#undef KVQ_FN
#undef KVQ_FT
#undef KVQ_FQ
  return occupancy_wgs_per_cu(fn);
}

hipError_t launch_decode_mfma(const Geom& g, const Planes& p, const ChunkPlan& cp, const __half* q,
                              float sm_scale, float* ws, hipStream_t s) {
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
    a.q_pos = 0;
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
    const bool blk = g.scheme == KVQ_BLOCK128_SYM;
#define KVQ_MF(GG, BB, BL) hipLaunchKernelGGL((decode_mfma_kernel<GG, BB, BL>), grid, block, 0, s, a)
#define KVQ_MT(GG) hipLaunchKernelGGL((decode_mfma_kernel<GG, 4, true, true>), grid, block, 0, s, a)
#define KVQ_MQ(GG, BB) hipLaunchKernelGGL((decode_mfma_kernel<GG, BB, true, false, true>), grid, block, 0, s, a)
    if (g.tbq4) {
      if (g.G == 1) KVQ_MT(1);
      else if (g.G == 2) KVQ_MT(2);
      else KVQ_MT(4);
    } else if (g.q40 && rp.bits == 8) {
      if (g.G == 1) KVQ_MQ(1, 8);
      else if (g.G == 2) KVQ_MQ(2, 8);
      else KVQ_MQ(4, 8);
    } else if (g.q40) {
      if (g.G == 1) KVQ_MQ(1, 4);
      else if (g.G == 2) KVQ_MQ(2, 4);
      else KVQ_MQ(4, 4);
    } else if (blk && rp.bits == 3) {
      if (g.G == 1) KVQ_MF(1, 3, true);
      else if (g.G == 2) KVQ_MF(2, 3, true);
      else KVQ_MF(4, 3, true);
    } else if (blk) {
      if (g.G == 1) KVQ_MF(1, 4, true);
      else if (g.G == 2) KVQ_MF(2, 4, true);
      else KVQ_MF(4, 4, true);
    } else if (rp.bits == 4) {
      if (g.G == 1) KVQ_MF(1, 4, false);
      else if (g.G == 2) KVQ_MF(2, 4, false);
      else KVQ_MF(4, 4, false);
    } else if (rp.bits == 3) {
      if (g.G == 1) KVQ_MF(1, 3, false);
      else if (g.G == 2) KVQ_MF(2, 3, false);
      else KVQ_MF(4, 3, false);
    } else {
      if (g.G == 1) KVQ_MF(1, 2, false);
      else if (g.G == 2) KVQ_MF(2, 2, false);
      else KVQ_MF(4, 2, false);
    }
#undef KVQ_MF
#undef KVQ_MT
#undef KVQ_MQ
  }
  return hipGetLastError();
}

}  // namespace kvq
