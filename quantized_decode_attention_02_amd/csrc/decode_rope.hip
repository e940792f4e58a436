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
// softmax").  Values, softmax, window and partials are those of the other
// MFMA decode (decode_common.h).
#include "decode_common.h"

namespace kvq {
namespace {

__device__ __forceinline__ f4_t mfma1(float x, float y, f4_t c) {
  return __builtin_amdgcn_mfma_f32_4x4x1f32(x, y, c, 0, 0, 0);
}

template <int B>
__device__ __forceinline__ float ubyte_f32(uint32_t v) {   // byte B of v as fp32 (pure ALU)
  float r;
  if (B == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(v));
  else if (B == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(v));
  else if (B == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(v));
  else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(v));
  return r;
}
template <int BITS, int K>
__device__ __forceinline__ float key_int(uint32_t w) {
  constexpr int SH = BITS == 4 ? 4 * (K & 1) : 2 * (K & 3);
  constexpr int BYTE = BITS == 4 ? (K >> 1) : (K >> 2);
  const uint32_t src = (w >> SH) & (BITS == 4 ? 0x0F0F0F0Fu : 0x03030303u);
  return ubyte_f32<BYTE>(src);
}
template <int BITS>
__device__ __forceinline__ void codes_int(uint32_t w, float* n) {
  constexpr int CPW = 32 / BITS;
  if constexpr (BITS == 4) {
    n[0] = key_int<4, 0>(w); n[1] = key_int<4, 1>(w); n[2] = key_int<4, 2>(w); n[3] = key_int<4, 3>(w);
    n[4] = key_int<4, 4>(w); n[5] = key_int<4, 5>(w); n[6] = key_int<4, 6>(w); n[7] = key_int<4, 7>(w);
  } else {
    n[0] = key_int<2, 0>(w); n[1] = key_int<2, 1>(w); n[2] = key_int<2, 2>(w); n[3] = key_int<2, 3>(w);
    n[4] = key_int<2, 4>(w); n[5] = key_int<2, 5>(w); n[6] = key_int<2, 6>(w); n[7] = key_int<2, 7>(w);
    n[8] = key_int<2, 8>(w); n[9] = key_int<2, 9>(w); n[10] = key_int<2, 10>(w); n[11] = key_int<2, 11>(w);
    n[12] = key_int<2, 12>(w); n[13] = key_int<2, 13>(w); n[14] = key_int<2, 14>(w); n[15] = key_int<2, 15>(w);
  }
  (void)CPW;
}

template <int G, int BITS>
__global__ __launch_bounds__(256, 2) void decode_rope_kernel(MfmaArgs a) {
  constexpr int HL = (G <= 2) ? 1 : 2;   // value-side MFMAs per k-step (hi/lo of p')
  constexpr int NDG = 4;                 // value scale groups per token
  constexpr int TB = 512 * BITS;         // tile bytes
  constexpr int CPW = 32 / BITS;         // channels per code word
  const Geom& g = a.g;
  __shared__ __attribute__((aligned(16))) float DT[32][32][4];     // [j / 2][d]: cos, sin of j, j + 1
  // per wave: waves never wait for each other after the table above.  Rows
  // are padded by 16 bytes so that the rows one read gathers (group and head
  // of QA, group of KSZ) fall in different banks.
  __shared__ __attribute__((aligned(16))) float QA[4][2][4][kD + 4];   // [wave][group][head][channel]
  // [wave][group][j]: the fp16 (s, z) words of channels j and j + 64, as
  // stored; 66 rows so that the two groups' rows fall in different banks
  __shared__ __attribute__((aligned(16))) uint32_t KSZ[4][2][66][2];
  using PTab = ATab<HL, 16, G == 4, G == 4>;
  __shared__ __attribute__((aligned(16))) _Float16 PL[4][NDG * PTab::T];

  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index is uniform: read it into a scalar register, so that the
  // tile walk and its addresses stay on the scalar unit
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gh = lane >> 5, tl = lane & 31, row = lane & 3;
  const float* rope_tab = reinterpret_cast<const float*>(a.p.p[KVQ_PLANE_ROPE]);
  float qx[G], qy[G];   // R(q_pos) q, scaled: channels lane and lane + 64 of every head

  // ---------------- offset table (rows 0..31 of the RoPE table: the plane
  // always holds at least 32 rows; rows at or past the cache length are only
  // used for masked tokens), zeroed tables
  for (int e = tid; e < 32 * 32; e += 256) {
    const int jp = e >> 5, d = e & 31;
    *reinterpret_cast<float4*>(&DT[jp][d][0]) = *reinterpret_cast<const float4*>(rope_tab + d * 128 + 4 * jp);
  }
  for (int e = lane; e < (int)(sizeof(QA[0]) / 4); e += 64) (&QA[w][0][0][0])[e] = 0.0f;
  for (int e = lane; e < (int)(sizeof(PL[0]) / 2); e += 64) PL[w][e] = (_Float16)0.0f;
  lds_barrier();

  // the query of (b, h) at q_pos: R(q_pos) q (fp64 angles), scaled; lane j
  // takes channel pair j of every head
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

  // RoPE table rows of a tile's group starts t0 and t0 + 32 (t0 twice when
  // the tile has one group): lane j loads the cos / sin of pair j
  auto group_rows = [&](int64_t t0, bool second, float2* cs) {
    cs[0] = *reinterpret_cast<const float2*>(rope_tab + t0 * 128 + 2 * lane);
    cs[1] = *reinterpret_cast<const float2*>(rope_tab + (second ? t0 + 32 : t0) * 128 + 2 * lane);
  };
  // query tables of the two groups of a tile from their rows: u = R(-t0) qs,
  // lane j writes channels j and j + 64 of every head
  auto build_query_rows = [&](const float2* rows) {
    for (int gg = 0; gg < 2; ++gg) {
      const float2 cs = rows[gg];
      for (int m = 0; m < G; ++m) {
        const float x = qx[m], y = qy[m];
        QA[w][gg][m][lane] = x * cs.x + y * cs.y;
        QA[w][gg][m][lane + 64] = y * cs.x - x * cs.y;
      }
    }
    wave_sync();
  };
  auto build_query = [&](int64_t t0, bool second) {
    float2 rows[2];
    group_rows(t0, second, rows);
    build_query_rows(rows);
  };

  float m_run[G], l_acc[G];
  float zacc[G][NDG];
  f4_t o0, o1, o2, o3;
  auto reset = [&]() {
    for (int m = 0; m < G; ++m) {
      m_run[m] = -INFINITY;
      l_acc[m] = 0.0f;
      for (int d = 0; d < NDG; ++d) zacc[m][d] = 0.0f;
    }
    o0 = f4_t{0, 0, 0, 0}; o1 = o0; o2 = o0; o3 = o0;
  };
  reset();

  // Scores of this lane's token from its 128 key values x_c (fp32), rotated
  // by d = tl: four accumulator chains, one MFMA per channel.
  auto score_pairs = [&](const float* xl, const float* xh, int j0, int np, f4_t* acc) {
    for (int k = 0; k < np; k += 2) {
      const int j = j0 + k;
      const float4 cs = *reinterpret_cast<const float4*>(&DT[j >> 1][tl][0]);
      const float4 qa = *reinterpret_cast<const float4*>(&QA[w][gh][row][j & ~3]);
      const float4 qb = *reinterpret_cast<const float4*>(&QA[w][gh][row][64 + (j & ~3)]);
      const float qal[4] = {qa.x, qa.y, qa.z, qa.w}, qbl[4] = {qb.x, qb.y, qb.z, qb.w};
      for (int e = 0; e < 2; ++e) {
        const float c = e ? cs.z : cs.x, s = e ? cs.w : cs.y;
        const float x = xl[k + e], y = xh[k + e];
        const float rl = x * c - y * s, rh = x * s + y * c;
        acc[2 * e] = mfma1(qal[(j + e) & 3], rl, acc[2 * e]);
        acc[2 * e + 1] = mfma1(qbl[(j + e) & 3], rh, acc[2 * e + 1]);
      }
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
      build_query(base, nvalid > 32);
      const bool tok_ok = lane < nvalid;
      const __half* krow = reinterpret_cast<const __half*>(a.p.p[KVQ_PLANE_K_WIN]) +
                           (pair * kRing + (base + lane) % kRing) * kD;
      f4_t acc[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
      for (int i = 0; i < 8; ++i) {   // channels 8i..8i+7 and 64 + 8i..
        float xl[8], xh[8];
        const uint4 lo = tok_ok ? *reinterpret_cast<const uint4*>(krow + 8 * i) : make_uint4(0, 0, 0, 0);
        const uint4 hi = tok_ok ? *reinterpret_cast<const uint4*>(krow + 64 + 8 * i) : make_uint4(0, 0, 0, 0);
        const __half* hl = reinterpret_cast<const __half*>(&lo);
        const __half* hh = reinterpret_cast<const __half*>(&hi);
        for (int e = 0; e < 8; ++e) {
          xl[e] = __half2float(hl[e]);
          xh[e] = __half2float(hh[e]);
        }
        score_pairs(xl, xh, 8 * i, 8, acc);
      }
      float p[G];
      for (int m = 0; m < G; ++m) {
        const float s = tok_ok ? (acc[0][m] + acc[1][m]) + (acc[2][m] + acc[3][m]) : -INFINITY;
        p[m] = softmax_step<G, HL, NDG>(m, s, tok_ok, m_run, l_acc, o0, o1, o2, o3, zacc);
      }
      stage_window_probs<G, HL>(p, PTab{PL[w]}, lane);
      wave_sync();
      const __half* vring = reinterpret_cast<const __half*>(a.p.p[KVQ_PLANE_V_WIN]) + pair * kD * kRing;
      window_value_mfma<HL>(vring, base, nvalid, PTab{PL[w]}, lane, row, o0, o1, o2, o3);
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

  TilePos cur_pos, nxt_pos;
  TileRaw<BITS, false> cur, nxt;
  float2 cur_rows[2], nxt_rows[2];   // group_rows() of the tile, loaded with it
  int64_t pair = -1, pk = 0;
  int pb = 0, ph = 0;

  // this member's partial of `pair`
  auto flush = [&]() {
    float add0[G], add1[G];
    for (int m = 0; m < G; ++m) {
      float zsum[NDG];
      for (int d = 0; d < NDG; ++d) zsum[d] = wave_sum64(zacc[m][d]);
      add0[m] = zsum[gh];
      add1[m] = zsum[gh + 2];
    }
    write_partial<G, HL>(a, pb, ph, a.slot_base + pk, lane, m_run, l_acc, o0, o1, o2, o3, 16777216.0f,
                         add0, add1);
    reset();
  };
  auto fetch = [&](TileRaw<BITS, false>& r, const TilePos& tp, int64_t pr) {
    load_tile<BITS, false, true>(r, tp, lane, kplane + pr * slots * TB, vplane + pr * slots * TB,
                                 a.p.p[KVQ_PLANE_K_META] + pr * g.gmax * 512,
                                 a.p.p[KVQ_PLANE_V_META] + pr * g.gmax * 512, nullptr, nullptr, 0, 0);
  };

  TileCursor cs;
  cursor_start(a, rank, cs, lane);
  tile_at(a, cs.t, slots, ring, cur_pos);
  fetch(cur, cur_pos, cs.pair);
  group_rows(cur_pos.base, cur_pos.nvalid > 32, cur_rows);
  bool fresh = true;   // the current tile opens an assignment
  // One tile: the next one's loads go out into n, then c is computed.  The
  // loop below alternates the two buffers, so no tile is copied.
  auto tile_step = [&](TileRaw<BITS, false>& c, const TilePos& c_pos, const float2* c_rows,
                       TileRaw<BITS, false>& n, TilePos& n_pos, float2* n_rows) -> bool {
    if (fresh) {
      pair = cs.pair;
      pk = cs.k;
      pb = (int)(pair / g.Hkv);
      ph = (int)(pair % g.Hkv);
      load_query(pb, ph);
    }
    // the next tile's loads go out before this one is computed
    bool ends = false;
    const bool more = cursor_next(a, cs, lane, &ends);
    if (more) {
      tile_at(a, cs.t, slots, ring, n_pos);
      fetch(n, n_pos, cs.pair);
      group_rows(n_pos.base, n_pos.nvalid > 32, n_rows);
    }
    const int nvalid = c_pos.nvalid;
    const bool tok_ok = lane < nvalid;
    float vs[NDG], vz[NDG];
    value_meta<BITS, false, NDG>(c, tok_ok, vs, vz);

    // key (s, z) words of both groups into KSZ (channel ch -> pair ch mod 64, half ch / 64)
    {
      const uint32_t mw[4] = {c.kmr.x, c.kmr.y, c.kmr.z, c.kmr.w};
      for (int e = 0; e < 4; ++e) {
        const int ch = 4 * tl + e;
        KSZ[w][gh][ch & 63][ch >> 6] = mw[e];
      }
    }
    build_query_rows(c_rows);   // its wave barrier also covers KSZ

    // ---------------- scores
    f4_t acc[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
    uint32_t kw[4 * BITS];
    for (int j = 0; j < BITS; ++j) {
      kw[4 * j] = c.kc[j].x; kw[4 * j + 1] = c.kc[j].y;
      kw[4 * j + 2] = c.kc[j].z; kw[4 * j + 3] = c.kc[j].w;
    }
#pragma unroll
    for (int i = 0; i < 2 * BITS; ++i) {   // words of channels [CPW i, CPW (i + 1)) and 64 + ...
      float xl[CPW], xh[CPW];
      float nl[CPW], nh[CPW];   // the codes as exact fp32 integers
      codes_int<BITS>(kw[i], nl);
      codes_int<BITS>(kw[i + 2 * BITS], nh);
      for (int k = 0; k < CPW; k += 2) {
        // the (s, z) words of channels k, k + 1 and their partners k + 64, k + 65
        const uint4 sz = *reinterpret_cast<const uint4*>(&KSZ[w][gh][CPW * i + k][0]);
        const uint32_t szw[4] = {sz.x, sz.y, sz.z, sz.w};
        for (int e = 0; e < 2; ++e) {
          const h2_t lo = __builtin_bit_cast(h2_t, szw[2 * e]), hi = __builtin_bit_cast(h2_t, szw[2 * e + 1]);
          // x = n s + z with one rounding (the product is exact)
          xl[k + e] = __builtin_fmaf(nl[k + e], (float)lo.x, (float)lo.y);
          xh[k + e] = __builtin_fmaf(nh[k + e], (float)hi.x, (float)hi.y);
        }
      }
      score_pairs(xl, xh, CPW * i, CPW, acc);
    }
    float p[G];
    for (int m = 0; m < G; ++m) {
      const float s = tok_ok ? (acc[0][m] + acc[1][m]) + (acc[2][m] + acc[3][m]) : -INFINITY;
      p[m] = softmax_step<G, HL, NDG>(m, s, tok_ok, m_run, l_acc, o0, o1, o2, o3, zacc);
    }

    // ---------------- values
    stage_probs<G, BITS, false, HL, NDG>(p, vs, vz, PTab{PL[w]}, zacc, tl, gh);
    wave_sync();
    value_mfma<G, BITS, false, HL, NDG>(c.vc, PTab{PL[w]}, row, gh, o0, o1, o2, o3);
    wave_sync();

    if (ends) flush();
    fresh = ends;
    return more;
  };
  for (;;) {
    if (!tile_step(cur, cur_pos, cur_rows, nxt, nxt_pos, nxt_rows)) break;
    if (!tile_step(nxt, nxt_pos, nxt_rows, cur, cur_pos, cur_rows)) break;
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
