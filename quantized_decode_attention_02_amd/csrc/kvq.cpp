// libkvq C ABI: argument validation, plane layout, tier bookkeeping and
// kernel dispatch.  No device allocation, no synchronization and no mutable
// global state (the TBQ4 codebook is computed once and never changes).  The
// contract of every function is in include/kvq.h.
//
// Sources cited here:
//   [troisinh] "KV Cache Quantization — Nén cache INT4/INT3, mở khóa
//              ultra-long context" (troisinh.com).
//   [nalar]    "Kuantisasi KV Cache dengan Error Budget yang Eksplisit"
//              (nalar.dev).
#include <algorithm>
#include <cmath>
#include <cstring>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr uint64_t kAlign = 16;

bool aligned(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) % kAlign) == 0; }

kvq_status validate_config(const kvq_config* c) {
  if (c == nullptr) return KVQ_ERR_INVALID_ARG;
  if (c->head_dim <= 0 || c->num_q_heads <= 0 || c->num_kv_heads <= 0) return KVQ_ERR_INVALID_ARG;
  if (c->num_q_heads % c->num_kv_heads != 0) return KVQ_ERR_INVALID_ARG;
  if (c->scheme != KVQ_KIVI_ASYM && !block_scheme(c->scheme)) return KVQ_ERR_INVALID_ARG;
  if (c->k_bits <= 0 || c->v_bits <= 0) return KVQ_ERR_INVALID_ARG;
  if (c->hadamard != 0 && c->hadamard != 1) return KVQ_ERR_INVALID_ARG;
  if (c->pre_rope_keys != 0 && c->pre_rope_keys != 1) return KVQ_ERR_INVALID_ARG;
  if (c->pre_rope_keys && !(c->rope_theta > 0.0f && std::isfinite(c->rope_theta)))
    return KVQ_ERR_INVALID_ARG;
  if (c->int4_window != -1 && (c->int4_window <= 0 || c->int4_window % kGroup != 0))
    return KVQ_ERR_INVALID_ARG;
  const int G = c->num_q_heads / c->num_kv_heads;
  if (c->head_dim != kD) return KVQ_ERR_UNSUPPORTED;
  if (G != 1 && G != 2 && G != 4) return KVQ_ERR_UNSUPPORTED;
  if (c->k_group_tokens != kGroup || c->v_group_dims != 32) return KVQ_ERR_UNSUPPORTED;
  if (c->v_bits != c->k_bits) return KVQ_ERR_UNSUPPORTED;
  if (c->hadamard && c->pre_rope_keys) return KVQ_ERR_UNSUPPORTED;
  if (!c->hadamard)
    for (int i = 0; i < 4; ++i)
      if (c->hadamard_sign_in[i] != 0 || c->hadamard_sign_out[i] != 0) return KVQ_ERR_INVALID_ARG;
  if (c->scheme == KVQ_KIVI_ASYM) {
    if (c->k_bits != 4 && c->k_bits != 3 && c->k_bits != 2) return KVQ_ERR_UNSUPPORTED;
    if (c->fp16_window != kWindow) return KVQ_ERR_UNSUPPORTED;
    // tiers: INT4 newest, INT2 or INT3 older
    if (c->int4_window >= 0 && (c->k_bits != 4 || (c->low_bits != 2 && c->low_bits != 3)))
      return KVQ_ERR_UNSUPPORTED;
    // 3-bit codes (a 3-bit cache or a 3-bit low tier): keys stored after RoPE (or rotated)
    if ((c->k_bits == 3 || (c->int4_window >= 0 && c->low_bits == 3)) && c->pre_rope_keys)
      return KVQ_ERR_UNSUPPORTED;
  } else {
    // 3 bits: the 50-byte block of the format table (symmetric block scheme only)
    // 8 bits: Q8_0 (and only Q8_0)
    if ((c->scheme == KVQ_Q8_0) != (c->k_bits == 8)) return KVQ_ERR_UNSUPPORTED;
    if (c->k_bits != 4 && c->k_bits != 8 && !(c->k_bits == 3 && c->scheme == KVQ_BLOCK128_SYM))
      return KVQ_ERR_UNSUPPORTED;
    if (c->fp16_window != 0 || c->int4_window != -1) return KVQ_ERR_UNSUPPORTED;
    if (c->pre_rope_keys) return KVQ_ERR_UNSUPPORTED;
    // TBQ4's levels assume the near-normal coordinates of a rotated block
    if (c->scheme == KVQ_TBQ4 && !c->hadamard) return KVQ_ERR_UNSUPPORTED;
  }
  return KVQ_OK;
}

int64_t quantized_prefix(const kvq_config* c, int64_t length) {
  if (block_scheme(c->scheme)) return length;
  const int64_t r = length - kWindow;
  if (r <= 0) return 0;
  return (r / kGroup) * kGroup;
}

int64_t groups_for(int64_t max_tokens) { return (max_tokens + kGroup - 1) / kGroup; }

// The TBQ4 codebook ([trefon] "Jak 4-bitowemu cache to uchodzi: najpierw
// obrót": 16 Lloyd-Max levels fitted to N(0, 1/sqrt(128))).  Lloyd's
// iteration on the unit normal in fp64 from evenly spaced levels on [-3, 3]:
// every boundary the midpoint of its neighbours, every level the normal's
// mean over its cell, (phi(a) - phi(b)) / (Phi(b) - Phi(a)), until no level
// moves by 1e-14 (the iteration contracts by ~0.965 a step, so the levels end
// ~3e-13 from the fixed point, far inside their fp32 rounding margins).  Then
// level_k = fl32(unit level * 1/sqrt(128)), boundary_k = fl32 of the exact
// midpoint of two fp32 levels.  Computed once, immutable afterwards.
struct Tbq4Codebook {
  float level[16];
  float bound[15];
  uint32_t lut[8];
};

const Tbq4Codebook& tbq4_codebook() {
  static const Tbq4Codebook cb = [] {
    const double inv_sqrt2 = 1.0 / std::sqrt(2.0);
    auto phi = [](double x) { return std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI); };
    // Phi(b) - Phi(a), from the tail that keeps it accurate
    auto mass = [&](double a, double b) {
      if (a >= 0.0) return 0.5 * (std::erfc(a * inv_sqrt2) - std::erfc(b * inv_sqrt2));
      if (b <= 0.0) return 0.5 * (std::erfc(-b * inv_sqrt2) - std::erfc(-a * inv_sqrt2));
      return 1.0 - 0.5 * std::erfc(-a * inv_sqrt2) - 0.5 * std::erfc(b * inv_sqrt2);
    };
    double c[16];
    for (int k = 0; k < 16; ++k) c[k] = -3.0 + 6.0 * (k + 0.5) / 16.0;
    for (int it = 0; it < 10000; ++it) {
      double b[17];
      b[0] = -HUGE_VAL;
      b[16] = HUGE_VAL;
      for (int k = 0; k < 15; ++k) b[k + 1] = 0.5 * (c[k] + c[k + 1]);
      double moved = 0.0;
      double nc[16];
      for (int k = 0; k < 16; ++k) {
        const double plo = std::isinf(b[k]) ? 0.0 : phi(b[k]);
        const double phi_ = std::isinf(b[k + 1]) ? 0.0 : phi(b[k + 1]);
        nc[k] = (plo - phi_) / mass(b[k], b[k + 1]);
        moved = std::max(moved, std::fabs(nc[k] - c[k]));
      }
      for (int k = 0; k < 16; ++k) c[k] = nc[k];
      if (moved < 1e-14) break;
    }
    Tbq4Codebook r{};
    const double sigma = 1.0 / std::sqrt(128.0);
    for (int k = 0; k < 16; ++k) r.level[k] = (float)(c[k] * sigma);
    for (int k = 0; k < 15; ++k) r.bound[k] = (float)(((double)r.level[k] + (double)r.level[k + 1]) / 2.0);
    // decode's v_perm tables: each magnitude as hi = fp16(level) and
    // lo = fp16(level - hi), split into low and high bytes
    for (int m = 0; m < 8; ++m) {
      const __half hh = __float2half_rn(r.level[8 + m]);
      const uint16_t h = __half_as_ushort(hh);
      const uint16_t l = __half_as_ushort(__float2half_rn(r.level[8 + m] - __half2float(hh)));
      r.lut[m >> 2] |= (uint32_t)(h & 0xFF) << (8 * (m & 3));
      r.lut[2 + (m >> 2)] |= (uint32_t)(h >> 8) << (8 * (m & 3));
      r.lut[4 + (m >> 2)] |= (uint32_t)(l & 0xFF) << (8 * (m & 3));
      r.lut[6 + (m >> 2)] |= (uint32_t)(l >> 8) << (8 * (m & 3));
    }
    return r;
  }();
  return cb;
}

Geom make_geom(const kvq_config* c, int64_t batch, int64_t max_tokens, int64_t length) {
  Geom g;
  g.B = (int)batch;
  g.Hq = c->num_q_heads;
  g.Hkv = c->num_kv_heads;
  g.G = c->num_q_heads / c->num_kv_heads;
  g.scheme = c->scheme;
  g.hi_bits = c->k_bits;
  g.lo_bits = (c->scheme == KVQ_KIVI_ASYM && c->int4_window >= 0) ? c->low_bits : c->k_bits;
  g.hadamard = c->hadamard;
  g.tbq4 = c->scheme == KVQ_TBQ4;
  g.q40 = c->scheme == KVQ_Q4_0 || c->scheme == KVQ_Q8_0;
  {
    const Tbq4Codebook& cb = tbq4_codebook();
    for (int k = 0; k < 16; ++k) g.cb_level[k] = cb.level[k];
    for (int k = 0; k < 15; ++k) g.cb_bound[k] = cb.bound[k];
    for (int k = 0; k < 8; ++k) g.cb_lut[k] = cb.lut[k];
  }
  g.hsigned = 0;
  for (int i = 0; i < 4; ++i) {
    g.sign_in.w[i] = c->hadamard_sign_in[i];
    g.sign_out.w[i] = c->hadamard_sign_out[i];
    if (c->hadamard_sign_in[i] != 0 || c->hadamard_sign_out[i] != 0) g.hsigned = 1;
  }
  g.pre_rope = c->pre_rope_keys;
  g.rope_theta = c->rope_theta;
  g.gmax = groups_for(max_tokens);
  g.hi_slots = (c->scheme == KVQ_KIVI_ASYM && c->int4_window >= 0) ? c->int4_window / kGroup : g.gmax;
  g.length = length;
  g.Tq = quantized_prefix(c, length);
  g.hi_start = (c->scheme == KVQ_KIVI_ASYM && c->int4_window >= 0)
                   ? (g.Tq > c->int4_window ? g.Tq - c->int4_window : 0)
                   : 0;
  return g;
}

void plane_sizes(const kvq_config* c, int64_t batch, int64_t max_tokens, uint64_t* sz) {
  for (int i = 0; i < KVQ_MAX_PLANES; ++i) sz[i] = 0;
  const uint64_t pairs = (uint64_t)batch * c->num_kv_heads;
  const uint64_t G = (uint64_t)groups_for(max_tokens);
  if (c->scheme == KVQ_KIVI_ASYM) {
    const uint64_t hs = c->int4_window >= 0 ? (uint64_t)(c->int4_window / kGroup) : G;
    sz[KVQ_PLANE_K_HI] = pairs * hs * 512 * c->k_bits;
    sz[KVQ_PLANE_V_HI] = pairs * hs * 512 * c->v_bits;
    if (c->int4_window >= 0) {
      sz[KVQ_PLANE_K_LO] = pairs * G * 512 * c->low_bits;
      sz[KVQ_PLANE_V_LO] = pairs * G * 512 * c->low_bits;
    }
    sz[KVQ_PLANE_K_META] = pairs * G * 512;
    sz[KVQ_PLANE_V_META] = pairs * G * 512;
    sz[KVQ_PLANE_K_WIN] = pairs * kRing * kD * 2;
    sz[KVQ_PLANE_V_WIN] = pairs * kRing * kD * 2;
  } else {
    sz[KVQ_PLANE_K_HI] = pairs * G * 512 * c->k_bits;
    sz[KVQ_PLANE_V_HI] = pairs * G * 512 * c->v_bits;
    const uint64_t per_token = (c->scheme == KVQ_Q4_0 || c->scheme == KVQ_Q8_0) ? 4 : 1;   // fp16 scales
    sz[KVQ_PLANE_K_META] = pairs * G * kGroup * 2 * per_token;
    sz[KVQ_PLANE_V_META] = pairs * G * kGroup * 2 * per_token;
  }
  if (c->pre_rope_keys) sz[KVQ_PLANE_ROPE] = G * kGroup * 64 * 2 * 4;
}

kvq_status validate_cache(const kvq_config* c, const kvq_cache* cache, Planes* planes) {
  if (cache == nullptr) return KVQ_ERR_INVALID_ARG;
  if (cache->batch <= 0 || cache->batch > 65535 || cache->max_tokens < 0) return KVQ_ERR_INVALID_ARG;
  if (cache->length < 0 || cache->length > cache->max_tokens) return KVQ_ERR_INVALID_ARG;
  uint64_t sz[KVQ_MAX_PLANES];
  plane_sizes(c, cache->batch, cache->max_tokens, sz);
  for (int i = 0; i < KVQ_NUM_PLANES; ++i) {
    planes->p[i] = static_cast<uint8_t*>(cache->planes[i]);
    if (sz[i] > 0 && (cache->planes[i] == nullptr || !aligned(cache->planes[i])))
      return KVQ_ERR_INVALID_ARG;
  }
  return KVQ_OK;
}

kvq_status from_hip(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP; }

// Workspace bytes of a decode call: the chunk counters, then the partials.
uint64_t workspace_need(const Geom& g, const ChunkPlan& cp) {
  if (cp.n == 0) return 0;
  return ((uint64_t)cp.ctr_floats + (uint64_t)g.B * g.Hq * cp.n * kPartial) * sizeof(float);
}

struct DecodeSetup {
  Geom g;
  Planes p;
  ChunkPlan cp;
  float scale;
};

kvq_status decode_setup(const kvq_config* cfg, const kvq_cache* cache, const void* q, void* out,
                        void* workspace, uint64_t workspace_bytes, float sm_scale, DecodeSetup* st) {
  kvq_status s = validate_config(cfg);
  if (s != KVQ_OK) return s;
  s = validate_cache(cfg, cache, &st->p);
  if (s != KVQ_OK) return s;
  if (q == nullptr || out == nullptr || !aligned(q) || !aligned(out)) return KVQ_ERR_INVALID_ARG;
  if (!std::isfinite(sm_scale)) return KVQ_ERR_INVALID_ARG;
  st->g = make_geom(cfg, cache->batch, cache->max_tokens, cache->length);
  st->cp = plan_chunks(st->g);
  const uint64_t need = workspace_need(st->g, st->cp);
  if (need > 0 && (workspace == nullptr || !aligned(workspace))) return KVQ_ERR_INVALID_ARG;
  if (workspace_bytes < need) return KVQ_ERR_WORKSPACE;
  st->scale = sm_scale > 0.0f ? sm_scale : 1.0f / std::sqrt((float)kD);
  return KVQ_OK;
}

}  // namespace

// Split-K plan.  The quantized tokens form up to two ranges of one code width
// each (low-bit tier, high-bit tier), one launch each.  A launch runs as many
// waves as fit on the device at once, as a team of equal size per pair (one
// wave handles several pairs in turn when pairs outnumber waves); a team is
// no larger than half its pair's tile count (a wave's set-up, the query and
// its partial record, then serves at least two tiles: the INT4 window range
// of an INT4-over-INT2 cache, 64 tiles a pair, took 26 of cfg3's 274 us at one
// tile a wave).  Chunks are one tile, or two where
// every member gets at least 8 chunks on average, so that a claim has a
// tile's time to come back; teams above 2 * kTeamPerChunkTile waves take
// team / kTeamPerChunkTile tiles per chunk.  The last team tiles of a pair
// go as single-tile chunks, so that its members' last claims are short and
// they finish close together.  The fp16 window rides on the last launch:
// one more work-group per pair.
#ifndef KVQ_DECODE_CHUNK_MIN
#define KVQ_DECODE_CHUNK_MIN 1
#endif
#ifndef KVQ_DECODE_CHUNK_MAX
#define KVQ_DECODE_CHUNK_MAX 2
#endif
#ifndef KVQ_MIN_TILES_PER_WAVE
#define KVQ_MIN_TILES_PER_WAVE 2
#endif
constexpr int64_t kMinTilesPerWave = KVQ_MIN_TILES_PER_WAVE;
#ifndef KVQ_TEAM_PER_CHUNK_TILE
#define KVQ_TEAM_PER_CHUNK_TILE 16
#endif
constexpr int64_t kTeamPerChunkTile = KVQ_TEAM_PER_CHUNK_TILE;
// Single-tile chunks at the end of a pair's range, per team member.
#ifndef KVQ_DECODE_TAIL_TILES_PER_MEMBER
#define KVQ_DECODE_TAIL_TILES_PER_MEMBER 1
#endif

// Asked of the runtime on every plan (a pure function of the kernel binary
// and the current device; nothing is cached).
int occupancy_wgs_per_cu(const void* kernel) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, 256, 0) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    n = 2;   // no device: a plan that is valid everywhere, if not the fastest
  }
  return n;
}

int device_compute_units() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    cus = 256;
  }
  return cus;
}

ChunkPlan plan_chunks(const Geom& g) {
  // the device's resident waves for the kernel of the widest range (ranges
  // of one call differ only in code width; each is capped by its own kernel)
  return plan_chunks(g, -1);
}

ChunkPlan plan_chunks(const Geom& g, int64_t cap_waves) {
  ChunkPlan cp;
  cp.nr = 0;
  const int64_t pairs = (int64_t)g.B * g.Hkv;
  const bool window = g.scheme == KVQ_KIVI_ASYM && g.length > g.Tq;
  const int64_t lo_end = g.scheme == KVQ_KIVI_ASYM ? g.hi_start : 0;
  auto add = [&](int64_t t_lo, int64_t t_hi, int bits, int hi_tier) {
    RangePlan& r = cp.r[cp.nr++];
    r.t_lo = t_lo;
    r.t_hi = t_hi;
    r.bits = bits;
    r.hi_tier = hi_tier;
    r.tiles_pp = (t_hi - t_lo + 63) / 64;
    r.pwgs = 0;
    r.window = 0;
    r.team = 0;
    r.chunk = 1;
    r.n_chunks = 0;
    r.n_big = 0;
    if (r.tiles_pp > 0) {
      int64_t cap = cap_waves;   // waves
      if (cap <= 0) {
        const int per_cu = g.pre_rope ? decode_rope_wgs_per_cu(g, bits) : decode_mfma_wgs_per_cu(g, bits);
        cap = 4 * (int64_t)per_cu * device_compute_units();
      }
      if (cap > kMaxPlanWaves) cap = kMaxPlanWaves;
      int64_t team = pairs <= cap ? cap / pairs : 1;
      const int64_t most = (r.tiles_pp + kMinTilesPerWave - 1) / kMinTilesPerWave;
      if (team > most) team = most;
      r.chunk = (KVQ_DECODE_CHUNK_MAX >= 2 && r.tiles_pp >= 16 * team) ? 2 : 1;
      if (r.chunk < KVQ_DECODE_CHUNK_MIN && r.tiles_pp >= 8 * team * KVQ_DECODE_CHUNK_MIN)
        r.chunk = KVQ_DECODE_CHUNK_MIN;
      // large teams: fewer, longer chunks, so one counter is not claimed more
      // often than its atomics can be served
      const int64_t wide = team / kTeamPerChunkTile;
      if (wide > r.chunk && r.tiles_pp >= 8 * team * wide) r.chunk = wide;
      // the last team * KVQ_DECODE_TAIL_TILES_PER_MEMBER tiles (or fewer) go
      // as single-tile chunks
      const int64_t tail = r.chunk > 1 ? team * KVQ_DECODE_TAIL_TILES_PER_MEMBER : 0;
      r.n_big = r.tiles_pp > tail ? (r.tiles_pp - tail) / r.chunk : 0;
      r.n_chunks = r.n_big + (r.tiles_pp - r.n_big * r.chunk);
      if (team > r.n_chunks) team = r.n_chunks;
      r.team = team;
      const int64_t waves = pairs * team < cap ? pairs * team : cap;
      r.pwgs = (waves + 3) / 4;
    }
  };
  if (lo_end > 0) add(0, lo_end, g.lo_bits, 0);
  if (g.Tq > lo_end || window) add(lo_end, g.Tq, g.hi_bits, 1);
  int64_t slot = 0;
  for (int i = 0; i < cp.nr; ++i) {
    cp.r[i].slot_base = slot;
    slot += cp.r[i].team;
  }
  cp.nq = slot;
  if (window) cp.r[cp.nr - 1].window = 1;
  cp.n = cp.nq + (window ? 4 : 0);
  cp.ctr_floats = counter_words(pairs);
  return cp;
}

}  // namespace kvq

using namespace kvq;

extern "C" {

int32_t kvq_abi_version(void) { return KVQ_ABI_VERSION; }

const char* kvq_strerror(kvq_status status) {
  switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID_ARG: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVQ_ERR_CAPACITY: return "cache capacity exceeded";
    case KVQ_ERR_WORKSPACE: return "workspace too small";
    case KVQ_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

kvq_status kvq_layout(const kvq_config* cfg, int64_t batch, int64_t max_tokens, kvq_layout_t* out) {
  kvq_status s = validate_config(cfg);
  if (s != KVQ_OK) return s;
  if (out == nullptr || batch <= 0 || batch > 65535 || max_tokens < 0) return KVQ_ERR_INVALID_ARG;
  std::memset(out, 0, sizeof(*out));
  plane_sizes(cfg, batch, max_tokens, out->plane_bytes);
  out->alignment = kAlign;
  out->groups = groups_for(max_tokens);
  out->hi_slots = (cfg->scheme == KVQ_KIVI_ASYM && cfg->int4_window >= 0) ? cfg->int4_window / kGroup
                                                                           : out->groups;
  return KVQ_OK;
}

kvq_status kvq_workspace_bytes(const kvq_config* cfg, int64_t batch, int64_t length, uint64_t* bytes) {
  kvq_status s = validate_config(cfg);
  if (s != KVQ_OK) return s;
  if (bytes == nullptr || batch <= 0 || batch > 65535 || length < 0) return KVQ_ERR_INVALID_ARG;
  // the plan of the largest launch any device may run: a team per pair is
  // never smaller on a larger device, so this covers every device's plan
  const Geom g = make_geom(cfg, batch, length, length);
  const ChunkPlan cp = plan_chunks(g, kMaxPlanWaves);
  *bytes = workspace_need(g, cp);
  return KVQ_OK;
}

kvq_status kvq_append(const kvq_config* cfg, kvq_cache* cache, const void* k_new, const void* v_new,
                      int64_t n_new, void* stream) {
  kvq_status s = validate_config(cfg);
  if (s != KVQ_OK) return s;
  Planes p;
  s = validate_cache(cfg, cache, &p);
  if (s != KVQ_OK) return s;
  if (n_new < 0) return KVQ_ERR_INVALID_ARG;
  if (n_new == 0) return KVQ_OK;
  if (k_new == nullptr || v_new == nullptr || !aligned(k_new) || !aligned(v_new))
    return KVQ_ERR_INVALID_ARG;
  const int64_t T0 = cache->length, T1 = T0 + n_new;
  if (T1 > cache->max_tokens) return KVQ_ERR_CAPACITY;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Geom g = make_geom(cfg, cache->batch, cache->max_tokens, T0);
  const __half* kn = static_cast<const __half*>(k_new);
  const __half* vn = static_cast<const __half*>(v_new);
  hipError_t e = hipSuccess;
  if (cfg->pre_rope_keys) {
    e = launch_rope_table(g, p, T0, T1, st);
    if (e != hipSuccess) return from_hip(e);
  }
  if (block_scheme(cfg->scheme)) {
    e = launch_block128_append(g, p, kn, vn, n_new, T0, st);
  } else {
    // Tier bookkeeping ([troisinh] "Ý tưởng cốt lõi", "Mixed Precision"): the
    // quantized prefix grows by whole 32-token groups; groups older than the
    // high-bit window drop to low_bits.
    const int64_t Tq0 = quantized_prefix(cfg, T0), Tq1 = quantized_prefix(cfg, T1);
    int64_t h0 = 0, h1 = 0, d1 = 0;
    if (cfg->int4_window >= 0) {
      h0 = Tq0 > cfg->int4_window ? Tq0 - cfg->int4_window : 0;
      h1 = Tq1 > cfg->int4_window ? Tq1 - cfg->int4_window : 0;
      d1 = (Tq0 < h1 ? Tq0 : h1);
    }
    if (n_new <= kSmallAppendMax) {
      // decode-sized append: one fused launch (the window write starts at T0,
      // since fewer than 128 new tokens never reach the quantized prefix)
      e = launch_kivi_small_append(g, p, kn, vn, n_new, T0, h0 / kGroup, d1 / kGroup, Tq0 / kGroup,
                                   Tq1 / kGroup, h1, st);
    } else {
      if (d1 > h0) {
        e = launch_kivi_demote(g, p, h0 / kGroup, d1 / kGroup, st);
        if (e != hipSuccess) return from_hip(e);
      }
      e = launch_kivi_quantize(g, p, kn, vn, n_new, T0, Tq0 / kGroup, Tq1 / kGroup, h1, st);
      if (e != hipSuccess) return from_hip(e);
      const int64_t w0 = T0 > Tq1 ? T0 : Tq1;
      e = launch_window_write(g, p, kn, vn, n_new, T0, w0, T1, st);
    }
  }
  if (e != hipSuccess) return from_hip(e);
  cache->length = T1;
  return KVQ_OK;
}

kvq_status kvq_decode_partials(const kvq_config* cfg, const kvq_cache* cache, const void* q,
                               int64_t q_pos, float sm_scale, void* out, void* workspace,
                               uint64_t workspace_bytes, void* stream) {
  DecodeSetup st;
  kvq_status s = decode_setup(cfg, cache, q, out, workspace, workspace_bytes, sm_scale, &st);
  if (s != KVQ_OK) return s;
  return from_hip(launch_decode_partials(st.g, st.p, st.cp, static_cast<const __half*>(q), q_pos,
                                         st.scale, static_cast<float*>(workspace),
                                         static_cast<hipStream_t>(stream)));
}

kvq_status kvq_decode_merge(const kvq_config* cfg, const kvq_cache* cache, const void* q,
                            int64_t q_pos, float sm_scale, void* out, void* workspace,
                            uint64_t workspace_bytes, void* stream) {
  DecodeSetup st;
  kvq_status s = decode_setup(cfg, cache, q, out, workspace, workspace_bytes, sm_scale, &st);
  if (s != KVQ_OK) return s;
  (void)q_pos;
  return from_hip(launch_decode_merge(st.g, st.cp, static_cast<float*>(workspace),
                                      static_cast<float*>(out), static_cast<hipStream_t>(stream)));
}

kvq_status kvq_decode_attn(const kvq_config* cfg, const kvq_cache* cache, const void* q,
                           int64_t q_pos, float sm_scale, void* out, void* workspace,
                           uint64_t workspace_bytes, void* stream) {
  kvq_status s = kvq_decode_partials(cfg, cache, q, q_pos, sm_scale, out, workspace, workspace_bytes,
                                     stream);
  if (s != KVQ_OK) return s;
  return kvq_decode_merge(cfg, cache, q, q_pos, sm_scale, out, workspace, workspace_bytes, stream);
}

kvq_status kvq_decode_attn_static(const kvq_config* cfg, const kvq_cache* cache, const void* q,
                                  int64_t q_pos, float sm_scale, void* out, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KVQ_ERR_HIP;
  if (st != nullptr) {
    // the workspace address below is the current device's: the stream must
    // belong to it
    hipDevice_t sdev = 0;
    if (hipStreamGetDevice(st, &sdev) != hipSuccess) return KVQ_ERR_HIP;
    if ((int)sdev != dev) return KVQ_ERR_INVALID_ARG;
  }
  void* ws = nullptr;
  if (static_workspace(dev, &ws) != hipSuccess) return KVQ_ERR_HIP;
  DecodeSetup su;
  // KVQ_ERR_WORKSPACE here: the call needs more than the static array holds
  const kvq_status s = decode_setup(cfg, cache, q, out, ws, KVQ_STATIC_WORKSPACE_BYTES, sm_scale, &su);
  if (s != KVQ_OK) return s;
  float* w = static_cast<float*>(ws);
  hipError_t e = launch_zero_counters(su.cp, w, st);
  if (e == hipSuccess)
    e = launch_decode_partials(su.g, su.p, su.cp, static_cast<const __half*>(q), q_pos, su.scale, w, st);
  if (e == hipSuccess) e = launch_decode_merge(su.g, su.cp, w, static_cast<float*>(out), st);
  return from_hip(e);
}

kvq_status kvq_dequant(const kvq_config* cfg, const kvq_cache* cache, int64_t t0, int64_t t1,
                       void* k_out, void* v_out, void* stream) {
  kvq_status s = validate_config(cfg);
  if (s != KVQ_OK) return s;
  Planes p;
  s = validate_cache(cfg, cache, &p);
  if (s != KVQ_OK) return s;
  if (t0 < 0 || t1 < t0 || t1 > cache->length) return KVQ_ERR_INVALID_ARG;
  if (t1 == t0) return KVQ_OK;
  if (k_out == nullptr || v_out == nullptr || !aligned(k_out) || !aligned(v_out))
    return KVQ_ERR_INVALID_ARG;
  const Geom g = make_geom(cfg, cache->batch, cache->max_tokens, cache->length);
  return from_hip(launch_dequant(g, p, t0, t1, static_cast<float*>(k_out), static_cast<float*>(v_out),
                                 static_cast<hipStream_t>(stream)));
}

}  // extern "C"
