// Internal declarations shared by the C ABI (kvq.cpp) and the HIP kernels.
// Not part of the public interface; see include/kvq.h for the contract.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

constexpr int kD = 128;        // head dim
constexpr int kGroup = 32;     // tokens per key group / tile
constexpr int kRing = 160;     // fp16 window ring rows (>= 128 + 31)
constexpr int kWindow = 128;   // fp16 window length

// 128 sign bits: bit i of w[i / 32] negates coordinate i.
struct Mask128 {
  uint32_t w[4];
};

// Everything a kernel needs to address one cache.  Plain values, passed by
// value to every launch.
struct Geom {
  int B, Hq, Hkv, G;           // G = Hq / Hkv
  int scheme;                  // KVQ_KIVI_ASYM / KVQ_BLOCK128_SYM / KVQ_TBQ4 / KVQ_Q4_0 / KVQ_Q8_0
  int hi_bits, lo_bits;
  int hadamard, pre_rope;
  int hsigned;                 // 1: the rotation is randomized (a mask is nonzero)
  Mask128 sign_in, sign_out;   // D_in, D_out of D_out H D_in / sqrt(128)
  int tbq4;                    // 1: KVQ_TBQ4 blocks (norm + Lloyd-Max indices)
  int q40;                     // 1: four 32-value blocks per token (KVQ_Q4_0 at 4 bits,
                               // KVQ_Q8_0 at 8 bits)
  float cb_bound[15];          // TBQ4 decision boundaries (fp32 midpoints)
  float cb_level[16];          // TBQ4 levels, ascending
  uint32_t cb_lut[8];          // levels 8..15 (the magnitudes) as hi + lo
                               // fp16: low bytes of hi of 8..11, of 12..15,
                               // high bytes of hi of 8..11, of 12..15, then
                               // the same four for lo (v_perm tables)
  float rope_theta;
  int64_t gmax;                // groups per (sequence, head)
  int64_t hi_slots;            // K_HI / V_HI tiles per (sequence, head)
  int64_t length;              // cached tokens
  int64_t Tq;                  // quantized tokens [0, Tq)
  int64_t hi_start;            // first high-bit token (KIVI)
};

struct Planes {
  uint8_t* p[KVQ_NUM_PLANES];
};

// One token range of a decode call with a single code width and tier.  Each
// pair's tiles form n_chunks chunks of `chunk` tiles worked by a team of
// `team` waves (decode_common.h); pwgs work-groups of 4 waves hold them.
struct RangePlan {
  int64_t t_lo, t_hi;  // tokens [t_lo, t_hi), t_lo a multiple of 32
  int bits;            // code bits
  int hi_tier;         // 1: high-bit planes (ring), 0: low-bit planes
  int64_t tiles_pp;    // 64-token tiles per (sequence, kv head)
  int64_t team;        // waves per pair = partial slots per query head
  int64_t chunk;       // tiles per chunk
  int64_t n_chunks;    // chunks per pair (>= team)
  int64_t n_big;       // chunks [0, n_big) hold `chunk` tiles, the rest one tile each
  int64_t pwgs;        // work-groups of the quantized tiles
  int64_t slot_base;   // first partial slot
  int window;          // 1: this launch also attends the fp16 window (one
                       // work-group per pair, 4 slots after all ranges')
};

// Split-K plan of one decode call: quantized tokens as up to two tier-pure
// ranges (one launch each); the fp16 window rides on the last launch.
// Slots [0, nq) hold quantized tokens, [nq, n) the window.  The workspace
// starts with the chunk counters, one per 256-byte line (range r of pair p
// at uint32 index (r * pairs + p) * kCounterStride), ctr_floats 4-byte words
// in all; the partials follow.
struct ChunkPlan {
  RangePlan r[2];
  int nr;
  int64_t nq;          // partial slots of quantized tokens
  int64_t n;           // all slots (nq + the window's)
  int64_t ctr_floats;  // workspace words before the partials
};

// Counters one to a 256-byte line: claims on one pair do not queue behind
// claims on its neighbours.
constexpr int64_t kCounterStride = 64;
// Workspace words holding the chunk counters of `pairs` pairs.
inline int64_t counter_words(int64_t pairs) { return 2 * pairs * kCounterStride; }

// Waves a decode launch may run at once, at most (2048 threads per compute
// unit on 256 compute units).  The workspace size is that of the plan with
// this many waves, so it depends on (config, batch, length) only; a plan on
// a device holds at most as many waves and needs no more workspace.
constexpr int64_t kMaxPlanWaves = 8192;

// Split-K plan for a launch of at most cap_waves waves (<= kMaxPlanWaves).
ChunkPlan plan_chunks(const Geom& g, int64_t cap_waves);
// The same with the waves the current device keeps resident.
ChunkPlan plan_chunks(const Geom& g);

// Schemes with one 128-value block per token (no window, no tiers).
__host__ __device__ inline bool block_scheme(int scheme) {
  return scheme == KVQ_BLOCK128_SYM || scheme == KVQ_TBQ4 || scheme == KVQ_Q4_0 || scheme == KVQ_Q8_0;
}

// Launchers (kernels in append.hip, decode.hip, dequant.hip).  Each returns
// hipGetLastError() after its launches.
hipError_t launch_rope_table(const Geom& g, const Planes& p, int64_t t0, int64_t t1,
                             hipStream_t s);
hipError_t launch_kivi_demote(const Geom& g, const Planes& p, int64_t g0, int64_t g1,
                              hipStream_t s);
hipError_t launch_kivi_quantize(const Geom& g, const Planes& p, const __half* k_new,
                                const __half* v_new, int64_t n_new, int64_t T0, int64_t g0,
                                int64_t g1, int64_t hi_start_new, hipStream_t s);
// Appends of 1..kSmallAppendMax tokens: demote, quantize and window copy
// fused into one launch of one work-group per (sequence, kv head).
// KIVI groups [g0, g1) that lie wholly in the new tokens, at 4 or 2 bits
// (append_kivi.hip); supported: the code widths and the source size allow it.
bool kivi_groups_supported(const Geom& g, int64_t n_new);
hipError_t launch_kivi_groups(const Geom& g, const Planes& p, const __half* k_new, const __half* v_new,
                              int64_t n_new, int64_t T0, int64_t g0, int64_t g1, int64_t hi_start_new,
                              hipStream_t s);
constexpr int kSmallAppendMax = 32;
hipError_t launch_kivi_small_append(const Geom& g, const Planes& p, const __half* k_new,
                                    const __half* v_new, int64_t n_new, int64_t T0, int64_t d0,
                                    int64_t d1, int64_t q0, int64_t q1, int64_t hi_start_new,
                                    hipStream_t s);
hipError_t launch_window_write(const Geom& g, const Planes& p, const __half* k_new,
                               const __half* v_new, int64_t n_new, int64_t T0, int64_t w0,
                               int64_t w1, hipStream_t s);
hipError_t launch_block128_append(const Geom& g, const Planes& p, const __half* k_new,
                                  const __half* v_new, int64_t n_new, int64_t T0,
                                  hipStream_t s);
hipError_t launch_decode_partials(const Geom& g, const Planes& p, const ChunkPlan& cp,
                                  const __half* q, int64_t q_pos, float sm_scale, float* ws,
                                  hipStream_t s);
hipError_t launch_decode_mfma(const Geom& g, const Planes& p, const ChunkPlan& cp, const __half* q,
                              float sm_scale, float* ws, hipStream_t s);
// Work-groups of the partials kernel for (g, bits) that fit on one compute
// unit at once, and the device's compute units (fallbacks when no device).
int decode_mfma_wgs_per_cu(const Geom& g, int bits);
int decode_rope_wgs_per_cu(const Geom& g, int bits);
int occupancy_wgs_per_cu(const void* kernel);
int device_compute_units();
hipError_t launch_decode_rope(const Geom& g, const Planes& p, const ChunkPlan& cp, const __half* q,
                              int64_t q_pos, float sm_scale, float* ws, hipStream_t s);
hipError_t launch_decode_merge(const Geom& g, const ChunkPlan& cp, float* ws, float* out,
                               hipStream_t s);
// Zeroes the chunk counters at the head of a workspace (a fill kernel).
hipError_t launch_zero_counters(const ChunkPlan& cp, float* ws, hipStream_t s);
// Device address of the static workspace on device dev (looked up once per
// device; dev must be the current device on the first call).
hipError_t static_workspace(int dev, void** ptr);
hipError_t launch_dequant(const Geom& g, const Planes& p, int64_t t0, int64_t t1, float* k_out,
                          float* v_out, hipStream_t s);

// Partial record per (sequence, q head, chunk): m, l, o[128] (fp32, log2 domain).
constexpr int kPartial = 2 + kD;

}  // namespace kvq
