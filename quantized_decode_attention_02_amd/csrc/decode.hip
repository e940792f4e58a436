// Split-K single-query decode attention over the packed cache, and the merge.
//
// Sources cited here:
//   [troisinh] "KV Cache Quantization — Nén cache INT4/INT3, mở khóa
//              ultra-long context" (troisinh.com).
//   [nalar]    "Kuantisasi KV Cache dengan Error Budget yang Eksplisit"
//              (nalar.dev).
//   [trefon]   "Matematyka cache KV: ile kosztuje długi kontekst i co daje
//              4-bitowy cache" (trefon.com).
//
// For one query head: s_i = q . k_i * scale, p = softmax(s), out = sum p_i v_i
// ([nalar] "Error pada key mengubah input softmax", "Error pada value masuk
// setelah attention probability").  Keys and values are dequantized inside
// the attention kernel, never written back ([nalar] "Biaya dequantization
// harus masuk ke model latency").  Hadamard caches are attended in the
// rotated domain: q is rotated once per work-group and the merged output
// rotated back once ([trefon] "Jak 4-bitowemu cache to uchodzi: najpierw
// obrót").  Pre-RoPE keys get split-half RoPE at their position on the fly
// ([troisinh] "Tại sao nó hoạt động", item 3).
//
// Work split: one work-group per (chunk of key groups, kv head, sequence)
// computes, for every query head of the GQA group, the running max m (log2
// domain), the sum l of exp2(s - m) and the unnormalized output o[128]; the
// fp16 window is one more chunk.  The merge combines chunks by log-sum-exp.
#include "kvq_device.h"

namespace kvq {
namespace {

struct DecodeArgs {
  Geom g;
  Planes p;
  const __half* q;
  float* ws;
  int64_t q_pos;
  float scale_log2;  // sm_scale * log2(e)
  int64_t gpc, nq, n;
  int64_t c0;  // chunk index of blockIdx.x == 0
};

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Dequantized stored-domain key values of token `tok` (row in its tile / ring)
// for the 16 channels `ch[i]` this thread owns.
template <bool ROPE>
__device__ __forceinline__ void channels_of(int sl, int* ch) {
  if (ROPE) {
    for (int i = 0; i < 8; ++i) {
      ch[i] = 8 * sl + i;
      ch[i + 8] = 64 + 8 * sl + i;
    }
  } else {
    for (int i = 0; i < 16; ++i) ch[i] = 16 * sl + i;
  }
}

template <int G, bool ROPE>
__global__ __launch_bounds__(256) void decode_partials_v0(DecodeArgs a) {
  const Geom& g = a.g;
  const int64_t c = a.c0 + blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int64_t pair = pair_index(g, b, h);
  const bool window_chunk = c >= a.nq;

  __shared__ float qs[G][kD];
  __shared__ float sc[G][kGroup];
  __shared__ float pr[G][kGroup];
  __shared__ float alpha_s[G];
  __shared__ float ml[G][2];
  __shared__ float ored[G][kD];

  for (int e = tid; e < G * kD; e += 256) {
    const int i = e / kD, d = e % kD;
    qs[i][d] = __half2float(a.q[((int64_t)b * g.Hq + h * G + i) * kD + d]);
  }
  __syncthreads();
  if (ROPE) {
    for (int e = tid; e < G * 64; e += 256) {
      const int i = e / 64, j = e % 64;
      const double theta = pow((double)g.rope_theta, -2.0 * (double)j / 128.0);
      const double ang = (double)a.q_pos * theta;
      const float cs = (float)cos(ang), sn = (float)sin(ang);
      const float x1 = qs[i][j], x2 = qs[i][j + 64];
      qs[i][j] = x1 * cs - x2 * sn;
      qs[i][j + 64] = x1 * sn + x2 * cs;
    }
    __syncthreads();
  }
  if (g.hadamard && !window_chunk) fwht128_lds(&qs[0][0], G, tid, 256);
  for (int e = tid; e < G * kD; e += 256) (&qs[0][0])[e] *= a.scale_log2;
  if (tid < G) {
    ml[tid][0] = -INFINITY;
    ml[tid][1] = 0.0f;
  }
  __syncthreads();

  int64_t t_begin, t_end;
  if (window_chunk) {
    t_begin = g.Tq;
    t_end = g.length;
  } else {
    t_begin = c * a.gpc * kGroup;
    t_end = min((c + 1) * a.gpc * kGroup, g.Tq);
  }

  const int tok = tid >> 3, sl = tid & 7;       // key side
  const int vd = tid & 127, vhalf = tid >> 7;   // value side
  int ch[16];
  channels_of<ROPE>(sl, ch);
  float o[G];
  for (int i = 0; i < G; ++i) o[i] = 0.0f;

  for (int64_t base = t_begin; base < t_end; base += kGroup) {
    const int nvalid = (int)min((int64_t)kGroup, t_end - base);
    const int64_t grp = base / kGroup;
    // ---------------- keys: dequantize, (RoPE), partial dot products
    float part[G];
    for (int i = 0; i < G; ++i) part[i] = 0.0f;
    if (tok < nvalid) {
      const int64_t t = base + tok;
      float kx[16];
      if (window_chunk) {
        const __half* row = reinterpret_cast<const __half*>(a.p.p[KVQ_PLANE_K_WIN]) +
                            (pair * kRing + t % kRing) * kD;
        for (int i = 0; i < 16; ++i) kx[i] = __half2float(row[ch[i]]);
      } else if (g.scheme == KVQ_BLOCK128_SYM) {
        const uint8_t* tile = a.p.p[KVQ_PLANE_K_HI] + (pair * g.gmax + grp) * 2048;
        const float s = half_bits_to_float(reinterpret_cast<const uint16_t*>(
            a.p.p[KVQ_PLANE_K_META])[pair * g.gmax * kGroup + t]);
        for (int i = 0; i < 16; ++i) {
          const int d = ch[i];
          const int n = (tile[ktile_offset(tok, d >> 1)] >> (4 * (d & 1))) & 15;
          kx[i] = (float)(n - 8) * s;
        }
      } else {
        int bits;
        const uint8_t* tile = tile_ptr(g, a.p, KVQ_PLANE_K_HI, KVQ_PLANE_K_LO, pair, grp, &bits);
        const uint16_t* meta =
            reinterpret_cast<const uint16_t*>(a.p.p[KVQ_PLANE_K_META] + (pair * g.gmax + grp) * 512);
        const int per = 8 / bits, mask = (1 << bits) - 1;
        for (int i = 0; i < 16; ++i) {
          const int d = ch[i];
          const int code = (tile[ktile_offset(tok, d / per)] >> (bits * (d % per))) & mask;
          kx[i] = (float)code * half_bits_to_float(meta[2 * d]) + half_bits_to_float(meta[2 * d + 1]);
        }
      }
      if (ROPE) {
        const float* tab = reinterpret_cast<const float*>(a.p.p[KVQ_PLANE_ROPE]) + t * 128;
        for (int i = 0; i < 8; ++i) {
          const int j = ch[i];
          const float cs = tab[2 * j], sn = tab[2 * j + 1];
          const float x1 = kx[i], x2 = kx[i + 8];
          kx[i] = x1 * cs - x2 * sn;
          kx[i + 8] = x1 * sn + x2 * cs;
        }
      }
      for (int i = 0; i < G; ++i)
        for (int k = 0; k < 16; ++k) part[i] += qs[i][ch[k]] * kx[k];
    }
    for (int i = 0; i < G; ++i) {
      part[i] += __shfl_xor(part[i], 1, 64);
      part[i] += __shfl_xor(part[i], 2, 64);
      part[i] += __shfl_xor(part[i], 4, 64);
    }
    if (sl == 0)
      for (int i = 0; i < G; ++i) sc[i][tok] = tok < nvalid ? part[i] : -INFINITY;
    __syncthreads();
    // ---------------- online softmax (first wave)
    if (tid < 64) {
      for (int i = 0; i < G; ++i) {
        const float s = tid < kGroup ? sc[i][tid] : -INFINITY;
        const float gm = wave_max(s);
        const float m_old = ml[i][0];
        const float m_new = fmaxf(m_old, gm);
        const float alpha = m_old == -INFINITY ? 0.0f : exp2f(m_old - m_new);
        const float pv = (tid < kGroup && s != -INFINITY) ? exp2f(s - m_new) : 0.0f;
        const float ps = wave_sum(pv);
        if (tid < kGroup) pr[i][tid] = pv;
        if (tid == 0) {
          ml[i][0] = m_new;
          ml[i][1] = ml[i][1] * alpha + ps;
          alpha_s[i] = alpha;
        }
      }
    }
    __syncthreads();
    // ---------------- values: dequantize, accumulate p * v
    float vx[16];
    const int64_t t0 = base + 16 * vhalf;
    if (window_chunk) {
      const __half* ring = reinterpret_cast<const __half*>(a.p.p[KVQ_PLANE_V_WIN]) + pair * kRing * kD;
      for (int k = 0; k < 16; ++k) {
        const int64_t t = t0 + k;
        vx[k] = (16 * vhalf + k < nvalid) ? __half2float(ring[vd * kRing + t % kRing]) : 0.0f;
      }
    } else if (g.scheme == KVQ_BLOCK128_SYM) {
      const uint8_t* tile = a.p.p[KVQ_PLANE_V_HI] + (pair * g.gmax + grp) * 2048;
      const uint16_t* sp = reinterpret_cast<const uint16_t*>(a.p.p[KVQ_PLANE_V_META]) + pair * g.gmax * kGroup;
      for (int k = 0; k < 16; ++k) {
        const int j = 16 * vhalf + k;
        const int n = (tile[vd * 16 + (j >> 1)] >> (4 * (j & 1))) & 15;
        vx[k] = j < nvalid ? (float)(n - 8) * half_bits_to_float(sp[base + j]) : 0.0f;
      }
    } else {
      int bits;
      const uint8_t* tile = tile_ptr(g, a.p, KVQ_PLANE_V_HI, KVQ_PLANE_V_LO, pair, grp, &bits);
      const uint16_t* meta =
          reinterpret_cast<const uint16_t*>(a.p.p[KVQ_PLANE_V_META] + (pair * g.gmax + grp) * 512);
      const int per = 8 / bits, mask = (1 << bits) - 1, rb = 4 * bits;
      const int dg = vd >> 5;
      for (int k = 0; k < 16; ++k) {
        const int j = 16 * vhalf + k;
        const int code = (tile[vd * rb + j / per] >> (bits * (j % per))) & mask;
        vx[k] = (float)code * half_bits_to_float(meta[2 * (j * 4 + dg)]) +
                half_bits_to_float(meta[2 * (j * 4 + dg) + 1]);
      }
    }
    for (int i = 0; i < G; ++i) {
      float acc = o[i] * alpha_s[i];
      for (int k = 0; k < 16; ++k) acc += pr[i][16 * vhalf + k] * vx[k];
      o[i] = acc;
    }
    __syncthreads();
  }
  if (vhalf == 1)
    for (int i = 0; i < G; ++i) ored[i][vd] = o[i];
  __syncthreads();
  if (vhalf == 0) {
    for (int i = 0; i < G; ++i) {
      float* rec = a.ws + (((int64_t)b * g.Hq + h * G + i) * a.n + c) * kPartial;
      rec[2 + vd] = o[i] + ored[i][vd];
      if (vd == 0) {
        rec[0] = ml[i][0];
        rec[1] = ml[i][1];
      }
    }
  }
}

// Log-sum-exp merge of the chunk partials of one (sequence, query head):
// M = max m_c, L = sum l_c 2^(m_c - M), out = sum o_c 2^(m_c - M) / L.
// Hadamard caches: the quantized chunks (slots < nq) were attended with the
// rotated query, so their sum is rotated back once (H/sqrt(128) is its own
// inverse); the fp16 window slots were attended unrotated.
// 256 threads: the slot loops are strided over threads so their loads are
// independent; two threads per output channel.
__device__ __forceinline__ float block_reduce(float v, float* red, int tid, bool is_max) {
  red[tid] = v;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] = is_max ? fmaxf(red[tid], red[tid + s]) : red[tid] + red[tid + s];
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(256) void decode_merge_kernel(Geom g, const float* ws, float* out,
                                                           int64_t nq, int64_t n) {
  __shared__ float red[256];
  __shared__ float wsh[1024];
  __shared__ float acc[2][2][kD];
  const int hq = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const float* base = ws + ((int64_t)b * g.Hq + hq) * n * kPartial;
  float M = -INFINITY;
  for (int64_t c = tid; c < n; c += 256) M = fmaxf(M, base[c * kPartial]);
  M = block_reduce(M, red, tid, true);
  float L = 0.0f;
  if (M != -INFINITY) {
    for (int64_t c = tid; c < n; c += 256) {
      const float m = base[c * kPartial];
      if (m != -INFINITY) L += base[c * kPartial + 1] * exp2f(m - M);
    }
  }
  L = block_reduce(L, red, tid, false);
  const int d = tid & 127, hf = tid >> 7;
  float oq = 0.0f, ow = 0.0f;
  for (int64_t c0 = 0; c0 < n; c0 += 1024) {
    const int cnt = (int)min((int64_t)1024, n - c0);
    for (int i = tid; i < cnt; i += 256) {
      const float m = base[(c0 + i) * kPartial];
      wsh[i] = (m == -INFINITY) ? 0.0f : exp2f(m - M);
    }
    __syncthreads();
#pragma unroll 8
    for (int i = hf; i < cnt; i += 2) {
      const float v = base[(c0 + i) * kPartial + 2 + d] * wsh[i];
      if (c0 + i < nq) oq += v; else ow += v;
    }
    __syncthreads();
  }
  acc[0][hf][d] = oq;
  acc[1][hf][d] = ow;
  __syncthreads();
  if (g.hadamard) {
    if (tid < kD) red[tid] = acc[0][0][tid] + acc[0][1][tid];
    __syncthreads();
    fwht128_lds(red, 1, tid, 256);
  }
  if (tid < kD) {
    const float q_part = g.hadamard ? red[tid] : acc[0][0][tid] + acc[0][1][tid];
    const float w_part = acc[1][0][tid] + acc[1][1][tid];
    out[((int64_t)b * g.Hq + hq) * kD + tid] = L > 0.0f ? (q_part + w_part) / L : 0.0f;
  }
}

}  // namespace

hipError_t launch_decode_partials(const Geom& g, const Planes& p, const ChunkPlan& cp,
                                  const __half* q, int64_t q_pos, float sm_scale, float* ws,
                                  hipStream_t s) {
  if (cp.n == 0) return hipGetLastError();
  DecodeArgs a;
  a.g = g;
  a.p = p;
  a.q = q;
  a.ws = ws;
  a.q_pos = q_pos;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.gpc = cp.gpc;
  a.nq = cp.nq;
  a.n = cp.n;
  a.c0 = 0;
  unsigned nblocks = (unsigned)cp.n;
  if (cp.mode == 1) return launch_decode_mfma(g, p, cp, q, sm_scale, ws, s);
  const dim3 grid(nblocks, g.Hkv, g.B), block(256);
#define KVQ_LAUNCH(GG, RR) hipLaunchKernelGGL((decode_partials_v0<GG, RR>), grid, block, 0, s, a)
  if (g.pre_rope) {
    if (g.G == 1) KVQ_LAUNCH(1, true);
    else if (g.G == 2) KVQ_LAUNCH(2, true);
    else KVQ_LAUNCH(4, true);
  } else {
    if (g.G == 1) KVQ_LAUNCH(1, false);
    else if (g.G == 2) KVQ_LAUNCH(2, false);
    else KVQ_LAUNCH(4, false);
  }
#undef KVQ_LAUNCH
  return hipGetLastError();
}

hipError_t launch_decode_merge(const Geom& g, const ChunkPlan& cp, float* ws, float* out,
                               hipStream_t s) {
  hipLaunchKernelGGL(decode_merge_kernel, dim3(g.Hq, g.B), dim3(256), 0, s, g, ws, out, cp.nq, cp.n);
  return hipGetLastError();
}

}  // namespace kvq
