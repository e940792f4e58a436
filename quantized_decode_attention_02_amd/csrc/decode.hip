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
//
// One pass over the workspace: wave w takes slots w, w + 4, w + 8, ... in batches
// of 64 (lane j reads the (m, l) of the batch's j-th slot), folds a batch into
// its running (M, L, o) with one max and one sum over the wave, then streams
// the batch's o[128] rows (two channels per lane) with the weights broadcast
// from the lane that holds them.  The four waves combine in LDS.  Quantized
// slots (below nq) and window slots are summed apart so that a Hadamard cache
// rotates back only the quantized part.
__global__ __launch_bounds__(256) void decode_merge_kernel(Geom g, const float* ws, float* out,
                                                           int64_t nq, int64_t n) {
  __shared__ float wml[4][2];
  __shared__ float wo[4][2][kD];
  __shared__ float rot[kD];
  const int hq = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const float* base = ws + ((int64_t)b * g.Hq + hq) * n * kPartial;
  float M = -INFINITY, L = 0.0f;
  float q0 = 0.0f, q1 = 0.0f, w0 = 0.0f, w1 = 0.0f;
  for (int64_t first = w; first < n; first += 256) {
    const int64_t mine = first + 4 * (int64_t)lane;
    float m = -INFINITY, l = 0.0f;
    if (mine < n) {
      m = base[mine * kPartial];
      l = base[mine * kPartial + 1];
    }
    const float Mb = fmaxf(M, wave_max64(m));
    if (Mb == -INFINITY) continue;  // nothing attended so far
    const float r = M == -INFINITY ? 0.0f : exp2f(M - Mb);
    const float wt = m == -INFINITY ? 0.0f : exp2f(m - Mb);
    L = L * r + wave_sum64(l * wt);
    q0 *= r; q1 *= r; w0 *= r; w1 *= r;
    M = Mb;
    // eight rows in flight per step; steps past the batch end reread its
    // last row with weight 0, so the body has no branch to wait behind
    const int cnt = (int)min((int64_t)64, (n - first + 3) / 4);
    for (int i0 = 0; i0 < cnt; i0 += 8) {
      float2 v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int64_t slot = first + 4 * (int64_t)min(i0 + k, cnt - 1);
        v[k] = *reinterpret_cast<const float2*>(base + slot * kPartial + 2 + 2 * lane);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int i = min(i0 + k, cnt - 1);
        const float wr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt), i));
        const float wi = i0 + k < cnt ? wr : 0.0f;
        const float wq = first + 4 * (int64_t)i < nq ? wi : 0.0f;
        const float ww = wi - wq;
        q0 += wq * v[k].x;
        q1 += wq * v[k].y;
        w0 += ww * v[k].x;
        w1 += ww * v[k].y;
      }
    }
  }
  if (lane == 0) {
    wml[w][0] = M;
    wml[w][1] = L;
  }
  wo[w][0][2 * lane] = q0;
  wo[w][0][2 * lane + 1] = q1;
  wo[w][1][2 * lane] = w0;
  wo[w][1][2 * lane + 1] = w1;
  __syncthreads();
  float Mt = -INFINITY;
  for (int i = 0; i < 4; ++i) Mt = fmaxf(Mt, wml[i][0]);
  float sc[4], Lt = 0.0f;
  for (int i = 0; i < 4; ++i) {
    sc[i] = wml[i][0] == -INFINITY ? 0.0f : exp2f(wml[i][0] - Mt);
    Lt += sc[i] * wml[i][1];
  }
  float qp = 0.0f, wp = 0.0f;
  if (tid < kD) {
    for (int i = 0; i < 4; ++i) {
      qp += sc[i] * wo[i][0][tid];
      wp += sc[i] * wo[i][1][tid];
    }
    rot[tid] = qp;
  }
  __syncthreads();
  if (g.hadamard) fwht128_lds(rot, 1, tid, 256);
  if (tid < kD) {
    const float q_part = g.hadamard ? rot[tid] : qp;
    out[((int64_t)b * g.Hq + hq) * kD + tid] = Lt > 0.0f ? (q_part + wp) / Lt : 0.0f;
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
