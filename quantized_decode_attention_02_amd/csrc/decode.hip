// Split-K single-query decode attention: dispatch of the partials kernels
// and the merge.
//
// Sources cited here:
//   [nalar]    "Kuantisasi KV Cache dengan Error Budget yang Eksplisit"
//              (nalar.dev).
//   [trefon]   "Matematyka cache KV: ile kosztuje długi kontekst i co daje
//              4-bitowy cache" (trefon.com).
//
// For one query head: s_i = q . k_i * scale, p = softmax(s), out = sum p_i v_i
// ([nalar] "Error pada key mengubah input softmax", "Error pada value masuk
// setelah attention probability").  The partials kernels (decode_mfma.hip,
// decode_rope.hip) split the tokens into chunks; each wave writes, for every
// query head of its GQA group, the running max m (log2 domain), the sum l of
// exp2(s - m) and the unnormalized output o[128].  The merge below combines
// them by log-sum-exp.
#include <mutex>

#include "kvq_device.h"

// Workspace of kvq_decode_attn_static: split-K partials and chunk counters of
// a decode call for callers that cannot allocate.  Each GPU holds its own
// copy from the library's load until the process ends.  In host code this
// name is only a handle for hipGetSymbolAddress: the device address of the
// current GPU's copy comes from static_workspace() below, and kernels take
// that address.
static __device__ __align__(256) uint8_t scratch[KVQ_STATIC_WORKSPACE_BYTES];

namespace kvq {
namespace {

// Zeroes n 32-bit words (the chunk counters a decode call starts from).  A
// kernel rather than hipMemsetAsync, so that the call can be captured in a
// HIP graph.
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

// Log-sum-exp merge of the chunk partials of one (sequence, query head):
// M = max m_c, L = sum l_c 2^(m_c - M), out = sum o_c 2^(m_c - M) / L.
// Hadamard caches: the quantized chunks (slots < nq) were attended with the
// rotated query R q, so their sum is rotated back once with R^T (R =
// D_out H D_in / sqrt(128), R^T = D_in H D_out / sqrt(128); the plain H /
// sqrt(128) is its own inverse); the fp16 window slots were attended
// unrotated.
//
// One pass over the workspace: wave w takes slots w, w + 4, w + 8, ... in batches
// of 64 (lane j reads the (m, l) of the batch's j-th slot), folds a batch into
// its running (M, L, o) with one max and one sum over the wave, then streams
// the batch's o[128] rows (two channels per lane) with the weights broadcast
// from the lane that holds them.  The four waves combine in LDS.  Quantized
// slots (below nq) and window slots are summed apart so that a Hadamard cache
// rotates back only the quantized part.
__global__ __launch_bounds__(256) void decode_merge_kernel(Geom g, float* ws, float* out,
                                                           int64_t nq, int64_t n) {
  __shared__ float wml[4][2];
  __shared__ float wo[4][2][kD];
  __shared__ float rot[kD];
  const int hq = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  float* base = ws + ((int64_t)b * g.Hq + hq) * n * kPartial;
  float M = -INFINITY, L = 0.0f;
  float q0 = 0.0f, q1 = 0.0f, w0 = 0.0f, w1 = 0.0f;
  for (int64_t first = w; first < n; first += 256) {
    const int64_t mine = first + 4 * (int64_t)lane;
    // eight rows in flight per step; steps past the batch end reread its
    // last row with weight 0, so the body has no branch to wait behind.
    // The first step's rows go out with the (m, l) loads, so a head with at
    // most 32 partials needs one round trip.
    const int cnt = (int)min((int64_t)64, (n - first + 3) / 4);
    float2 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t slot = first + 4 * (int64_t)min(k, cnt - 1);
      v[k] = *reinterpret_cast<const float2*>(base + slot * kPartial + 2 + 2 * lane);
    }
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
    for (int i0 = 0; i0 < cnt; i0 += 8) {
      if (i0 > 0) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int64_t slot = first + 4 * (int64_t)min(i0 + k, cnt - 1);
          v[k] = *reinterpret_cast<const float2*>(base + slot * kPartial + 2 + 2 * lane);
        }
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
  // every record of this head has been read: zero them, so that a finished
  // call leaves the whole workspace zero (the chunk counters of any later
  // call, whatever its cache, start from zero)
  for (int64_t e = tid; e < n * kPartial / 2; e += 256) reinterpret_cast<float2*>(base)[e] = make_float2(0.0f, 0.0f);
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
  // the inverse of D_out H D_in / sqrt(128) is D_in H D_out / sqrt(128)
  if (g.hadamard) fwht128_rows(rot, 1, tid, 256, g.sign_out, g.sign_in, g.hsigned);
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
  return g.pre_rope ? launch_decode_rope(g, p, cp, q, q_pos, sm_scale, ws, s)
                    : launch_decode_mfma(g, p, cp, q, sm_scale, ws, s);
}

hipError_t launch_zero_counters(const ChunkPlan& cp, float* ws, hipStream_t s) {
  if (cp.ctr_floats <= 0) return hipGetLastError();
  const int64_t blocks = std::min<int64_t>((cp.ctr_floats + 255) / 256, 1024);
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<uint32_t*>(ws), cp.ctr_floats);
  return hipGetLastError();
}

// Device address of `scratch` on device `dev` (the current device), looked
// up once per device with hipGetSymbolAddress and kept: host code never
// passes the array's name itself to a kernel.
hipError_t static_workspace(int dev, void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* a = nullptr;
    const hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (a == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode_merge(const Geom& g, const ChunkPlan& cp, float* ws, float* out,
                               hipStream_t s) {
  hipLaunchKernelGGL(decode_merge_kernel, dim3(g.Hq, g.B), dim3(256), 0, s, g, ws + cp.ctr_floats, out,
                     cp.nq, cp.n);
  return hipGetLastError();
}

}  // namespace kvq
