/*
 * kvq.h — C ABI of libkvq: low-bit KV-cache quantization and single-query
 * decode attention over the packed cache, for AMD Instinct MI355X (gfx950).
 *
 * Sources (the pages this library implements; sections are their headings):
 *   [troisinh] "KV Cache Quantization — Nén cache INT4/INT3, mở khóa
 *              ultra-long context" (troisinh.com).
 *   [nalar]    "Kuantisasi KV Cache dengan Error Budget yang Eksplisit"
 *              (nalar.dev).
 *   [trefon]   "Matematyka cache KV: ile kosztuje długi kontekst i co daje
 *              4-bitowy cache" (trefon.com).
 *   [nexus]    "NexusQuant: Cách nén KV Cache của LLM lên tới 33 lần mà
 *              không cần huấn luyện" (lehuy.net).
 *
 * Conventions for every call:
 *   - Plain C types only.  Device pointers are HIP device addresses owned by
 *     the caller; `stream` is a hipStream_t passed as void* (NULL = the null
 *     stream).  Work is enqueued asynchronously on `stream`; no call
 *     allocates device memory, synchronizes, or keeps global mutable state,
 *     so calls on different streams with different buffers are independent.
 *   - Every argument is validated on the host before anything is launched;
 *     a call that returns an error has enqueued nothing.  KVQ_ERR_HIP means a
 *     launch was rejected by the HIP runtime (hipGetLastError after launch).
 *   - All device buffers must be 16-byte aligned (256 recommended); tensors
 *     are dense row-major, fp16 = IEEE binary16, fp32 = IEEE binary32.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_ABI_VERSION 2
#define KVQ_MAX_PLANES 16

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARG = -1, /* bad pointer, size, alignment or config value */
  KVQ_ERR_UNSUPPORTED = -2, /* a valid but unimplemented combination */
  KVQ_ERR_CAPACITY = -3,    /* length + n_new would exceed max_tokens */
  KVQ_ERR_WORKSPACE = -4,   /* workspace smaller than the call needs (for
                               kvq_decode_attn_static: more than its static
                               array holds) */
  KVQ_ERR_HIP = -5          /* the HIP runtime rejected a launch */
} kvq_status;

/* Cache schemes.
 * KVQ_KIVI_ASYM: keys quantized per channel over groups of 32 tokens, values
 *   per token over groups of 32 dims, asymmetric with an fp16 scale and zero
 *   point ([troisinh] "Tại sao nó hoạt động", item 1; [trefon] "Dlaczego cache
 *   trudniej skwantyzować niż wagi"), plus a 128-token fp16 window of recent
 *   tokens ([nalar] "Evaluasi harus memisahkan peningkatan kapasitas dari
 *   dampak model").  Tokens [Tq, length) are fp16 with
 *   Tq = max(0, floor((length - 128) / 32) * 32).  Codes have 4, 3 or 2
 *   bits (the INT4 / INT3 caches of [troisinh] "KV Cache Quantization - Nén
 *   cache INT4/INT3"); 3-bit rows are one little-endian bit string (code c at
 *   bits 3c); 3-bit codes (a 3-bit cache, or the older tier below an INT4
 *   window) need keys stored after RoPE.
 * KVQ_BLOCK128_SYM: each token's 128-value head vector is one block of an
 *   fp16 scale and 128 symmetric 4-bit codes, 66 bytes, 4.125 bits per value
 *   ([trefon] "Przykład: model 27B przy 262K"); every token is quantized.
 *   With k_bits = 3, the format table's 50-byte block: codes in [-3, 3]
 *   stored + 4, scale = absmax / 3, 3.125 bits per value; a row's codes are
 *   one little-endian bit string (code c at bits 3c), so codes straddle
 *   bytes.
 * KVQ_TBQ4: the same 66-byte container holding an fp16 norm and 128 4-bit
 *   indices into 16 Lloyd-Max levels of N(0, 1/sqrt(128)), taken after the
 *   (randomized) Hadamard rotation, which is required ([trefon] "Jak
 *   4-bitowemu cache to uchodzi: najpierw obrót").  The levels are the fixed
 *   point of Lloyd's iteration in fp64, rounded to fp32; the norm is
 *   fp16(min(fl32(sqrt(sum y^2)), 65504)) with the sum and the root in fp64;
 *   an index counts the fp32 midpoints between consecutive levels that lie
 *   strictly below fl32(y / norm); a value decodes to fl32(norm * level).
 * KVQ_Q4_0: each token's 128-value head vector is four 32-value blocks of an
 *   fp16 scale and 32 symmetric 4-bit codes, 18 bytes per 32 values, 4.5 bits
 *   per value (the Q4_0 row of the format table, [trefon] "Przykład: model
 *   27B przy 262K"); the quantizer of KVQ_BLOCK128_SYM per 32-value slice.
 *   Rotation optional.
 * KVQ_Q8_0: the same four 32-value blocks at 8 bits (k_bits = 8): an fp16
 *   scale absmax / 127 and 32 codes in [-127, 127] stored as the byte c + 128,
 *   34 bytes per 32 values, 8.5 bits per value (the Q8_0 row of the same
 *   table).  Rotation optional. */
enum { KVQ_KIVI_ASYM = 0, KVQ_BLOCK128_SYM = 1, KVQ_TBQ4 = 2, KVQ_Q4_0 = 3, KVQ_Q8_0 = 4 };

/* Cache planes (caller-allocated device buffers; byte image per plane is the
 * documented layout, sizes from kvq_layout):
 *   K_HI/V_HI   key/value code tiles of the high-bit tier (KIVI; a ring of
 *               int4_window/32 slots when int4_window >= 0) or of every token
 *               (BLOCK128, TBQ4, Q4_0, Q8_0).  A tile is 32 tokens x 128 channels at b bits:
 *               keys token-major with 16-byte chunks interleaved across the
 *               32 tokens, values channel-major.
 *   K_LO/V_LO   low-bit tiles (KIVI with int4_window >= 0), one per group.
 *   K_META      KIVI: per group 128 fp16 (scale, zero) pairs, one per
 *               channel.  BLOCK128: one fp16 scale per token; TBQ4: one fp16
 *               norm per token; Q4_0, Q8_0: four fp16 scales per token (32-value
 *               slices in order).
 *   V_META      KIVI: per group, token-major: for each of the 32 tokens the
 *               fp16 (scale, zero) of its four 32-dim slices.  BLOCK128: one
 *               fp16 scale per token; TBQ4: one fp16 norm per token; Q4_0, Q8_0:
 *               four fp16 scales per token.
 *   K_WIN       KIVI: fp16 key ring of 160 rows x 128 channels per
 *               (sequence, kv head); token t lives in row t mod 160.
 *   V_WIN       KIVI: fp16 value ring, channel-major: 128 rows x 160 slots
 *               per (sequence, kv head); token t lives in slot t mod 160.
 *   ROPE        pre-RoPE keys only: fp32 (cos, sin) of t * theta_j, row t,
 *               j = 0..63, written by kvq_append for the appended positions.
 * Every plane is indexed [sequence][kv head][...] except ROPE (shared). */
enum {
  KVQ_PLANE_K_HI = 0,
  KVQ_PLANE_V_HI = 1,
  KVQ_PLANE_K_LO = 2,
  KVQ_PLANE_V_LO = 3,
  KVQ_PLANE_K_META = 4,
  KVQ_PLANE_V_META = 5,
  KVQ_PLANE_K_WIN = 6,
  KVQ_PLANE_V_WIN = 7,
  KVQ_PLANE_ROPE = 8,
  KVQ_NUM_PLANES = 9
};

typedef struct kvq_config {
  int32_t head_dim;       /* must be 128 */
  int32_t num_q_heads;    /* Hq */
  int32_t num_kv_heads;   /* Hkv; Hq / Hkv must be 1, 2 or 4 (GQA, [trefon]
                             "Bajty na token"), q head h reads kv head h / (Hq/Hkv) */
  int32_t scheme;         /* KVQ_KIVI_ASYM, KVQ_BLOCK128_SYM, KVQ_TBQ4,
                             KVQ_Q4_0 or KVQ_Q8_0 */
  int32_t k_bits;         /* bits of the high-bit tier: 4, 3 or 2 (KIVI); 4
                             or 3 (BLOCK128); 4 (TBQ4, Q4_0); 8 (Q8_0) */
  int32_t v_bits;         /* must equal k_bits */
  int32_t k_group_tokens; /* must be 32 */
  int32_t v_group_dims;   /* must be 32 */
  int32_t fp16_window;    /* 128 for KIVI, 0 for the block schemes */
  int32_t int4_window;    /* KIVI: -1 = every quantized token at k_bits; else a
                             positive multiple of 32: the newest int4_window
                             quantized tokens keep k_bits (4) and older ones
                             drop to low_bits ([troisinh] "Ý tưởng cốt lõi",
                             "Mixed Precision").  Block schemes: -1. */
  int32_t low_bits;       /* 2 or 3 (used only when int4_window >= 0) */
  int32_t hadamard;       /* 1: rotate each 128-vector by H_128/sqrt(128)
                             (Sylvester order, fixed fp32 butterfly order
                             h = 1,2,...,64) before quantizing ([troisinh]
                             "Tại sao nó hoạt động", item 2; [trefon] "Jak
                             4-bitowemu cache to uchodzi: najpierw obrót"),
                             randomized by the sign masks below */
  int32_t pre_rope_keys;  /* 1: keys are stored before RoPE and rotated on the
                             fly at decode, split-half pairs (j, j+64)
                             ([troisinh] "Tại sao nó hoạt động", item 3;
                             [nexus] "Các mô hình được hỗ trợ").  Not with
                             hadamard. */
  float rope_theta;       /* RoPE base (> 0 when pre_rope_keys) */
  uint32_t hadamard_sign_in[4];  /* randomized Hadamard ([trefon] "Jak
                             4-bitowemu cache to uchodzi: najpierw obrót":
                             signs, transform, signs): the rotation is
                             D_out H D_in / sqrt(128) with D = diag(+-1); bit
                             i of word i / 32 set negates coordinate i of the
                             input (D_in) ... */
  uint32_t hadamard_sign_out[4]; /* ... and of the output (D_out).  Sign flips
                             are exact, so codes stay bit-exact.  All zero:
                             the plain rotation.  Must be all zero unless
                             hadamard (else KVQ_ERR_INVALID_ARG).  The masks
                             are part of the cache's format: append, decode
                             and dequant of one cache take the same ones. */
} kvq_config;

typedef struct kvq_layout_t {
  uint64_t plane_bytes[KVQ_MAX_PLANES]; /* 0 = plane unused */
  uint64_t alignment;                   /* required base alignment (bytes) */
  int64_t groups;                       /* ceil(max_tokens / 32) */
  int64_t hi_slots;                     /* tiles per (sequence, head) in K_HI */
} kvq_layout_t;

typedef struct kvq_cache {
  void* planes[KVQ_MAX_PLANES]; /* device pointers, caller-owned */
  int64_t batch;                /* sequences */
  int64_t max_tokens;           /* capacity per sequence */
  int64_t length;               /* tokens cached per sequence (host-side; the
                                   same for every sequence).  kvq_append
                                   advances it.  The caller may set it back
                                   from L1 to L0 < L1 only if L1 - Tq(L0) <= 160
                                   and no group was demoted since L0 (KIVI); the
                                   tokens [L0, L1) are then forgotten. */
} kvq_cache;

/* Sizes of the cache planes for `batch` sequences of up to `max_tokens`
 * tokens.  Writes *out; no device work.  Cache size follows from the stored
 * element count and the bits per element plus metadata ([nalar] "Ukuran cache
 * mengikuti jumlah elemen tersimpan dan bit width"). */
kvq_status kvq_layout(const kvq_config* cfg, int64_t batch, int64_t max_tokens,
                      kvq_layout_t* out);

/* Bytes of the device workspace kvq_decode_attn needs for `batch` sequences
 * of `length` cached tokens.  Writes *bytes.  A pure function of (cfg, batch,
 * length): the size is that of the split-K plan with the most waves a launch
 * may run at once (8192), which no device's plan exceeds, so the same number
 * serves every device and call.  The workspace starts with
 * KVQ_COUNTER_BYTES(batch * num_kv_heads) bytes of work counters; the split-K
 * partials follow (running max, sum and 128 accumulators per query head and
 * partial).  The workspace must be all zero before its first use: every
 * completed decode (kvq_decode_attn, or kvq_decode_partials followed by
 * kvq_decode_merge) leaves every byte it used zero again, so one workspace,
 * zeroed once when it is allocated, serves caches of any shape. */
#define KVQ_COUNTER_BYTES(pairs) (2 * (uint64_t)(pairs) * 256)
kvq_status kvq_workspace_bytes(const kvq_config* cfg, int64_t batch, int64_t length,
                               uint64_t* bytes);

/* Append n_new tokens to every sequence: quantize on append, computing every
 * range from the values themselves, no calibration ([nalar] "Pertumbuhan
 * cache dinamis mengubah persoalan kalibrasi"; [trefon] "Dlaczego cache
 * trudniej skwantyzować niż wagi").
 *   k_new, v_new: device fp16 [batch][n_new][num_kv_heads][128], keys before
 *                 RoPE when pre_rope_keys.
 * KIVI: 32-token groups leaving the fp16 window are quantized (keys per
 * channel, values per token; after the Hadamard rotation if configured);
 * groups leaving the high-bit window are requantized to low_bits from their
 * dequantized values; new groups go straight to the tier of their age.
 * BLOCK128, TBQ4, Q4_0, Q8_0: every new token becomes one block (four for Q4_0 and Q8_0).  pre_rope_keys: ROPE rows for
 * the new positions are written.  Advances cache->length on success.
 * Errors: KVQ_ERR_CAPACITY if length + n_new > max_tokens; n_new == 0 is a
 * no-op.  Output is bit-exact with the documented fp32 round-to-nearest-even
 * arithmetic and byte layout. */
kvq_status kvq_append(const kvq_config* cfg, kvq_cache* cache, const void* k_new,
                      const void* v_new, int64_t n_new, void* stream);

/* Single-query decode attention over the packed cache, dequantizing on the
 * fly inside the attention kernel ([nalar] "Biaya dequantization harus masuk
 * ke model latency").  For query head h of sequence b:
 *   s_i = (q . k_i) * sm_scale over every cached token i (no mask),
 *   out = sum_i softmax(s)_i v_i
 * ([nalar] "Error pada key mengubah input softmax", "Error pada value masuk
 * setelah attention probability").  Hadamard caches are attended in the
 * rotated domain: q is rotated once and the output rotated back once, since
 * q.k = (Hq).(Hk) ([trefon] "Jak 4-bitowemu cache to uchodzi").  Pre-RoPE
 * keys are rotated to their positions and q to q_pos.
 *   q:   device fp16 [batch][num_q_heads][128] (before RoPE if pre_rope_keys)
 *   out: device fp32 [batch][num_q_heads][128]
 *   sm_scale <= 0 means 1/sqrt(128).
 *   workspace: device, >= kvq_workspace_bytes(cfg, batch, length), its
 *              counters zero (see kvq_workspace_bytes).  Calls that overlap
 *              in time must not share a workspace.
 * Accuracy: within |d| <= 2e-3 + 1e-2 |ref| of fp64 attention over the same
 * dequantized cache.  length == 0 writes zeros.  Waves take token chunks
 * dynamically, so the grouping of the fp32 partial sums, and with it the
 * last bits of out, can differ from call to call. */
kvq_status kvq_decode_attn(const kvq_config* cfg, const kvq_cache* cache, const void* q,
                           int64_t q_pos, float sm_scale, void* out, void* workspace,
                           uint64_t workspace_bytes, void* stream);

/* The two launches of kvq_decode_attn, exposed so a caller can time them
 * apart: kvq_decode_partials streams the cache and writes per-chunk partials
 * into the workspace; kvq_decode_merge combines them into `out`.  Same
 * arguments and errors as kvq_decode_attn; call them in this order on one
 * stream with the same workspace. */
kvq_status kvq_decode_partials(const kvq_config* cfg, const kvq_cache* cache, const void* q,
                               int64_t q_pos, float sm_scale, void* out, void* workspace,
                               uint64_t workspace_bytes, void* stream);
kvq_status kvq_decode_merge(const kvq_config* cfg, const kvq_cache* cache, const void* q,
                            int64_t q_pos, float sm_scale, void* out, void* workspace,
                            uint64_t workspace_bytes, void* stream);

/* kvq_decode_attn without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments (minus the workspace),
 * output, accuracy and errors as kvq_decode_attn.  The partials and chunk
 * counters live in a static device array of KVQ_STATIC_WORKSPACE_BYTES that
 * each GPU holds from the library's load until the process ends; the call
 * allocates nothing and starts by clearing the counters with a fill kernel.
 * Every call on one GPU uses that GPU's one array: calls that overlap in time
 * on one GPU (other streams, other threads) race, and the caller must order
 * them.  The stream must belong to the current device (KVQ_ERR_INVALID_ARG
 * otherwise).  KVQ_ERR_WORKSPACE: the call needs more than
 * KVQ_STATIC_WORKSPACE_BYTES (at most kvq_workspace_bytes of the same
 * arguments). */
#define KVQ_STATIC_WORKSPACE_BYTES (32u << 20)
kvq_status kvq_decode_attn_static(const kvq_config* cfg, const kvq_cache* cache, const void* q,
                                  int64_t q_pos, float sm_scale, void* out, void* stream);

/* Dequantize tokens [t0, t1) to fp32 in the stored domain (rotated when
 * hadamard, before RoPE when pre_rope_keys; window tokens are their fp16
 * values), the dequantize-first path of [nalar] "Biaya dequantization harus
 * masuk ke model latency", for tests and inspection.
 *   k_out, v_out: device fp32 [batch][t1 - t0][num_kv_heads][128].
 * Bit-exact: x = c * scale + zero (KIVI), (n - 8) * scale (BLOCK128, n - 4 at
 * 3 bits; Q4_0, and n - 128 for Q8_0, with the scale of the value's slice),
 * norm * level[n] (TBQ4). */
kvq_status kvq_dequant(const kvq_config* cfg, const kvq_cache* cache, int64_t t0, int64_t t1,
                       void* k_out, void* v_out, void* stream);

/* Static, never NULL. */
const char* kvq_strerror(kvq_status status);

/* KVQ_ABI_VERSION of the loaded library. */
int32_t kvq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
