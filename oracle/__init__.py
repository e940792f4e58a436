"""CPU oracle for low-bit KV-cache quantization and single-query decode attention.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously-correct
restatement of what the GPU library computes.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with the HIP library or its Python binding and
imports neither; the only code both sides use is the seeded input generator
(``quantized_decode_attention_02_amd.workloads``), which holds no arithmetic of
the method.

Numerics (fixed here because the pages fix none of them):
  * quantize / pack / dequantize run in float32 with IEEE round-to-nearest-even,
    one IEEE operation at a time (NumPy float32 arithmetic), division correctly
    rounded, ``np.rint`` for rounding, fp32->fp16 casts RNE;
  * attention runs in float64 on the dequantized cache;
  * min / max are exact, so their reduction order is free.

Sources (the pages this oracle restates; sections are the pages' own headings):
  [troisinh] "KV Cache Quantization — Nén cache INT4/INT3, mở khóa ultra-long
             context" (troisinh.com, AI Tech Decoded, level 2).
  [nalar]    "Kuantisasi KV Cache dengan Error Budget yang Eksplisit" (nalar.dev).
  [trefon]   "Matematyka cache KV: ile kosztuje długi kontekst i co daje
             4-bitowy cache" (trefon.com).
  [nexus]    "NexusQuant: Cách nén KV Cache của LLM lên tới 33 lần mà không cần
             huấn luyện" (lehuy.net).

Modules:
  tiers      -- which tokens are fp16 / high-bit / low-bit for a cache length
  hadamard   -- fixed-order fp32 FWHT-128 and the dense fp64 Sylvester matrix
  quant      -- asymmetric group quantizer (4, 3, 2 bits), symmetric 128-block
                quantizer (4, 3 bits), symmetric 32-value blocks (Q4_0, Q8_0), dequant
  codebook   -- TBQ4: Lloyd-Max levels of N(0, 1/sqrt(128)), norm + index blocks
  layout     -- the documented byte image of every cache plane, plane sizes
  attention  -- fp64 split-half RoPE and scaled-dot-product decode attention
  cache      -- a whole cache: append (with demotion), dequant, decode
  sizes      -- bytes-per-token accounting for the formats the pages tabulate

Parity status: every function here is pinned by a test in ``tests/`` against
values the pages print, closed forms, library routines or brute force.  Two
things stay unpinned because the pages fix neither: bit-level agreement with
third-party implementations of KIVI or TBQ4 (the bit conventions here are this
package's own, stated in each docstring) and model quality (perplexity, task
scores), which needs trained weights.
"""

from . import tiers, hadamard, quant, codebook, layout, attention, cache, sizes  # noqa: F401
