"""kvq: low-bit KV-cache quantization and single-query decode attention on MI355X.

The compute path is the C-ABI library ``libkvq.so`` (HIP kernels for gfx950);
``kvq`` is its thin ctypes binding (torch tensors in, device pointers out) and
``workloads`` holds the seeded synthetic inputs.  Import ``kvq`` explicitly:

    from quantized_decode_attention_02_amd import kvq, workloads
"""

__all__ = ["kvq", "workloads"]
