"""ctypes binding of libkvq (include/kvq.h): argument marshalling only.

Every step of the method runs in the HIP library; this module turns torch
tensors into device pointers and the current torch stream into a hipStream_t.
Importing it fails loudly when ``_lib/libkvq.so`` has not been built
(``python -m quantized_decode_attention_02_amd.build``); there is no fallback.
"""

import ctypes
import os

import torch

# KVQ_LIBRARY may point at another build of the same library (e.g. a tuning
# variant); by default the in-tree build is loaded.
_LIB_PATH = os.environ.get("KVQ_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "_lib", "libkvq.so")

KIVI_ASYM, BLOCK128_SYM, TBQ4, Q4_0, Q8_0 = 0, 1, 2, 3, 4
MAX_PLANES = 16
NUM_PLANES = 9
PLANE_NAMES = ["K_HI", "V_HI", "K_LO", "V_LO", "K_META", "V_META", "K_WIN", "V_WIN", "ROPE"]
STATUS = {0: "OK", -1: "INVALID_ARG", -2: "UNSUPPORTED", -3: "CAPACITY", -4: "WORKSPACE", -5: "HIP"}

# every symbol include/kvq.h declares
EXPORTS = ["kvq_layout", "kvq_workspace_bytes", "kvq_append", "kvq_decode_attn",
           "kvq_decode_partials", "kvq_decode_merge", "kvq_dequant", "kvq_decode_attn_static",
           "kvq_strerror", "kvq_abi_version"]
STATIC_WORKSPACE_BYTES = 32 << 20


class KvqError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({strerror(status)})")


class Config(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("scheme", ctypes.c_int32),
                ("k_bits", ctypes.c_int32), ("v_bits", ctypes.c_int32),
                ("k_group_tokens", ctypes.c_int32), ("v_group_dims", ctypes.c_int32),
                ("fp16_window", ctypes.c_int32), ("int4_window", ctypes.c_int32),
                ("low_bits", ctypes.c_int32), ("hadamard", ctypes.c_int32),
                ("pre_rope_keys", ctypes.c_int32), ("rope_theta", ctypes.c_float),
                ("hadamard_sign_in", ctypes.c_uint32 * 4), ("hadamard_sign_out", ctypes.c_uint32 * 4)]


class Layout(ctypes.Structure):
    _fields_ = [("plane_bytes", ctypes.c_uint64 * MAX_PLANES), ("alignment", ctypes.c_uint64),
                ("groups", ctypes.c_int64), ("hi_slots", ctypes.c_int64)]


class CacheStruct(ctypes.Structure):
    _fields_ = [("planes", ctypes.c_void_p * MAX_PLANES), ("batch", ctypes.c_int64),
                ("max_tokens", ctypes.c_int64), ("length", ctypes.c_int64)]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"libkvq.so is not built ({_LIB_PATH}); run "
                          "python -m quantized_decode_attention_02_amd.build")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER
    vp, i64, u64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64
    lib.kvq_layout.argtypes = [P(Config), i64, i64, P(Layout)]
    lib.kvq_workspace_bytes.argtypes = [P(Config), i64, i64, P(u64)]
    lib.kvq_append.argtypes = [P(Config), P(CacheStruct), vp, vp, i64, vp]
    dec = [P(Config), P(CacheStruct), vp, i64, ctypes.c_float, vp, vp, u64, vp]
    lib.kvq_decode_attn.argtypes = dec
    lib.kvq_decode_partials.argtypes = dec
    lib.kvq_decode_merge.argtypes = dec
    lib.kvq_dequant.argtypes = [P(Config), P(CacheStruct), i64, i64, vp, vp, vp]
    lib.kvq_decode_attn_static.argtypes = [P(Config), P(CacheStruct), vp, i64, ctypes.c_float, vp, vp]
    lib.kvq_strerror.argtypes = [ctypes.c_int]
    lib.kvq_strerror.restype = ctypes.c_char_p
    lib.kvq_abi_version.restype = ctypes.c_int32
    for name in EXPORTS[:8]:
        getattr(lib, name).restype = ctypes.c_int
    return lib


LIB = _load()
LIB_PATH = _LIB_PATH


def strerror(status):
    return LIB.kvq_strerror(status).decode()


def _check(status, what):
    if status != 0:
        raise KvqError(status, what)


def make_config(d):
    """kvq_config from a plain dict (keys as in workloads.library_config)."""
    scheme = {"kivi": KIVI_ASYM, "block128": BLOCK128_SYM, "tbq4": TBQ4, "q4_0": Q4_0,
              "q8_0": Q8_0}[d["scheme"]]
    return Config(head_dim=d.get("head_dim", 128), num_q_heads=d["num_q_heads"],
                  num_kv_heads=d["num_kv_heads"], scheme=scheme, k_bits=d.get("k_bits", 4),
                  v_bits=d.get("v_bits", 4), k_group_tokens=d.get("group", 32),
                  v_group_dims=d.get("vdims", 32),
                  fp16_window=d.get("window", 128 if scheme == KIVI_ASYM else 0),
                  int4_window=d.get("hi_window", -1), low_bits=d.get("low_bits", 2),
                  hadamard=int(bool(d.get("hadamard", False))),
                  pre_rope_keys=int(bool(d.get("pre_rope", False))),
                  rope_theta=float(d.get("rope_theta", 10000.0)),
                  hadamard_sign_in=(ctypes.c_uint32 * 4)(*(d.get("sign_in") or [0, 0, 0, 0])),
                  hadamard_sign_out=(ctypes.c_uint32 * 4)(*(d.get("sign_out") or [0, 0, 0, 0])))


def layout(cfg, batch, max_tokens):
    lay = Layout()
    _check(LIB.kvq_layout(ctypes.byref(cfg), batch, max_tokens, ctypes.byref(lay)), "kvq_layout")
    return lay


def workspace_bytes(cfg, batch, length):
    n = ctypes.c_uint64()
    _check(LIB.kvq_workspace_bytes(ctypes.byref(cfg), batch, length, ctypes.byref(n)),
           "kvq_workspace_bytes")
    return n.value


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, shape, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)}, got "
                         f"{t.dtype} {tuple(t.shape)}")


class KVCache:
    """A cache of ``batch`` sequences of up to ``max_tokens`` tokens.

    The planes are zero-initialized torch uint8 tensors sized by kvq_layout."""

    def __init__(self, cfg_dict, batch, max_tokens, device="cuda"):
        self.cfg_dict = dict(cfg_dict)
        self.cfg = make_config(cfg_dict)
        self.batch, self.max_tokens = batch, max_tokens
        self.layout = layout(self.cfg, batch, max_tokens)
        self.planes = []
        self.struct = CacheStruct()
        for i in range(NUM_PLANES):
            n = int(self.layout.plane_bytes[i])
            t = torch.zeros(n, dtype=torch.uint8, device=device) if n else None
            self.planes.append(t)
            self.struct.planes[i] = t.data_ptr() if t is not None else 0
        self.struct.batch = batch
        self.struct.max_tokens = max_tokens
        self.struct.length = 0

    @property
    def length(self):
        return self.struct.length

    @length.setter
    def length(self, v):
        self.struct.length = int(v)

    @property
    def hkv(self):
        return self.cfg.num_kv_heads

    @property
    def hq(self):
        return self.cfg.num_q_heads

    def append(self, k_new, v_new, stream=None):
        """k_new, v_new: fp16 [batch, n, Hkv, 128] device tensors."""
        n = k_new.shape[1]
        shape = (self.batch, n, self.hkv, 128)
        _need(k_new, torch.float16, shape, "k_new")
        _need(v_new, torch.float16, shape, "v_new")
        _check(LIB.kvq_append(ctypes.byref(self.cfg), ctypes.byref(self.struct), _ptr(k_new),
                              _ptr(v_new), n, _stream(stream)), "kvq_append")

    def workspace_bytes(self):
        return workspace_bytes(self.cfg, self.batch, self.length)

    def new_workspace(self):
        # zero: the leading work counters must start at zero (every decode
        # call leaves them so)
        return torch.zeros(max(1, self.workspace_bytes() // 4), dtype=torch.float32, device="cuda")

    def _decode_args(self, q, q_pos, sm_scale, out, workspace):
        _need(q, torch.float16, (self.batch, self.hq, 128), "q")
        if out is None:
            out = torch.empty((self.batch, self.hq, 128), dtype=torch.float32, device=q.device)
        _need(out, torch.float32, (self.batch, self.hq, 128), "out")
        if workspace is None:
            workspace = self.new_workspace()
        pos = self.length if q_pos is None else int(q_pos)
        return (ctypes.byref(self.cfg), ctypes.byref(self.struct), _ptr(q), pos,
                ctypes.c_float(sm_scale), _ptr(out), _ptr(workspace),
                workspace.numel() * workspace.element_size()), out

    def decode(self, q, q_pos=None, sm_scale=0.0, out=None, workspace=None, stream=None):
        """fp32 [batch, Hq, 128] attention output (both launches)."""
        args, out = self._decode_args(q, q_pos, sm_scale, out, workspace)
        _check(LIB.kvq_decode_attn(*args, _stream(stream)), "kvq_decode_attn")
        return out

    def decode_partials(self, q, workspace, out, q_pos=None, sm_scale=0.0, stream=None):
        args, _ = self._decode_args(q, q_pos, sm_scale, out, workspace)
        _check(LIB.kvq_decode_partials(*args, _stream(stream)), "kvq_decode_partials")

    def decode_merge(self, q, workspace, out, q_pos=None, sm_scale=0.0, stream=None):
        args, _ = self._decode_args(q, q_pos, sm_scale, out, workspace)
        _check(LIB.kvq_decode_merge(*args, _stream(stream)), "kvq_decode_merge")

    def decode_static(self, q, q_pos=None, sm_scale=0.0, out=None, stream=None):
        """As decode(), through kvq_decode_attn_static: no workspace argument,
        the library's static per-GPU array instead (nothing is allocated
        beyond ``out`` when it is not given)."""
        _need(q, torch.float16, (self.batch, self.hq, 128), "q")
        if out is None:
            out = torch.empty((self.batch, self.hq, 128), dtype=torch.float32, device=q.device)
        _need(out, torch.float32, (self.batch, self.hq, 128), "out")
        pos = self.length if q_pos is None else int(q_pos)
        _check(LIB.kvq_decode_attn_static(ctypes.byref(self.cfg), ctypes.byref(self.struct), _ptr(q), pos,
                                          ctypes.c_float(sm_scale), _ptr(out), _stream(stream)),
               "kvq_decode_attn_static")
        return out

    def dequant(self, t0=0, t1=None, stream=None):
        """fp32 [batch, t1 - t0, Hkv, 128] keys and values in the stored domain."""
        t1 = self.length if t1 is None else t1
        shape = (self.batch, max(0, t1 - t0), self.hkv, 128)
        k = torch.empty(shape, dtype=torch.float32, device="cuda")
        v = torch.empty(shape, dtype=torch.float32, device="cuda")
        _check(LIB.kvq_dequant(ctypes.byref(self.cfg), ctypes.byref(self.struct), t0, t1, _ptr(k),
                               _ptr(v), _stream(stream)), "kvq_dequant")
        return k, v
