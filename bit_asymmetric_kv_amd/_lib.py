"""ctypes binding of libkvq.so (the C ABI declared in include/kvq.h).

Argument marshalling only: every step of quantization, packing and attention runs
in the library's HIP kernels. PyTorch supplies device memory and the stream.
The library must have been built (bit_asymmetric_kv_amd.build_lib); there is no
fallback path, so a missing library raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

KVQ_OK = 0
KVQ_ERR_INVALID_ARG = -1
KVQ_ERR_CAPACITY = -2
KVQ_ERR_OOM = -3
KVQ_ERR_HIP = -4
KVQ_ERR_NO_DEVICE = -5
KVQ_ERR_EMPTY = -6

KVQ_PART_GROUPS = 0
KVQ_PART_RING_K = 1
KVQ_PART_RING_V = 2

EXPORTED = (
    "kvq_cache_bytes", "kvq_create", "kvq_append", "kvq_decode_attention", "kvq_set_decode_split",
    "kvq_destroy", "kvq_seq_len", "kvq_group_bytes", "kvq_read_state", "kvq_last_error",
    "kvq_set_profile_events", "kvq_decode_step", "kvq_stream_read", "kvq_fp16_workspace_bytes", "kvq_fp16_decode_attention",
    "kvq_set_pages", "kvq_reset_sequence", "kvq_fp16_decode_attention_noalloc",
)


class KVQConfig(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("bits", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("residual", ctypes.c_int32),
        ("rotate", ctypes.c_int32),
        ("max_tokens", ctypes.c_int64),
        ("softmax_scale", ctypes.c_float),
        ("sink", ctypes.c_int32),
        ("rope", ctypes.c_int32),
        ("rope_base", ctypes.c_float),
        ("page_groups", ctypes.c_int32),
        ("pool_pages", ctypes.c_int64),
    ]


class KVQFp16Config(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("t_cap", ctypes.c_int64),
        ("softmax_scale", ctypes.c_float),
    ]


class KVQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"kvq status {status}: {message}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libkvq.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    # KVQ_LIBRARY names another build of the same library (the host-sanitizer build
    # that the CPU tests load in a child process)
    path = os.environ.get("KVQ_LIBRARY", LIB_PATH)
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m bit_asymmetric_kv_amd.build_lib`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    cfgp = ctypes.POINTER(KVQConfig)
    lib.kvq_cache_bytes.argtypes = [cfgp, ctypes.POINTER(sz)]
    lib.kvq_create.argtypes = [cfgp, vp, sz, vp, ctypes.POINTER(vp)]
    lib.kvq_append.argtypes = [vp, vp, vp, ctypes.POINTER(i32), i32, vp]
    lib.kvq_decode_attention.argtypes = [vp, vp, vp, vp]
    lib.kvq_decode_step.argtypes = [vp, vp, vp, ctypes.POINTER(i32), i32, vp, vp, vp]
    lib.kvq_set_decode_split.argtypes = [vp, i32]
    lib.kvq_set_profile_events.argtypes = [vp, vp, vp]
    lib.kvq_destroy.argtypes = [vp]
    lib.kvq_destroy.restype = None
    lib.kvq_seq_len.argtypes = [vp, i32, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.kvq_group_bytes.argtypes = [i32]
    lib.kvq_group_bytes.restype = sz
    lib.kvq_read_state.argtypes = [vp, i32, i32, i32, sz, vp, sz, vp]
    lib.kvq_last_error.argtypes = []
    lib.kvq_last_error.restype = ctypes.c_char_p
    f16p = ctypes.POINTER(KVQFp16Config)
    lib.kvq_stream_read.argtypes = [vp, sz, vp, i32, vp]
    lib.kvq_fp16_workspace_bytes.argtypes = [f16p, ctypes.POINTER(sz)]
    lib.kvq_fp16_decode_attention.argtypes = [f16p, vp, vp, vp, i64, vp, vp, vp, sz, vp]
    lib.kvq_fp16_decode_attention_noalloc.argtypes = [f16p, vp, vp, vp, i64, vp, vp, vp]
    lib.kvq_set_pages.argtypes = [vp, i32, ctypes.POINTER(i32), i32, vp]
    lib.kvq_reset_sequence.argtypes = [vp, i32]
    for name in ("kvq_cache_bytes", "kvq_create", "kvq_append", "kvq_decode_attention",
                 "kvq_set_decode_split", "kvq_seq_len", "kvq_read_state", "kvq_set_profile_events",
                 "kvq_decode_step", "kvq_stream_read", "kvq_fp16_workspace_bytes", "kvq_fp16_decode_attention",
                 "kvq_set_pages", "kvq_reset_sequence", "kvq_fp16_decode_attention_noalloc"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != KVQ_OK:
        raise KVQError(status, load().kvq_last_error().decode())


def make_config(batch, num_q_heads, num_kv_heads, head_dim=128, bits=2, group=32, residual=128,
                rotate=False, max_tokens=4096, softmax_scale=0.0, sink=False, rope=False,
                rope_base=0.0, page_groups=0, pool_pages=0) -> KVQConfig:
    def flag(x):
        return int(bool(x)) if x in (True, False) else int(x)
    return KVQConfig(batch, num_q_heads, num_kv_heads, head_dim, bits, group, residual, flag(rotate),
                     max_tokens, softmax_scale, flag(sink), flag(rope), rope_base, page_groups, pool_pages)


def cache_bytes(cfg: KVQConfig) -> int:
    out = ctypes.c_size_t(0)
    check(load().kvq_cache_bytes(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def group_bytes(bits: int) -> int:
    return int(load().kvq_group_bytes(bits))


def _stream_ptr(torch, device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


class KVCache:
    """A low-bit KV cache on one GPU, owning its device memory as a torch tensor."""

    def __init__(self, batch, num_q_heads, num_kv_heads, head_dim=128, bits=2, group=32, residual=128,
                 rotate=False, max_tokens=4096, softmax_scale=0.0, device="cuda", sink=False, rope=False,
                 rope_base=0.0, page_groups=0, pool_pages=0):
        import torch
        self._torch = torch
        self.cfg = make_config(batch, num_q_heads, num_kv_heads, head_dim, bits, group, residual,
                               rotate, max_tokens, softmax_scale, sink, rope, rope_base, page_groups, pool_pages)
        self.device = torch.device(device)
        nbytes = cache_bytes(self.cfg)
        self.mem = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        ptr = self.mem.data_ptr()
        self._base = (ptr + 255) & ~255
        self._handle = ctypes.c_void_p(0)
        check(load().kvq_create(ctypes.byref(self.cfg), ctypes.c_void_p(self._base), nbytes,
                                ctypes.c_void_p(_stream_ptr(torch, self.device)), ctypes.byref(self._handle)))

    # -- properties -------------------------------------------------------
    @property
    def batch(self):
        return self.cfg.batch

    @property
    def ring_len(self):
        return self.cfg.residual + self.cfg.group + self.cfg.sink

    def _check_tensor(self, t, shape, dtype, name):
        torch = self._torch
        if t.device != self.device and not (t.is_cuda and self.device.type == "cuda"):
            raise ValueError(f"{name} must be on {self.device}")
        if t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        del torch

    # -- ABI calls ---------------------------------------------------------
    def append(self, k, v, n_tokens=None):
        """k, v: fp16 [B, n_max, Hkv, D] on the device; n_tokens: per-sequence counts or None."""
        torch = self._torch
        n_max = k.shape[1]
        shape = (self.cfg.batch, n_max, self.cfg.num_kv_heads, self.cfg.head_dim)
        self._check_tensor(k, shape, torch.float16, "k")
        self._check_tensor(v, shape, torch.float16, "v")
        arr = None
        if n_tokens is not None:
            vals = [int(x) for x in n_tokens]
            if len(vals) != self.cfg.batch:
                raise ValueError("n_tokens must have one entry per sequence")
            arr = (ctypes.c_int32 * self.cfg.batch)(*vals)
        check(load().kvq_append(self._handle, ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                                arr, n_max, ctypes.c_void_p(_stream_ptr(torch, self.device))))

    def decode(self, q, out=None):
        """q: fp16 [B, Hq, D] on the device -> fp32 [B, Hq, D]."""
        torch = self._torch
        shape = (self.cfg.batch, self.cfg.num_q_heads, self.cfg.head_dim)
        self._check_tensor(q, shape, torch.float16, "q")
        if out is None:
            out = torch.empty(shape, dtype=torch.float32, device=self.device)
        else:
            self._check_tensor(out, shape, torch.float32, "out")
        check(load().kvq_decode_attention(self._handle, ctypes.c_void_p(q.data_ptr()),
                                          ctypes.c_void_p(out.data_ptr()),
                                          ctypes.c_void_p(_stream_ptr(torch, self.device))))
        return out

    def step(self, k, v, q, n_tokens=None, out=None):
        """Append k, v (fp16 [B, n_max, Hkv, D]; n_tokens per sequence or None) and
        decode q (fp16 [B, Hq, D]) in one library call -> fp32 [B, Hq, D]."""
        torch = self._torch
        n_max = k.shape[1]
        kshape = (self.cfg.batch, n_max, self.cfg.num_kv_heads, self.cfg.head_dim)
        self._check_tensor(k, kshape, torch.float16, "k")
        self._check_tensor(v, kshape, torch.float16, "v")
        qshape = (self.cfg.batch, self.cfg.num_q_heads, self.cfg.head_dim)
        self._check_tensor(q, qshape, torch.float16, "q")
        if out is None:
            out = torch.empty(qshape, dtype=torch.float32, device=self.device)
        else:
            self._check_tensor(out, qshape, torch.float32, "out")
        arr = None
        if n_tokens is not None:
            vals = [int(x) for x in n_tokens]
            if len(vals) != self.cfg.batch:
                raise ValueError("n_tokens must have one entry per sequence")
            arr = (ctypes.c_int32 * self.cfg.batch)(*vals)
        check(load().kvq_decode_step(self._handle, ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                                     arr, n_max, ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                     ctypes.c_void_p(_stream_ptr(torch, self.device))))
        return out

    def set_decode_split(self, groups_per_split: int):
        check(load().kvq_set_decode_split(self._handle, int(groups_per_split)))

    def set_pages(self, b: int, pages):
        """Paged caches: the pool pages of sequence b, in group order."""
        arr = (ctypes.c_int32 * max(1, len(pages)))(*[int(p) for p in pages])
        check(load().kvq_set_pages(self._handle, int(b), arr, len(pages),
                                   ctypes.c_void_p(_stream_ptr(self._torch, self.device))))

    def reset_sequence(self, b: int):
        """Start sequence b over (a paged cache frees its pages)."""
        check(load().kvq_reset_sequence(self._handle, int(b)))

    def set_profile_events(self, start_event: int, stop_event: int):
        """Raw hipEvent_t handles recorded around the decode split kernel (0, 0 to stop)."""
        check(load().kvq_set_profile_events(self._handle, ctypes.c_void_p(start_event or None),
                                            ctypes.c_void_p(stop_event or None)))

    def seq_len(self, b):
        T, Q = ctypes.c_int64(0), ctypes.c_int64(0)
        check(load().kvq_seq_len(self._handle, b, ctypes.byref(T), ctypes.byref(Q)))
        return T.value, Q.value

    def _read(self, part, b, h, offset, nbytes):
        buf = np.empty(nbytes, dtype=np.uint8)
        check(load().kvq_read_state(self._handle, part, b, h, offset, buf.ctypes.data_as(ctypes.c_void_p),
                                    nbytes, ctypes.c_void_p(_stream_ptr(self._torch, self.device))))
        return buf

    def read_groups(self, b, h, first, count):
        """Packed blocks of groups [first, first + count) of (b, h): uint8 [count, group_bytes]."""
        gb = group_bytes(self.cfg.bits)
        return self._read(KVQ_PART_GROUPS, b, h, first * gb, count * gb).reshape(count, gb)

    def read_ring(self, b, h, which="k"):
        """FP16 window of (b, h): fp16 [R + G, D]; token t sits in slot t % (R + G)."""
        part = KVQ_PART_RING_K if which == "k" else KVQ_PART_RING_V
        n = self.ring_len * self.cfg.head_dim * 2
        return self._read(part, b, h, 0, n).view(np.float16).reshape(self.ring_len, self.cfg.head_dim)

    def close(self):
        if getattr(self, "_handle", None) and self._handle.value:
            load().kvq_destroy(self._handle)
            self._handle = ctypes.c_void_p(0)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# -- comparison kernels -------------------------------------------------------

def stream_read(buf, fold):
    """Stream-read every byte of the device tensor `buf` once with one workgroup per
    element of the int32 device tensor `fold`, which receives their xor folds (the xor
    of all elements equals the xor of every 32-bit word of `buf`). Asynchronous on the
    current stream."""
    import torch
    if fold.dtype != torch.int32 or not fold.is_contiguous() or not fold.is_cuda:
        raise ValueError("fold must be a contiguous int32 device tensor")
    check(load().kvq_stream_read(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                                 ctypes.c_void_p(fold.data_ptr()), int(fold.numel()),
                                 ctypes.c_void_p(_stream_ptr(torch, buf.device))))


class Fp16Decode:
    """Decode attention over a plain FP16 cache k, v [B, Hkv, t_cap, D] (comparison
    baseline of the quantized path). Owns its workspace as a torch tensor."""

    def __init__(self, batch, num_q_heads, num_kv_heads, t_cap, head_dim=128, softmax_scale=0.0, device="cuda",
                 static_scratch=False):
        """static_scratch: call kvq_fp16_decode_attention_noalloc, whose split partials
        live in the library's static per-GPU scratch (no workspace is allocated)."""
        import torch
        self._torch = torch
        self.device = torch.device(device)
        self.cfg = KVQFp16Config(batch, num_q_heads, num_kv_heads, head_dim, t_cap, softmax_scale)
        self.static_scratch = bool(static_scratch)
        self.workspace = None
        if not self.static_scratch:
            nbytes = ctypes.c_size_t(0)
            check(load().kvq_fp16_workspace_bytes(ctypes.byref(self.cfg), ctypes.byref(nbytes)))
            self.workspace = torch.empty(nbytes.value, dtype=torch.uint8, device=self.device)

    def __call__(self, k, v, seq_lens, max_len, q, out=None):
        """k, v: fp16 [B, Hkv, t_cap, D]; seq_lens: int32 [B] on the device; q: fp16 [B, Hq, D]."""
        torch = self._torch
        c = self.cfg
        for t, shape, dt, name in ((k, (c.batch, c.num_kv_heads, c.t_cap, c.head_dim), torch.float16, "k"),
                                   (v, (c.batch, c.num_kv_heads, c.t_cap, c.head_dim), torch.float16, "v"),
                                   (seq_lens, (c.batch,), torch.int32, "seq_lens"),
                                   (q, (c.batch, c.num_q_heads, c.head_dim), torch.float16, "q")):
            if t.dtype != dt or tuple(t.shape) != shape or not t.is_contiguous() or not t.is_cuda:
                raise ValueError(f"{name} must be a contiguous {dt} device tensor of shape {shape}")
        if out is None:
            out = torch.empty((c.batch, c.num_q_heads, c.head_dim), dtype=torch.float32, device=self.device)
        elif (out.dtype != torch.float32 or tuple(out.shape) != (c.batch, c.num_q_heads, c.head_dim)
              or not out.is_contiguous() or not out.is_cuda):
            raise ValueError("out must be a contiguous float32 device tensor of shape [B, Hq, D]")
        stream = ctypes.c_void_p(_stream_ptr(torch, self.device))
        if self.static_scratch:
            check(load().kvq_fp16_decode_attention_noalloc(
                ctypes.byref(c), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                ctypes.c_void_p(seq_lens.data_ptr()), int(max_len), ctypes.c_void_p(q.data_ptr()),
                ctypes.c_void_p(out.data_ptr()), stream))
        else:
            check(load().kvq_fp16_decode_attention(
                ctypes.byref(c), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                ctypes.c_void_p(seq_lens.data_ptr()), int(max_len), ctypes.c_void_p(q.data_ptr()),
                ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(self.workspace.data_ptr()),
                self.workspace.numel(), stream))
        return out
