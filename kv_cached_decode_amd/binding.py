"""Thin ctypes binding over libkvdecode.so (the C ABI in include/kvdecode.h).

Argument marshalling only: every function checks that the torch tensors it is
given are on the ROCm device, contiguous and of the expected dtype, then
passes their data pointers, the sizes and torch's current HIP stream to the C
entry point of the same name. Nothing here computes any step of the path, and
there is no fallback: when the library is missing every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from ctypes import c_float, c_int, c_int32, c_size_t, c_void_p

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvdecode.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "kvdecode.h")

F32, F16, BF16 = 0, 1, 2
DTYPE_CODE = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
CODE_DTYPE = {v: k for k, v in DTYPE_CODE.items()}
HEAD_DIM = 64


class KvdCache(ctypes.Structure):
    _fields_ = [("k", c_void_p), ("v", c_void_p), ("B", c_int32), ("H", c_int32),
                ("S_max", c_int32), ("D", c_int32), ("dtype", c_int32)]


class KVDError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")
        self.status = status


_lib = None

_SIGNATURES = {
    "kv_append": (c_int, [ctypes.POINTER(KvdCache), c_void_p, c_void_p, c_int32, c_int32,
                          c_float, c_void_p]),
    "kv_reorder": (c_int, [ctypes.POINTER(KvdCache), c_void_p, c_int32, c_void_p, c_void_p]),
    "kv_append_ragged": (c_int, [ctypes.POINTER(KvdCache), c_void_p, c_void_p, c_void_p, c_int32,
                                 c_float, c_void_p, c_void_p]),
    "decode_attn_self_ragged": (c_int, [c_void_p, c_int32, c_int32, ctypes.POINTER(KvdCache),
                                        c_void_p, c_int32, c_float, c_float, c_void_p, c_void_p,
                                        c_size_t, c_void_p, c_void_p]),
    "decode_step_self_ragged": (c_int, [c_void_p, c_void_p, c_void_p, c_int32, c_int32,
                                        ctypes.POINTER(KvdCache), c_void_p, c_int32, c_float,
                                        c_float, c_void_p, c_void_p, c_size_t, c_void_p,
                                        c_void_p]),
    "decode_attn_self": (c_int, [c_void_p, c_int32, c_int32, ctypes.POINTER(KvdCache), c_int32,
                                 c_float, c_float, c_void_p, c_void_p, c_size_t, c_void_p]),
    "decode_step_self": (c_int, [c_void_p, c_void_p, c_void_p, c_int32, c_int32,
                                 ctypes.POINTER(KvdCache), c_int32, c_float, c_float, c_void_p,
                                 c_void_p, c_size_t, c_void_p]),
    "decode_step_self_beams": (c_int, [c_void_p, c_void_p, c_void_p, c_int32, c_int32,
                                       ctypes.POINTER(KvdCache), ctypes.POINTER(KvdCache),
                                       c_void_p, c_int32, c_float, c_float, c_void_p, c_void_p,
                                       c_size_t, c_void_p, c_void_p]),
    "decode_attn_cross": (c_int, [c_void_p, c_int32, c_int32, c_int32, ctypes.POINTER(KvdCache),
                                  c_int32, c_float, c_void_p, c_void_p, c_size_t, c_void_p]),
    "verify_accept": (c_int, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p, c_int32,
                              c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "kvd_attn_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32, c_int32]),
    "verify_accept_masked": (c_int, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p,
                                     c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_size_t, c_void_p]),
    "kvd_verify_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32]),
    "beam_select": (c_int, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p, c_int32,
                            c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                            c_void_p, c_size_t, c_void_p]),
    "kvd_beam_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32]),
    "kvd_status_string": (ctypes.c_char_p, [c_int]),
    "kvd_time_next_launch": (c_int, [c_void_p, c_void_p]),
    "kvd_read_probe": (c_int, [c_void_p, c_void_p, c_size_t, c_void_p, c_void_p]),
    "kvd_read_probe_ex": (c_int, [c_void_p, c_void_p, c_size_t, c_void_p, c_int32, c_size_t,
                                  c_void_p]),
    "kvd_set_plan_override": (c_int, [c_int32, c_int32, c_int32]),
    "decode_step_self_static": (c_int, [c_void_p, c_void_p, c_void_p, c_int32, c_int32,
                                        ctypes.POINTER(KvdCache), c_int32, c_float, c_float,
                                        c_void_p, c_void_p]),
    "kvd_static_scratch_bytes": (c_size_t, []),
}


def lib() -> ctypes.CDLL:
    """Open libkvdecode.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m kv_cached_decode_amd.build` (no fallback exists)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def declared_functions() -> list[str]:
    """Names of the functions include/kvdecode.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)


def status_string(status: int) -> str:
    return lib().kvd_status_string(int(status)).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise KVDError(fn, status)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, name: str, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the ROCm device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


class Cache:
    """One layer's K/V cache preallocated to capacity: k, v [B, H, S_max, D]."""

    def __init__(self, B: int, H: int, S_max: int, dtype=torch.float16, device="cuda",
                 D: int = HEAD_DIM):
        self.k = torch.zeros((B, H, S_max, D), dtype=dtype, device=device)
        self.v = torch.zeros((B, H, S_max, D), dtype=dtype, device=device)
        self._desc = None

    @classmethod
    def wrap(cls, k: torch.Tensor, v: torch.Tensor) -> "Cache":
        c = cls.__new__(cls)
        c.k, c.v, c._desc = k, v, None
        return c

    @property
    def B(self):
        return self.k.shape[0]

    @property
    def H(self):
        return self.k.shape[1]

    @property
    def S_max(self):
        return self.k.shape[2]

    @property
    def dtype(self):
        return self.k.dtype

    def desc(self) -> KvdCache:
        if self._desc is None:
            if self.k.dim() != 4 or self.k.shape != self.v.shape or self.k.dtype != self.v.dtype:
                raise ValueError("k and v must be [B, H, S_max, D] tensors of one dtype")
            if self.k.dtype not in DTYPE_CODE:
                raise ValueError(f"unsupported cache dtype {self.k.dtype}")
            B, H, S, D = self.k.shape
            self._desc = KvdCache(_dev(self.k, "cache.k"), _dev(self.v, "cache.v"),
                                  B, H, S, D, DTYPE_CODE[self.k.dtype])
        return self._desc


def time_next_launch(start: "torch.cuda.Event", stop: "torch.cuda.Event"):
    """The next kernel launch of this thread records `start` at kernel begin
    and `stop` at kernel end (both events must have been recorded once, which
    creates them)."""
    _check("kvd_time_next_launch", lib().kvd_time_next_launch(start.cuda_event, stop.cuda_event))


def read_probe(a: torch.Tensor, b: torch.Tensor | None, nbytes: int, sink: torch.Tensor,
               unroll: int = 4, blocks: int = 0):
    """Plain streaming read of nbytes from a (and from b): the attainable
    rate for one launch that reads that much. unroll: loads in flight per
    thread; blocks: workgroups of 256 threads (0: one round of loads)."""
    _check("kvd_read_probe_ex", lib().kvd_read_probe_ex(
        _dev(a, "a"), _dev(b, "b") if b is not None else None, int(nbytes), _dev(sink, "sink"),
        int(unroll), int(blocks), _stream()))


class plan_override:
    """Context manager that forces the attention split plan of the calls made
    inside it (a testing hook: kvd_set_plan_override). mfma=0 keeps 16-bit
    caches on the streaming kernel; waves / chunk force the waves per
    workgroup and the keys per split; None leaves each as planned. Workspace
    sizes queried inside the block follow the forced plan."""

    def __init__(self, mfma: int | None = None, waves: int | None = None, chunk: int | None = None):
        self.args = (-1 if mfma is None else int(mfma), 0 if waves is None else int(waves),
                     0 if chunk is None else int(chunk))

    def __enter__(self):
        _check("kvd_set_plan_override", lib().kvd_set_plan_override(*self.args))
        return self

    def __exit__(self, *exc):
        _check("kvd_set_plan_override", lib().kvd_set_plan_override(-1, 0, 0))
        return False


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A zero-filled device workspace (the counters at its start must be zero
    before first use; the kernels leave them that way)."""
    return torch.zeros(max(int(nbytes), 16384), dtype=torch.uint8, device=device)


def attn_workspace_bytes(B: int, Hq: int, N: int, len_max: int) -> int:
    return int(lib().kvd_attn_workspace_bytes(B, Hq, N, len_max))


def verify_workspace_bytes(B: int, R: int, V: int) -> int:
    return int(lib().kvd_verify_workspace_bytes(B, R, V))


def kv_append(cache: Cache, k_new: torch.Tensor, v_new: torch.Tensor, pos: int,
              rope_base: float = 0.0):
    d = cache.desc()
    if k_new.dim() != 4 or k_new.shape != v_new.shape:
        raise ValueError("k_new and v_new must be [B, H, T, D] of one shape")
    T = k_new.shape[2]
    if (k_new.shape[0], k_new.shape[1], k_new.shape[3]) != (d.B, d.H, d.D):
        raise ValueError(f"k_new shape {tuple(k_new.shape)} does not match the cache")
    _check("kv_append", lib().kv_append(
        ctypes.byref(d), _dev(k_new, "k_new", cache.dtype), _dev(v_new, "v_new", cache.dtype),
        pos, T, rope_base, _stream()))


def kv_reorder(cache: Cache, parent: torch.Tensor, length: int,
               dev_status: torch.Tensor | None = None):
    d = cache.desc()
    if parent.numel() != d.B:
        raise ValueError("parent must hold one index per beam")
    st = _dev(dev_status, "dev_status", torch.int32) if dev_status is not None else None
    _check("kv_reorder", lib().kv_reorder(ctypes.byref(d), _dev(parent, "parent", torch.int32),
                                          length, st, _stream()))


def _attn_out(q: torch.Tensor, out):
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    return out


def decode_attn_self(q: torch.Tensor, cache: Cache, length: int, scale: float,
                     rope_base: float = 0.0, out: torch.Tensor | None = None,
                     ws: torch.Tensor | None = None) -> torch.Tensor:
    d = cache.desc()
    if q.dim() != 4 or q.shape[0] != d.B or q.shape[3] != d.D:
        raise ValueError(f"q must be [B={d.B}, Hq, N, {d.D}], got {tuple(q.shape)}")
    Hq, N = q.shape[1], q.shape[2]
    out = _attn_out(q, out)
    if ws is None:
        ws = workspace(attn_workspace_bytes(d.B, Hq, N, length), q.device)
    _check("decode_attn_self", lib().decode_attn_self(
        _dev(q, "q", cache.dtype), Hq, N, ctypes.byref(d), length, scale, rope_base,
        _dev(out, "out", torch.float32), _dev(ws, "ws"), ws.numel() * ws.element_size(),
        _stream()))
    return out


def decode_step_self(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, cache: Cache,
                     length: int, scale: float, rope_base: float = 0.0,
                     out: torch.Tensor | None = None,
                     ws: torch.Tensor | None = None) -> torch.Tensor:
    """kv_append of the N new rows at [length - N, length) plus decode_attn_self,
    one launch for N <= 16."""
    d = cache.desc()
    if q.dim() != 4 or q.shape[0] != d.B or q.shape[3] != d.D:
        raise ValueError(f"q must be [B={d.B}, Hq, N, {d.D}], got {tuple(q.shape)}")
    Hq, N = q.shape[1], q.shape[2]
    if tuple(k_new.shape) != (d.B, d.H, N, d.D) or k_new.shape != v_new.shape:
        raise ValueError(f"k_new/v_new must be [{d.B}, {d.H}, {N}, {d.D}]")
    out = _attn_out(q, out)
    if ws is None:
        ws = workspace(attn_workspace_bytes(d.B, Hq, N, length), q.device)
    _check("decode_step_self", lib().decode_step_self(
        _dev(q, "q", cache.dtype), _dev(k_new, "k_new", cache.dtype),
        _dev(v_new, "v_new", cache.dtype), Hq, N, ctypes.byref(d), length, scale, rope_base,
        _dev(out, "out", torch.float32), _dev(ws, "ws"), ws.numel() * ws.element_size(),
        _stream()))
    return out


def decode_step_self_static(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                            cache: Cache, length: int, scale: float, rope_base: float = 0.0,
                            out: torch.Tensor | None = None) -> torch.Tensor:
    """decode_step_self with no workspace: the library's static device array
    serves the split merge (nothing is allocated by the call; `out` is
    allocated here when not given)."""
    d = cache.desc()
    if q.dim() != 4 or q.shape[0] != d.B or q.shape[3] != d.D:
        raise ValueError(f"q must be [B={d.B}, Hq, N, {d.D}], got {tuple(q.shape)}")
    Hq, N = q.shape[1], q.shape[2]
    if tuple(k_new.shape) != (d.B, d.H, N, d.D) or k_new.shape != v_new.shape:
        raise ValueError(f"k_new/v_new must be [{d.B}, {d.H}, {N}, {d.D}]")
    out = _attn_out(q, out)
    _check("decode_step_self_static", lib().decode_step_self_static(
        _dev(q, "q", cache.dtype), _dev(k_new, "k_new", cache.dtype),
        _dev(v_new, "v_new", cache.dtype), Hq, N, ctypes.byref(d), length, scale, rope_base,
        _dev(out, "out", torch.float32), _stream()))
    return out


def static_scratch_bytes() -> int:
    return int(lib().kvd_static_scratch_bytes())


def _rows(t: torch.Tensor, B: int, name: str):
    if t.numel() != B:
        raise ValueError(f"{name} must hold one int32 per batch row ({B})")
    return _dev(t, name, torch.int32)


def kv_append_ragged(cache: Cache, k_new: torch.Tensor, v_new: torch.Tensor, pos: torch.Tensor,
                     rope_base: float = 0.0, dev_status: torch.Tensor | None = None):
    """kv_append with batch row b written at [pos[b], pos[b] + T) (pos: device
    int32 [B])."""
    d = cache.desc()
    if k_new.dim() != 4 or k_new.shape != v_new.shape:
        raise ValueError("k_new and v_new must be [B, H, T, D] of one shape")
    if (k_new.shape[0], k_new.shape[1], k_new.shape[3]) != (d.B, d.H, d.D):
        raise ValueError(f"k_new shape {tuple(k_new.shape)} does not match the cache")
    st = _dev(dev_status, "dev_status", torch.int32) if dev_status is not None else None
    _check("kv_append_ragged", lib().kv_append_ragged(
        ctypes.byref(d), _dev(k_new, "k_new", cache.dtype), _dev(v_new, "v_new", cache.dtype),
        _rows(pos, d.B, "pos"), k_new.shape[2], rope_base, st, _stream()))


def decode_attn_self_ragged(q: torch.Tensor, cache: Cache, lens: torch.Tensor, len_max: int,
                            scale: float, rope_base: float = 0.0, out: torch.Tensor | None = None,
                            ws: torch.Tensor | None = None,
                            dev_status: torch.Tensor | None = None) -> torch.Tensor:
    """decode_attn_self with per-row lengths (lens: device int32 [B], each in
    [N, len_max])."""
    d = cache.desc()
    if q.dim() != 4 or q.shape[0] != d.B or q.shape[3] != d.D:
        raise ValueError(f"q must be [B={d.B}, Hq, N, {d.D}], got {tuple(q.shape)}")
    Hq, N = q.shape[1], q.shape[2]
    out = _attn_out(q, out)
    if ws is None:
        ws = workspace(attn_workspace_bytes(d.B, Hq, N, len_max), q.device)
    st = _dev(dev_status, "dev_status", torch.int32) if dev_status is not None else None
    _check("decode_attn_self_ragged", lib().decode_attn_self_ragged(
        _dev(q, "q", cache.dtype), Hq, N, ctypes.byref(d), _rows(lens, d.B, "lens"), len_max,
        scale, rope_base, _dev(out, "out", torch.float32), _dev(ws, "ws"),
        ws.numel() * ws.element_size(), st, _stream()))
    return out


def decode_step_self_ragged(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                            cache: Cache, lens: torch.Tensor, len_max: int, scale: float,
                            rope_base: float = 0.0, out: torch.Tensor | None = None,
                            ws: torch.Tensor | None = None,
                            dev_status: torch.Tensor | None = None) -> torch.Tensor:
    """kv_append_ragged of the N new rows at [lens[b] - N, lens[b]) plus
    decode_attn_self_ragged, one launch (N <= 16)."""
    d = cache.desc()
    if q.dim() != 4 or q.shape[0] != d.B or q.shape[3] != d.D:
        raise ValueError(f"q must be [B={d.B}, Hq, N, {d.D}], got {tuple(q.shape)}")
    Hq, N = q.shape[1], q.shape[2]
    if tuple(k_new.shape) != (d.B, d.H, N, d.D) or k_new.shape != v_new.shape:
        raise ValueError(f"k_new/v_new must be [{d.B}, {d.H}, {N}, {d.D}]")
    out = _attn_out(q, out)
    if ws is None:
        ws = workspace(attn_workspace_bytes(d.B, Hq, N, len_max), q.device)
    st = _dev(dev_status, "dev_status", torch.int32) if dev_status is not None else None
    _check("decode_step_self_ragged", lib().decode_step_self_ragged(
        _dev(q, "q", cache.dtype), _dev(k_new, "k_new", cache.dtype),
        _dev(v_new, "v_new", cache.dtype), Hq, N, ctypes.byref(d), _rows(lens, d.B, "lens"),
        len_max, scale, rope_base, _dev(out, "out", torch.float32), _dev(ws, "ws"),
        ws.numel() * ws.element_size(), st, _stream()))
    return out


def decode_step_self_beams(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                           src: Cache, dst: Cache, parent: torch.Tensor, length: int,
                           scale: float, rope_base: float = 0.0,
                           out: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                           dev_status: torch.Tensor | None = None) -> torch.Tensor:
    """One beam step on two caches used in turn: dst rows [0, length - N) of
    beam b become src rows of beam parent[b], the N new rows are appended at
    [length - N, length) of dst and the queries attend over dst; one launch
    (N <= 16)."""
    d, s = dst.desc(), src.desc()
    if q.dim() != 4 or q.shape[0] != d.B or q.shape[3] != d.D:
        raise ValueError(f"q must be [B={d.B}, Hq, N, {d.D}], got {tuple(q.shape)}")
    Hq, N = q.shape[1], q.shape[2]
    if tuple(k_new.shape) != (d.B, d.H, N, d.D) or k_new.shape != v_new.shape:
        raise ValueError(f"k_new/v_new must be [{d.B}, {d.H}, {N}, {d.D}]")
    out = _attn_out(q, out)
    if ws is None:
        ws = workspace(attn_workspace_bytes(d.B, Hq, N, length), q.device)
    st = _dev(dev_status, "dev_status", torch.int32) if dev_status is not None else None
    _check("decode_step_self_beams", lib().decode_step_self_beams(
        _dev(q, "q", dst.dtype), _dev(k_new, "k_new", dst.dtype),
        _dev(v_new, "v_new", dst.dtype), Hq, N, ctypes.byref(s), ctypes.byref(d),
        _rows(parent, d.B, "parent"), length, scale, rope_base,
        _dev(out, "out", torch.float32), _dev(ws, "ws"), ws.numel() * ws.element_size(), st,
        _stream()))
    return out


def decode_attn_cross(q: torch.Tensor, xcache: Cache, frames: int, scale: float,
                      out: torch.Tensor | None = None,
                      ws: torch.Tensor | None = None) -> torch.Tensor:
    d = xcache.desc()
    if q.dim() != 4 or q.shape[3] != d.D:
        raise ValueError(f"q must be [B, Hq, N, {d.D}], got {tuple(q.shape)}")
    B, Hq, N = q.shape[0], q.shape[1], q.shape[2]
    out = _attn_out(q, out)
    if ws is None:
        ws = workspace(attn_workspace_bytes(B, Hq, N, frames), q.device)
    _check("decode_attn_cross", lib().decode_attn_cross(
        _dev(q, "q", xcache.dtype), B, Hq, N, ctypes.byref(d), frames, scale,
        _dev(out, "out", torch.float32), _dev(ws, "ws"), ws.numel() * ws.element_size(),
        _stream()))
    return out


def verify_accept(logits: torch.Tensor, draft: torch.Tensor,
                  argmax_out: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                  accept_len: torch.Tensor | None = None,
                  next_token: torch.Tensor | None = None):
    """Returns (accept_len int32[B], next_token int32[B], argmax int32[B, R] or None)."""
    if logits.dim() != 3 or draft.dim() != 2 or draft.shape[0] != logits.shape[0]:
        raise ValueError("logits must be [B, R, V] and draft [B, N]")
    if logits.dtype not in DTYPE_CODE:
        raise ValueError(f"unsupported logits dtype {logits.dtype}")
    B, R, V = logits.shape
    N = draft.shape[1]
    dev = logits.device
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if next_token is None:
        next_token = torch.empty(B, dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(verify_workspace_bytes(B, R, V), dev)
    am = _dev(argmax_out, "argmax_out", torch.int32) if argmax_out is not None else None
    _check("verify_accept", lib().verify_accept(
        _dev(logits, "logits"), DTYPE_CODE[logits.dtype], B, R, V,
        _dev(draft, "draft", torch.int32), N, am, _dev(accept_len, "accept_len", torch.int32),
        _dev(next_token, "next_token", torch.int32), _dev(ws, "ws"),
        ws.numel() * ws.element_size(), _stream()))
    return accept_len, next_token, argmax_out


def token_bitmap(tokens, V: int, device="cuda") -> torch.Tensor:
    """Suppression bitmap for verify_accept_masked: ceil(V / 32) words, bit
    t % 32 of word t / 32 set for every token t listed (held as int32)."""
    ids = np.asarray(list(tokens), dtype=np.int64)
    if ids.size and (ids.min() < 0 or ids.max() >= V):
        raise ValueError("token ids must lie in [0, V)")
    bits = np.zeros((V + 31) // 32, dtype=np.uint32)
    np.bitwise_or.at(bits, ids >> 5, (np.uint32(1) << (ids & 31).astype(np.uint32)))
    return torch.from_numpy(bits.view(np.int32)).to(device)


def verify_accept_masked(logits: torch.Tensor, draft: torch.Tensor | None,
                         suppress: torch.Tensor | None = None,
                         suppress_first: torch.Tensor | None = None,
                         argmax_out: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                         accept_len: torch.Tensor | None = None,
                         next_token: torch.Tensor | None = None):
    """verify_accept after the logit filters: `suppress` (every row) and
    `suppress_first` (row 0 of each batch row) are token_bitmap() tensors or
    None; draft may be None or [B, 0] (then R = 1: a masked argmax). Returns
    (accept_len, next_token, argmax_out)."""
    if logits.dim() != 3:
        raise ValueError("logits must be [B, R, V]")
    if logits.dtype not in DTYPE_CODE:
        raise ValueError(f"unsupported logits dtype {logits.dtype}")
    B, R, V = logits.shape
    N = 0 if draft is None else draft.shape[1]
    if draft is not None and (draft.dim() != 2 or draft.shape[0] != B):
        raise ValueError("draft must be [B, N]")
    words = (V + 31) // 32
    for m, name in ((suppress, "suppress"), (suppress_first, "suppress_first")):
        if m is not None and m.numel() != words:
            raise ValueError(f"{name} must hold ceil(V / 32) = {words} words")
    dev = logits.device
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if next_token is None:
        next_token = torch.empty(B, dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(verify_workspace_bytes(B, R, V), dev)
    am = _dev(argmax_out, "argmax_out", torch.int32) if argmax_out is not None else None
    dr = _dev(draft, "draft", torch.int32) if N > 0 else None
    sp = _dev(suppress, "suppress", torch.int32) if suppress is not None else None
    sf = _dev(suppress_first, "suppress_first", torch.int32) if suppress_first is not None else None
    _check("verify_accept_masked", lib().verify_accept_masked(
        _dev(logits, "logits"), DTYPE_CODE[logits.dtype], B, R, V, dr, N, sp, sf, am,
        _dev(accept_len, "accept_len", torch.int32), _dev(next_token, "next_token", torch.int32),
        _dev(ws, "ws"), ws.numel() * ws.element_size(), _stream()))
    return accept_len, next_token, argmax_out


def beam_workspace_bytes(B: int, K: int, V: int) -> int:
    return int(lib().kvd_beam_workspace_bytes(B, K, V))


def beam_select(logits: torch.Tensor, sum_logprobs: torch.Tensor, eot: int,
                ws: torch.Tensor | None = None, out: dict | None = None) -> dict:
    """One beam-search update: logits [B, K, V], running scores sum_logprobs
    fp32 [B, K]. Returns a dict of device tensors: parent, token, score
    [B, K]; finished_count [B]; finished_parent, finished_score [B, K]."""
    if logits.dim() != 3 or tuple(sum_logprobs.shape) != tuple(logits.shape[:2]):
        raise ValueError("logits must be [B, K, V] and sum_logprobs [B, K]")
    if logits.dtype not in DTYPE_CODE:
        raise ValueError(f"unsupported logits dtype {logits.dtype}")
    B, K, V = logits.shape
    dev = logits.device
    if out is None:
        out = {"parent": torch.empty((B, K), dtype=torch.int32, device=dev),
               "token": torch.empty((B, K), dtype=torch.int32, device=dev),
               "score": torch.empty((B, K), dtype=torch.float32, device=dev),
               "finished_count": torch.empty(B, dtype=torch.int32, device=dev),
               "finished_parent": torch.empty((B, K), dtype=torch.int32, device=dev),
               "finished_score": torch.empty((B, K), dtype=torch.float32, device=dev)}
    if ws is None:
        ws = workspace(beam_workspace_bytes(B, K, V), dev)
    _check("beam_select", lib().beam_select(
        _dev(logits, "logits"), DTYPE_CODE[logits.dtype], B, K, V,
        _dev(sum_logprobs, "sum_logprobs", torch.float32), int(eot),
        _dev(out["parent"], "parent", torch.int32), _dev(out["token"], "token", torch.int32),
        _dev(out["score"], "score", torch.float32),
        _dev(out["finished_count"], "finished_count", torch.int32),
        _dev(out["finished_parent"], "finished_parent", torch.int32),
        _dev(out["finished_score"], "finished_score", torch.float32),
        _dev(ws, "ws"), ws.numel() * ws.element_size(), _stream()))
    return out

