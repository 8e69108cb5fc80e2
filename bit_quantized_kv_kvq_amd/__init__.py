"""Python binding of libkvq (quantized KV cache + fused dequant decode attention on MI355X).

Argument marshalling only: every step of the path runs in the HIP kernels of libkvq.so.
PyTorch provides device memory and the stream.  The functions below carry the C ABI's
names (include/kvq.h); `Cache` bundles the device buffer and the handle.
"""
from __future__ import annotations

import ctypes
import re
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkvq.so")

KVQ_OK, KVQ_EINVAL, KVQ_ECAPACITY, KVQ_ENOSPACE, KVQ_EHIP, KVQ_ESTATE = 0, -1, -2, -3, -4, -5
FMT = {"fp16": 0, "int2": 2, "int4": 4, "int8": 8, "nvfp4": 16, "fp8": 32, "mxfp4": 64}
GROUP_SIZE = {"int2": 64, "int4": 64, "int8": 64, "nvfp4": 16, "fp8": 0, "fp16": 0, "mxfp4": 32}
REGION_RESIDUAL, REGION_YOUNG, REGION_OLD = 0, 1, 2

# every symbol include/kvq.h declares
EXPORTS = ("kvq_cache_bytes", "kvq_cache_create", "kvq_cache_destroy", "kvq_cache_reset", "kvq_append",
           "kvq_append_seq", "kvq_flush_residual", "kvq_decode_workspace_bytes", "kvq_decode_attn",
           "kvq_append_decode_attn", "kvq_decode_attn_noalloc", "kvq_seq_len", "kvq_seq_info", "kvq_layout",
           "kvq_set_plan_only", "kvq_set_deterministic", "kvq_read_probe_sink_bytes", "kvq_read_probe",
           "kvq_last_error")


class KvqError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"kvq error {code}: {msg}")
        self.code = code


class kvq_config(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("max_tokens", ctypes.c_int64), ("format", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("residual_len", ctypes.c_int32), ("old_format", ctypes.c_int32),
                ("old_after", ctypes.c_int64), ("k_per_channel", ctypes.c_int32), ("demote_young", ctypes.c_int32)]


class kvq_seq_info_t(ctypes.Structure):
    _fields_ = [("length", ctypes.c_int64), ("residual", ctypes.c_int64), ("young_first_block", ctypes.c_int64),
                ("young_tokens", ctypes.c_int64), ("old_tokens", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libkvq.so; raises if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "or python bit_quantized_kv_kvq_amd/_build.py")
    # torch must load its HIP runtime first: libkvq then binds to that same instance
    # (libamdhip64.so.7), so device memory, streams and kernels share one runtime.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    P = ctypes.POINTER
    L.kvq_cache_bytes.argtypes = [P(kvq_config)]; L.kvq_cache_bytes.restype = sz
    L.kvq_cache_create.argtypes = [P(kvq_config), vp, sz, P(vp)]; L.kvq_cache_create.restype = ctypes.c_int
    L.kvq_cache_destroy.argtypes = [vp]; L.kvq_cache_destroy.restype = ctypes.c_int
    L.kvq_cache_reset.argtypes = [vp]; L.kvq_cache_reset.restype = ctypes.c_int
    L.kvq_append.argtypes = [vp, i32, vp, vp, i64, vp]; L.kvq_append.restype = ctypes.c_int
    L.kvq_append_seq.argtypes = [vp, i32, i32, vp, vp, i64, vp]; L.kvq_append_seq.restype = ctypes.c_int
    L.kvq_flush_residual.argtypes = [vp, i32, vp]; L.kvq_flush_residual.restype = ctypes.c_int
    L.kvq_decode_workspace_bytes.argtypes = [vp, i32]; L.kvq_decode_workspace_bytes.restype = sz
    L.kvq_decode_attn.argtypes = [vp, i32, vp, i32, ctypes.c_float, vp, i32, vp, sz, vp]
    L.kvq_decode_attn.restype = ctypes.c_int
    L.kvq_decode_attn_noalloc.argtypes = [vp, i32, vp, i32, ctypes.c_float, vp, i32, vp]
    L.kvq_decode_attn_noalloc.restype = ctypes.c_int
    L.kvq_append_decode_attn.argtypes = [vp, i32, vp, vp, i64, vp, i32, ctypes.c_float, vp, i32, vp, sz, vp]
    L.kvq_append_decode_attn.restype = ctypes.c_int
    L.kvq_seq_len.argtypes = [vp, i32, P(i64), P(i64)]; L.kvq_seq_len.restype = ctypes.c_int
    L.kvq_layout.argtypes = [vp, i32, i32, P(sz), P(sz), P(i64)]; L.kvq_layout.restype = ctypes.c_int
    L.kvq_seq_info.argtypes = [vp, i32, i32, P(kvq_seq_info_t)]; L.kvq_seq_info.restype = ctypes.c_int
    L.kvq_set_plan_only.argtypes = [vp, i32]; L.kvq_set_plan_only.restype = ctypes.c_int
    L.kvq_set_deterministic.argtypes = [vp, i32]; L.kvq_set_deterministic.restype = ctypes.c_int
    L.kvq_read_probe_sink_bytes.argtypes = []; L.kvq_read_probe_sink_bytes.restype = sz
    L.kvq_read_probe.argtypes = [vp, sz, vp, sz, vp]; L.kvq_read_probe.restype = ctypes.c_int
    L.kvq_last_error.argtypes = []; L.kvq_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(code: int):
    if code != KVQ_OK:
        raise KvqError(code, lib().kvq_last_error().decode())


def read_probe_sink_bytes() -> int:
    return lib().kvq_read_probe_sink_bytes()


def read_probe(buf, sink, stream=None):
    """kvq_read_probe: one kernel reading every byte of the uint8 device tensor `buf` once
    (measurement aid); `sink` (uint8 device tensor of read_probe_sink_bytes()) receives one
    uint32 per lane, the XOR of the words it read."""
    _check(lib().kvq_read_probe(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                                ctypes.c_void_p(sink.data_ptr()), sink.numel() * sink.element_size(),
                                ctypes.c_void_p(_stream_ptr(stream))))


def parse_format(name: str):
    """(format code, group size) of a format name: "int4" (groups of 64), "int4g32", "int2g128",
    "nvfp4", "mxfp4", "fp8", "fp16"."""
    m = re.fullmatch(r"(int[248])g(32|64|128)", name)
    if m:
        return FMT[m.group(1)], int(m.group(2))
    m = re.fullmatch(r"(int[248])kc", name)      # K per channel over 128-token windows, V in groups of 64
    if m:
        return FMT[m.group(1)], 64
    if name not in FMT:
        raise ValueError(f"unknown cache format {name!r}")
    return FMT[name], GROUP_SIZE[name]


def make_config(num_layers, batch, num_kv_heads, max_tokens, fmt="int4", residual_len=128,
                old_fmt=None, old_after=0, head_dim=128, demote=False) -> kvq_config:
    """An affine old tier shares the young tier's group size when the young format is affine
    (64 otherwise): old_fmt must name that group size.  demote: young blocks move to the old
    tier as they age (demote_young)."""
    code, gs = parse_format(fmt)
    old_code, old_gs = parse_format(old_fmt or fmt)
    if old_fmt and old_code in (2, 4, 8) and old_gs != (gs if code in (2, 4, 8) else 64):
        raise ValueError(f"old tier {old_fmt!r} must use the group size of the young tier ({fmt!r})")
    kc = fmt.endswith("kc")
    if old_fmt and old_code in (2, 4, 8) and old_fmt.endswith("kc") != kc:
        raise ValueError(f"old tier {old_fmt!r} must quantize K like the young tier ({fmt!r})")
    return kvq_config(num_layers, batch, num_kv_heads, head_dim, max_tokens, code, gs, residual_len,
                      old_code, old_after, int(kc), int(bool(demote)))


def kvq_cache_bytes(cfg: kvq_config) -> int:
    return lib().kvq_cache_bytes(ctypes.byref(cfg))


def _stream_ptr(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


class Cache:
    """A kvq cache over a torch uint8 device buffer.

    `plan_only=True` creates the handle without a GPU over a fake (never touched)
    address, for bookkeeping checks on machines without a device."""

    def __init__(self, cfg: kvq_config, device="cuda", plan_only=False):
        import torch
        self.cfg = cfg
        self.nbytes = kvq_cache_bytes(cfg)
        if self.nbytes == 0:
            raise KvqError(KVQ_EINVAL, lib().kvq_last_error().decode())
        self.plan_only = plan_only
        if plan_only:
            self.buf = None
            ptr = 1 << 40                     # 256-aligned placeholder, never dereferenced
        else:
            self.buf = torch.empty(self.nbytes + 256, dtype=torch.uint8, device=device)
            ptr = (self.buf.data_ptr() + 255) // 256 * 256
        self.base_ptr = ptr
        self.base_off = ptr - (self.buf.data_ptr() if self.buf is not None else ptr)
        h = ctypes.c_void_p()
        _check(lib().kvq_cache_create(ctypes.byref(cfg), ctypes.c_void_p(ptr), self.nbytes, ctypes.byref(h)))
        self.h = h
        if plan_only:
            _check(lib().kvq_set_plan_only(self.h, 1))

    def __del__(self):
        h = getattr(self, "h", None)
        if h is not None and _lib is not None:
            _lib.kvq_cache_destroy(h)
            self.h = None

    # -- calls
    def append(self, layer: int, k, v, stream=None):
        n = k.shape[2] if k is not None else 0
        kp = k.data_ptr() if k is not None else None
        vp_ = v.data_ptr() if v is not None else None
        s = None if self.plan_only else _stream_ptr(stream)
        _check(lib().kvq_append(self.h, layer, kp, vp_, n, s))

    def append_plan(self, layer: int, n: int):
        """Bookkeeping-only append of n tokens (plan-only caches)."""
        assert self.plan_only
        _check(lib().kvq_append(self.h, layer, 1 << 40, 1 << 40, n, None))

    def append_seq(self, layer: int, seq: int, k, v, stream=None):
        """kvq_append_seq: k, v fp16 [kv_heads, n, 128] appended to sequence seq alone."""
        n = k.shape[-2]
        if self.plan_only:
            _check(lib().kvq_append_seq(self.h, layer, seq, 1 << 40, 1 << 40, n, None))
            return
        assert k.is_contiguous() and v.is_contiguous()
        _check(lib().kvq_append_seq(self.h, layer, seq, k.data_ptr(), v.data_ptr(), n, _stream_ptr(stream)))

    def append_seq_plan(self, layer: int, seq: int, n: int):
        """Bookkeeping-only kvq_append_seq of n tokens (plan-only caches)."""
        assert self.plan_only
        _check(lib().kvq_append_seq(self.h, layer, seq, 1 << 40, 1 << 40, n, None))

    def flush(self, layer: int, stream=None):
        _check(lib().kvq_flush_residual(self.h, layer, None if self.plan_only else _stream_ptr(stream)))

    def reset(self):
        _check(lib().kvq_cache_reset(self.h))

    def set_deterministic(self, on: bool = True):
        """Decode with chunks assigned up front (bitwise reproducible output) instead of
        shared through the workspace cursor (the default)."""
        _check(lib().kvq_set_deterministic(self.h, 1 if on else 0))

    def workspace_bytes(self, num_q_heads: int) -> int:
        return lib().kvq_decode_workspace_bytes(self.h, num_q_heads)

    def decode(self, layer: int, q, softmax_scale: float, out, workspace, stream=None):
        import torch
        out_fp32 = 1 if out.dtype == torch.float32 else 0
        _check(lib().kvq_decode_attn(self.h, layer, q.data_ptr(), q.shape[1], float(softmax_scale), out.data_ptr(),
                                     out_fp32, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                     _stream_ptr(stream)))

    def decode_noalloc(self, layer: int, q, softmax_scale: float, out, stream=None):
        """kvq_decode_attn_noalloc: decode with the library's per-GPU scratch as workspace."""
        import torch
        out_fp32 = 1 if out.dtype == torch.float32 else 0
        _check(lib().kvq_decode_attn_noalloc(self.h, layer, q.data_ptr(), q.shape[1], float(softmax_scale),
                                             out.data_ptr(), out_fp32, _stream_ptr(stream)))

    def decode_noalloc_plan(self, layer: int, num_q_heads: int):
        """Host-side checks of kvq_decode_attn_noalloc (plan-only caches: nothing is launched)."""
        assert self.plan_only
        _check(lib().kvq_decode_attn_noalloc(self.h, layer, 1 << 40, num_q_heads, 0.125, 1 << 40, 1, None))

    def append_decode(self, layer: int, k, v, q, softmax_scale: float, out, workspace, stream=None):
        """kvq_append_decode_attn: append k, v (fp16 [B, H, n, 128]) then attend with q."""
        import torch
        out_fp32 = 1 if out.dtype == torch.float32 else 0
        for t in (k, v, q):
            assert t.is_contiguous() and t.dtype == torch.float16
        _check(lib().kvq_append_decode_attn(self.h, layer, k.data_ptr(), v.data_ptr(), k.shape[2], q.data_ptr(),
                                            q.shape[1], float(softmax_scale), out.data_ptr(), out_fp32,
                                            workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                            _stream_ptr(stream)))

    def seq_len(self, layer: int) -> tuple[int, int]:
        t, r = ctypes.c_int64(), ctypes.c_int64()
        _check(lib().kvq_seq_len(self.h, layer, ctypes.byref(t), ctypes.byref(r)))
        return t.value, r.value

    def layout(self, layer: int, region: int) -> tuple[int, int, int]:
        """(byte offset in the cache buffer, bytes, slots used per (batch, kv_head))."""
        off, nb, tok = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_int64()
        _check(lib().kvq_layout(self.h, layer, region, ctypes.byref(off), ctypes.byref(nb), ctypes.byref(tok)))
        return off.value, nb.value, tok.value

    def seq_info(self, layer: int, seq: int = 0) -> dict:
        """kvq_seq_info: one sequence's host counters."""
        i = kvq_seq_info_t()
        _check(lib().kvq_seq_info(self.h, layer, seq, ctypes.byref(i)))
        return {f: getattr(i, f) for f, _ in kvq_seq_info_t._fields_}

    def first_block(self, layer: int, region: int, seq: int = 0) -> int:
        """First live block of a region's arena for one sequence (the young tier's blocks before
        it were demoted)."""
        return self.seq_info(layer, seq)["young_first_block"] if region == REGION_YOUNG else 0

    def region_tensor(self, layer: int, region: int):
        """uint8 device view [batch, kv_heads, bytes per (b, h)] of a region."""
        off, nb, _ = self.layout(layer, region)
        B, H = self.cfg.batch, self.cfg.num_kv_heads
        t = self.buf[self.base_off + off:self.base_off + off + nb]
        return t.view(B, H, nb // (B * H)) if nb else t.view(B, H, 0)
