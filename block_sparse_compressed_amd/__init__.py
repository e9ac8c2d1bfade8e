"""Python binding of libhca.so -- MI355X (gfx950) Heavily Compressed Attention.

Thin ctypes layer over the C ABI declared in ``include/hca.h``: the functions
below carry the same names and marshal arguments (torch tensors become device
pointers, the current torch stream becomes the HIP stream).  Every step of the
computation runs inside libhca.so; nothing here computes attention, and there
is no fallback: importing this package fails if the library is missing.

PyTorch is used for device memory and streams only.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhca.so")

HCA_OK, HCA_ERR_INVALID_ARG, HCA_ERR_UNSUPPORTED = 0, 1, 2
HCA_ERR_WORKSPACE, HCA_ERR_HIP, HCA_ERR_NOMEM, HCA_ERR_STATE = 3, 4, 5, 6
HCA_F32, HCA_BF16 = 0, 1
HCA_COMPSEG_STRICT, HCA_COMPSEG_LAST = 0, 1
HCA_TILE_EMPTY, HCA_TILE_PARTIAL, HCA_TILE_FULL = 0, 1, 2

# Declared in include/hca.h; the ABI test checks the header and this list agree.
EXPORTS = (
    "hca_block_mask_build", "hca_block_mask_build_gqa", "hca_block_mask_build_masked",
    "hca_block_mask_build_topk", "hca_plan_get_info",
    "hca_plan_export_tiles",
    "hca_plan_export_rows", "hca_plan_export_items", "hca_plan_upload", "hca_plan_destroy",
    "hca_attn_fwd", "hca_attn_fwd_noalloc",
    "hca_attn_bwd", "hca_timing_enable", "hca_timing_read", "hca_status_string",
    "hca_last_error",
)


class HcaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class HcaInvalidArgument(HcaError, ValueError):
    pass


class HcaUnsupported(HcaError, NotImplementedError):
    pass


class _TileCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "bq", "bk_raw", "bk_comp", "half_items_min", "comp_item_chunks", "kv_keys")]


class _PlanInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "B", "S", "H", "D", "r", "W", "S_c", "dtype", "comp_mode", "bq", "bk_raw", "bk_comp",
        "nqt", "nkt_raw", "nkt_comp", "kernel_ok")] + [(n, ctypes.c_int64) for n in (
        "tiles_raw", "tiles_comp", "full_raw", "full_comp", "pairs_raw", "pairs_comp")] + [
        (n, ctypes.c_uint64) for n in ("device_bytes", "ws_fwd_bytes", "ws_bwd_bytes")] + [
        (n, ctypes.c_int64) for n in ("items", "items_half", "part_blocks")] + [
        (n, ctypes.c_int32) for n in ("comp_item_chunks", "kv_heads", "comp_masked",
                                      "kv_keys")] + [("ws_pds_bytes", ctypes.c_uint64)]


class _KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64),
                ("total_ms", ctypes.c_double)]


def _load_library():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libhca.so is not built (%s); run block_sparse_compressed_amd/_build.py" % LIB_PATH)
    # One HIP runtime per process: PyTorch ships its own libamdhip64, and if
    # libhca.so were loaded first it would pull in the system copy as well; the
    # two runtimes then disagree about the device.  Importing torch first makes
    # libhca.so bind to the runtime torch has already loaded.
    import torch  # noqa: F401

    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64
    lib.hca_block_mask_build.argtypes = [i32, i32, i32, i32, i32, vp, vp, i32, i32, i32, i32,
                                         vp, ctypes.POINTER(vp)]
    lib.hca_block_mask_build.restype = ctypes.c_int
    lib.hca_block_mask_build_gqa.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, i32, i32,
                                             i32, i32, vp, ctypes.POINTER(vp)]
    lib.hca_block_mask_build_gqa.restype = ctypes.c_int
    lib.hca_block_mask_build_masked.argtypes = [i32, i32, i32, i32, vp, vp, i32, i32, i32, vp,
                                                vp, ctypes.POINTER(vp)]
    lib.hca_block_mask_build_masked.restype = ctypes.c_int
    lib.hca_block_mask_build_topk.argtypes = [i32, i32, i32, i32, vp, vp, i32, i32, i32, vp,
                                              i32, vp, ctypes.POINTER(vp)]
    lib.hca_block_mask_build_topk.restype = ctypes.c_int
    lib.hca_plan_get_info.argtypes = [vp, ctypes.POINTER(_PlanInfo)]
    lib.hca_plan_get_info.restype = ctypes.c_int
    lib.hca_plan_export_tiles.argtypes = [vp, vp, vp]
    lib.hca_plan_export_tiles.restype = ctypes.c_int
    lib.hca_plan_export_rows.argtypes = [vp, vp]
    lib.hca_plan_export_rows.restype = ctypes.c_int
    lib.hca_plan_export_items.argtypes = [vp, vp, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]
    lib.hca_plan_export_items.restype = ctypes.c_int
    lib.hca_plan_upload.argtypes = [vp, vp, u64, vp]
    lib.hca_plan_upload.restype = ctypes.c_int
    lib.hca_plan_destroy.argtypes = [vp]
    lib.hca_plan_destroy.restype = None
    lib.hca_attn_fwd.argtypes = [vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, u64, vp]
    lib.hca_attn_fwd.restype = ctypes.c_int
    lib.hca_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, ctypes.c_float, vp, vp, vp]
    lib.hca_attn_fwd_noalloc.restype = ctypes.c_int
    lib.hca_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp,
                                 u64, vp]
    lib.hca_attn_bwd.restype = ctypes.c_int
    lib.hca_timing_enable.argtypes = [i32]
    lib.hca_timing_enable.restype = ctypes.c_int
    lib.hca_timing_read.argtypes = [ctypes.POINTER(_KernelTime), i32, ctypes.POINTER(i32)]
    lib.hca_timing_read.restype = ctypes.c_int
    lib.hca_status_string.argtypes = [ctypes.c_int]
    lib.hca_status_string.restype = ctypes.c_char_p
    lib.hca_last_error.argtypes = []
    lib.hca_last_error.restype = ctypes.c_char_p
    return lib


_lib = _load_library()


def library():
    return _lib


def _check(status: int):
    if status == HCA_OK:
        return
    msg = "%s: %s" % (_lib.hca_status_string(status).decode(), _lib.hca_last_error().decode())
    if status == HCA_ERR_INVALID_ARG:
        raise HcaInvalidArgument(status, msg)
    if status == HCA_ERR_UNSUPPORTED:
        raise HcaUnsupported(status, msg)
    raise HcaError(status, msg)


def hca_status_string(status: int) -> str:
    return _lib.hca_status_string(status).decode()


def hca_last_error() -> str:
    return _lib.hca_last_error().decode()


@dataclass(frozen=True)
class PlanInfo:
    B: int; S: int; H: int; D: int; r: int; W: int; S_c: int
    dtype: int; comp_mode: int; bq: int; bk_raw: int; bk_comp: int
    nqt: int; nkt_raw: int; nkt_comp: int; kernel_ok: int
    tiles_raw: int; tiles_comp: int; full_raw: int; full_comp: int
    pairs_raw: int; pairs_comp: int
    device_bytes: int; ws_fwd_bytes: int; ws_bwd_bytes: int
    items: int; items_half: int; part_blocks: int; comp_item_chunks: int; kv_heads: int
    comp_masked: int; kv_keys: int; ws_pds_bytes: int


class Plan:
    """Owns an ``hca_plan*``; released when the object is collected."""

    def __init__(self, handle: int):
        self._h = ctypes.c_void_p(handle)
        # Held by the object so that a plan collected at interpreter exit, after
        # the module's globals are cleared, can still be released.
        self._destroy = _lib.hca_plan_destroy
        self.device_buffer = None  # keeps the uploaded torch buffer alive
        self.info_cache = None  # PlanInfo (a plan never changes after it is built)

    @property
    def handle(self):
        return self._h

    def __del__(self):
        h = getattr(self, "_h", None)
        destroy = getattr(self, "_destroy", None)
        if h is not None and h.value and destroy is not None:
            destroy(h)
            h.value = None


def _i32(a: Optional[Sequence[int]]):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _cfg(tiles):
    if tiles is None:
        return None
    return _TileCfg(*(tuple(tiles) + (0,) * (6 - len(tiles))))


def hca_block_mask_build(B, S, r, W, S_c, seg_starts=None, seg_counts=None, H=1, D=64,
                         dtype=HCA_BF16, mode=HCA_COMPSEG_STRICT, tiles=None) -> Plan:
    """tiles: None or (bq, bk_raw, bk_comp[, half_items_min[, comp_item_chunks[, kv_keys]]]),
    0 = library choice (see hca_tile_cfg in include/hca.h)."""
    starts, counts = _i32(seg_starts), _i32(seg_counts)
    cfg = _cfg(tiles)
    out = ctypes.c_void_p()
    _check(_lib.hca_block_mask_build(
        B, S, r, W, S_c,
        starts.ctypes.data if starts is not None else None,
        counts.ctypes.data if counts is not None else None,
        H, D, dtype, mode, ctypes.byref(cfg) if cfg is not None else None, ctypes.byref(out)))
    return Plan(out.value)


def hca_block_mask_build_gqa(B, kv_heads, S, r, W, S_c, seg_starts=None, seg_counts=None, H=1,
                             D=64, dtype=HCA_BF16, mode=HCA_COMPSEG_STRICT, tiles=None) -> Plan:
    """Plan with kv_heads key/value heads (query head h uses kv head h // (H // kv_heads))."""
    starts, counts = _i32(seg_starts), _i32(seg_counts)
    cfg = _cfg(tiles)
    out = ctypes.c_void_p()
    _check(_lib.hca_block_mask_build_gqa(
        B, kv_heads, S, r, W, S_c,
        starts.ctypes.data if starts is not None else None,
        counts.ctypes.data if counts is not None else None,
        H, D, dtype, mode, ctypes.byref(cfg) if cfg is not None else None, ctypes.byref(out)))
    return Plan(out.value)


def hca_block_mask_build_masked(B, S, W, S_c, comp_mask, seg_starts=None, seg_counts=None, H=1,
                                D=512, dtype=HCA_BF16, tiles=None) -> Plan:
    """Plan whose compressed-key visibility is the host mask comp_mask [B, S, S_c]
    (nonzero = visible); the raw window keeps its rule."""
    mask = np.ascontiguousarray(np.asarray(comp_mask) != 0, dtype=np.uint8)
    if mask.shape != (B, S, S_c):
        raise HcaInvalidArgument(HCA_ERR_INVALID_ARG, "comp_mask must be [B, S, S_c]")
    starts, counts = _i32(seg_starts), _i32(seg_counts)
    cfg = _cfg(tiles)
    out = ctypes.c_void_p()
    _check(_lib.hca_block_mask_build_masked(
        B, S, W, S_c, starts.ctypes.data if starts is not None else None,
        counts.ctypes.data if counts is not None else None, H, D, dtype, mask.ctypes.data,
        ctypes.byref(cfg) if cfg is not None else None, ctypes.byref(out)))
    return Plan(out.value)


def hca_block_mask_build_topk(B, S, W, S_c, idx, seg_starts=None, seg_counts=None, H=1, D=512,
                              dtype=HCA_BF16, tiles=None) -> Plan:
    """Plan for attention over the per-query compressed entries idx [B, S, K]
    (negative = none) plus the raw window."""
    ix = np.ascontiguousarray(np.asarray(idx), dtype=np.int32)
    if ix.ndim != 3 or ix.shape[:2] != (B, S):
        raise HcaInvalidArgument(HCA_ERR_INVALID_ARG, "idx must be [B, S, K]")
    starts, counts = _i32(seg_starts), _i32(seg_counts)
    cfg = _cfg(tiles)
    out = ctypes.c_void_p()
    _check(_lib.hca_block_mask_build_topk(
        B, S, W, S_c, starts.ctypes.data if starts is not None else None,
        counts.ctypes.data if counts is not None else None, H, D, dtype, ix.ctypes.data,
        ix.shape[2], ctypes.byref(cfg) if cfg is not None else None, ctypes.byref(out)))
    return Plan(out.value)


def hca_plan_get_info(plan: Plan) -> PlanInfo:
    if plan.info_cache is None:
        info = _PlanInfo()
        _check(_lib.hca_plan_get_info(plan.handle, ctypes.byref(info)))
        plan.info_cache = PlanInfo(**{n: getattr(info, n) for n, _ in _PlanInfo._fields_})
    return plan.info_cache


def hca_plan_export_tiles(plan: Plan):
    """Returns (raw [B * kv_heads, nqt, nkt_raw], comp [B * kv_heads, nqt, nkt_comp])
    uint8 tables."""
    i = hca_plan_get_info(plan)
    nb = i.B * i.kv_heads
    raw = np.empty((nb, i.nqt, i.nkt_raw), dtype=np.uint8)
    comp = np.empty((nb, i.nqt, i.nkt_comp), dtype=np.uint8)
    _check(_lib.hca_plan_export_tiles(plan.handle, raw.ctypes.data if raw.size else None,
                                      comp.ctypes.data if comp.size else None))
    return raw, comp


def hca_plan_export_rows(plan: Plan) -> np.ndarray:
    """Per-position intervals [B * kv_heads, S, 3] int32: raw_lo, comp_lo, comp_hi."""
    i = hca_plan_get_info(plan)
    rows = np.empty((i.B * i.kv_heads, i.S, 3), dtype=np.int32)
    _check(_lib.hca_plan_export_rows(plan.handle, rows.ctypes.data))
    return rows


def hca_plan_export_items(plan: Plan) -> np.ndarray:
    """Key-stationary work items [n, 8] int64: batch row, kind, first key, keys per
    item, first and last listed query tile, halves, partial-block offset."""
    n = ctypes.c_int64(0)
    _check(_lib.hca_plan_export_items(plan.handle, None, 0, ctypes.byref(n)))
    items = np.empty((n.value, 8), dtype=np.int64)
    _check(_lib.hca_plan_export_items(plan.handle, items.ctypes.data if items.size else None,
                                      n.value, ctypes.byref(n)))
    return items


def _stream(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def hca_plan_upload(plan: Plan, dev_buf, stream=None):
    """Uploads the plan's device image into ``dev_buf`` (a uint8 CUDA tensor)."""
    _check(_lib.hca_plan_upload(plan.handle, _ptr(dev_buf), _nbytes(dev_buf), _stream(stream)))
    plan.device_buffer = dev_buf


def _expect(t, name, shape, dtype):
    """Host-side check that a torch tensor matches the plan before its pointer is passed."""
    import torch

    if t is None:
        return
    # Fast path: the checks below, in one expression, for the common case.
    if (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == dtype and t.shape == shape
            and t.is_contiguous()):
        return
    if not isinstance(t, torch.Tensor):
        raise HcaInvalidArgument(HCA_ERR_INVALID_ARG, "%s must be a torch tensor" % name)
    if t.device.type != "cuda" or not t.is_contiguous():
        raise HcaInvalidArgument(HCA_ERR_INVALID_ARG, "%s must be a contiguous device tensor" % name)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise HcaInvalidArgument(
            HCA_ERR_INVALID_ARG, "%s: expected %s %s, got %s %s" % (name, tuple(shape), dtype,
                                                                   tuple(t.shape), t.dtype))


def _kv_shape(info, n):
    """Shape of kv / dkv (n = S) or kv_comp / dkv_comp (n = S_c)."""
    if info.kv_heads == 1:
        return (info.B, n, info.D)
    return (info.B, info.kv_heads, n, info.D)


def _elem_dtype(info):
    import torch

    return torch.bfloat16 if info.dtype == HCA_BF16 else torch.float32


def hca_attn_fwd(plan: Plan, q, kv, kv_comp, scale, o, lse, ws, stream=None):
    import torch

    i = hca_plan_get_info(plan)
    et = _elem_dtype(i)
    _expect(q, "q", (i.B, i.H, i.S, i.D), et)
    _expect(kv, "kv", _kv_shape(i, i.S), et)
    if i.S_c > 0:
        _expect(kv_comp, "kv_comp", _kv_shape(i, i.S_c), et)
    _expect(o, "o", (i.B, i.H, i.S, i.D), et)
    _expect(lse, "lse", (i.B, i.H, i.S), torch.float32)
    _check(_lib.hca_attn_fwd(plan.handle, _ptr(q), _ptr(kv), _ptr(kv_comp), float(scale),
                             _ptr(o), _ptr(lse), _ptr(ws), _nbytes(ws), _stream(stream)))


# Scratch the library holds per device for hca_attn_fwd_noalloc (include/hca.h).
NOALLOC_SCRATCH_BYTES = 64 << 20


def hca_attn_fwd_noalloc(plan: Plan, q, kv, kv_comp, scale, o, lse, stream=None):
    """Forward with the library's own scratch as workspace (no workspace argument,
    no device allocation in the call); plans with ws_fwd_bytes above
    NOALLOC_SCRATCH_BYTES are refused."""
    import torch

    i = hca_plan_get_info(plan)
    et = _elem_dtype(i)
    _expect(q, "q", (i.B, i.H, i.S, i.D), et)
    _expect(kv, "kv", _kv_shape(i, i.S), et)
    if i.S_c > 0:
        _expect(kv_comp, "kv_comp", _kv_shape(i, i.S_c), et)
    _expect(o, "o", (i.B, i.H, i.S, i.D), et)
    _expect(lse, "lse", (i.B, i.H, i.S), torch.float32)
    _check(_lib.hca_attn_fwd_noalloc(plan.handle, _ptr(q), _ptr(kv), _ptr(kv_comp), float(scale),
                                     _ptr(o), _ptr(lse), _stream(stream)))


def hca_attn_bwd(plan: Plan, q, kv, kv_comp, o, lse, dout, scale, dq, dkv, dkv_comp, ws,
                 stream=None):
    import torch

    i = hca_plan_get_info(plan)
    et = _elem_dtype(i)
    for t, n in ((q, "q"), (o, "o"), (dout, "dout"), (dq, "dq")):
        _expect(t, n, (i.B, i.H, i.S, i.D), et)
    for t, n in ((kv, "kv"), (dkv, "dkv")):
        _expect(t, n, _kv_shape(i, i.S), et)
    if i.S_c > 0:
        _expect(kv_comp, "kv_comp", _kv_shape(i, i.S_c), et)
        _expect(dkv_comp, "dkv_comp", _kv_shape(i, i.S_c), et)
    _expect(lse, "lse", (i.B, i.H, i.S), torch.float32)
    _check(_lib.hca_attn_bwd(plan.handle, _ptr(q), _ptr(kv), _ptr(kv_comp), _ptr(o), _ptr(lse),
                             _ptr(dout), float(scale), _ptr(dq), _ptr(dkv), _ptr(dkv_comp),
                             _ptr(ws), _nbytes(ws), _stream(stream)))


def hca_timing_enable(enable: bool = True):
    _check(_lib.hca_timing_enable(1 if enable else 0))


def hca_timing_read() -> dict:
    """{kernel name: (launches, total_ms)} since the last read (waits for the events)."""
    buf = (_KernelTime * 16)()
    n = ctypes.c_int32()
    _check(_lib.hca_timing_read(buf, 16, ctypes.byref(n)))
    return {buf[k].name.decode(): (int(buf[k].launches), float(buf[k].total_ms))
            for k in range(min(n.value, 16))}


class HcaAttention:
    """Convenience holder: one plan, its device image and workspaces (torch-allocated).

    All computation goes through hca_attn_fwd / hca_attn_bwd.
    """

    def __init__(self, B, S, H, D, r, W, dtype="bf16", seg_starts=None, seg_counts=None,
                 mode=HCA_COMPSEG_STRICT, tiles=None, device="cuda", kv_heads=1, plan=None):
        """plan: a plan built elsewhere (for instance hca_block_mask_build_masked);
        r is then unused and S_c comes from the plan."""
        import torch

        self.B, self.S, self.H, self.D, self.r, self.W = B, S, H, D, r, W
        self.S_c = S // r if plan is None else hca_plan_get_info(plan).S_c
        self.kv_heads = kv_heads
        self.dtype = HCA_BF16 if dtype == "bf16" else HCA_F32
        self.torch_dtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        if plan is not None:
            self.plan = plan
        elif kv_heads == 1:
            self.plan = hca_block_mask_build(B, S, r, W, self.S_c, seg_starts, seg_counts, H, D,
                                             self.dtype, mode, tiles)
        else:
            self.plan = hca_block_mask_build_gqa(B, kv_heads, S, r, W, self.S_c, seg_starts,
                                                 seg_counts, H, D, self.dtype, mode, tiles)
        self.info = hca_plan_get_info(self.plan)
        self.device = torch.device(device)
        buf = torch.empty(max(1, self.info.device_bytes), dtype=torch.uint8, device=self.device)
        hca_plan_upload(self.plan, buf)
        # One workspace serves both passes: the backward's layout starts with the
        # forward's (ws_bwd_bytes >= ws_fwd_bytes), and the calls run in turn on
        # one stream.
        self.ws = torch.empty(max(16, self.info.ws_bwd_bytes, self.info.ws_fwd_bytes),
                              dtype=torch.uint8, device=self.device)

    def new_outputs(self):
        import torch

        o = torch.empty((self.B, self.H, self.S, self.D), dtype=self.torch_dtype,
                        device=self.device)
        lse = torch.empty((self.B, self.H, self.S), dtype=torch.float32, device=self.device)
        return o, lse

    def new_grads(self):
        import torch

        dq = torch.empty((self.B, self.H, self.S, self.D), dtype=self.torch_dtype,
                         device=self.device)
        dkv = torch.empty(_kv_shape(self.info, self.S), dtype=self.torch_dtype,
                          device=self.device)
        dkvc = torch.empty(_kv_shape(self.info, self.S_c), dtype=self.torch_dtype,
                           device=self.device)
        return dq, dkv, dkvc

    def forward(self, q, kv, kv_comp, scale, o=None, lse=None, stream=None):
        if o is None:
            o, lse = self.new_outputs()
        hca_attn_fwd(self.plan, q, kv, kv_comp if self.S_c > 0 else None, scale, o, lse,
                     self.ws, stream)
        return o, lse

    def backward(self, q, kv, kv_comp, o, lse, dout, scale, grads=None, stream=None):
        dq, dkv, dkvc = grads if grads is not None else self.new_grads()
        hca_attn_bwd(self.plan, q, kv, kv_comp if self.S_c > 0 else None, o, lse, dout, scale,
                     dq, dkv, dkvc if self.S_c > 0 else None, self.ws, stream)
        return dq, dkv, dkvc
