"""CPU oracle for DeepSeek-V4 Heavily Compressed Attention (HCA).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__`` and the benchmark's ``cpu_baseline`` leg may import this
package.  The product library never imports, links or calls it, and this
package imports nothing from the product library: the two share no code.

The arithmetic lives in ``hca_oracle.c`` (plain C, fp64, OpenMP), which states
the definitions it follows and where on the pages they come from.  This module
only marshals numpy arrays into it.

Inputs are numpy arrays holding float32 or float64 values, or bfloat16 bit
patterns (``uint16``); the C side widens every element to double exactly.
Layouts: q, dout ``[B, H, S, D]``; kv ``[B, S, D]``; kvc ``[B, Sc, D]``;
seg ``[B, S]`` int32 per-token document id.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(library routines, closed forms, invariants, finite differences, hand-derived
visible sets) except the STRICT/LAST choice for a compressed window that
straddles a document boundary, which is a convention the pages leave open
(parity unpinned for that choice; both modes are tested for consistency).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hca_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libhca_oracle.so")

STRICT = 0
LAST = 1
MASK = 2  # compressed visibility from a given dense mask [B, S, Sc]
EMPTY, PARTIAL, FULL = 0, 1, 2


def build(force: bool = False) -> str:
    """Compiles the oracle with gcc (OpenMP, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
             "-o", tmp, _SRC, "-lm"]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("S", ctypes.c_int32), ("H", ctypes.c_int32),
        ("D", ctypes.c_int32), ("r", ctypes.c_int32), ("W", ctypes.c_int32),
        ("Sc", ctypes.c_int32), ("comp_mode", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32), ("pad_", ctypes.c_int32),
        ("scale", ctypes.c_double), ("seg", ctypes.c_void_p), ("comp_mask", ctypes.c_void_p),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        # HCA_ORACLE_LIB lets the mutation test load a deliberately broken copy.
        lib = ctypes.CDLL(os.environ.get("HCA_ORACLE_LIB") or build())
        P = ctypes.POINTER(_Problem)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        lib.hco_vis_raw.argtypes = [P, i32, i64, i64]
        lib.hco_vis_raw.restype = ctypes.c_int
        lib.hco_vis_comp.argtypes = [P, i32, i64, i64]
        lib.hco_vis_comp.restype = ctypes.c_int
        lib.hco_rows.argtypes = [P, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp]
        lib.hco_rows.restype = None
        lib.hco_keys.argtypes = [P, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp]
        lib.hco_keys.restype = None
        lib.hco_tile_state.argtypes = [P, i32, i32, i64, i64, i32, i32]
        lib.hco_tile_state.restype = ctypes.c_uint8
        lib.hco_tile_states.argtypes = [P, i32, i32, i32, vp]
        lib.hco_tile_states.restype = None
        lib.hco_tile_states_at.argtypes = [P, i32, i32, i32, i64, vp, vp]
        lib.hco_tile_states_at.restype = None
        lib.hco_count_pairs.argtypes = [P, i32]
        lib.hco_count_pairs.restype = i64
        lib.hco_num_threads.argtypes = []
        lib.hco_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Problem:
    """Parameters of one HCA problem plus the per-token document ids."""

    def __init__(self, B, S, H, D, r, W, Sc, scale, seg=None, comp_mode=STRICT,
                 in_dtype="f32", comp_mask=None):
        if seg is None:
            seg = np.zeros((B, S), dtype=np.int32)
        self.seg = np.ascontiguousarray(seg, dtype=np.int32)
        assert self.seg.shape == (B, S)
        self.comp_mask = None
        if comp_mode == MASK:
            self.comp_mask = np.ascontiguousarray(comp_mask, dtype=np.uint8)
            assert self.comp_mask.shape == (B, S, Sc)
        self.B, self.S, self.H, self.D = B, S, H, D
        self.r, self.W, self.Sc = r, W, Sc
        self.scale = float(scale)
        self.comp_mode = comp_mode
        self.in_dtype = in_dtype
        self._c = _Problem(B, S, H, D, r, W, Sc, comp_mode,
                           {"f32": 0, "bf16": 1, "f64": 2}[in_dtype], 0, self.scale,
                           self.seg.ctypes.data,
                           None if self.comp_mask is None else self.comp_mask.ctypes.data)

    def with_dtype(self, in_dtype):
        return Problem(self.B, self.S, self.H, self.D, self.r, self.W, self.Sc,
                       self.scale, self.seg, self.comp_mode, in_dtype, self.comp_mask)

    @property
    def c(self):
        return ctypes.byref(self._c)


def _check_input(prob, a, shape, name):
    if a is None:
        return None
    want = {"f32": np.float32, "bf16": np.uint16, "f64": np.float64}[prob.in_dtype]
    if a.dtype != want:
        raise TypeError(f"{name}: expected {want}, got {a.dtype}")
    if tuple(a.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {shape}, got {a.shape}")
    return np.ascontiguousarray(a)


def _inputs(prob, q, kv, kvc, dout):
    B, S, H, D, Sc = prob.B, prob.S, prob.H, prob.D, prob.Sc
    q = _check_input(prob, q, (B, H, S, D), "q")
    kv = _check_input(prob, kv, (B, S, D), "kv")
    kvc = _check_input(prob, kvc, (B, Sc, D), "kvc") if Sc > 0 else (
        np.zeros((B, 1, D), dtype=q.dtype))
    dout = _check_input(prob, dout, (B, H, S, D), "dout")
    return q, kv, kvc, dout


def vis_raw(prob, b, i, t):
    return bool(_load().hco_vis_raw(prob.c, b, i, t))


def vis_comp(prob, b, i, c):
    return bool(_load().hco_vis_comp(prob.c, b, i, c))


def rows(prob, q, kv, kvc, dout=None, row_index=None, need_grad=True):
    """Row pass.  row_index: flat indices (b*H + h)*S + i (default: all rows).

    Returns (o [n, D], lse [n], delta [n] or None, dq [n, D] or None), fp64.
    """
    lib = _load()
    q, kv, kvc, dout = _inputs(prob, q, kv, kvc, dout)
    if row_index is None:
        row_index = np.arange(prob.B * prob.H * prob.S, dtype=np.int64)
    row_index = np.ascontiguousarray(row_index, dtype=np.int64)
    n = row_index.size
    o = np.empty((n, prob.D), dtype=np.float64)
    lse = np.empty(n, dtype=np.float64)
    grad = need_grad and dout is not None
    delta = np.empty(n, dtype=np.float64) if grad else None
    dq = np.empty((n, prob.D), dtype=np.float64) if grad else None
    lib.hco_rows(prob.c, _ptr(q), _ptr(kv), _ptr(kvc), _ptr(dout) if grad else None,
                 n, _ptr(row_index), _ptr(o), _ptr(lse), _ptr(delta), _ptr(dq))
    return o, lse, delta, dq


def keys(prob, q, kv, kvc, dout, kinds, bs, idx, lse_all=None, delta_all=None):
    """Key pass: dKV rows for listed keys (kind 0 raw, 1 compressed), fp64 [n, D].

    lse_all / delta_all: [B, H, S] fp64 from a full row pass, or None to
    recompute every row that sees each key.
    """
    lib = _load()
    q, kv, kvc, dout = _inputs(prob, q, kv, kvc, dout)
    kinds = np.ascontiguousarray(kinds, dtype=np.int32)
    bs = np.ascontiguousarray(bs, dtype=np.int32)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    n = kinds.size
    if lse_all is not None:
        lse_all = np.ascontiguousarray(lse_all, dtype=np.float64).reshape(-1)
        delta_all = np.ascontiguousarray(delta_all, dtype=np.float64).reshape(-1)
        assert lse_all.size == prob.B * prob.H * prob.S
    out = np.empty((n, prob.D), dtype=np.float64)
    lib.hco_keys(prob.c, _ptr(q), _ptr(kv), _ptr(kvc), _ptr(dout), _ptr(lse_all),
                 _ptr(delta_all), n, _ptr(kinds), _ptr(bs), _ptr(idx), _ptr(out))
    return out


def full(prob, q, kv, kvc, dout):
    """Every output of the method, dense (small problems only).

    Returns dict o [B,H,S,D], lse [B,H,S], delta [B,H,S], dq [B,H,S,D],
    dkv [B,S,D], dkvc [B,Sc,D]; all fp64.
    """
    B, S, H, D, Sc = prob.B, prob.S, prob.H, prob.D, prob.Sc
    o, lse, delta, dq = rows(prob, q, kv, kvc, dout)
    kinds = np.concatenate([np.zeros(B * S, np.int32), np.ones(B * Sc, np.int32)])
    bs = np.concatenate([np.repeat(np.arange(B, dtype=np.int32), S),
                         np.repeat(np.arange(B, dtype=np.int32), Sc)])
    idx = np.concatenate([np.tile(np.arange(S, dtype=np.int32), B),
                          np.tile(np.arange(Sc, dtype=np.int32), B)])
    g = keys(prob, q, kv, kvc, dout, kinds, bs, idx, lse, delta)
    return dict(
        o=o.reshape(B, H, S, D), lse=lse.reshape(B, H, S),
        delta=delta.reshape(B, H, S), dq=dq.reshape(B, H, S, D),
        dkv=g[: B * S].reshape(B, S, D), dkvc=g[B * S:].reshape(B, Sc, D),
    )


def full_gqa(prob, kv_heads, q, kv, kvc, dout):
    """Every output with several key/value heads: query head h attends to
    key/value head h // (H // kv_heads).  Each key/value head with its group of
    query heads is an independent single-head (MQA) problem with the same
    documents, so this is the MQA oracle run once per group: prob.H is the total
    number of query heads; kv [B, G, S, D], kvc [B, G, Sc, D] (G = kv_heads).

    The pages dispatch the single-KV-head kernel only when there is one KV head
    ("Add HCA Static Compilation for Splash Attention [Deepseek v4]",
    Description); a layer with several key/value heads groups its query heads
    over them (grouped-query attention).  Returns the dict of full() with dkv
    [B, G, S, D] and dkvc [B, G, Sc, D].
    """
    G = kv_heads
    B, S, H, D, Sc = prob.B, prob.S, prob.H, prob.D, prob.Sc
    assert H % G == 0 and kv.shape == (B, G, S, D)
    Hg = H // G
    sub = Problem(B, S, Hg, D, prob.r, prob.W, Sc, prob.scale, prob.seg, prob.comp_mode,
                  prob.in_dtype, prob.comp_mask)
    out = {k: [] for k in ("o", "lse", "delta", "dq", "dkv", "dkvc")}
    for g in range(G):
        hs = slice(g * Hg, (g + 1) * Hg)
        kvc_g = kvc[:, g] if Sc > 0 else None
        r = full(sub, np.ascontiguousarray(q[:, hs]), np.ascontiguousarray(kv[:, g]),
                 None if kvc_g is None else np.ascontiguousarray(kvc_g),
                 np.ascontiguousarray(dout[:, hs]))
        for k in out:
            out[k].append(r[k])
    return dict(o=np.concatenate(out["o"], 1), lse=np.concatenate(out["lse"], 1),
                delta=np.concatenate(out["delta"], 1), dq=np.concatenate(out["dq"], 1),
                dkv=np.stack(out["dkv"], 1), dkvc=np.stack(out["dkvc"], 1))


def topk_mask(B, S, Sc, idx):
    """Dense compressed-key mask [B, S, Sc] uint8 of a per-query selection:
    idx [B, S, K] int, entry idx[b, i, k] selected for query i (negative =
    none; repeats select once)."""
    idx = np.asarray(idx)
    mask = np.zeros((B, S, Sc), np.uint8)
    b, i, _ = np.nonzero(idx >= 0)
    mask[b, i, idx[idx >= 0]] = 1
    return mask


def tile_states(prob, kind, bq, bk):
    """Brute-force tile table [B, ceil(S/bq), ceil(N/bk)] uint8 (0/1/2)."""
    lib = _load()
    nkeys = prob.S if kind == 0 else prob.Sc
    nqt = -(-prob.S // bq)
    nkt = -(-nkeys // bk)
    out = np.empty((prob.B, nqt, nkt), dtype=np.uint8)
    if out.size:
        lib.hco_tile_states(prob.c, kind, bq, bk, _ptr(out))
    return out


def tile_states_at(prob, kind, bq, bk, flat_tiles):
    lib = _load()
    flat_tiles = np.ascontiguousarray(flat_tiles, dtype=np.int64)
    out = np.empty(flat_tiles.size, dtype=np.uint8)
    lib.hco_tile_states_at(prob.c, kind, bq, bk, flat_tiles.size, _ptr(flat_tiles),
                           _ptr(out))
    return out


def count_pairs(prob, kind):
    return int(_load().hco_count_pairs(prob.c, kind))


def num_threads():
    return int(_load().hco_num_threads())
