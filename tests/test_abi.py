"""C ABI: exported symbols match include/hca.h, and every error path returns the
documented status before any HIP call (so these run on a CPU-only host)."""

import ctypes
import os
import re

import numpy as np
import pytest

import block_sparse_compressed_amd as hca

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hca.h")
lib = hca.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hca_\w+)\s*\(", text)))


def test_header_and_library_agree():
    names = declared_functions()
    assert names == sorted(hca.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_library_exports_via_nm():
    import subprocess

    out = subprocess.run(["nm", "-D", "--defined-only", hca.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (hca_\w+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def status_of(fn, *args):
    return fn(*args)


def build_raw(B=1, S=64, r=8, W=4, Sc=None, starts=None, counts=None, H=4, D=64,
              dtype=hca.HCA_BF16, mode=0, tiles=None):
    out = ctypes.c_void_p()
    st = np.asarray(starts, np.int32) if starts is not None else None
    ct = np.asarray(counts, np.int32) if counts is not None else None
    cfg = hca._TileCfg(*(tuple(tiles) + (0,) * (5 - len(tiles)))) if tiles is not None else None
    s = lib.hca_block_mask_build(B, S, r, W, (S // r if r > 0 else 0) if Sc is None else Sc,
                                 st.ctypes.data if st is not None else None,
                                 ct.ctypes.data if ct is not None else None, H, D, dtype, mode,
                                 ctypes.byref(cfg) if cfg is not None else None,
                                 ctypes.byref(out))
    return s, out


@pytest.mark.parametrize("kw", [
    dict(S=0), dict(B=0), dict(H=0), dict(D=0), dict(r=0), dict(W=-1), dict(Sc=7),
    dict(S=64, r=8, Sc=9), dict(starts=[0, 10], counts=None), dict(starts=None, counts=[1]),
    dict(starts=[1, 10], counts=[2]), dict(starts=[0, 10, 10], counts=[3]),
    dict(starts=[0, 30, 20], counts=[3]), dict(starts=[0, 64], counts=[2]),
    dict(starts=[0], counts=[0]), dict(dtype=7), dict(mode=5), dict(tiles=(-1, 0, 0)),
])
def test_build_rejects_invalid(kw):
    s, out = build_raw(**kw)
    assert s == hca.HCA_ERR_INVALID_ARG
    assert out.value is None
    assert lib.hca_last_error().decode()


def test_build_null_out():
    assert lib.hca_block_mask_build(1, 8, 2, 2, 4, None, None, 1, 64, 1, 0, None, None) == \
        hca.HCA_ERR_INVALID_ARG


def test_python_layer_raises_value_error():
    with pytest.raises(ValueError):
        hca.hca_block_mask_build(1, 64, 8, 4, 7, H=4, D=64)


FAKE = 0x100000  # an aligned address that is never dereferenced: checks fail first


def fwd_args(plan, **over):
    a = dict(q=FAKE, kv=FAKE, kvc=FAKE, scale=0.125, o=FAKE, lse=FAKE, ws=FAKE,
             ws_bytes=1 << 40)
    a.update(over)
    return (plan.handle, a["q"], a["kv"], a["kvc"], ctypes.c_float(a["scale"]), a["o"],
            a["lse"], a["ws"], ctypes.c_uint64(a["ws_bytes"]), None)


def bwd_args(plan, **over):
    a = dict(q=FAKE, kv=FAKE, kvc=FAKE, o=FAKE, lse=FAKE, dout=FAKE, scale=0.125, dq=FAKE,
             dkv=FAKE, dkvc=FAKE, ws=FAKE, ws_bytes=1 << 40)
    a.update(over)
    return (plan.handle, a["q"], a["kv"], a["kvc"], a["o"], a["lse"], a["dout"],
            ctypes.c_float(a["scale"]), a["dq"], a["dkv"], a["dkvc"], a["ws"],
            ctypes.c_uint64(a["ws_bytes"]), None)


@pytest.fixture
def plan():
    return hca.hca_block_mask_build(1, 64, 8, 4, 8, H=4, D=64, dtype=hca.HCA_BF16, tiles=(32, 32, 32))


def test_plan_is_kernel_ready(plan):
    assert hca.hca_plan_get_info(plan).kernel_ok == 1


@pytest.mark.parametrize("over,status", [
    (dict(q=None), hca.HCA_ERR_INVALID_ARG), (dict(kv=FAKE + 8), hca.HCA_ERR_INVALID_ARG),
    (dict(kvc=None), hca.HCA_ERR_INVALID_ARG), (dict(o=None), hca.HCA_ERR_INVALID_ARG),
    (dict(lse=FAKE + 4), hca.HCA_ERR_INVALID_ARG), (dict(scale=0.0), hca.HCA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), hca.HCA_ERR_INVALID_ARG),
    (dict(), hca.HCA_ERR_STATE),
])
def test_fwd_error_paths(plan, over, status):
    assert lib.hca_attn_fwd(*fwd_args(plan, **over)) == status
    assert lib.hca_last_error().decode()


def test_fwd_workspace_size_checked():
    """The head dim 512 forward needs its tile-image workspace; a head dim 64
    forward needs none (it stages the row-major K itself)."""
    p512 = hca.hca_block_mask_build(1, 64, 8, 4, 8, H=4, D=512, dtype=hca.HCA_BF16,
                                    tiles=(32, 32, 32))
    assert hca.hca_plan_get_info(p512).ws_fwd_bytes > 16
    assert lib.hca_attn_fwd(*fwd_args(p512, ws_bytes=16)) == hca.HCA_ERR_WORKSPACE
    assert "workspace" in lib.hca_last_error().decode()
    assert lib.hca_attn_fwd(*fwd_args(p512, ws=None)) == hca.HCA_ERR_INVALID_ARG
    p64 = hca.hca_block_mask_build(1, 64, 8, 4, 8, H=4, D=64, dtype=hca.HCA_BF16,
                                   tiles=(32, 32, 32))
    assert hca.hca_plan_get_info(p64).ws_fwd_bytes == 0
    # no workspace needed: any size and a NULL pointer pass (next: not uploaded)
    assert lib.hca_attn_fwd(*fwd_args(p64, ws_bytes=0)) == hca.HCA_ERR_STATE
    assert lib.hca_attn_fwd(*fwd_args(p64, ws=None)) == hca.HCA_ERR_STATE


@pytest.mark.parametrize("over,status", [
    (dict(dout=None), hca.HCA_ERR_INVALID_ARG), (dict(dq=FAKE + 2), hca.HCA_ERR_INVALID_ARG),
    (dict(dkv=None), hca.HCA_ERR_INVALID_ARG), (dict(dkvc=None), hca.HCA_ERR_INVALID_ARG),
    (dict(o=None), hca.HCA_ERR_INVALID_ARG), (dict(scale=-1.0), hca.HCA_ERR_INVALID_ARG),
    (dict(ws_bytes=100), hca.HCA_ERR_WORKSPACE), (dict(), hca.HCA_ERR_STATE),
])
def test_bwd_error_paths(plan, over, status):
    assert lib.hca_attn_bwd(*bwd_args(plan, **over)) == status


def test_null_plan():
    assert lib.hca_attn_fwd(None, FAKE, FAKE, FAKE, ctypes.c_float(1.0), FAKE, FAKE, FAKE,
                            ctypes.c_uint64(1 << 40), None) == hca.HCA_ERR_INVALID_ARG
    assert lib.hca_plan_get_info(None, None) == hca.HCA_ERR_INVALID_ARG
    lib.hca_plan_destroy(None)


def test_compressed_pointers_optional_without_entries():
    plan = hca.hca_block_mask_build(1, 64, 100, 4, 0, H=4, D=64, dtype=hca.HCA_BF16,
                                    tiles=(32, 32, 32))
    # kv_comp = NULL is fine when S_c = 0: the call proceeds to the upload check
    assert lib.hca_attn_fwd(*fwd_args(plan, kvc=None)) == hca.HCA_ERR_STATE
    assert lib.hca_attn_bwd(*bwd_args(plan, kvc=None, dkvc=None)) == hca.HCA_ERR_STATE


@pytest.mark.parametrize("kw", [
    dict(dtype=hca.HCA_BF16, H=3, D=64),        # 128 rows per tile not reachable
    dict(dtype=hca.HCA_BF16, H=4, D=96),        # head dim without a kernel
    dict(dtype=hca.HCA_F32, H=4, D=96),
    dict(dtype=hca.HCA_BF16, H=4, D=64, tiles=(32, 16, 32)),
])
def test_unsupported_configurations(kw):
    plan = hca.hca_block_mask_build(1, 64, 8, 4, 8, **kw)
    assert hca.hca_plan_get_info(plan).kernel_ok == 0
    assert lib.hca_attn_fwd(*fwd_args(plan)) == hca.HCA_ERR_UNSUPPORTED
    assert lib.hca_attn_bwd(*bwd_args(plan)) == hca.HCA_ERR_UNSUPPORTED


@pytest.mark.parametrize("S,H,ok", [(1048544, 8, 1), (1048545, 8, 0), (2097184, 1, 0)])
def test_sizes_past_32bit_image_offsets_unsupported(S, H, ok):
    """Head dim 512 kernels address the tile images with 32-bit offsets: a plan
    whose padded keys x 2048 bytes reach 2^31 is marked unsupported and both
    passes return HCA_ERR_UNSUPPORTED (with the reason) instead of computing
    on wrapped offsets."""
    plan = hca.hca_block_mask_build(1, S, 128, 128, S // 128, H=H, D=512, dtype=hca.HCA_BF16)
    assert hca.hca_plan_get_info(plan).kernel_ok == ok
    if not ok:
        assert lib.hca_attn_fwd(*fwd_args(plan)) == hca.HCA_ERR_UNSUPPORTED
        assert "32-bit" in lib.hca_last_error().decode()
        assert lib.hca_attn_bwd(*bwd_args(plan)) == hca.HCA_ERR_UNSUPPORTED


def test_negative_comp_item_chunks_rejected():
    s, out = build_raw(tiles=(0, 0, 0, 0, -1))
    assert s == hca.HCA_ERR_INVALID_ARG and out.value is None


def test_fwd_noalloc_error_paths(plan):
    """The allocation-free forward checks its arguments like hca_attn_fwd, and
    refuses a plan whose forward workspace exceeds the library's scratch, all
    before any HIP call."""
    f = lib.hca_attn_fwd_noalloc
    args = lambda **o: fwd_args(plan, **o)[:7] + (None,)
    assert f(*args()) == hca.HCA_ERR_STATE
    assert f(*args(q=None)) == hca.HCA_ERR_INVALID_ARG
    assert f(*args(lse=FAKE + 4)) == hca.HCA_ERR_INVALID_ARG
    assert f(*args(scale=0.0)) == hca.HCA_ERR_INVALID_ARG
    assert f(None, FAKE, FAKE, FAKE, ctypes.c_float(1.0), FAKE, FAKE, None) == \
        hca.HCA_ERR_INVALID_ARG
    # S = 40000 at D = 512: 80 MiB of tile images, past the 64 MiB scratch
    big = hca.hca_block_mask_build(1, 40000, 128, 128, 312, H=8, D=512, dtype=hca.HCA_BF16)
    assert hca.hca_plan_get_info(big).ws_fwd_bytes > hca.NOALLOC_SCRATCH_BYTES
    assert f(*(fwd_args(big)[:7] + (None,))) == hca.HCA_ERR_WORKSPACE
    assert "scratch" in lib.hca_last_error().decode()
    unsup = hca.hca_block_mask_build(1, 64, 8, 4, 8, H=3, D=64, dtype=hca.HCA_BF16)
    assert f(*(fwd_args(unsup)[:7] + (None,))) == hca.HCA_ERR_UNSUPPORTED


def test_gqa_build_checks_and_tables():
    """hca_block_mask_build_gqa: kv_heads must divide H; the plan's tables hold
    one MQA problem per (batch row, kv head) with the batch row's documents,
    identical to the single-head plan of the same documents; pair counts stay
    per batch row."""
    out = ctypes.c_void_p()
    for G, H in ((0, 8), (3, 8), (-1, 8)):
        assert lib.hca_block_mask_build_gqa(1, G, 64, 8, 4, 8, None, None, H, 64, hca.HCA_BF16, 0,
                                            None, ctypes.byref(out)) == hca.HCA_ERR_INVALID_ARG
    starts, counts = [0, 40, 0, 10, 70], [2, 3]
    one = hca.hca_block_mask_build(2, 100, 8, 20, 12, starts, counts, H=16, D=512)
    gqa = hca.hca_block_mask_build_gqa(2, 4, 100, 8, 20, 12, starts, counts, H=64, D=512)
    i1, ig = hca.hca_plan_get_info(one), hca.hca_plan_get_info(gqa)
    assert ig.kv_heads == 4 and i1.kv_heads == 1 and ig.kernel_ok == 1
    assert (ig.pairs_raw, ig.pairs_comp) == (i1.pairs_raw, i1.pairs_comp)
    assert ig.tiles_raw == 4 * i1.tiles_raw and ig.items == 4 * i1.items
    r1, c1 = hca.hca_plan_export_tiles(one)
    rg, cg = hca.hca_plan_export_tiles(gqa)
    np.testing.assert_array_equal(rg, np.repeat(r1, 4, axis=0))
    np.testing.assert_array_equal(cg, np.repeat(c1, 4, axis=0))
    np.testing.assert_array_equal(hca.hca_plan_export_rows(gqa),
                                  np.repeat(hca.hca_plan_export_rows(one), 4, axis=0))
    # kernel support follows the heads per kv head (D = 64: bq x H / G = 128)
    p = hca.hca_block_mask_build_gqa(1, 2, 64, 8, 4, 8, H=6, D=64)
    assert hca.hca_plan_get_info(p).kernel_ok == 0


def test_upload_checks(plan):
    info = hca.hca_plan_get_info(plan)
    assert lib.hca_plan_upload(plan.handle, None, info.device_bytes, None) == \
        hca.HCA_ERR_INVALID_ARG
    assert lib.hca_plan_upload(plan.handle, FAKE + 1, info.device_bytes, None) == \
        hca.HCA_ERR_INVALID_ARG
    assert lib.hca_plan_upload(plan.handle, FAKE, info.device_bytes - 1, None) == \
        hca.HCA_ERR_WORKSPACE
    assert lib.hca_plan_upload(None, FAKE, info.device_bytes, None) == hca.HCA_ERR_INVALID_ARG


def test_status_strings():
    for s in range(7):
        assert hca.hca_status_string(s).startswith("HCA_")


def test_binding_binds_to_torch_hip_runtime():
    """Importing the binding on its own loads torch first, so libhca.so binds to the
    HIP runtime torch ships instead of pulling in a second one."""
    import subprocess
    import sys

    code = ("import sys; import block_sparse_compressed_amd; "
            "print('torch' in sys.modules)")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         cwd=ROOT, check=True).stdout
    assert out.strip().splitlines()[-1] == "True"


def test_timing_read_checks_and_empty():
    """hca_timing_read: NULL count (or NULL output with a capacity) is an
    invalid argument; with nothing timed it reports zero kernel families, and
    enabling / disabling makes no HIP call."""
    n = ctypes.c_int32(-1)
    assert lib.hca_timing_read(None, 4, ctypes.byref(n)) == hca.HCA_ERR_INVALID_ARG
    assert lib.hca_timing_read(None, 0, None) == hca.HCA_ERR_INVALID_ARG
    assert lib.hca_timing_enable(1) == hca.HCA_OK
    assert lib.hca_timing_enable(0) == hca.HCA_OK
    assert lib.hca_timing_read(None, 0, ctypes.byref(n)) == hca.HCA_OK and n.value == 0
    assert hca.hca_timing_read() == {}
