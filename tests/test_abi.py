"""C ABI of libhs2.so on the host: exported symbols, workspace sizing and argument
validation.  Nothing here launches a kernel on a GPU."""
import ctypes
import dataclasses
import os
import re

import pytest

hs2 = pytest.importorskip("kv_reuse_amd.hs2")

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "hs2.h")

FAKE = ctypes.c_void_p(0x10000)     # never dereferenced: every call below fails validation first


def declared_functions():
    src = open(HEADER, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hs2_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert len(names) == 13
    lib = hs2.raw()
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(hs2.EXPORTED) == names


def test_shape_struct_layout():
    assert ctypes.sizeof(hs2.Shape) == 64
    assert hs2.Shape.scale.offset == 8 and hs2.Shape.batch.offset == 16
    assert hs2.Shape.kv_capacity.offset == 48 and hs2.Shape.decode_splits.offset == 56


def good():
    return hs2.ShapeArgs(batch=2, n_q_tokens=1, n_q_heads=16, n_kv_heads=2, head_dim=128,
                         ctx_len=5000, top_k=64, window=16)


def test_workspace_bytes_valid_and_monotone():
    s = good()
    n0 = hs2.workspace_bytes(s, 0)
    n4 = hs2.workspace_bytes(s, 4)
    assert n0 > 0 and n4 >= n0
    big = hs2.ShapeArgs(batch=1, n_q_tokens=1, n_q_heads=32, n_kv_heads=4, head_dim=128,
                        ctx_len=1 << 20)
    # per key row: subtile maxima (2 B), candidate list (12 B) and the 32-bit key of
    # the scores path (4 B) dominate; the K/V cache itself is 512 B per key and head
    n = hs2.workspace_bytes(big, 8)
    assert 18 * 4 * (1 << 20) <= n < 64 * 4 * (1 << 20)
    # a cache allocated for a longer context does not change the workspace
    assert hs2.workspace_bytes(dataclasses.replace(big, kv_capacity=(1 << 20) + 4096), 8) == n


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 64, hs2.HS2_ERR_UNSUPPORTED),
    ("n_q_heads", 8, hs2.HS2_ERR_UNSUPPORTED),        # G = 4
    ("n_q_heads", 17, hs2.HS2_ERR_INVALID_ARG),       # not a multiple of Hkv
    ("top_k", 5000, hs2.HS2_ERR_UNSUPPORTED),         # k + w > 4096
    ("top_k", -1, hs2.HS2_ERR_INVALID_ARG),
    ("window", -3, hs2.HS2_ERR_INVALID_ARG),
    ("ctx_len", 0, hs2.HS2_ERR_INVALID_ARG),
    ("ctx_len", 1 << 31, hs2.HS2_ERR_UNSUPPORTED),
    ("n_q_tokens", 6000, hs2.HS2_ERR_INVALID_ARG),    # T > S
    ("batch", 0, hs2.HS2_ERR_INVALID_ARG),
    ("scale", -1.0, hs2.HS2_ERR_INVALID_ARG),
    ("scale", float("nan"), hs2.HS2_ERR_INVALID_ARG),
    ("select_block", 7, hs2.HS2_ERR_INVALID_ARG),       # not a power of two
    ("select_block", 8, hs2.HS2_ERR_INVALID_ARG),       # below 16
    ("select_block", 512, hs2.HS2_ERR_INVALID_ARG),     # above 256
    ("select_block", 128, hs2.HS2_ERR_INVALID_ARG),     # top_k = 64 is not a multiple
    ("kv_capacity", 4999, hs2.HS2_ERR_INVALID_ARG),   # smaller than ctx_len
    ("kv_capacity", -1, hs2.HS2_ERR_INVALID_ARG),
    ("kv_capacity", 1 << 40, hs2.HS2_ERR_UNSUPPORTED),
    ("decode_splits", -1, hs2.HS2_ERR_INVALID_ARG),
    ("decode_select", 3, hs2.HS2_ERR_INVALID_ARG),
    ("decode_select", -1, hs2.HS2_ERR_INVALID_ARG),
])
def test_bad_shapes_rejected(field, value, code):
    c = good().c()
    setattr(c, field, value)
    lib = hs2.raw()
    assert lib.hs2_workspace_bytes(ctypes.byref(c), 2) == 0
    st = lib.hs2_full_attn_scores(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 40, None)
    assert st == code
    st = lib.hs2_cross_decoder_step(ctypes.byref(c), 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    FAKE, None, None, FAKE, 1 << 40, None)
    assert st == code


def test_null_pointers_and_workspace_errors():
    lib = hs2.raw()
    c = good().c()
    need = lib.hs2_workspace_bytes(ctypes.byref(c), 3)
    E = hs2.HS2_ERR_INVALID_ARG
    assert lib.hs2_full_attn_scores(None, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, need, None) == E
    assert lib.hs2_full_attn_scores(ctypes.byref(c), None, FAKE, FAKE, FAKE, None, None, FAKE, need, None) == E
    assert lib.hs2_full_attn_scores(ctypes.byref(c), FAKE, FAKE, FAKE, None, None, None, FAKE, need, None) == E
    assert lib.hs2_topk_select(ctypes.byref(c), None, FAKE, FAKE, FAKE, need, None) == E
    assert lib.hs2_topk_select(ctypes.byref(c), FAKE, FAKE, None, FAKE, need, None) == E
    assert lib.hs2_sparse_attn(ctypes.byref(c), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == E
    assert lib.hs2_sparse_attn(ctypes.byref(c), 3, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, need, None) == E
    # sparse layers requested without their tensors
    assert lib.hs2_cross_decoder_step(ctypes.byref(c), 3, FAKE, None, FAKE, FAKE, FAKE, None, FAKE,
                                      FAKE, None, None, FAKE, need, None) == E
    # workspace: too small, missing, misaligned
    W = hs2.HS2_ERR_WORKSPACE
    assert lib.hs2_cross_decoder_step(ctypes.byref(c), 3, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      FAKE, None, None, FAKE, need - 1, None) == W
    assert lib.hs2_topk_select(ctypes.byref(c), FAKE, FAKE, FAKE, None, need, None) == E
    assert lib.hs2_topk_select(ctypes.byref(c), FAKE, FAKE, FAKE, ctypes.c_void_p(0x10010), need, None) == E
    # timed variant validates the same way
    ms = (ctypes.c_float * 4)()
    assert lib.hs2_cross_decoder_step_timed(ctypes.byref(c), 3, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                            FAKE, FAKE, FAKE, need, None, 0, ms) == E


@pytest.mark.parametrize("T", [1, 4])
def test_workspace_regions(T):
    """The introspection regions lie inside the workspace, 256-byte aligned,
    with the documented sizes; unknown regions and null pointers are rejected."""
    s = dataclasses.replace(good(), n_q_tokens=T)
    total = hs2.workspace_bytes(s, 2)
    rows = s.batch * T * s.n_kv_heads
    parts = 1 if rows >= 256 else -(-(s.top_k + s.window) // 128)   # sparse slices per row
    for region, size in ((hs2.HS2_WS_LSE2, rows * 8 * 8), (hs2.HS2_WS_REFINE, rows * 16),
                         (hs2.HS2_WS_INDEX_CHECK, rows * parts * 4)):
        off, nb = hs2.workspace_region(s, 2, region)
        assert nb == size and off % 256 == 0 and off + nb <= total
    lib = hs2.raw()
    o, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    c = s.c()
    assert lib.hs2_workspace_region(ctypes.byref(c), 2, 99, ctypes.byref(o), ctypes.byref(b)) == \
        hs2.HS2_ERR_INVALID_ARG
    assert lib.hs2_workspace_region(ctypes.byref(c), 2, hs2.HS2_WS_LSE2, None, ctypes.byref(b)) == \
        hs2.HS2_ERR_INVALID_ARG
    c.batch = 0
    assert lib.hs2_workspace_region(ctypes.byref(c), 2, hs2.HS2_WS_LSE2, ctypes.byref(o),
                                    ctypes.byref(b)) == hs2.HS2_ERR_INVALID_ARG


def test_decode_split_override_changes_the_plan():
    """A caller's split count changes the decode plan (and so the workspace of
    the per-split partial results); it is clamped to the context's 128-key
    splits; a prefill chunk ignores it."""
    base = hs2.ShapeArgs(batch=1, n_q_tokens=1, n_q_heads=8, n_kv_heads=1, head_dim=128,
                         ctx_len=100000, top_k=64, window=16)
    sizes = {n: hs2.workspace_bytes(dataclasses.replace(base, decode_splits=n), 0)
             for n in (1, 7, 300, 100000)}
    assert sizes[1] < sizes[7] < sizes[300] <= sizes[100000]
    assert sizes[100000] == hs2.workspace_bytes(dataclasses.replace(base, decode_splits=782), 0)
    chunk = dataclasses.replace(base, n_q_tokens=4)
    assert hs2.workspace_bytes(dataclasses.replace(chunk, decode_splits=3), 0) == \
        hs2.workspace_bytes(chunk, 0)


def test_block_selection_on_a_chunk_lists_a_band_entry_per_block():
    """Block selection in a prefill chunk ranks any band of blocks exactly: the
    per-row band list (a 32-bit index and a 64-bit key per entry) grows to one
    entry per block where that exceeds the token path's 8192."""
    tok = dataclasses.replace(good(), n_q_tokens=4, ctx_len=200000, top_k=1024, window=128)
    rows = tok.batch * 4 * tok.n_kv_heads
    extra = rows * (200000 // 16 - 8192) * 12
    d = hs2.workspace_bytes(dataclasses.replace(tok, select_block=16), 0) - \
        hs2.workspace_bytes(tok, 0)
    assert extra <= d < extra + 4096
    # blocks of 128: 1563 blocks, within the token path's list
    assert hs2.workspace_bytes(dataclasses.replace(tok, select_block=128), 0) == \
        hs2.workspace_bytes(tok, 0)


def test_status_strings():
    lib = hs2.raw()
    for code in (0, -1, -2, -3, -4):
        assert lib.hs2_status_string(code).decode() != "unknown status"
    assert lib.hs2_status_string(99).decode() == "unknown status"


def test_valid_call_without_gpu_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    lib = hs2.raw()
    c = good().c()
    need = lib.hs2_workspace_bytes(ctypes.byref(c), 0)
    st = lib.hs2_topk_select(ctypes.byref(c), FAKE, FAKE, FAKE, ctypes.c_void_p(0x100000), need, None)
    assert st == hs2.HS2_ERR_HIP
    assert lib.hs2_last_hip_error() != 0


def good_bridge():
    return hs2.BridgeShape(kv_capacity=1000, pos0=990, batch=2, n_tokens=10, d_model=512,
                           n_kv_heads=4, head_dim=128, reserved=0)


def test_bridge_shape_struct_layout():
    assert ctypes.sizeof(hs2.BridgeShape) == 40
    assert hs2.BridgeShape.batch.offset == 16 and hs2.BridgeShape.reserved.offset == 36


@pytest.mark.parametrize("field,value,code", [
    ("pos0", 991, hs2.HS2_ERR_INVALID_ARG),           # rows past the capacity
    ("pos0", -1, hs2.HS2_ERR_INVALID_ARG),
    ("n_tokens", 0, hs2.HS2_ERR_INVALID_ARG),
    ("batch", 0, hs2.HS2_ERR_INVALID_ARG),
    ("kv_capacity", 0, hs2.HS2_ERR_INVALID_ARG),
    ("reserved", 1, hs2.HS2_ERR_INVALID_ARG),
    ("d_model", 0, hs2.HS2_ERR_INVALID_ARG),
    ("d_model", 100, hs2.HS2_ERR_UNSUPPORTED),         # not a multiple of 64
    ("d_model", (1 << 20) + 64, hs2.HS2_ERR_UNSUPPORTED),  # beyond the supported hidden size
    ("head_dim", 64, hs2.HS2_ERR_UNSUPPORTED),
])
def test_bridge_bad_shapes_rejected(field, value, code):
    c = good_bridge()
    setattr(c, field, value)
    assert hs2.raw().hs2_kv_bridge(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, None) == code


def test_bridge_null_pointers_rejected():
    c = good_bridge()
    lib = hs2.raw()
    assert lib.hs2_kv_bridge(None, FAKE, FAKE, FAKE, FAKE, None) == hs2.HS2_ERR_INVALID_ARG
    for i in range(4):
        ptrs = [FAKE] * 4
        ptrs[i] = None
        assert lib.hs2_kv_bridge(ctypes.byref(c), *ptrs, None) == hs2.HS2_ERR_INVALID_ARG


def test_block_selection_limits():
    lib = hs2.raw()
    c = good().c()
    c.select_block = 32                      # top_k = 64: two blocks
    assert lib.hs2_workspace_bytes(ctypes.byref(c), 2) > 0
    c.ctx_len = 16384 * 32 + 1               # more than 16384 blocks
    assert lib.hs2_workspace_bytes(ctypes.byref(c), 2) == 0


def test_static_step_rejects_shapes_beyond_its_scratch():
    """A shape whose workspace exceeds the library-held buffer gets
    HS2_ERR_SCRATCH before anything touches a device; one that fits passes the
    size check (and then fails on a null pointer, still before any device call)."""
    lib = hs2.raw()
    big = hs2.ShapeArgs(batch=4, n_q_tokens=1, n_q_heads=32, n_kv_heads=4, head_dim=128,
                        ctx_len=1 << 20)
    assert hs2.workspace_bytes(big, 8) > hs2.HS2_STATIC_SCRATCH_BYTES
    args = [FAKE] * 8 + [None, None, None]
    st = lib.hs2_cross_decoder_step_static(ctypes.byref(big.c()), 8, *args)
    assert st == hs2.HS2_ERR_SCRATCH
    assert "static scratch" in lib.hs2_status_string(st).decode()
    small = hs2.ShapeArgs(batch=1, n_q_tokens=1, n_q_heads=8, n_kv_heads=1, head_dim=128,
                          ctx_len=4096)
    assert hs2.workspace_bytes(small, 1) <= hs2.HS2_STATIC_SCRATCH_BYTES
    st = lib.hs2_cross_decoder_step_static(ctypes.byref(small.c()), 1, FAKE, None, *([FAKE] * 6),
                                           None, None, None)
    assert st == hs2.HS2_ERR_INVALID_ARG     # q_sparse is NULL with one sparse layer
