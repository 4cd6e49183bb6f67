"""The C ABI on the CPU: the library loads, exports what rkv.h declares, and
rejects every invalid argument before touching a GPU (no compute calls here)."""
import ctypes
import os
import re

import numpy as np
import pytest

from decode_kv_cache_03_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return _lib.load()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "rkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rkv_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert names == sorted(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def dense(**kw):
    base = dict(num_heads=4, n_cand=1152, head_dim=128, gqa_group=4, window=8, budget=1024,
                mix_lambda=0.1, dtype=_lib.RKV_BF16, kv_head_stride=0, out_head_stride=0)
    base.update(kw)
    return _lib.DenseDesc(**base)


def call_dense(lib, d, ws_bytes=1 << 30, K=FAKE, V=ctypes.c_void_p(0x20000000),
               Q=FAKE, kept=FAKE, Ko=ctypes.c_void_p(0x40000000), Vo=ctypes.c_void_p(0x60000000),
               ws=ctypes.c_void_p(0x100000)):
    return lib.rkv_compress(ctypes.byref(d), K, V, Q, kept, Ko, Vo, None, None, None, ws, ws_bytes,
                            None)


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 64, _lib.RKV_EINVAL),
    ("gqa_group", 0, _lib.RKV_EINVAL),
    ("window", 0, _lib.RKV_EINVAL),
    ("window", 33, _lib.RKV_EUNSUPPORTED),
    ("budget", 8, _lib.RKV_EINVAL),
    ("budget", 3, _lib.RKV_EINVAL),
    ("n_cand", 0, _lib.RKV_EINVAL),
    ("num_heads", -1, _lib.RKV_EINVAL),
    ("dtype", 7, _lib.RKV_EINVAL),
    ("mix_lambda", float("nan"), _lib.RKV_EINVAL),
    ("mix_lambda", float("inf"), _lib.RKV_EINVAL),
    ("gqa_group", 17, _lib.RKV_EUNSUPPORTED),
    ("kv_head_stride", 1000, _lib.RKV_EINVAL),
    ("out_head_stride", 1000, _lib.RKV_EINVAL),
    ("variant", 8, _lib.RKV_EINVAL),
    ("variant", 0x80000001, _lib.RKV_EINVAL),
    ("select_group", -1, _lib.RKV_EINVAL),
    ("select_group", 3, _lib.RKV_EINVAL),        # 4 units are not a multiple of 3
])
def test_dense_desc_errors(lib, field, value, code):
    d = dense(**{field: value})
    assert lib.rkv_workspace_size(ctypes.byref(d)) == 0
    assert call_dense(lib, d) == code
    assert _lib.last_error() != ""


def test_fp32_query_rows_limit(lib):
    d = dense(dtype=_lib.RKV_F32, gqa_group=16)
    assert call_dense(lib, d) == _lib.RKV_EUNSUPPORTED
    d = dense(dtype=_lib.RKV_F32, gqa_group=8)     # queries and fp32 tiles exceed the LDS
    assert call_dense(lib, d) == _lib.RKV_EUNSUPPORTED
    d = dense(dtype=_lib.RKV_F32, gqa_group=6)
    assert lib.rkv_workspace_size(ctypes.byref(d)) > 0
    d = dense(dtype=_lib.RKV_BF16, gqa_group=16)    # bf16 tiles leave room for 128 query rows
    assert lib.rkv_workspace_size(ctypes.byref(d)) > 0


def test_workspace_errors(lib):
    d = dense()
    need = lib.rkv_workspace_size(ctypes.byref(d))
    assert need > 0
    assert call_dense(lib, d, ws_bytes=need - 1) == _lib.RKV_EWORKSPACE
    assert call_dense(lib, d, ws=None) == _lib.RKV_EWORKSPACE
    assert call_dense(lib, d, ws=ctypes.c_void_p(0x100010)) == _lib.RKV_EWORKSPACE  # misaligned


def test_null_pointers(lib):
    d = dense()
    for kw in ("K", "V", "Q", "kept", "Ko", "Vo"):
        assert call_dense(lib, d, **{kw: None}) == _lib.RKV_EINVAL, kw


def test_aliasing_rejected(lib):
    d = dense()
    assert call_dense(lib, d, Ko=FAKE) == _lib.RKV_EINVAL          # K_out over K
    assert call_dense(lib, d, Vo=ctypes.c_void_p(0x40000000)) == _lib.RKV_EINVAL  # V_out over K_out


def test_zero_heads_needs_nothing(lib):
    d = dense(num_heads=0)
    assert lib.rkv_workspace_size(ctypes.byref(d)) > 0
    assert lib.rkv_compress(ctypes.byref(d), None, None, None, None, None, None, None, None, None,
                            None, 0, None) == _lib.RKV_OK


def test_variants_and_groups_accepted(lib):
    for v in range(8):
        assert lib.rkv_workspace_size(ctypes.byref(dense(variant=v))) > 0
    plain = lib.rkv_workspace_size(ctypes.byref(dense(select_group=1)))
    assert lib.rkv_workspace_size(ctypes.byref(dense(select_group=0))) == plain
    # head-shared selection adds the summed scores of each group
    assert lib.rkv_workspace_size(ctypes.byref(dense(select_group=2))) >= plain + 2 * 1152 * 4
    assert lib.rkv_workspace_size(ctypes.byref(dense(select_group=4))) > plain


def test_struct_layouts_match_header():
    """Field order and offsets of the ctypes views follow rkv.h (natural
    alignment: 8-byte members at multiples of 8)."""
    d = _lib.DenseDesc
    assert [f[0] for f in d._fields_] == ["num_heads", "n_cand", "head_dim", "gqa_group", "window",
                                          "budget", "mix_lambda", "dtype", "kv_head_stride",
                                          "out_head_stride", "variant", "select_group"]
    assert d.kv_head_stride.offset == 32 and d.variant.offset == 48 and ctypes.sizeof(d) == 56
    p = _lib.PagedDesc
    assert p.page_stride.offset == 40 and p.variant.offset == 64 and ctypes.sizeof(p) == 72
    text = open(os.path.join(ROOT, "include", "rkv.h")).read()
    for name in ("variant;", "select_group;"):
        assert name in text


def test_workspace_grows_with_units(lib):
    a = lib.rkv_workspace_size(ctypes.byref(dense(num_heads=8)))
    b = lib.rkv_workspace_size(ctypes.byref(dense(num_heads=16)))
    assert b > a > 0


# ---- paged -----------------------------------------------------------------------
def paged(**kw):
    base = dict(num_seqs=3, num_kv_heads=2, head_dim=128, gqa_group=2, window=8, page_size=16,
                max_pages_per_seq=8, num_pages=64, mix_lambda=0.1, dtype=_lib.RKV_BF16,
                page_stride=0, head_stride=0, slot_stride=0)
    base.update(kw)
    return _lib.PagedDesc(**base)


def arr(x):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int32))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def call_paged(lib, d, lens, buds, free_cap=100, free_count=0, ws_bytes=1 << 30, Kp=FAKE,
               Vp=ctypes.c_void_p(0x20000000)):
    _, lp = arr(lens)
    _, bp = arr(buds)
    cnt = ctypes.c_int32(free_count)
    rc = lib.rkv_compress_paged(ctypes.byref(d), Kp, Vp, FAKE, lp, bp, FAKE, FAKE, FAKE, free_cap,
                                ctypes.byref(cnt), None, ctypes.c_void_p(0x100000), ws_bytes, None)
    return rc, cnt.value


@pytest.mark.parametrize("lens,buds,code", [
    ([100, 50, 70], [64, 32, 48], _lib.RKV_OK),         # valid (only sized here)
    ([100, 50, 70], [60, 32, 48], _lib.RKV_EINVAL),     # budget not a page multiple
    ([100, 50, 70], [8, 32, 48], _lib.RKV_EINVAL),      # budget not above window
    ([0, 50, 70], [64, 32, 48], _lib.RKV_EINVAL),       # empty sequence
    ([200, 50, 70], [64, 32, 48], _lib.RKV_EINVAL),     # needs more than 8 pages
])
def test_paged_size_validation(lib, lens, buds, code):
    _, lp = arr(lens)
    _, bp = arr(buds)
    n = lib.rkv_paged_workspace_size(ctypes.byref(paged()), lp, bp)
    assert (n > 0) == (code == _lib.RKV_OK)
    if code != _lib.RKV_OK:
        assert call_paged(lib, paged(), lens, buds)[0] == code


def test_paged_free_list_overflow(lib):
    # pages freed: ceil(100/16)-4 = 3, ceil(50/16)-2 = 2, ceil(70/16)-3 = 2 -> 7
    lens, buds = [100, 50, 70], [64, 32, 48]
    rc, cnt = call_paged(lib, paged(), lens, buds, free_cap=10, free_count=4)
    assert rc == _lib.RKV_EFREELIST and cnt == 4
    rc, _ = call_paged(lib, paged(), lens, buds, free_cap=10, free_count=11)
    assert rc == _lib.RKV_EINVAL


@pytest.mark.parametrize("field,value", [("page_size", 12), ("page_size", 0), ("num_kv_heads", 0),
                                         ("head_dim", 96), ("window", 0), ("num_pages", 0),
                                         ("slot_stride", 64), ("variant", 16)])
def test_paged_desc_errors(lib, field, value):
    d = paged(**{field: value})
    rc, _ = call_paged(lib, d, [100, 50, 70], [64, 32, 48])
    assert rc in (_lib.RKV_EINVAL, _lib.RKV_EUNSUPPORTED)


def test_paged_shared_heads_accepted(lib):
    """RKV_VARIANT_SHARED_HEADS is a paged variant (alone or with the reading
    variants); its workspace adds the per-sequence sums of Z (one float per
    candidate of every sequence). The dense call refuses the bit and names
    its own way of sharing."""
    lens, buds = [100, 50, 70], [64, 32, 48]
    _, lp = arr(lens)
    _, bp = arr(buds)
    plain = lib.rkv_paged_workspace_size(ctypes.byref(paged()), lp, bp)
    for v in range(8):
        d = paged(variant=v | _lib.RKV_VARIANT_SHARED_HEADS)
        need = lib.rkv_paged_workspace_size(ctypes.byref(d), lp, bp)
        assert need >= plain + 4 * sum(lens), (v, need, plain)
    d = dense(variant=_lib.RKV_VARIANT_SHARED_HEADS)
    assert lib.rkv_workspace_size(ctypes.byref(d)) == 0
    assert b"select_group" in lib.rkv_last_error()


def test_paged_workspace_too_small(lib):
    lens, buds = [100, 50, 70], [64, 32, 48]
    _, lp = arr(lens)
    _, bp = arr(buds)
    need = lib.rkv_paged_workspace_size(ctypes.byref(paged()), lp, bp)
    rc, _ = call_paged(lib, paged(), lens, buds, ws_bytes=need - 1)
    assert rc == _lib.RKV_EWORKSPACE


def test_paged_same_pools_rejected(lib):
    rc, _ = call_paged(lib, paged(), [100, 50, 70], [64, 32, 48], Vp=FAKE)
    assert rc == _lib.RKV_EINVAL


def test_python_binding_refuses_cpu_tensors(lib):
    import torch
    import decode_kv_cache_03_amd as rkv
    K = torch.zeros((1, 100, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        rkv.compress(K, K, torch.zeros((1, 4, 8, 128), dtype=torch.bfloat16), 64)


def test_static_entry_point_rejects_before_any_gpu_call(lib):
    """rkv_compress_static validates like rkv_compress and refuses a call whose
    workspace would not fit its static scratch, all before touching a GPU."""
    far = [ctypes.c_void_p(k << 44) for k in range(1, 5)]   # disjoint even for 33 GB inputs

    def call(d, K=far[0]):
        return lib.rkv_compress_static(ctypes.byref(d), K, far[1], FAKE, FAKE, far[2], far[3],
                                       None, None, None, None)
    assert call(dense(head_dim=64)) == _lib.RKV_EINVAL
    assert call(dense(budget=8)) == _lib.RKV_EINVAL
    assert call(dense(), K=None) == _lib.RKV_EINVAL
    assert call(dense(num_heads=0)) == _lib.RKV_OK
    big = dense(num_heads=16384, n_cand=8000, budget=6000)
    assert lib.rkv_workspace_size(ctypes.byref(big)) > _lib.STATIC_SCRATCH_BYTES
    assert call(big) == _lib.RKV_EWORKSPACE
    assert b"static scratch" in lib.rkv_last_error()
