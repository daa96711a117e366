"""CPU-side checks of the C ABI: the library loads, exports every function the header
declares, and rejects bad arguments before touching the device (so these run without a GPU)."""
import ctypes as C
import os
import re

import pytest
import torch

from top_chunk_sparse_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tcsparse.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.findall(r"^\s*(?:tcs_status|const char\s*\*|int)\s+\**\s*(\w+)\s*\(", src, flags=re.M)


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) >= {"sparse_attn_decode", "sparse_attn_prefill", "tcs_status_str",
                          "tcs_abi_version", "tcs_decode_workspace_size",
                          "tcs_prefill_workspace_size"}
    lib = ops.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(ops.EXPORTS)


def test_abi_version_and_status_strings():
    assert ops.lib().tcs_abi_version() == 9
    # the header's constant, which the build entry point checks the library against
    with open(os.path.join(os.path.dirname(__file__), "..", "include", "tcsparse.h")) as f:
        assert "#define TCS_ABI_VERSION 9\n" in f.read()
    for code in range(7):
        assert ops.status_str(code)
    assert ops.status_str(99) == "unknown status"


def P(**kw):
    base = dict(B=2, Hq=8, Hkv=2, d=128, N=1000, C_=64, g=4, k=4, num_pages=32)
    base.update(kw)
    return ops.decode_params(**base)


def test_selected_gists_need_fewer_partial_slots():
    # without gist slices the partial buffer shrinks; the scores, selection and chunk
    # attention parts are unchanged
    a = ops.decode_workspace_size(P(N=64 * 500))
    b = ops.decode_workspace_size(P(N=64 * 500, gist_mode=1))
    assert 0 < b < a


def test_selected_gists_two_levels_slots():
    # two levels with selected gists: no level-2 slices among the partial slots, one slot per
    # chosen group (its own level-2 gists) as with every gist
    kw = dict(N=64 * 500, levels=2, J=8, k2=4)
    a = ops.decode_workspace_size(P(**kw))
    b = ops.decode_workspace_size(P(gist_mode=1, **kw))
    assert 0 < b < a


def test_per_head_selection_workspace():
    # G candidate lists per slice and G * k union entries per unit
    a = ops.decode_workspace_size(P(N=64 * 500))
    b = ops.decode_workspace_size(P(N=64 * 500, select_mode=1))
    assert 0 < a < b
    assert ops.decode_workspace_size(P(select_mode=1, C_=16, g=1, N=16 * 65536 + 1)) > 0


def test_adaptive_k_keeps_the_caller_strides():
    # the budget only lowers the selected count: sel / sel_groups / gamma keep k and k2
    for kw in (dict(N=64 * 500, k=40, gate=1), dict(N=64 * 500, levels=2, J=8, k2=9, k=40)):
        a = ops.decode_workspace_size(P(**kw))
        b = ops.decode_workspace_size(P(k_mode=1, **kw))
        assert 0 < b <= a


def test_workspace_size_grows_with_work():
    a = ops.decode_workspace_size(P())
    b = ops.decode_workspace_size(P(k=16))
    c = ops.decode_workspace_size(P(B=4, num_pages=64))
    assert 0 < a < b and a < c
    assert a % 256 == 0


@pytest.mark.parametrize("kw,code", [
    (dict(Hq=6, Hkv=4), ops.TCS_ERR_SHAPE),
    (dict(d=96), ops.TCS_ERR_UNSUPPORTED),
    (dict(Hq=24, Hkv=2), ops.TCS_ERR_UNSUPPORTED),       # G = 12
    (dict(k=-1), ops.TCS_ERR_SHAPE),
    (dict(N=0), ops.TCS_ERR_SHAPE),
    (dict(C_=0), ops.TCS_ERR_SHAPE),
    (dict(g=0), ops.TCS_ERR_SHAPE),
    (dict(g=65), ops.TCS_ERR_UNSUPPORTED),
    (dict(max_chunks=10), ops.TCS_ERR_SHAPE),            # M = 16
    (dict(gist_cap=3), ops.TCS_ERR_SHAPE),
    (dict(levels=3), ops.TCS_ERR_SHAPE),
    (dict(levels=2, J=0), ops.TCS_ERR_SHAPE),
    (dict(levels=2, J=4, k2=2, gate=1), ops.TCS_ERR_UNSUPPORTED),
    (dict(levels=2, J=4, k2=65, N=64 * 4 * 70), ops.TCS_ERR_UNSUPPORTED),  # 69 groups
    (dict(levels=2, J=300, k2=1), ops.TCS_ERR_UNSUPPORTED),              # J*g > 1024
    (dict(gate=2), ops.TCS_ERR_SHAPE),
    (dict(scale=-1.0), ops.TCS_ERR_SHAPE),
    (dict(num_pages=0), ops.TCS_ERR_SHAPE),
    (dict(B=4097, Hkv=4, Hq=16), ops.TCS_ERR_UNSUPPORTED),   # 16388 units
    (dict(gist_mode=2), ops.TCS_ERR_SHAPE),
    (dict(top_p=-0.1), ops.TCS_ERR_SHAPE),
    (dict(top_p=1.5), ops.TCS_ERR_SHAPE),
    (dict(top_p=float("nan")), ops.TCS_ERR_SHAPE),
    (dict(top_p=0.5, levels=2, J=4, k2=2, k=257), ops.TCS_ERR_UNSUPPORTED),
    (dict(top_p=0.5, k=257), ops.TCS_ERR_UNSUPPORTED),
    (dict(gist_mode=1, C_=1024, g=8, N=5000), ops.TCS_ERR_UNSUPPORTED),  # C + g > 1024
    (dict(select_mode=1, gate=1), ops.TCS_ERR_UNSUPPORTED),       # per-head selection: no gate
    (dict(select_mode=1, top_p=0.5), ops.TCS_ERR_UNSUPPORTED),    # ... no top-p
    (dict(select_mode=1, levels=2, J=4, k2=2), ops.TCS_ERR_UNSUPPORTED),   # ... one level
    (dict(select_mode=1, C_=16, g=1, N=16 * 65537 + 1), ops.TCS_ERR_UNSUPPORTED),   # H > 65536
    (dict(select_mode=2), ops.TCS_ERR_SHAPE),
    (dict(k_mode=2), ops.TCS_ERR_SHAPE),
    (dict(k_mode=-1), ops.TCS_ERR_SHAPE),
    (dict(k_mode=1, top_p=0.5), ops.TCS_ERR_UNSUPPORTED),     # adaptive k: no top-p
])
def test_decode_rejects_bad_params(kw, code):
    p = P(**kw)
    n = C.c_size_t(0)
    assert ops.lib().tcs_decode_workspace_size(C.byref(p), C.byref(n)) == code
    st = ops.lib().sparse_attn_decode(C.byref(p), *([None] * 14), 0, None)
    assert st == code


def test_decode_struct_size_checked():
    p = P()
    p.struct_size = 12
    n = C.c_size_t(0)
    assert ops.lib().tcs_decode_workspace_size(C.byref(p), C.byref(n)) == ops.TCS_ERR_SHAPE


def test_decode_null_and_workspace_errors():
    p = P()
    need = ops.decode_workspace_size(p)
    fake = 0x100000  # never dereferenced: the checks fail first
    args = [fake] * 6 + [None, None, fake, None, None, None, None]
    lib = ops.lib()
    # q missing
    assert lib.sparse_attn_decode(C.byref(p), None, *args[1:], fake, need, None) == ops.TCS_ERR_NULL
    # workspace too small / misaligned / missing
    assert lib.sparse_attn_decode(C.byref(p), *args, fake, need - 1, None) == ops.TCS_ERR_WORKSPACE
    assert lib.sparse_attn_decode(C.byref(p), *args, fake + 4, need, None) == ops.TCS_ERR_WORKSPACE
    assert lib.sparse_attn_decode(C.byref(p), *args, None, need, None) == ops.TCS_ERR_WORKSPACE
    # gists required when there are historical chunks
    a2 = list(args)
    a2[4] = None
    assert lib.sparse_attn_decode(C.byref(p), *a2, fake, need, None) == ops.TCS_ERR_NULL
    # two levels need level-2 gists
    p2 = P(levels=2, J=4, k2=2)
    need2 = ops.decode_workspace_size(p2)
    assert lib.sparse_attn_decode(C.byref(p2), *args, fake, need2, None) == ops.TCS_ERR_NULL


def PP(**kw):
    base = dict(B=1, Hq=8, Hkv=2, d=128, T=1024, blk=64, k=4, gate=1)
    base.update(kw)
    return ops.prefill_params(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(T=1000), ops.TCS_ERR_SHAPE),
    (dict(blk=32), ops.TCS_ERR_UNSUPPORTED),
    (dict(d=64), ops.TCS_ERR_UNSUPPORTED),
    (dict(Hq=6, Hkv=4), ops.TCS_ERR_SHAPE),
    (dict(k=-2), ops.TCS_ERR_SHAPE),
    (dict(gate=5), ops.TCS_ERR_SHAPE),
])
def test_prefill_rejects_bad_params(kw, code):
    p = PP(**kw)
    n = C.c_size_t(0)
    assert ops.lib().tcs_prefill_workspace_size(C.byref(p), C.byref(n)) == code
    assert ops.lib().sparse_attn_prefill(C.byref(p), *([None] * 8), 0, None) == code


def test_prefill_null_and_workspace_errors():
    p = PP()
    need = ops.prefill_workspace_size(p)
    fake = 0x100000
    lib = ops.lib()
    assert lib.sparse_attn_prefill(C.byref(p), None, fake, fake, fake, fake, None, None,
                                   fake, need, None) == ops.TCS_ERR_NULL
    assert lib.sparse_attn_prefill(C.byref(p), fake, fake, fake, None, fake, None, None,
                                   fake, need, None) == ops.TCS_ERR_NULL     # S needed for k > 0
    assert lib.sparse_attn_prefill(C.byref(p), fake, fake, fake, fake, fake, None, None,
                                   fake, need - 8, None) == ops.TCS_ERR_WORKSPACE


@pytest.mark.parametrize("kw,code", [
    (dict(T=1000), ops.TCS_ERR_SHAPE),
    (dict(blk=32), ops.TCS_ERR_UNSUPPORTED),
    (dict(d=64), ops.TCS_ERR_UNSUPPORTED),
    (dict(k=-2), ops.TCS_ERR_SHAPE),
])
def test_prefill_backward_rejects_bad_params(kw, code):
    p = PP(**kw)
    n = C.c_size_t(0)
    assert ops.lib().tcs_prefill_backward_workspace_size(C.byref(p), C.byref(n)) == code
    assert ops.lib().sparse_attn_prefill_backward(C.byref(p), *([None] * 13), 0, None) == code


def test_prefill_backward_null_and_workspace_errors():
    p = PP()
    need = ops.prefill_backward_workspace_size(p)
    assert need > ops.prefill_workspace_size(p)
    fake = 0x100000   # never dereferenced: the checks fail first
    lib = ops.lib()
    full = [fake] * 7 + [None] + [fake] * 4   # q k v S out lse dout, dlse, dq dk dv dS
    assert lib.sparse_attn_prefill_backward(C.byref(p), *full, fake, need - 8,
                                            None) == ops.TCS_ERR_WORKSPACE
    for miss in (0, 1, 2, 3, 4, 5, 6, 8, 9, 10):   # every required pointer
        args = list(full)
        args[miss] = None
        assert lib.sparse_attn_prefill_backward(C.byref(p), *args, fake, need,
                                                None) == ops.TCS_ERR_NULL, miss


def GP(**kw):
    base = dict(B=1, Hq=8, Hkv=2, d=128, M=8, L=128, g=4)
    base.update(kw)
    return ops.gist_prefill_params(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(L=100), ops.TCS_ERR_UNSUPPORTED),      # L not a multiple of 64
    (dict(g=3), ops.TCS_ERR_UNSUPPORTED),        # 64 not a multiple of g
    (dict(g=128), ops.TCS_ERR_UNSUPPORTED),
    (dict(d=64), ops.TCS_ERR_UNSUPPORTED),
    (dict(g=0), ops.TCS_ERR_SHAPE),
    (dict(M=0), ops.TCS_ERR_SHAPE),
    (dict(Hq=6, Hkv=4), ops.TCS_ERR_SHAPE),
    (dict(scale=-1.0), ops.TCS_ERR_SHAPE),
])
def test_gist_prefill_rejects_bad_params(kw, code):
    p = GP(**kw)
    n = C.c_size_t(0)
    assert ops.lib().tcs_gist_prefill_workspace_size(C.byref(p), C.byref(n)) == code
    assert ops.lib().sparse_attn_gist_prefill(C.byref(p), *([None] * 6), 0, None) == code


def test_gist_prefill_null_and_workspace_errors():
    p = GP()
    need = ops.gist_prefill_workspace_size(p)
    assert need == 2 * 2 * 2 * 64 * 128   # gathered gist K and V: 2 heads x 64 rows, padded
    fake = 0x100000
    lib = ops.lib()
    for miss in (0, 1, 2, 3):
        args = [fake] * 4 + [None]
        args[miss] = None
        assert lib.sparse_attn_gist_prefill(C.byref(p), *args, fake, need,
                                            None) == ops.TCS_ERR_NULL
    assert lib.sparse_attn_gist_prefill(C.byref(p), *([fake] * 4), None, fake, need - 8,
                                        None) == ops.TCS_ERR_WORKSPACE


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(ops, "_lib", None)
    monkeypatch.setattr(ops, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="missing"):
        ops.lib()


def test_workspace_init_checks_alignment():
    lib = ops.lib()
    assert lib.tcs_workspace_init(None, 0, None) == ops.TCS_OK
    assert lib.tcs_workspace_init(None, 256, None) == ops.TCS_ERR_WORKSPACE
    assert lib.tcs_workspace_init(0x100004, 256, None) == ops.TCS_ERR_WORKSPACE


def test_stage_counts():
    assert ops.decode_stage_count(P()) == 2
    assert ops.decode_stage_count(P(levels=2, J=4, k2=2)) == 3
    assert ops.decode_stage_count(P(d=96)) == -1


def test_noalloc_rejects_beyond_its_scratch_before_device_work():
    # the shape check comes before any device call: placeholder (never dereferenced) pointers
    big = P(B=256, Hq=32, Hkv=8, N=131072, C_=128, g=4, k=16, num_pages=256 * 1024)
    assert ops.decode_workspace_size(big) > ops.NOALLOC_SCRATCH_BYTES
    fake = C.c_void_p(4096)
    st = ops.lib().sparse_attn_decode_noalloc(C.byref(big), *([fake] * 10), None, None, None, None)
    assert st == ops.TCS_ERR_TOO_LARGE
    assert "scratch" in ops.status_str(st)
    assert ops.lib().sparse_attn_decode_noalloc(C.byref(P()), *([None] * 14)) == ops.TCS_ERR_NULL
