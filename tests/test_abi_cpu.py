"""The C-ABI library loads and exports every symbol include/eagle3.h declares,
and argument validation returns the documented codes before anything is
launched (no GPU needed: these paths never reach a HIP call)."""
import ctypes
import os
import re
import shutil

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "eagle3.h")


@pytest.fixture(scope="module")
def blib():
    from eagle_draft_tree_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
            pytest.skip("library not built and no hipcc")
        from eagle_draft_tree_amd.build import build
        build()
    return binding


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(eagle3_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_five_calls():
    fns = declared_functions()
    for f in ("eagle3_fuse", "eagle3_draft_step", "eagle3_tree_expand", "eagle3_verify", "eagle3_ttt_forward"):
        assert f in fns


def test_library_exports_every_declared_symbol(blib):
    lib = ctypes.CDLL(blib.LIB_PATH)
    missing = [f for f in declared_functions() if not hasattr(lib, f)]
    assert not missing, missing


def test_strerror_and_version(blib):
    lib = blib.load()
    assert lib.eagle3_strerror(blib.ECAPACITY) == b"capacity exceeded"
    assert lib.eagle3_version().startswith(b"eagle3")


def test_tree_limits(blib):
    assert blib.tree_state_size(1, 10, 6) > 0
    with pytest.raises(blib.Eagle3Error) as e:
        blib.tree_state_size(1, 17, 2)          # k > 16
    assert e.value.code == blib.ECAPACITY
    with pytest.raises(blib.Eagle3Error) as e:
        blib.tree_state_size(1, 10, 8)          # (D-1)k = 70 > 64 slots
    assert e.value.code == blib.ECAPACITY


def test_dims_validation(blib):
    from workloads.configs import L8B_SHAPE, tiny_shape
    d = blib.dims_of(L8B_SHAPE)
    assert blib.workspace_size(d, 1, 10, 2048) > 0
    bad = blib.dims_of(tiny_shape(d=256, hq=4, hkv=4, hd=96, ffn=512, vocab=1024, dtype="bf16"))
    with pytest.raises(blib.Eagle3Error) as e:
        blib.workspace_size(bad, 1, 1, 16)      # head_dim 96
    assert e.value.code == blib.EUNSUPPORTED
    bad2 = blib.dims_of(tiny_shape(d=256, hq=6, hkv=4, hd=64, ffn=512, vocab=1024, dtype="bf16"))
    with pytest.raises(blib.Eagle3Error) as e:
        blib.workspace_size(bad2, 1, 1, 16)     # Hq not a multiple of Hkv
    assert e.value.code == blib.EINVAL


def test_call_validation_happens_before_launch(blib):
    lib = blib.load()
    # NULL dims, NULL weights, bad mode: all rejected on the host
    assert lib.eagle3_fuse(None, None, None, 1, None, None, 0, None) == blib.EINVAL
    assert lib.eagle3_verify(1, 70, 100, 6, None, None, None, 0, ctypes.c_float(1.0), None, None, None, None, None,
                             None, None, 0, None) == blib.ECAPACITY
    assert lib.eagle3_tree_expand(7, 1, 2, 3, 4, *([None] * 14), None) == blib.EINVAL
    assert lib.eagle3_topk(None, 1, 10, 2, None, None, None, None, 0, None) == blib.EINVAL
    assert b"NULL" in lib.eagle3_last_error() or lib.eagle3_last_error() != b""


def test_verify_workspace_layout(blib):
    """The verify workspace keeps its arrival counters from byte
    (ws_bytes / 6 * 5) & ~255 on: for every shape, a buffer of the queried
    size holds that call's partials (24 bytes per row and 4096-wide vocab
    slice) below the counter region and its counters inside it (one per
    verify row and one per request, 64 bytes apart), and so does any larger
    buffer."""
    for B in (1, 2, 3, 8, 64, 257, 1000):
        for m in (0, 3, 12, 59, 63):
            for V in (1, 100, 4096, 5000, 32000, 128256):
                S = blib.verify_workspace_size(B, m, V)
                n = B * (m + 1) * (-(-V // 4096))
                for size in (S, S + 1, S + 255, 3 * S + 7):
                    off = (size // 6 * 5) & ~255
                    assert 24 * n <= off and off + 64 * (B * (m + 1) + B) <= size, (B, m, V, size)
