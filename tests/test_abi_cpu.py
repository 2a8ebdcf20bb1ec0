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


# ---------------------------------------------------------------- documented error codes
# Dummy non-NULL device pointers: every call below fails validation on the
# host, before anything is launched or dereferenced.
_P = ctypes.c_void_p(0x10000)


def _fake_weights(blib, layout=0):
    return blib.Weights(*([0x10000] * 11), layout)


def _fake_kv(blib, paged=False):
    return blib.KV(0x10000, 0x10000, 0 if paged else 4096, 0x10000 if paged else None, 256 if paged else 0,
                   16 if paged else 0, 0x10000, 0x10000, 0x10000)


def test_workspace_too_small_is_eworkspace(blib):
    from workloads.configs import L8B_SHAPE
    lib = blib.load()
    d = blib.dims_of(L8B_SHAPE)
    w = _fake_weights(blib)
    kv = _fake_kv(blib)
    assert lib.eagle3_fuse(ctypes.byref(d), ctypes.byref(w), _P, 1, _P, _P, 1, None) == blib.EWORKSPACE
    need = blib.workspace_size(d, 1, 10, 4096 - 10)
    assert lib.eagle3_draft_step(ctypes.byref(d), ctypes.byref(w), ctypes.byref(kv), blib.TREE, 1, 10, None, _P, _P,
                                 _P, _P, 0, 10, blib.TOPK_ALL, _P, _P, _P, None, _P, need - 1,
                                 None) == blib.EWORKSPACE
    assert b"workspace" in lib.eagle3_last_error()
    vneed = blib.verify_workspace_size(1, 60, 128256)
    assert lib.eagle3_verify(1, 60, 128256, 6, _P, _P, _P, blib.GREEDY, ctypes.c_float(1.0), None, None, _P, _P, _P,
                             _P, _P, vneed - 1, None) == blib.EWORKSPACE
    assert lib.eagle3_topk(_P, 4, 128256, 10, _P, _P, None, _P, 16, None) == blib.EWORKSPACE
    tneed = blib.ttt_workspace_size(d, 1, 128, 2)
    assert lib.eagle3_ttt_forward(ctypes.byref(d), ctypes.byref(w), _P, _P, 1, 128, 2, None, _P, _P, _P, _P,
                                  tneed - 1, None) == blib.EWORKSPACE
    assert lib.eagle3_pack_weights(ctypes.byref(d), ctypes.byref(w), _P, 100, ctypes.byref(blib.Weights()),
                                   None) == blib.EWORKSPACE


@pytest.mark.parametrize("T", [0.0, -1.0, float("nan")])
def test_sampling_temperature_must_be_positive(blib, T):
    lib = blib.load()
    vneed = blib.verify_workspace_size(1, 8, 4096)
    assert lib.eagle3_verify(1, 8, 4096, 3, _P, _P, _P, blib.SAMPLE, ctypes.c_float(T), _P, _P, _P, _P, _P, _P, _P,
                             vneed, None) == blib.EINVAL
    assert b"temperature" in lib.eagle3_last_error()


def test_dtype_mismatches(blib):
    from workloads.configs import L8B_SHAPE, TINY_SHAPE
    lib = blib.load()
    sz = ctypes.c_size_t(0)
    bad = blib.dims_of(L8B_SHAPE)
    bad.dtype = 7                                            # no such dtype
    assert lib.eagle3_workspace_size(ctypes.byref(bad), 1, 1, 16, ctypes.byref(sz)) == blib.EINVAL
    f32 = blib.dims_of(TINY_SHAPE)
    packed = _fake_weights(blib, layout=blib.LAYOUT_PACKED)  # packed weights with an fp32 drafter
    assert lib.eagle3_fuse(ctypes.byref(f32), ctypes.byref(packed), _P, 1, _P, _P, 1 << 30, None) == blib.EINVAL
    w = _fake_weights(blib)
    kv = _fake_kv(blib, paged=True)                          # paged KV needs bf16
    assert lib.eagle3_draft_step(ctypes.byref(f32), ctypes.byref(w), ctypes.byref(kv), blib.COMMIT, 1, 1, _P, None,
                                 _P, _P, None, 0, 2, blib.TOPK_LAST, _P, _P, _P, None, _P, 1 << 30,
                                 None) == blib.EUNSUPPORTED
    assert lib.eagle3_ttt_forward(ctypes.byref(f32), ctypes.byref(w), _P, _P, 1, 64, 2, None, _P, _P, _P, _P,
                                  1 << 30, None) == blib.EUNSUPPORTED
    assert lib.eagle3_packed_weights_size(ctypes.byref(f32), ctypes.byref(sz)) == blib.EUNSUPPORTED


def test_model_width_above_row_kernel_limit(blib):
    """The row kernels hold a row as 1024 threads x 8 elements: d = 8224 (a
    multiple of 32 above 8192) is rejected by every call that takes dims."""
    from workloads.configs import tiny_shape
    lib = blib.load()
    d = blib.dims_of(tiny_shape(d=8224, hq=64, hkv=8, hd=128, ffn=28672, vocab=128256, dtype="bf16"))
    with pytest.raises(blib.Eagle3Error) as e:
        blib.workspace_size(d, 1, 10, 4096)
    assert e.value.code == blib.EUNSUPPORTED
    w = _fake_weights(blib)
    kv = _fake_kv(blib)
    assert lib.eagle3_draft_step(ctypes.byref(d), ctypes.byref(w), ctypes.byref(kv), blib.COMMIT, 1, 1, _P, None,
                                 _P, _P, None, 0, 10, blib.TOPK_LAST, _P, _P, _P, None, _P, 1 << 40,
                                 None) == blib.EUNSUPPORTED
    assert lib.eagle3_fuse(ctypes.byref(d), ctypes.byref(w), _P, 1, _P, _P, 1 << 40, None) == blib.EUNSUPPORTED
    d.d = 8192
    assert blib.workspace_size(d, 1, 10, 4096) > 0


def test_efficient_head_argument_checks(blib):
    """eagle3_draft_step_lowrank rejects bad low-rank heads on the host."""
    from workloads.configs import L8B_SHAPE, TINY_SHAPE
    lib = blib.load()
    d = blib.dims_of(L8B_SHAPE)
    w = _fake_weights(blib)
    kv = _fake_kv(blib)
    ws = 1 << 40

    def call(head, dims=d, rows=10, k=10, topk_rows=None):
        return lib.eagle3_draft_step_lowrank(
            ctypes.byref(dims), ctypes.byref(w), ctypes.byref(kv), blib.TREE, 1, rows, None, _P, _P, _P, _P, 0, k,
            blib.TOPK_ALL if topk_rows is None else topk_rows, _P, _P, _P, None,
            ctypes.byref(head) if head is not None else None, None, None, _P, ws, None)
    H = lambda rank=256, c=64, layout=0, a=0x10000: blib.LowrankHead(a, 0x10000, rank, c, layout)
    assert call(None) == blib.EINVAL                      # no head
    assert call(H(a=0)) == blib.EINVAL                    # NULL factor
    assert call(H(rank=96)) == blib.EUNSUPPORTED          # rank not a multiple of 64
    assert call(H(rank=8192)) == blib.EUNSUPPORTED        # rank above d
    assert call(H(c=8)) == blib.EINVAL                    # fewer candidates than k
    assert call(H(c=300)) == blib.EINVAL                  # more than 256 candidates
    assert call(H(layout=5)) == blib.EINVAL
    assert call(H(), rows=65) == blib.ECAPACITY           # more than 64 rows (draft-step limit)
    f32 = blib.dims_of(TINY_SHAPE)
    assert call(H(rank=64), dims=f32, k=2) == blib.EUNSUPPORTED  # fp32 drafter
    assert lib.eagle3_pack_matrix(_P, 100, 64, _P, 1 << 20, None) == blib.EINVAL
    assert lib.eagle3_pack_matrix(_P, 128, 64, _P, 100, None) == blib.EWORKSPACE


def _fake_target(blib, n_layers=2, feat=(1, 2, 2), layout=0):
    arr = (blib.TargetLayer * n_layers)()
    for i in range(n_layers):
        arr[i] = blib.TargetLayer(*([0x10000] * 6))
    t = blib.Target(n_layers, ctypes.cast(arr, ctypes.POINTER(blib.TargetLayer)), 0x10000, 0x10000, 0x10000, layout,
                    (ctypes.c_int32 * 3)(*feat))
    return t, arr


def test_target_forward_argument_checks(blib):
    """eagle3_target_forward / eagle3_kv_commit / the target packing calls
    reject bad arguments on the host with the documented codes."""
    from workloads.configs import L8B_SHAPE, TINY_SHAPE
    lib = blib.load()
    d = blib.dims_of(L8B_SHAPE)
    t, _arr = _fake_target(blib)
    kv = blib.kv_array([_fake_kv(blib), _fake_kv(blib)])
    ws = 1 << 40

    def fwd(target=t, kvs=kv, B=1, rows=61, begin=0, end=2, feats=_P, ws_bytes=ws, dims=d):
        return lib.eagle3_target_forward(ctypes.byref(dims), ctypes.byref(target) if target is not None else None,
                                         kvs, B, rows, _P, _P, _P, begin, end, _P, feats, _P, _P, ws_bytes, None)
    assert fwd(target=None) == blib.EINVAL
    assert fwd(rows=65) == blib.ECAPACITY                     # more than 64 verify rows
    assert fwd(begin=1, end=0) == blib.EINVAL                 # empty/negative range
    assert fwd(end=3) == blib.EINVAL                          # past the last layer
    t_bad, _a2 = _fake_target(blib, feat=(0, 1, 2))
    assert fwd(target=t_bad) == blib.EINVAL                   # feature layer 0 (layers count from 1)
    t_pk, _a3 = _fake_target(blib, layout=blib.LAYOUT_PACKED)
    assert fwd(target=t_pk, dims=blib.dims_of(TINY_SHAPE), rows=8) == blib.EINVAL   # packed fp32
    big = blib.kv_array([blib.KV(0x10000, 0x10000, 40000, None, 0, 0, 0x10000, 0x10000, 0x10000)] * 2)
    assert fwd(kvs=big) == blib.EUNSUPPORTED                   # capacity above the attention's limit
    no_slots = blib.kv_array([blib.KV(0x10000, 0x10000, 4096, None, 0, 0, 0x10000, None, None)] * 2)
    assert fwd(kvs=no_slots) == blib.EINVAL                    # tree slots are required
    need = blib.target_workspace_size(d, 1, 61, 4096)
    assert fwd(ws_bytes=need - 1) == blib.EWORKSPACE
    assert blib.target_workspace_size(d, 64, 4, 2048) > 0
    with pytest.raises(blib.Eagle3Error) as e:
        blib.target_workspace_size(d, 1, 65, 2048)
    assert e.value.code == blib.ECAPACITY
    # KV commit
    assert lib.eagle3_kv_commit(ctypes.byref(d), 2, kv, 1, 61, _P, _P, 6, _P, None, None, None,
                                None) == blib.EINVAL           # feats without feats_next
    assert lib.eagle3_kv_commit(ctypes.byref(d), 2, kv, 1, 65, _P, _P, 6, None, None, None, None,
                                None) == blib.ECAPACITY
    assert lib.eagle3_kv_commit(ctypes.byref(d), 2, kv, 1, 61, None, _P, 6, None, None, None, None,
                                None) == blib.EINVAL
    assert lib.eagle3_kv_commit(ctypes.byref(d), 2, big, 1, 61, _P, _P, 6, None, None, None, None,
                                None) == blib.EUNSUPPORTED
    # packing
    sz = ctypes.c_size_t(0)
    assert lib.eagle3_target_layer_packed_size(ctypes.byref(d), ctypes.byref(sz)) == 0
    assert sz.value == 2 * (6144 * 4096 + 4096 * 4096 + 2 * 14336 * 4096 + 4096 * 14336)
    layer = blib.TargetLayer(*([0x10000] * 6))
    assert lib.eagle3_pack_target_layer(ctypes.byref(d), ctypes.byref(layer), _P, sz.value - 1,
                                        ctypes.byref(blib.TargetLayer()), None) == blib.EWORKSPACE
    f32 = blib.dims_of(TINY_SHAPE)
    assert lib.eagle3_target_layer_packed_size(ctypes.byref(f32), ctypes.byref(sz)) == blib.EUNSUPPORTED


def test_harness_rules_native_equal_oracle(blib):
    """The library's EAGLE-4 Harness rules (host code) take the oracle's
    decisions on random cost tables and confidences."""
    import numpy as np

    from oracle import eagle3_oracle as O
    rng = np.random.default_rng(17)
    agree = {"cost": 0, "continue": 0, "verify": 0, "branch": 0}
    for trial in range(60):
        nb, nc, nt = int(rng.integers(1, 4)), int(rng.integers(1, 4)), int(rng.integers(2, 7))
        batch = np.sort(rng.choice(np.arange(1, 129), nb, replace=False))
        ctx = np.sort(rng.choice(np.arange(64, 8193), nc, replace=False))
        tok = np.sort(rng.choice(np.arange(1, 65), nt, replace=False))
        base = rng.uniform(0.05, 2.0, size=(nb, nc, 1))
        draft = (base + np.cumsum(rng.uniform(0.0, 0.3, size=(nb, nc, nt)), axis=2)).astype(np.float32)
        verify = (2 * base + np.cumsum(rng.uniform(0.0, 0.5, size=(nb, nc, nt)), axis=2)).astype(np.float32)
        if trial % 5 == 0:   # a flat stretch: zero extra time
            verify[..., -1] = verify[..., -2]
        t = blib.HarnessTable(batch, ctx, tok, draft, verify)
        td = t.as_dict()
        B = int(rng.integers(1, 9))
        c = int(rng.integers(1, 9000))
        for kind in (0, 1):
            n = float(rng.uniform(0, 70))
            assert blib.harness_cost(t, kind, B, c, n) == pytest.approx(O.harness_cost(td, kind, B, c, np.float32(n)),
                                                                          rel=1e-12, abs=1e-12)
            agree["cost"] += 1
        k = int(rng.integers(1, 9))
        front = np.log(rng.uniform(1e-4, 1.0, size=(B, k))).astype(np.float32)
        tau0, alpha, depth = float(rng.uniform(0, 3)), float(rng.uniform(0, 1)), int(rng.integers(1, 6))
        want, _ = O.harness_continue(td, B, c, k, depth, front, tau0, alpha)
        assert blib.harness_continue(t, B, c, k, depth, front, tau0, alpha) == want
        agree["continue"] += 1
        m_max = int(rng.integers(1, 40))
        lc = -np.sort(-np.log(rng.uniform(1e-4, 1.0, size=(B, m_max))), axis=1).astype(np.float32)
        tau = float(rng.uniform(0, 5))
        assert blib.harness_verify_count(t, B, c, lc, tau) == O.harness_verify_count(td, B, c, lc, tau)
        agree["verify"] += 1
        lp = np.sort(np.log(rng.dirichlet(np.ones(8) * 0.5, size=B)), axis=1)[:, ::-1].astype(np.float32)
        tau = float(rng.uniform(0, 2))
        assert blib.harness_branch_cap(t, B, c, lp, tau) == O.harness_branch_cap(td, B, c, lp, tau)
        agree["branch"] += 1
    assert all(v >= 60 for v in agree.values())


def test_harness_argument_checks(blib):
    import numpy as np
    lib = blib.load()
    t = blib.HarnessTable([1, 8], [512], [1, 4], np.ones((2, 1, 2)), np.ones((2, 1, 2)))
    ms = ctypes.c_double(0)
    assert lib.eagle3_harness_cost(ctypes.byref(t.struct), 2, 1, 1, ctypes.c_float(1.0), ctypes.byref(ms)) == blib.EINVAL
    bad = blib.HarnessTable([8, 1], [512], [1, 4], np.ones((2, 1, 2)), np.ones((2, 1, 2)))   # not ascending
    assert lib.eagle3_harness_cost(ctypes.byref(bad.struct), 0, 1, 1, ctypes.c_float(1.0), ctypes.byref(ms)) == blib.EINVAL
    assert lib.eagle3_harness_cost(None, 0, 1, 1, ctypes.c_float(1.0), ctypes.byref(ms)) == blib.EINVAL
    go = ctypes.c_int(0)
    assert lib.eagle3_harness_continue(ctypes.byref(t.struct), 0, 1, 4, 1, _P, ctypes.c_double(1.0),
                                       ctypes.c_double(0.0), ctypes.byref(go)) == blib.EINVAL
    assert lib.eagle3_tree_confidence(1, 17, 2, 4, _P, _P, None, None) == blib.ECAPACITY
    assert lib.eagle3_tree_confidence(1, 4, 2, 4, None, _P, None, None) == blib.EINVAL


def test_ttt_train_argument_checks(blib):
    """eagle3_ttt_train validates before launching: workspace size, gradient
    pointers, the head-group and vocabulary restrictions, the dtype."""
    from workloads.configs import L8B_SHAPE, TINY_SHAPE, tiny_shape
    lib = blib.load()
    d = blib.dims_of(L8B_SHAPE)
    w = _fake_weights(blib)
    g = blib.Grads(*([0x1000] * len(blib.GRAD_NAMES)))
    need = blib.ttt_train_workspace_size(d, 8, 2048, 5)
    # the 8B shape at 8 x 2048 x 5 keeps ~45 GB of activations
    assert 30e9 < need < 60e9
    assert need > blib.ttt_workspace_size(d, 8, 2048, 5)

    def call(dims, grads, ws_bytes, S=128, R=2):
        return lib.eagle3_ttt_train(ctypes.byref(dims), ctypes.byref(w), _P, _P, 1, S, R, None, _P, _P, _P,
                                    ctypes.byref(grads), _P, ws_bytes, None)
    small = blib.ttt_train_workspace_size(d, 1, 128, 2)
    assert call(d, g, small - 1) == blib.EWORKSPACE
    nog = blib.Grads(*([0x1000] * (len(blib.GRAD_NAMES) - 1) + [0]))
    assert call(d, nog, small) == blib.EINVAL
    assert b"gradient" in lib.eagle3_last_error()
    assert call(d, g, small, S=96) == blib.EUNSUPPORTED                      # S % 64
    g3 = blib.dims_of(tiny_shape(d=384, hq=6, hkv=2, hd=64, ffn=512, vocab=2064, dtype="bf16"))
    assert call(g3, g, 1 << 40) == blib.EUNSUPPORTED                          # Hq/Hkv = 3
    assert b"Hq/Hkv" in lib.eagle3_last_error()
    v8 = blib.dims_of(tiny_shape(d=256, hq=4, hkv=2, hd=64, ffn=512, vocab=1048, dtype="bf16"))
    assert call(v8, g, 1 << 40) == blib.EUNSUPPORTED                          # vocab % 16
    f32 = blib.dims_of(TINY_SHAPE)
    assert call(f32, g, 1 << 40) == blib.EUNSUPPORTED                         # bf16 only
