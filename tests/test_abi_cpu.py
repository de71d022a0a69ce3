"""The C ABI on the host: the library loads, exports every declared symbol, and rejects
bad arguments before touching a device (no GPU needed)."""
import ctypes
import math
import os
import re

import pytest

from free_block_sparse_response_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparsepr.h")


@pytest.fixture(scope="module")
def lib():
    return L.load()


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(sparsepr_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.SYMBOLS)


def _cfg(**over):
    base = dict(batch=1, heads=2, seq_len=1000, head_dim=64, dtype="f32", n_sampled=32, n_key_groups=16,
                n_query_groups=12, n_probes=20, density=0.25)
    base.update(over)
    return L.make_config(**base)


def _create(lib, cfg):
    h = ctypes.c_void_p()
    st = lib.sparsepr_plan_create(ctypes.byref(cfg), ctypes.byref(h))
    return st, h


@pytest.mark.parametrize("over,want", [
    (dict(head_dim=96), L.SPARSEPR_ERR_UNSUPPORTED),
    (dict(dtype=7), L.SPARSEPR_ERR_UNSUPPORTED),
    (dict(n_sampled=0), L.SPARSEPR_ERR_INVALID_ARG),
    (dict(n_sampled=1001), L.SPARSEPR_ERR_INVALID_ARG),
    (dict(n_key_groups=0), L.SPARSEPR_ERR_INVALID_ARG),
    (dict(n_query_groups=1001), L.SPARSEPR_ERR_INVALID_ARG),
    (dict(seq_len=5000, n_key_groups=1025), L.SPARSEPR_ERR_UNSUPPORTED),
    (dict(n_probes=-1), L.SPARSEPR_ERR_INVALID_ARG),
    (dict(n_probes=1001), L.SPARSEPR_ERR_INVALID_ARG),
    (dict(density=0.0), L.SPARSEPR_ERR_INVALID_ARG),
    (dict(density=float("nan")), L.SPARSEPR_ERR_INVALID_ARG),
    (dict(ridge_lambda=-1.0), L.SPARSEPR_ERR_INVALID_ARG),
    (dict(kmeans_max_iter=0), L.SPARSEPR_ERR_INVALID_ARG),
    (dict(kmeans_tol=-1e-3), L.SPARSEPR_ERR_INVALID_ARG),
    (dict(seq_len=0), L.SPARSEPR_ERR_INVALID_ARG),
    (dict(batch=0), L.SPARSEPR_ERR_INVALID_ARG),
    (dict(assign_precision=2), L.SPARSEPR_ERR_INVALID_ARG),
    (dict(warm_iters=-1), L.SPARSEPR_ERR_INVALID_ARG),
    (dict(partition=3), L.SPARSEPR_ERR_INVALID_ARG),
    (dict(correction=-1), L.SPARSEPR_ERR_INVALID_ARG),
    (dict(probe_selector=3), L.SPARSEPR_ERR_INVALID_ARG),
    (dict(key_rank=-1), L.SPARSEPR_ERR_INVALID_ARG),
])
def test_plan_create_rejects(lib, over, want):
    st, h = _create(lib, _cfg(**over))
    assert st == want and not h.value


def test_plan_create_null_arguments(lib):
    h = ctypes.c_void_p()
    assert lib.sparsepr_plan_create(None, ctypes.byref(h)) == L.SPARSEPR_ERR_INVALID_ARG
    cfg = _cfg()
    assert lib.sparsepr_plan_create(ctypes.byref(cfg), None) == L.SPARSEPR_ERR_INVALID_ARG


def test_workspace_size_and_host_side_errors(lib):
    st, h = _create(lib, _cfg())
    assert st == L.SPARSEPR_OK and h.value
    try:
        ws = lib.sparsepr_workspace_bytes(h)
        assert ws > 0 and ws % 256 == 0
        fake = ctypes.c_void_p(0x100000)
        # missing, too small or misaligned workspace: rejected before any device work
        assert lib.sparsepr_plan(h, fake, fake, None, ws, None) == L.SPARSEPR_ERR_WORKSPACE
        assert lib.sparsepr_plan(h, fake, fake, fake, ws - 1, None) == L.SPARSEPR_ERR_WORKSPACE
        assert lib.sparsepr_plan(h, fake, fake, ctypes.c_void_p(0x100010), ws, None) == L.SPARSEPR_ERR_WORKSPACE
        assert lib.sparsepr_plan(h, None, fake, fake, ws, None) == L.SPARSEPR_ERR_INVALID_ARG
        # later stages before a plan; a warm start needs a previous plan in the same workspace
        assert lib.sparsepr_plan_warm(h, fake, fake, fake, ws, None) == L.SPARSEPR_ERR_STATE
        assert lib.sparsepr_plan_warm(h, None, fake, fake, ws, None) == L.SPARSEPR_ERR_INVALID_ARG
        assert lib.sparsepr_plan_set_probes(h, fake, None, fake, ws, None) == L.SPARSEPR_ERR_STATE
        assert lib.sparsepr_plan_set_probes(h, None, None, fake, ws, None) == L.SPARSEPR_ERR_INVALID_ARG
        assert lib.sparsepr_attend(h, fake, fake, fake, fake, fake, fake, None) == L.SPARSEPR_ERR_STATE
        assert lib.sparsepr_attend(h, fake, fake, fake, fake, fake, None, None) == L.SPARSEPR_ERR_INVALID_ARG
        assert lib.sparsepr_attend(h, fake, fake, fake, fake, None, fake, None) == L.SPARSEPR_ERR_INVALID_ARG
        assert lib.sparsepr_fit_residual(h, fake, fake, None, fake, None) == L.SPARSEPR_ERR_STATE
        assert lib.sparsepr_apply(h, fake, fake, fake, fake, None) == L.SPARSEPR_ERR_STATE
        assert lib.sparsepr_plan_export(h, 0, fake, 1 << 20, None) == L.SPARSEPR_ERR_STATE
        ms = (ctypes.c_float * 6)()
        assert lib.sparsepr_stage_times(h, ms, 6) == L.SPARSEPR_ERR_STATE
        assert lib.sparsepr_stage_times(h, ms, 7) == L.SPARSEPR_ERR_INVALID_ARG
        assert lib.sparsepr_set_stage_timing(None, 1) == L.SPARSEPR_ERR_INVALID_ARG
        info = (L.sparsepr_head_info * 2)()
        assert lib.sparsepr_plan_info(h, info, 2, None) == L.SPARSEPR_ERR_STATE
        assert lib.sparsepr_plan_info(h, info, 3, None) == L.SPARSEPR_ERR_INVALID_ARG
        # export sizes follow the documented shapes
        BH, N, S, Ck, Cq, M = 2, 1000, 32, 16, 12, 20
        want = {0: BH * S * 4, 1: BH * N * 4, 3: BH * N * 4, 5: BH * (Ck + 1) * 4, 6: BH * (Cq + 1) * 4,
                7: BH * (Cq + 1) * 4, 8: BH * Cq * Ck * 4, 9: BH * M * 4, 10: BH * M * 4, 11: BH * Cq * Ck * 8,
                12: BH * Ck * 64 * 4}
        for which, b in want.items():
            assert lib.sparsepr_export_bytes(h, which) == b
        assert lib.sparsepr_export_bytes(h, 99) == 0
    finally:
        lib.sparsepr_plan_destroy(h)


def test_workspace_grows_with_sequence(lib):
    sizes = []
    for n in (1000, 4000, 16000):
        st, h = _create(lib, _cfg(seq_len=n))
        sizes.append(lib.sparsepr_workspace_bytes(h))
        lib.sparsepr_plan_destroy(h)
    assert sizes[0] < sizes[1] < sizes[2]


def test_status_strings(lib):
    for s in range(7):
        assert lib.sparsepr_status_string(s)
    assert b"positive definite" in lib.sparsepr_status_string(L.SPARSEPR_ERR_NUMERICAL)


# ---------------------------------------------------------------- argument checks of the binding
def _t(shape, dtype=None, **kw):
    import torch

    return torch.zeros(shape, dtype=dtype or torch.bfloat16, **kw)


def test_binding_accepts_the_documented_layout():
    import torch

    from free_block_sparse_response_amd.call import check_tensor

    t = _t((1, 2, 8, 4))
    assert check_tensor(t, "q", [(1, 2, 8, 4)], torch.bfloat16, "cpu") is t
    lab = _t((2, 8), torch.int32)
    check_tensor(lab, "key_labels", [(2, 8), (1, 2, 8)], torch.int32, "cpu")


@pytest.mark.parametrize("case", ["device", "dtype", "shape", "transposed view", "not a tensor"])
def test_binding_refuses_what_the_kernels_would_misread(case):
    import torch

    from free_block_sparse_response_amd.call import check_tensor

    shape = [(1, 2, 8, 4)]
    if case == "device":           # a host tensor where a device pointer is expected
        t, dev = _t((1, 2, 8, 4)), "cuda"
    elif case == "dtype":          # float16 data for a bfloat16 configuration
        t, dev = _t((1, 2, 8, 4), torch.float16), "cpu"
    elif case == "shape":          # too few rows: the kernels would read past the allocation
        t, dev = _t((1, 2, 7, 4)), "cpu"
    elif case == "transposed view":  # the [B, N, H, d] activations of a video transformer
        t, dev = _t((1, 8, 2, 4)).transpose(1, 2), "cpu"
    else:
        t, dev = [[0.0]], "cpu"
    with pytest.raises(ValueError):
        check_tensor(t, "q", shape, torch.bfloat16, dev)


@pytest.mark.parametrize("dtype_name", ["int64 labels", "float weights as float64", "int32 masses"])
def test_binding_refuses_wrong_integer_and_weight_types(dtype_name):
    import torch

    from free_block_sparse_response_amd.call import check_tensor

    if dtype_name == "int64 labels":
        t, want, shape = _t((2, 8), torch.int64), torch.int32, (2, 8)
    elif dtype_name == "float weights as float64":
        t, want, shape = _t((2, 5), torch.float64), torch.float32, (2, 5)
    else:
        t, want, shape = _t((2, 3, 3), torch.int32), torch.int64, (2, 3, 3)
    with pytest.raises(ValueError):
        check_tensor(t, "x", [shape], want, "cpu")


def test_output_rank_and_tile_rows_are_validated(lib):
    for over, want in ((dict(output_rank=-1), L.SPARSEPR_ERR_INVALID_ARG), (dict(attn_tile_rows=96), L.SPARSEPR_ERR_INVALID_ARG),
                       (dict(output_rank=8, attn_tile_rows=256), L.SPARSEPR_OK)):
        st, h = _create(lib, _cfg(**over))
        assert st == want
        if st == L.SPARSEPR_OK:
            lib.sparsepr_plan_destroy(h)
