"""The C ABI on a machine without a GPU: the library loads, exports every symbol
include/fx.h declares, and rejects invalid descriptions and policies on the host
before any HIP call."""
import ctypes
import os
import re

import pytest

import block_sparse_decode_summary_amd as fx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fx.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fx_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fx.library_path()):
        pytest.skip("libfx.so not built (run __graft_entry__.build())")
    return fx.load_library()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("fx_build_summaries", "fx_select", "fx_sparse_decode", "fx_selection_delta",
              "fx_plan_create", "fx_plan_destroy", "fx_workspace_bytes", "fx_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings(lib):
    for s in range(5):
        assert fx.fx_status_string(s).startswith("FX_")
    assert "unknown" in fx.fx_status_string(99)


class P:
    def __init__(self, **kw):
        self.mode, self.block, self.sub_block, self.top_k, self.budget = 0, 64, 16, 8, 0.0
        self.k_evict = self.sink_tokens = self.local_tokens = 0
        self.force_sink = self.force_last = 1
        self.__dict__.update(kw)


def _create(desc_kw=None, pol_kw=None, units=None):
    d = dict(batch=1, num_q_heads=4, num_kv_heads=2, head_dim=128, t_cap=1024, dtype=fx.FX_BF16,
             split_tokens=0, pooling=fx.FX_POOL_KEY)
    d.update(desc_kw or {})
    n = d["batch"] * d["num_kv_heads"] if units is None else units
    pols = [P(**(pol_kw or {})) for _ in range(n)]
    return fx.fx_plan_create(d["batch"], d["num_q_heads"], d["num_kv_heads"], d["head_dim"],
                             d["t_cap"], d["dtype"], pols, d["split_tokens"], d["pooling"])


@pytest.mark.parametrize("desc_kw", [
    dict(batch=0), dict(num_kv_heads=0), dict(num_q_heads=6, num_kv_heads=4),   # not a multiple
    dict(num_q_heads=18, num_kv_heads=2),                                      # G = 9
    dict(head_dim=96), dict(t_cap=0), dict(t_cap=(1 << 24) + 1), dict(dtype=7),
    dict(split_tokens=100), dict(split_tokens=32), dict(split_tokens=4096),
    dict(pooling=3), dict(pooling=-1),
])
def test_invalid_descriptions(lib, desc_kw):
    with pytest.raises(fx.FxError) as e:
        _create(desc_kw=desc_kw)
    assert e.value.status == 1


@pytest.mark.parametrize("pol_kw", [
    dict(mode=5), dict(block=48), dict(block=512), dict(block=0), dict(sub_block=128),
    dict(sub_block=3), dict(force_sink=2), dict(top_k=-1), dict(top_k=0, budget=0.0),
    dict(top_k=0, budget=1.5), dict(mode=fx.FX_STREAMING, sink_tokens=-1),
    dict(mode=fx.FX_NOSA, top_k=0, k_evict=0), dict(mode=fx.FX_NOSA, k_evict=-3),
])
def test_invalid_policies(lib, pol_kw):
    with pytest.raises(fx.FxError) as e:
        _create(pol_kw=pol_kw)
    assert e.value.status == 1


@pytest.mark.parametrize("pooling", [fx.FX_POOL_SCORE_SUM, fx.FX_POOL_SCORE_MAX])
def test_score_side_pooling_limits_rows_per_block(lib, pooling):
    """Score-side pooling keeps block / sub_block summary rows per block, at most 64."""
    with pytest.raises(fx.FxError) as e:
        _create(desc_kw=dict(pooling=pooling), pol_kw=dict(block=256, sub_block=2))
    assert e.value.status == 2


def test_null_arguments_rejected_on_host(lib):
    # NULL plan / NULL output pointer: FX_E_INVALID without touching a device.
    assert lib.fx_plan_create(None, None, None) == 1
    assert lib.fx_build_summaries(None, None, None, 0, 1, None, None) == 1
    assert lib.fx_select(None, None, None, None, None, None, None, None, None, 0, None) == 1
    assert lib.fx_sparse_decode(None, None, None, None, None, None, None, ctypes.c_float(1.0),
                                None, None, None, 0, None) == 1
    assert lib.fx_selection_delta(None, *([None] * 9)) == 1
    assert lib.fx_workspace_bytes(None) == 0 and lib.fx_max_selected(None) == -1
    assert lib.fx_plan_destroy(None) == 0
    assert lib.fx_unit_block_offset(None, 0) == -1
    assert lib.fx_unit_summary_offset(None, 0) == -1
    assert lib.fx_unit_work_offset(None, 0) == -1 and lib.fx_unit_max_selected(None, 0) == -1
    assert lib.fx_work_bytes(None) == 0
    assert lib.fx_compact_update(None, *([None] * 10), 0, None) == 1
    assert lib.fx_sparse_decode_ed(None, *([None] * 7), ctypes.c_float(1.0), None, None, None, 0,
                                   None) == 1
