"""The C-ABI library loads, exports every symbol include/epoch.h declares, and rejects bad
arguments on the host before touching a GPU (CPU only)."""
import ctypes
import os
import re

import pytest

import synth
from block_diffusion_sparse_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "epoch.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(epoch_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libepoch.so not built")
    lib = ctypes.CDLL(B.LIB_PATH)
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/epoch.h but not exported"


def test_struct_layouts_match_header():
    src = open(os.path.join(ROOT, "include", "epoch.h")).read()
    body = src[src.index("typedef struct epoch_desc"):src.index("} epoch_desc;")]
    fields = re.findall(r"int32_t\s+([A-Za-z_0-9,\s]+);", body)
    names = [n.strip() for f in fields for n in f.split(",")]
    assert names == [f for f, _ in B.epoch_desc._fields_]
    body = src[src.index("typedef struct epoch_inspect"):src.index("} epoch_inspect;")]
    names = re.findall(r"\*\s*([a-z_]+);|int32_t\s+([a-z_]+);", body)
    names = [a or b for a, b in names]
    assert names == [f for f, _ in B.epoch_inspect._fields_]


def test_workspace_query_and_argument_errors():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libepoch.so not built")
    sizes = []
    for i in range(1, 6):
        d = B.make_desc(**synth.desc_fields(synth.workload(i)))
        sizes.append(B.epoch_plan_workspace_bytes(d))
    assert all(s > 0 and s % 256 == 0 for s in sizes)
    d = B.make_desc(**synth.desc_fields(synth.workload(2)))
    d2 = B.make_desc(**synth.desc_fields(synth.workload(2, batch=16)))
    assert B.epoch_plan_workspace_bytes(d2) > B.epoch_plan_workspace_bytes(d)
    bad = [dict(hidden=100), dict(top_k=0), dict(n_experts=2000), dict(staleness_R=0),
           dict(inter=100), dict(flags=1), dict(alpha_den=0), dict(q_num=200)]
    for b in bad:
        with pytest.raises(B.EpochError) as ei:
            B.epoch_plan_workspace_bytes(B.make_desc(**synth.desc_fields(synth.workload(2), **b)))
        assert ei.value.status == -2, b
    with pytest.raises(B.EpochError) as ei:
        B.epoch_plan_workspace_bytes(B.make_desc(**synth.desc_fields(synth.workload(2), act_dtype=7)))
    assert ei.value.status == -3
    # plan build checks the descriptor and the weights before any launch
    lw = [B.epoch_layer_weights()]
    with pytest.raises(B.EpochError) as ei:
        B.epoch_block_plan_build(d, lw, 256, 1 << 30, 0)
    assert ei.value.status == -1            # NULL router / expert weights
    with pytest.raises(B.EpochError) as ei:
        B.epoch_block_plan_build(d, lw, 100, 1 << 30, 0)
    assert ei.value.status == -4            # misaligned workspace
    assert B.epoch_status_string(0) == "ok"
    assert "workspace" in B.epoch_status_string(-4)
    assert B.load().epoch_block_plan_destroy(None) == 0
