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
    body = src[src.index("typedef struct epoch_decode_desc"):src.index("} epoch_decode_desc;")]
    names = re.findall(r"(?:int32_t|double)\s+([a-z_]+);", body)
    assert names == [f for f, _ in B.epoch_decode_desc._fields_]
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
           dict(inter=100), dict(flags=1), dict(alpha_den=0), dict(q_num=200), dict(routing=2),
           dict(atlas_period=3),                       # a period needs restricted routing
           dict(n_group=3, topk_group=1),              # 64 experts do not split in 3 groups
           dict(n_group=8, topk_group=9), dict(n_group=128, topk_group=4),
           dict(n_group=16, topk_group=3)]             # 3 groups of 4 < K_ext = 16 candidates
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


def test_decode_workspace_query_and_argument_errors():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libepoch.so not built")
    d = B.make_decode_desc(8, 32, 2048, 32768)
    n = B.epoch_decode_workspace_bytes(d)
    assert n % 256 == 0 and n >= 256 * (32768 // 256) * 12   # the partials of all 256 rows
    for kw, status in ((dict(vocab=100), -2), (dict(block=2000), -2), (dict(hidden=96), -2),
                       (dict(tau=0.0), -2), (dict(tau=1.5), -2), (dict(act_dtype=0), -3)):
        args = dict(batch=8, block=32, hidden=2048, vocab=32768)
        args.update(kw)
        with pytest.raises(B.EpochError) as ei:
            B.epoch_decode_workspace_bytes(B.make_decode_desc(**args))
        assert ei.value.status == status, kw
    with pytest.raises(B.EpochError) as ei:   # NULL tensors: checked before any launch
        B.epoch_live_decode(d, 0, 0, 0, 0, 0, None, 256, n, 0)
    assert ei.value.status == -1


def test_static_decode_rejects_shapes_beyond_its_scratch():
    """The workspace-free decoding call checks its shape against the static scratch array on
    the host and enqueues nothing for a shape that does not fit (no GPU involved)."""
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libepoch.so not built")
    cap = B.EPOCH_DECODE_STATIC_SCRATCH_BYTES
    fits = B.make_decode_desc(64, 32, 2048, 131072)          # 2048 positions
    big = B.make_decode_desc(256, 32, 2048, 131072)          # 8192 positions
    assert B.epoch_decode_workspace_bytes(fits) <= cap < B.epoch_decode_workspace_bytes(big)
    with pytest.raises(B.EpochError) as ei:   # aligned stand-in pointers: never dereferenced
        B.epoch_live_decode_static(big, 256, 256, 256, 256, 256, None, 0)
    assert ei.value.status == B.EPOCH_E_SCRATCH
    assert "static" in B.epoch_status_string(B.EPOCH_E_SCRATCH)
    with pytest.raises(B.EpochError) as ei:
        B.epoch_live_decode_static(fits, 0, 256, 256, 256, 256, None, 0)
    assert ei.value.status == -1
    with pytest.raises(B.EpochError) as ei:
        B.epoch_live_decode_static(fits, 8, 256, 256, 256, 256, None, 0)
    assert ei.value.status == -8
