"""ctypes binding of libepoch.so (include/epoch.h): argument marshalling only.

Every step of the layer runs in the HIP library; this module converts Python
values and torch tensors (device memory and streams only) into the C-ABI's
pointers and sizes, and turns a negative status into an exception.  It fails
loudly when the library has not been built: there is no other code path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libepoch.so")

EPOCH_GATE_SOFTMAX, EPOCH_GATE_SIGMOID = 0, 1
EPOCH_DTYPE_F32, EPOCH_DTYPE_BF16 = 0, 1
EPOCH_ROUTING_EXACT, EPOCH_ROUTING_RESTRICTED = 0, 1
EPOCH_NUM_COUNTERS = 20
EPOCH_TIMING_GROUPS = 9
EPOCH_E_SCRATCH = -9
EPOCH_DECODE_STATIC_SCRATCH_BYTES = 32 * 1024 * 1024
COUNTERS = ["cold", "hot_update", "hot_skip", "anomaly", "fresh_rows", "pairs", "unmet",
            "forced_rows", "due_rows", "support_size", "u_final", "repair_rounds", "touched",
            "forwards", "reserved14", "restricted", "coverage_fallback", "period_update",
            "big_experts", "big_pairs"]
TIMING_GROUPS = ["router", "plan", "place", "routed_gateup", "routed_down", "shared",
                 "combine", "routed_gateup_big", "routed_down_big"]

_i32 = ctypes.c_int32
_vp = ctypes.c_void_p


class epoch_desc(ctypes.Structure):
    _fields_ = [(n, _i32) for n in (
        "n_layers", "hidden", "n_experts", "top_k", "inter", "n_shared", "shared_inter", "batch",
        "block", "gate", "norm_topk", "act_dtype", "staleness_R", "atlas_m", "atlas_B", "atlas_c",
        "alpha_num", "alpha_den", "q_num", "q_den", "beta_num", "beta_den", "flags", "routing",
        "atlas_period", "n_group", "topk_group")]


class epoch_layer_weights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("router_w", "router_b", "w1", "w3", "w2", "sw1", "sw3", "sw2")]


class epoch_inspect(ctypes.Structure):
    _fields_ = [(n, _vp) for n in (
        "logits", "ids", "scores", "atlas_q", "weights", "fresh", "fresh_list", "n_fresh",
        "n_pairs", "wl_pos", "wl_k", "wl_w", "offs", "inv", "routed_ids", "routed_w",
        "in_support", "slot_of", "support", "support_size", "atlas", "cache", "valid",
        "last_fresh", "prev_decoded", "counters")] + [
        ("k_ext", _i32), ("iteration", _i32), ("last_forward_layer", _i32)]


class epoch_decode_desc(ctypes.Structure):
    _fields_ = [(n, _i32) for n in ("batch", "block", "hidden", "vocab", "act_dtype", "flags")] + [
        ("tau", ctypes.c_double)]


class EpochError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; "
                          "g.build()'` (hipcc, gfx950). There is no fallback path.")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.epoch_plan_workspace_bytes.argtypes = [P(epoch_desc), P(ctypes.c_size_t)]
    lib.epoch_block_plan_build.argtypes = [P(epoch_desc), P(epoch_layer_weights), _vp,
                                           ctypes.c_size_t, _vp, P(_vp)]
    lib.epoch_moe_fresh_forward.argtypes = [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.epoch_cache_update.argtypes = [_vp, _i32, _vp]
    lib.epoch_plan_inspect.argtypes = [_vp, _i32, P(epoch_inspect)]
    lib.epoch_block_plan_destroy.argtypes = [_vp]
    lib.epoch_status_string.argtypes = [_i32]
    lib.epoch_status_string.restype = ctypes.c_char_p
    lib.epoch_plan_set_timing.argtypes = [_vp, _i32]
    lib.epoch_plan_timing.argtypes = [_vp, P(ctypes.c_float), P(ctypes.c_int64), _i32]
    lib.epoch_decode_workspace_bytes.argtypes = [P(epoch_decode_desc), P(ctypes.c_size_t)]
    lib.epoch_live_decode.argtypes = [P(epoch_decode_desc), _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      ctypes.c_size_t, _vp]
    lib.epoch_live_decode_static.argtypes = [P(epoch_decode_desc), _vp, _vp, _vp, _vp, _vp, _vp,
                                             _vp]
    for fn in ("epoch_live_decode_static", "epoch_plan_workspace_bytes", "epoch_block_plan_build", "epoch_moe_fresh_forward",
               "epoch_cache_update", "epoch_plan_inspect", "epoch_block_plan_destroy",
               "epoch_plan_set_timing", "epoch_plan_timing", "epoch_decode_workspace_bytes",
               "epoch_live_decode"):
        getattr(lib, fn).restype = _i32
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != 0:
        raise EpochError(fn, status, load().epoch_status_string(status).decode())


def _ptr(t) -> Optional[int]:
    """A device pointer from a torch tensor, an int, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_desc(**kw) -> epoch_desc:
    d = epoch_desc()
    for k, v in kw.items():
        setattr(d, k, int(v))
    return d


def epoch_plan_workspace_bytes(desc: epoch_desc) -> int:
    out = ctypes.c_size_t(0)
    _check("epoch_plan_workspace_bytes", load().epoch_plan_workspace_bytes(ctypes.byref(desc),
                                                                           ctypes.byref(out)))
    return out.value


def layer_weights(router_w, router_b, w1, w3, w2, sw1=None, sw3=None, sw2=None) -> epoch_layer_weights:
    return epoch_layer_weights(*[_ptr(t) for t in (router_w, router_b, w1, w3, w2, sw1, sw3, sw2)])


def epoch_block_plan_build(desc: epoch_desc, weights: Sequence[epoch_layer_weights], workspace,
                           workspace_bytes: int, stream=None) -> int:
    arr = (epoch_layer_weights * len(weights))(*weights)
    plan = _vp(0)
    _check("epoch_block_plan_build",
           load().epoch_block_plan_build(ctypes.byref(desc), arr, _ptr(workspace),
                                         ctypes.c_size_t(workspace_bytes), _stream(stream),
                                         ctypes.byref(plan)))
    return plan.value


def epoch_moe_fresh_forward(plan: int, layer: int, x, decoded, force_fresh, y, y_routed=None,
                            stream=None):
    _check("epoch_moe_fresh_forward",
           load().epoch_moe_fresh_forward(plan, layer, _ptr(x), _ptr(decoded), _ptr(force_fresh),
                                          _ptr(y), _ptr(y_routed), _stream(stream)))


def epoch_cache_update(plan: int, layer: int, stream=None):
    _check("epoch_cache_update", load().epoch_cache_update(plan, layer, _stream(stream)))


def epoch_plan_inspect(plan: int, layer: int) -> epoch_inspect:
    out = epoch_inspect()
    _check("epoch_plan_inspect", load().epoch_plan_inspect(plan, layer, ctypes.byref(out)))
    return out


def epoch_block_plan_destroy(plan: int):
    _check("epoch_block_plan_destroy", load().epoch_block_plan_destroy(plan))


def epoch_status_string(status: int) -> str:
    return load().epoch_status_string(status).decode()


def epoch_plan_set_timing(plan: int, groups: int = -1):
    """groups: bitmask of TIMING_GROUPS indices (-1 = all, 0 = off)."""
    _check("epoch_plan_set_timing", load().epoch_plan_set_timing(plan, int(groups)))


def epoch_plan_timing(plan: int):
    ms = (ctypes.c_float * EPOCH_TIMING_GROUPS)()
    n = (ctypes.c_int64 * EPOCH_TIMING_GROUPS)()
    _check("epoch_plan_timing", load().epoch_plan_timing(plan, ms, n, EPOCH_TIMING_GROUPS))
    return {g: (float(ms[i]), int(n[i])) for i, g in enumerate(TIMING_GROUPS)}


def make_decode_desc(batch: int, block: int, hidden: int, vocab: int, tau: float = 0.95,
                     act_dtype: int = EPOCH_DTYPE_BF16) -> epoch_decode_desc:
    return epoch_decode_desc(batch=batch, block=block, hidden=hidden, vocab=vocab,
                             act_dtype=act_dtype, flags=0, tau=float(tau))


def epoch_decode_workspace_bytes(desc: epoch_decode_desc) -> int:
    out = ctypes.c_size_t(0)
    _check("epoch_decode_workspace_bytes",
           load().epoch_decode_workspace_bytes(ctypes.byref(desc), ctypes.byref(out)))
    return out.value


def epoch_live_decode(desc: epoch_decode_desc, h, w_vocab, decoded, decoded_next, tokens,
                      conf, workspace, workspace_bytes: int, stream=None):
    _check("epoch_live_decode",
           load().epoch_live_decode(ctypes.byref(desc), _ptr(h), _ptr(w_vocab), _ptr(decoded),
                                    _ptr(decoded_next), _ptr(tokens), _ptr(conf),
                                    _ptr(workspace), ctypes.c_size_t(workspace_bytes),
                                    _stream(stream)))


def epoch_live_decode_static(desc: epoch_decode_desc, h, w_vocab, decoded, decoded_next, tokens,
                             conf, stream=None):
    _check("epoch_live_decode_static",
           load().epoch_live_decode_static(ctypes.byref(desc), _ptr(h), _ptr(w_vocab),
                                           _ptr(decoded), _ptr(decoded_next), _ptr(tokens),
                                           _ptr(conf), _stream(stream)))
