"""Convenience wrapper over the C ABI: owns the workspace and weight references.

Torch supplies device memory and the stream; every computation is a call into
libepoch.so through `binding`.
"""
from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import binding as B

_NP = {"i32": (torch.int32, 4), "f32": (torch.float32, 4), "u8": (torch.uint8, 1),
       "i64": (torch.int64, 8)}


class EpochPlan:
    """One block plan: build (cold path), forward / commit per layer and iteration, inspect.

    desc: a binding.epoch_desc.  weights: per layer a dict of device tensors with keys
    router_w, router_b (or None), w1, w3, w2, sw1, sw3, sw2 (None without a shared expert).
    """

    def __init__(self, desc: B.epoch_desc, weights: Sequence[dict], device="cuda", stream=None):
        self.desc = desc
        self.M = desc.batch * desc.block
        self.act_size = 2 if desc.act_dtype == B.EPOCH_DTYPE_BF16 else 4
        self.nbytes = B.epoch_plan_workspace_bytes(desc)
        self.ws = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        self._weights = list(weights)  # keep the tensors alive for the plan's lifetime
        lw = [B.layer_weights(w["router_w"], w.get("router_b"), w["w1"], w["w3"], w["w2"],
                              w.get("sw1"), w.get("sw3"), w.get("sw2")) for w in self._weights]
        self.handle = B.epoch_block_plan_build(desc, lw, self.ws, self.nbytes, stream)

    def forward(self, layer: int, x, decoded, force=None, y=None, y_routed=None, stream=None):
        if y is None:
            y = torch.empty_like(x)
        B.epoch_moe_fresh_forward(self.handle, layer, x, decoded, force, y, y_routed, stream)
        return y

    def commit(self, layer: int, stream=None):
        B.epoch_cache_update(self.handle, layer, stream)

    def _view(self, ptr: int, n: int, kind: str) -> torch.Tensor:
        dt, size = _NP[kind]
        off = ptr - self.ws.data_ptr()
        assert 0 <= off and off + n * size <= self.nbytes
        return self.ws[off:off + n * size].view(dt)

    def inspect(self, layer: int) -> dict:
        """Torch views (no copies) of the stage outputs and the layer state."""
        d, M = self.desc, self.M
        E, K = d.n_experts, d.top_k
        ins = B.epoch_plan_inspect(self.handle, layer)
        kx = ins.k_ext
        v = self._view
        cache = self.ws[ins.cache - self.ws.data_ptr():][: M * d.hidden * self.act_size]
        return dict(
            logits=v(ins.logits, M * E, "f32").view(M, E),
            ids=v(ins.ids, M * kx, "i32").view(M, kx),
            scores=v(ins.scores, M * kx, "f32").view(M, kx),
            atlas_q=v(ins.atlas_q, M * kx, "i32").view(M, kx),
            weights=v(ins.weights, M * K, "f32").view(M, K),
            fresh=v(ins.fresh, M, "u8"),
            fresh_list=v(ins.fresh_list, M, "i32"),
            n_fresh=v(ins.n_fresh, 1, "i32"),
            n_pairs=v(ins.n_pairs, 1, "i32"),
            wl_pos=v(ins.wl_pos, M * K, "i32"),
            wl_k=v(ins.wl_k, M * K, "i32"),
            wl_w=v(ins.wl_w, M * K, "f32"),
            offs=v(ins.offs, E + 1, "i32"),
            inv=v(ins.inv, M * K, "i32").view(M, K),
            routed_ids=v(ins.routed_ids, M * K, "i32").view(M, K),
            routed_w=v(ins.routed_w, M * K, "f32").view(M, K),
            in_support=v(ins.in_support, E, "u8"),
            slot_of=v(ins.slot_of, E, "i32"),
            support=v(ins.support, E, "i32"),
            support_size=v(ins.support_size, 1, "i32"),
            atlas=v(ins.atlas, E, "u8"),
            cache=cache.view(torch.int16 if self.act_size == 2 else torch.float32).view(M, d.hidden),
            valid=v(ins.valid, M, "u8"),
            last_fresh=v(ins.last_fresh, M, "i32"),
            prev_decoded=v(ins.prev_decoded, M, "u8"),
            counters=v(ins.counters, B.EPOCH_NUM_COUNTERS, "i64"),
            k_ext=ins.k_ext, iteration=ins.iteration, last_forward_layer=ins.last_forward_layer,
        )

    def counters(self, layer: int) -> dict:
        c = self.inspect(layer)["counters"].cpu().tolist()
        return dict(zip(B.COUNTERS, c))

    def set_timing(self, groups: int = -1):
        B.epoch_plan_set_timing(self.handle, groups)

    def timing(self) -> dict:
        return B.epoch_plan_timing(self.handle)

    def close(self):
        if self.handle:
            B.epoch_block_plan_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
