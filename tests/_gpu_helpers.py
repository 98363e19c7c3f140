"""Shared set-up for the GPU parity tests: pools filled from the seeded generator,
device/host conversions, and the oracle side of each comparison."""
from __future__ import annotations

import numpy as np
import torch

from expert_slot_cache_amd import binding, synth
from oracle import lru as olru
from oracle import moe as omoe

DEV = torch.device("cuda:0")


def to_dev_act(a: np.ndarray, atype: str) -> torch.Tensor:
    """fp32 values or bf16 bits (uint16) -> device tensor of the activation type."""
    if atype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def from_dev_act(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float32)


class Rig:
    """A pool plus the host copies of its experts, for one workload shape."""

    def __init__(self, wl: synth.Workload, *, slots: int, layers: int | None = None,
                 resident: bool = False, rule: str = "distinct", max_tokens: int | None = None,
                 fast: bool = True, experts=None, std: float = 0.02, copy_streams: int = 1,
                 copy_chunk_bytes: int = 0, one_call: bool = False, timing: int = 0,
                 copy_engine: str = "kernel", policy: str = "host", read_through: bool = False,
                 evict: str = "lru", prefetch_slots: int = 0):
        self.wl = wl
        self.one_call = one_call   # one moe_pool_step call per layer instead of prepare + forward
        self.L = wl.layers if layers is None else layers
        self.E, self.K, self.H, self.I = wl.experts, wl.top_k, wl.hidden, wl.inter
        if experts is None:
            rng = synth.streams(wl)[1]
            experts = [[synth.draw_expert(rng, wl.wtype, self.H, self.I, std=std, fast=fast)
                        for _ in range(self.E)] for _ in range(self.L)]
        self.experts = experts
        self.pool = binding.MoePool(layers=self.L, experts=self.E, top_k=self.K, hidden=self.H,
                                    inter=self.I, slots=slots, wtype=wl.wtype, atype=wl.atype,
                                    rule=rule, resident=resident,
                                    max_tokens=max_tokens or wl.tokens, copy_streams=copy_streams,
                                    copy_chunk_bytes=copy_chunk_bytes, timing=timing,
                                    copy_engine=copy_engine, policy=policy, read_through=read_through,
                                    evict=evict, prefetch_slots=prefetch_slots)
        for l in range(self.L):
            for e in range(self.E):
                self.pool.load_expert(l, e, experts[l][e])

    def step(self, layer: int, ids: np.ndarray, x_dev, w_dev, resid_dev=None):
        """prepare + forward (or one step call); returns (path, misses, slot_ids
        host, out device)."""
        T = ids.shape[0]
        ids_d = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).to(DEV)
        slot_d = torch.empty_like(ids_d)
        dt = torch.float32 if self.wl.atype == "f32" else torch.bfloat16
        out = torch.empty((T, self.H), dtype=dt, device=DEV)
        if self.one_call:
            path, misses = self.pool.step(layer, ids_d, T, slot_d, x_dev, w_dev, out, resid=resid_dev)
        else:
            path, misses = self.pool.prepare(layer, ids_d, T, slot_d)
            self.pool.forward(layer, x_dev, slot_d, w_dev, out, T, resid=resid_dev)
        return path, misses, slot_d.cpu().numpy(), out

    def reference(self, layer: int, x: np.ndarray, ids: np.ndarray, w: np.ndarray, resid=None,
                  tokens=None):
        return omoe.moe_layer(x, ids, w, lambda e: self.experts[layer][e], self.wl.wtype,
                              self.H, self.I, resid=resid, atype=self.wl.atype, tokens=tokens)

    def close(self):
        self.pool.close()


def check_close(got: np.ndarray, ref: np.ndarray, atype: str, wtype: str, what: str = ""):
    tol = omoe.tolerance(atype, wtype)
    err = omoe.max_rel_err(got, ref)
    assert err <= tol, f"{what}: max|err|/max|ref| = {err:.3e} > {tol:.0e}"
    return err
