"""Host<->device helpers for the GPU tests (marshalling only)."""

from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import oracle
from workloads import make_workload


def say(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def to_dev_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


class DeviceInputs:
    def __init__(self, wl):
        self.wl = wl
        self.x = to_dev_bf16(wl.x)
        self.ids = to_dev(wl.expert_ids.astype(np.int32))
        self.w = to_dev(wl.routing_w.astype(np.float32))
        self.w_ug = to_dev_bf16(wl.w_ug)
        self.w_down = to_dev_bf16(wl.w_down)


@functools.lru_cache(maxsize=2)
def workload(name: str):
    return make_workload(name)


@functools.lru_cache(maxsize=2)
def oracle_result(name: str):
    wl = workload(name)
    say(f"[oracle] {name}: T={wl.T} k={wl.k} E={wl.E} d={wl.d} h={wl.h}")
    return oracle.moe_expert_forward(wl.x, wl.expert_ids, wl.routing_w, wl.w_ug, wl.w_down, keep_u=True)
