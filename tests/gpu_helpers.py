"""Shared helpers of the GPU tests: device banks built through the C ABI and
oracle counterparts for the same seeded inputs."""

from __future__ import annotations

import functools

import numpy as np

from awq_int4_mixture_amd import inputs


def torch_mod():
    import torch
    return torch


@functools.lru_cache(maxsize=8)
def bank_case(seed: int, E: int, H: int, I: int, rb: int, zero_hi: int = 16):
    """(dims, device bank, BankInputs) for seeded weights packed by awq_moe_prepare."""
    from awq_int4_mixture_amd import abi
    torch = torch_mod()
    bi = inputs.bank_inputs(seed, E, H, I, zero_hi=zero_hi)
    dims = abi.make_dims(E, H, I, rb)
    host = abi.prepare_from_inputs(dims, bi)
    dev = torch.from_numpy(host).to("cuda")
    return dims, dev, bi


def to_dev(a, dtype=None):
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda")


def f16_to_np(t) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.float16)


def say(*a):
    print("[case]", *a, flush=True)
