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
def bank_case(seed: int, E: int, H: int, I: int, rb: int, zero_hi: int = 16, wide: tuple | None = None):
    """(dims, device bank, BankInputs) for seeded weights packed by awq_moe_prepare.

    ``wide``: None for the default draws (``inputs.expert_weights`` with
    zeros below ``zero_hi``), else a tuple of (name, value) pairs passed to
    ``inputs.expert_weights_wide`` (zeros 0..255, scales of both signs)."""
    from awq_int4_mixture_amd import abi
    torch = torch_mod()
    if wide is None:
        bi = inputs.bank_inputs(seed, E, H, I, zero_hi=zero_hi)
    else:
        bi = inputs.bank_inputs(seed, E, H, I, draw=inputs.expert_weights_wide, **dict(wide))
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


def exact_in_fp32(v64) -> bool:
    """True when every float64 value is exactly representable in float32."""
    v = np.asarray(v64, dtype=np.float64)
    return bool(np.all(v.astype(np.float32).astype(np.float64) == v))


def say(*a):
    print("[case]", *a, flush=True)
