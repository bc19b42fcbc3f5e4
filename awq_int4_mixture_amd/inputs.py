"""Seeded synthetic inputs for the AWQ int4 MoE expert stage.

This module only draws random numbers. It holds none of the stage's
arithmetic (no dequantisation, no packing, no routing, no products), so both
the CPU oracle and the GPU path can take their inputs from it.

Shapes follow the layer share described on the pages (PR #520 "Narrow
Qwen3.8 AWQ active grouped decode", Purpose: 512 experts, top-k 10, hidden
2560, local intermediate 160, group 32). The pages measured on real layer-1
AWQ weights that are not available; the draws below stand in for them:

* packed values q ~ U{0..15}
* scales s = fp16(|N(0,1)| * 0.02)
* zeros z ~ U{0..15} (stored as u8)
* activations x = fp16(N(0,1))
* router weights = fp32 softmax of N(0,1) logits over the k selected experts

For parity over the whole record range the ABI admits there are also
``expert_weights_wide`` (zeros U{0..255}; scales with a random sign that
include +-0, subnormals and, in chosen K-groups, magnitudes in [32768, 65504];
or subnormal scales only) and activations that are tiny in chosen groups or
near the fp16 maximum (``activations_wide``, ``activations_near_max``).

Every expert draws from its own stream, ``PCG64(SeedSequence([seed, e]))``,
in the fixed order q_gate, q_up, q_down, s_gate, s_up, s_down, z_gate, z_up,
z_down, so one expert can be regenerated without drawing the others.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

GROUP = 32

# Layer shapes used by tests and the benchmark.
RANK_SHAPE = dict(num_experts=512, topk=10, hidden=2560, inter=160)
TINY_SHAPE = dict(num_experts=16, topk=2, hidden=256, inter=32)


@dataclass
class ExpertWeights:
    """Logical (unpacked) AWQ weights of one expert.

    Orientation is y = x @ W, i.e. W is [K][N]:
      q_gate, q_up : uint8 [hidden][inter]   values 0..15
      q_down       : uint8 [inter][hidden]   values 0..15
      s_*          : float16 [K/32][N]       group scales (group along K)
      z_*          : uint8  [K/32][N]        group zeros
    """

    q_gate: np.ndarray
    q_up: np.ndarray
    q_down: np.ndarray
    s_gate: np.ndarray
    s_up: np.ndarray
    s_down: np.ndarray
    z_gate: np.ndarray
    z_up: np.ndarray
    z_down: np.ndarray


def _expert_rng(seed: int, e: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(e)])))


def expert_weights(seed: int, e: int, hidden: int, inter: int,
                   scale_std: float = 0.02, zero_hi: int = 16) -> ExpertWeights:
    """Draw the logical weights of expert ``e`` from its own seeded stream."""
    rng = _expert_rng(seed, e)
    H, I = hidden, inter
    q_gate = rng.integers(0, 16, size=(H, I), dtype=np.uint8)
    q_up = rng.integers(0, 16, size=(H, I), dtype=np.uint8)
    q_down = rng.integers(0, 16, size=(I, H), dtype=np.uint8)
    s_gate = (np.abs(rng.standard_normal((H // GROUP, I))) * scale_std).astype(np.float16)
    s_up = (np.abs(rng.standard_normal((H // GROUP, I))) * scale_std).astype(np.float16)
    s_down = (np.abs(rng.standard_normal((I // GROUP, H))) * scale_std).astype(np.float16)
    z_gate = rng.integers(0, zero_hi, size=(H // GROUP, I), dtype=np.uint8)
    z_up = rng.integers(0, zero_hi, size=(H // GROUP, I), dtype=np.uint8)
    z_down = rng.integers(0, zero_hi, size=(I // GROUP, H), dtype=np.uint8)
    return ExpertWeights(q_gate, q_up, q_down, s_gate, s_up, s_down, z_gate, z_up, z_down)


@dataclass
class BankInputs:
    """Stacked logical weights of all experts of one layer (leading axis E)."""

    q_gate: np.ndarray
    q_up: np.ndarray
    q_down: np.ndarray
    s_gate: np.ndarray
    s_up: np.ndarray
    s_down: np.ndarray
    z_gate: np.ndarray
    z_up: np.ndarray
    z_down: np.ndarray

    def expert(self, e: int) -> ExpertWeights:
        return ExpertWeights(*(getattr(self, f)[e] for f in _FIELDS))


_FIELDS = ("q_gate", "q_up", "q_down", "s_gate", "s_up", "s_down", "z_gate", "z_up", "z_down")


def fp16_wide_scales(rng: np.random.Generator, shape, std: float = 0.002, frac_zero: float = 0.05,
                     frac_sub: float = 0.10) -> np.ndarray:
    """fp16 scales spread over the finite range a record admits.

    Every value gets a random sign bit (so +0 and -0 both occur). With
    probability ``frac_zero`` the magnitude is 0, with probability
    ``frac_sub`` it is a subnormal (exponent field 0, mantissa U{1..1023}),
    otherwise fp16(|N(0,1)| * std). Draw order: class, sign, normal, mantissa.
    """
    u = rng.random(shape)
    sign = (rng.integers(0, 2, size=shape).astype(np.uint16) << np.uint16(15)).astype(np.uint16)
    normal = (np.abs(rng.standard_normal(shape)) * std).astype(np.float16).view(np.uint16)
    sub = rng.integers(1, 1024, size=shape).astype(np.uint16)
    mag = np.where(u < frac_zero, np.uint16(0), np.where(u < frac_zero + frac_sub, sub, normal)).astype(np.uint16)
    return (mag | sign).view(np.float16)


def fp16_big_scales(rng: np.random.Generator, shape) -> np.ndarray:
    """fp16 scales at the top of the range: exponent field 30 (magnitudes
    32768 .. 65504), mantissa U{0..1023}, random sign. Draw order: mantissa, sign."""
    mant = rng.integers(0, 1024, size=shape).astype(np.uint16)
    sign = (rng.integers(0, 2, size=shape).astype(np.uint16) << np.uint16(15)).astype(np.uint16)
    return ((np.uint16(30 << 10) | mant) | sign).astype(np.uint16).view(np.float16)


def fp16_tiny_scales(rng: np.random.Generator, shape, mant_hi: int = 4) -> np.ndarray:
    """fp16 subnormal scales with mantissa U{1..mant_hi-1} (multiples of 2^-24)
    and a random sign. Draw order: mantissa, sign."""
    mant = rng.integers(1, mant_hi, size=shape).astype(np.uint16)
    sign = (rng.integers(0, 2, size=shape).astype(np.uint16) << np.uint16(15)).astype(np.uint16)
    return (mant | sign).astype(np.uint16).view(np.float16)


def expert_weights_wide(seed: int, e: int, hidden: int, inter: int, kind: str = "wide", kind_w2: str | None = None,
                        big_w13_groups=(), big_w2_groups=()) -> ExpertWeights:
    """Expert ``e`` with records over the whole admitted range: zeros
    U{0..255} and scales of both signs.

    ``kind`` sets the W13 scales and ``kind_w2`` (default: the same) the W2
    scales:
      "wide": ``fp16_wide_scales``, except the K-groups listed in
              ``big_w13_groups`` (W13) or ``big_w2_groups`` (W2), whose
              scales (every column) come from ``fp16_big_scales``;
      "tiny": ``fp16_tiny_scales`` (for activations near the fp16 maximum).
    Draw order: q_gate, q_up, q_down, z_gate, z_up, z_down, then the scales
    of gate, up and down (each: the base draw, then the big groups)."""
    rng = _expert_rng(seed, e)
    H, I = hidden, inter
    q_gate = rng.integers(0, 16, size=(H, I), dtype=np.uint8)
    q_up = rng.integers(0, 16, size=(H, I), dtype=np.uint8)
    q_down = rng.integers(0, 16, size=(I, H), dtype=np.uint8)
    z_gate = rng.integers(0, 256, size=(H // GROUP, I), dtype=np.uint8)
    z_up = rng.integers(0, 256, size=(H // GROUP, I), dtype=np.uint8)
    z_down = rng.integers(0, 256, size=(I // GROUP, H), dtype=np.uint8)
    scales = []
    kind_w2 = kind if kind_w2 is None else kind_w2
    for shape, big, kd in (((H // GROUP, I), big_w13_groups, kind), ((H // GROUP, I), big_w13_groups, kind),
                           ((I // GROUP, H), big_w2_groups, kind_w2)):
        if kd == "tiny":
            s = fp16_tiny_scales(rng, shape)
        elif kd == "wide":
            s = fp16_wide_scales(rng, shape)
            for g in big:
                s[g, :] = fp16_big_scales(rng, (shape[1],))
        else:
            raise ValueError(f"unknown kind {kd!r}")
        scales.append(s)
    return ExpertWeights(q_gate, q_up, q_down, scales[0], scales[1], scales[2], z_gate, z_up, z_down)


def bank_inputs(seed: int, num_experts: int, hidden: int, inter: int, draw=None, **kw) -> BankInputs:
    """Draw all experts of one layer (expert e from stream [seed, e]) with
    ``draw`` (``expert_weights`` unless given) and its keyword arguments."""
    draw = expert_weights if draw is None else draw
    E, H, I = num_experts, hidden, inter
    out = {
        "q_gate": np.empty((E, H, I), np.uint8), "q_up": np.empty((E, H, I), np.uint8),
        "q_down": np.empty((E, I, H), np.uint8),
        "s_gate": np.empty((E, H // GROUP, I), np.float16), "s_up": np.empty((E, H // GROUP, I), np.float16),
        "s_down": np.empty((E, I // GROUP, H), np.float16),
        "z_gate": np.empty((E, H // GROUP, I), np.uint8), "z_up": np.empty((E, H // GROUP, I), np.uint8),
        "z_down": np.empty((E, I // GROUP, H), np.uint8),
    }
    for e in range(E):
        w = draw(seed, e, H, I, **kw)
        for f in _FIELDS:
            out[f][e] = getattr(w, f)
    return BankInputs(**out)


def activations(rng: np.random.Generator, M: int, hidden: int) -> np.ndarray:
    """x = fp16(N(0,1)), shape [M][hidden]."""
    return rng.standard_normal((M, hidden)).astype(np.float16)


def activations_wide(rng: np.random.Generator, M: int, hidden: int, tiny_groups=()) -> np.ndarray:
    """x = fp16(N(0,1)), except the 32-value groups listed in ``tiny_groups``,
    which get fp16(N(0,1) * 2^-22): mostly subnormals of a few units of 2^-24,
    and zeros. Draw order: the normal matrix, then the tiny groups."""
    x = rng.standard_normal((M, hidden))
    for g in tiny_groups:
        x[:, GROUP * g:GROUP * (g + 1)] = rng.standard_normal((M, GROUP)) * 2.0 ** -22
    return x.astype(np.float16)


def activations_near_max(rng: np.random.Generator, M: int, hidden: int) -> np.ndarray:
    """x with |x| ~ U[2^14, 65504] rounded to fp16 and a random sign: the top
    two binades of the fp16 range. Draw order: magnitudes, signs."""
    mag = rng.uniform(2.0 ** 14, 65504.0, size=(M, hidden))
    sign = np.where(rng.integers(0, 2, size=(M, hidden)) == 1, -1.0, 1.0)
    return (mag * sign).astype(np.float16)


def router_weights(rng: np.random.Generator, M: int, k: int) -> np.ndarray:
    """fp32 softmax of N(0,1) logits over the k selected experts, [M][k].

    This only shapes the synthetic input distribution; the stage itself uses
    the weights exactly as given.
    """
    logits = rng.standard_normal((M, k))
    logits -= logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=1, keepdims=True)
    return p.astype(np.float32)


def ids_distinct(rng: np.random.Generator, M: int, k: int, E: int) -> np.ndarray:
    """Each token picks k distinct experts uniformly; tokens are independent."""
    return np.stack([rng.choice(E, size=k, replace=False) for _ in range(M)]).astype(np.int32)


def ids_shared_pool(rng: np.random.Generator, M: int, k: int, E: int, frac: float = 0.6) -> np.ndarray:
    """Tokens draw k distinct experts from a common pool of ceil(frac*M*k).

    This gives multi-row segments (experts shared by several tokens), the
    grouped-decode case of PR #520 (Purpose: multi-row active-expert segments).
    """
    pool_n = max(k, min(E, int(math.ceil(frac * M * k))))
    pool = rng.choice(E, size=pool_n, replace=False)
    return np.stack([rng.choice(pool, size=k, replace=False) for _ in range(M)]).astype(np.int32)


def ids_all_distinct(rng: np.random.Generator, M: int, k: int, E: int) -> np.ndarray:
    """All M*k slots pick different experts (upper bound on touched bytes)."""
    return rng.choice(E, size=M * k, replace=False).reshape(M, k).astype(np.int32)


def hot_experts(seed: int, k: int, E: int) -> np.ndarray:
    """The fixed set of k experts reused by every call of the hot workload."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), 0xA0])))
    return rng.choice(E, size=k, replace=False).astype(np.int32)


def rotating_ids(seed: int, calls: int, k: int, E: int) -> np.ndarray:
    """Call c uses experts perm[c*k:(c+1)*k] of one seeded permutation, [calls][1][k]."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), 0xB0])))
    perm = rng.permutation(E)
    assert calls * k <= E
    return perm[: calls * k].reshape(calls, 1, k).astype(np.int32)


def rotating_calls(seed: int, calls: int, M: int, k: int, E: int, banks: int, mode: str, frac: float = 0.6):
    """Ids for ``calls`` consecutive calls that keep weights cold across banks.

    Call j uses bank b = j % banks and the next window of P experts of that
    bank's own seeded permutation (windows advance cyclically, so a window
    comes back only after E / P calls on its bank, i.e. banks * E / P calls
    in all). mode "distinct": P = M*k, the window shuffled into [M][k] (all
    slots distinct); mode "pool": P = ceil(frac*M*k), each token draws k
    distinct experts from the window (shared experts, as ``ids_shared_pool``).
    Returns a list of (bank, ids int32 [M][k]). Draw order: the permutation of
    each bank, then per call the shuffle or the tokens' draws."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), 0xD0, M, k])))
    perms = [rng.permutation(E) for _ in range(banks)]
    P = M * k if mode == "distinct" else max(k, min(E, int(math.ceil(frac * M * k))))
    out = []
    for j in range(calls):
        b = j % banks
        start = ((j // banks) * P) % E
        win = perms[b][(start + np.arange(P)) % E]
        if mode == "distinct":
            ids = rng.permutation(win).reshape(M, k)
        elif mode == "pool":
            ids = np.stack([rng.choice(win, size=k, replace=False) for _ in range(M)])
        else:
            raise ValueError(f"unknown mode {mode!r}")
        out.append((b, ids.astype(np.int32)))
    return out


def router_logits(rng: np.random.Generator, M: int, E: int) -> np.ndarray:
    """fp32 router logits ~ N(0,1), [M][E]."""
    return rng.standard_normal((M, E)).astype(np.float32)


def call_rng(seed: int, tag: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), 0xC0, int(tag)])))


def device_bank(seed: int, num_experts: int, record_sections, expert_bytes: int, meta_bytes: int,
                device="cuda"):
    """A packed bank drawn directly on the device (for many-layer workloads).

    Uniform random bytes are uniform 4-bit values, so every byte of the bank
    is first drawn U{0..255}. Each record section ``(offset, count)`` of
    every expert block is then overwritten with ``count`` records of
    ``meta_bytes`` bytes: scale = fp16(|N(0,1)| * 0.02) (little endian),
    zero ~ U{0..15}, and a zero pad byte for 4-byte records. The draws come
    from one seeded torch generator in the order: bank bytes, then for each
    section the normals and then the zeros. Returns a uint8 device tensor.
    """
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    total = num_experts * expert_bytes
    bank = torch.randint(0, 256, (total,), dtype=torch.uint8, device=device, generator=g)
    blocks = bank.view(num_experts, expert_bytes)
    for off, count in record_sections:
        s = (torch.randn((num_experts, count), device=device, generator=g).abs() * 0.02).to(torch.float16)
        z = torch.randint(0, 16, (num_experts, count), dtype=torch.uint8, device=device, generator=g)
        rec = blocks[:, off:off + count * meta_bytes].view(num_experts, count, meta_bytes)
        rec[:, :, 0:2] = s.view(torch.uint8).view(num_experts, count, 2)
        rec[:, :, 2] = z
        if meta_bytes == 4:
            rec[:, :, 3] = 0
    return bank


def device_router_weights(seed: int, num_experts: int, hidden: int, device="cuda"):
    """Router weights for a many-layer workload, drawn on the device: fp16
    [num_experts][hidden] with entries N(0,1) / sqrt(hidden), so that a
    unit-RMS input row gives logits of about unit variance."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    w = torch.randn((num_experts, hidden), device=device, generator=g) / float(np.sqrt(hidden))
    return w.to(torch.float16)
