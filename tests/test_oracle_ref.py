"""Pins of the float64 oracle (CPU only).

Each pin comes from something other than the oracle's own code: scalar
loops written independently (``oracle.loops``), brute-force enumeration,
closed forms, torch's CPU float64 library routines for the textbook dense
SwiGLU FFN, exact integer arithmetic, and invariants of the definition.
"""

import itertools
import math

import numpy as np
import pytest
import torch

from awq_int4_mixture_amd import inputs
from oracle import loops as LP
from oracle import ref as R


# ---------------------------------------------------------------------------
# dequantisation
# ---------------------------------------------------------------------------

def test_dequant_matches_scalar_loops():
    w = inputs.expert_weights(3, 0, 64, 32, zero_hi=256)
    for q, s, z in ((w.q_gate, w.s_gate, w.z_gate), (w.q_down, w.s_down, w.z_down)):
        got = R.dequant(q, s, z)
        want = np.array(LP.dequant_loop(q.tolist(), s.astype(np.float64).tolist(), z.tolist()))
        np.testing.assert_array_equal(got, want)


def _wide_expert(seed=3, H=96, I=64):
    """Records over the whole admitted range: zeros 0..255, scales of both
    signs with +-0, subnormals, normals, and one K-group of scales near the
    fp16 maximum in each matrix."""
    return inputs.expert_weights_wide(seed, 0, H, I, big_w13_groups=(1,), big_w2_groups=(0,))


def test_wide_record_draws_cover_every_class():
    w = _wide_expert()
    s = np.concatenate([w.s_gate.ravel(), w.s_up.ravel(), w.s_down.ravel()])
    b = s.view(np.uint16)
    assert (b == 0x0000).any() and (b == 0x8000).any()                 # +0 and -0
    assert (((b & 0x7C00) == 0) & ((b & 0x03FF) != 0)).any()            # subnormals
    assert (np.abs(s.astype(np.float64)) >= 32768).any()                # near the top of the range
    assert (s < 0).any() and (s > 0).any()
    assert w.z_gate.max() > 200 and w.z_down.max() > 200
    assert np.isfinite(s.astype(np.float64)).all()
    t = inputs.expert_weights_wide(3, 0, 64, 32, kind="tiny")
    tb = t.s_gate.view(np.uint16) & 0x7FFF
    assert ((tb >= 1) & (tb <= 3)).all()                                  # subnormal multiples of 2^-24
    x = inputs.activations_near_max(np.random.default_rng(0), 2, 64).astype(np.float64)
    assert (np.abs(x) >= 2.0 ** 14).all() and (np.abs(x) <= 65504).all() and (x < 0).any()


def test_dequant_matches_scalar_loops_wide_records():
    """The same pin over zeros 0..255 and scales of both signs, +-0,
    subnormal and near 65504; each value is also exact in float32."""
    w = _wide_expert()
    for q, s, z in ((w.q_gate, w.s_gate, w.z_gate), (w.q_up, w.s_up, w.z_up), (w.q_down, w.s_down, w.z_down)):
        got = R.dequant(q, s, z)
        want = np.array(LP.dequant_loop(q.tolist(), s.astype(np.float64).tolist(), z.tolist()))
        np.testing.assert_array_equal(got, want)
        assert np.array_equal(got.astype(np.float32).astype(np.float64), got)
        # the sign of a zero scale survives: (q - z) * (-0.0) is -0.0 for q > z
        neg0 = (s.view(np.uint16) == 0x8000)[np.arange(q.shape[0]) // 32, :] & (q > z[np.arange(q.shape[0]) // 32, :])
        if neg0.any():
            assert np.signbit(got[neg0]).all() and (got[neg0] == 0).all()


def test_dequant_closed_form_values():
    q = np.array([[0], [15], [7], [8]] * 8, np.uint8)          # K=32, N=1
    s = np.array([[0.5]], np.float16)
    z = np.array([[8]], np.uint8)
    got = R.dequant(q, s, z)[:4, 0]
    np.testing.assert_array_equal(got, [-4.0, 3.5, -0.5, 0.0])


def test_dequant_exact_in_fp32_for_every_scale_and_offset():
    """(q - z) * s is exactly representable in fp32 for every finite fp16 s,
    every u8 zero and every 4-bit q (|q - z| <= 255 has 8 significant bits,
    an fp16 significand 11, and fp16's range sits inside fp32's normal range)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    s = bits.view(np.float16)
    s = s[np.isfinite(s)].astype(np.float64)
    assert s.size == 63488
    d = np.arange(-255, 16, dtype=np.float64)            # every q - z
    prod = d[:, None] * s[None, :]
    assert np.array_equal(prod.astype(np.float32).astype(np.float64), prod)


# ---------------------------------------------------------------------------
# routing compaction
# ---------------------------------------------------------------------------

def _check_route_against_brute(ids, E):
    got = R.route_compact(ids, E)
    want = LP.route_brute(ids.tolist(), E)
    A = got["num_active"]
    assert A == len(want["experts"])
    assert got["active_ids"][:A].tolist() == want["experts"]
    assert (got["active_ids"][A:] == -1).all()
    assert got["offsets"][:A + 1].tolist() == (want["offsets"] if A else [0])
    assert (got["offsets"][A + 1:] == got["num_valid"]).all()
    assert got["sorted_slots"].tolist() == want["sorted_slots"]
    assert got["status"] == want["status"]


def test_route_exhaustive_small():
    """All id tensors with E=4, k=2, M=1..3 (16 + 256 + 4096 cases)."""
    E, k = 4, 2
    count = 0
    for M in (1, 2, 3):
        for flat in itertools.product(range(E), repeat=M * k):
            _check_route_against_brute(np.array(flat, np.int32).reshape(M, k), E)
            count += 1
    assert count == 4368


def test_route_exhaustive_with_invalid_ids():
    """Values in {-1, 0..3, 4} with E=4, M=2, k=2: out-of-range ids set the status bit."""
    for flat in itertools.product(range(-1, 5), repeat=4):
        _check_route_against_brute(np.array(flat, np.int32).reshape(2, 2), 4)


def test_route_invariants_random():
    rng = np.random.default_rng(0)
    for _ in range(200):
        M = int(rng.integers(1, 9))
        k = int(rng.integers(1, 33))
        E = int(rng.integers(1, 600))
        ids = rng.integers(0, E, size=(M, k)).astype(np.int32)
        r = R.route_compact(ids, E)
        A, n = r["num_active"], M * k
        off = r["offsets"]
        assert off[0] == 0 and off[A] == n and (np.diff(off[:A + 1]) > 0).all()
        assert (np.diff(r["active_ids"][:A]) > 0).all()
        assert sorted(r["sorted_slots"].tolist()) == list(range(n))
        flat = ids.reshape(-1)
        for a in range(A):
            rows = r["sorted_slots"][off[a]:off[a + 1]]
            assert (flat[rows] == r["active_ids"][a]).all() and (np.diff(rows) > 0).all()


# ---------------------------------------------------------------------------
# the stage
# ---------------------------------------------------------------------------

def _micro(seed=1, E=4, H=64, I=32, M=3, k=2, zero_hi=16):
    bi = inputs.bank_inputs(seed, E, H, I, zero_hi=zero_hi)
    rng = inputs.call_rng(seed, 1)
    x = inputs.activations(rng, M, H)
    ids = inputs.ids_distinct(rng, M, k, E)
    w = inputs.router_weights(rng, M, k)
    return bi, x, ids, w


def test_stage_matches_scalar_loops_micro():
    """E=4, H=64, I=32, k=2, M=3 (scales 0.2 so the values are not tiny)."""
    bi, x, ids, w = _micro()
    for f in ("s_gate", "s_up", "s_down"):
        setattr(bi, f, (getattr(bi, f).astype(np.float32) * 10).astype(np.float16))
    got = R.moe_stage(x, ids, w, 4, bi.expert)
    want = np.array(LP.stage_loops(x.astype(np.float64).tolist(), ids.tolist(),
                                   w.astype(np.float64).tolist(), 4, bi.expert))
    assert np.abs(got - want).max() <= 1e-12 * np.abs(want).max()


def test_stage_matches_scalar_loops_wide_records():
    """E=3, H=96, I=64, k=2, M=3 with zeros 0..255, signed/zero/subnormal
    scales, one W13 K-group of scales near 65504 whose activations are tiny
    subnormals, and a second case with activations near the fp16 maximum and
    subnormal W13 scales."""
    E, H, I, M, k = 3, 96, 64, 3, 2
    cases = (
        (dict(big_w13_groups=(1,)), lambda rng: inputs.activations_wide(rng, M, H, tiny_groups=(1,))),
        (dict(kind="tiny", kind_w2="wide"), lambda rng: inputs.activations_near_max(rng, M, H)),
    )
    for kw, xdraw in cases:
        bi = inputs.bank_inputs(17, E, H, I, draw=inputs.expert_weights_wide, **kw)
        rng = inputs.call_rng(17, 2)
        x = xdraw(rng)
        ids = inputs.ids_distinct(rng, M, k, E)
        w = inputs.router_weights(rng, M, k)
        got = R.moe_stage(x, ids, w, E, bi.expert)
        want = np.array(LP.stage_loops(x.astype(np.float64).tolist(), ids.tolist(),
                                       w.astype(np.float64).tolist(), E, bi.expert))
        assert np.isfinite(got).all() and np.abs(got).max() > 1.0
        assert np.abs(got - want).max() <= 1e-12 * np.abs(want).max(), kw


def test_stage_with_duplicate_and_invalid_ids_matches_loops():
    bi, x, _, w = _micro(seed=2, E=4, k=3)
    ids = np.array([[1, 1, 3], [-1, 2, 7], [0, 0, 0]], np.int32)
    got = R.moe_stage(x, ids, w, 4, bi.expert)
    want = np.array(LP.stage_loops(x.astype(np.float64).tolist(), ids.tolist(),
                                   w.astype(np.float64).tolist(), 4, bi.expert))
    assert np.abs(got - want).max() <= 1e-12 * np.abs(want).max()


def test_one_hot_single_token_is_textbook_swiglu_ffn():
    """M=1, one-hot router weight: out = W2^T (silu(W1^T x) * (W3^T x)),
    computed with torch's CPU float64 silu and matmul."""
    bi, x, _, _ = _micro(seed=3, E=8, H=128, I=64, M=1, k=4)
    ids = np.array([[5, 2, 7, 0]], np.int32)
    w = np.array([[0.0, 1.0, 0.0, 0.0]], np.float32)
    got = R.moe_stage(x, ids, w, 8, bi.expert)
    Wg, Wu, Wd = (torch.from_numpy(a) for a in R.expert_dense(bi.expert(2)))
    xt = torch.from_numpy(x.astype(np.float64))
    want = (torch.nn.functional.silu(xt @ Wg) * (xt @ Wu)) @ Wd
    np.testing.assert_allclose(got, want.numpy(), rtol=1e-12, atol=1e-12 * float(want.abs().max()))


def test_w2_reduce_exact_integer_case():
    """s = 1, z = 8, integer activations in {-1, 0, 1}: every output is an exact
    integer; compare with Python integer arithmetic."""
    E, H, I, M, k = 3, 64, 64, 2, 2
    rng = np.random.default_rng(7)
    bi = inputs.bank_inputs(4, E, H, I)
    bi.s_down[:] = np.float16(1.0)
    bi.z_down[:] = 8
    ids = np.array([[2, 0], [0, 1]], np.int32)
    route = R.route_compact(ids, E)
    act = rng.integers(-1, 2, size=(M * k, I)).astype(np.float64)
    wts = np.array([[1.0, 2.0], [-1.0, 3.0]], np.float32)
    got = R.w2_reduce(act, wts, route, k, bi.expert, M, H)
    want = [[0] * H for _ in range(M)]
    for r, slot in enumerate(route["sorted_slots"].tolist()):
        t, j = divmod(slot, k)
        e = int(ids[t][j])
        for n in range(H):
            y = sum(int(act[r][i]) * (int(bi.q_down[e][i][n]) - 8) for i in range(I))
            want[t][n] += int(wts[t][j]) * y
    np.testing.assert_array_equal(got, np.array(want, np.float64))


def test_silu_closed_forms():
    from scipy.special import expit
    g = np.array([-800.0, -30.0, -1.0, -1e-300, 0.0, 1e-300, 0.5, 20.0, 800.0])
    np.testing.assert_allclose(R.silu(g), g * expit(g), rtol=1e-15, atol=0)
    assert R.silu(np.array([0.0]))[0] == 0.0
    assert R.silu(np.array([800.0]))[0] == 800.0
    assert R.silu(np.array([-800.0]))[0] == 0.0


def test_stage_linear_in_router_weights_and_permutation_invariant():
    bi, x, ids, _ = _micro(seed=5, E=6, k=3, M=2)
    rng = np.random.default_rng(1)
    wa = rng.standard_normal(ids.shape).astype(np.float32)
    wb = rng.standard_normal(ids.shape).astype(np.float32)
    oa = R.moe_stage(x, ids, wa, 6, bi.expert)
    ob = R.moe_stage(x, ids, wb, 6, bi.expert)
    oab = R.moe_stage(x, ids, (wa.astype(np.float64) + wb).astype(np.float64), 6, bi.expert)
    np.testing.assert_allclose(oab, oa + ob, rtol=1e-12, atol=1e-12 * np.abs(oab).max())
    perm = np.array([2, 0, 1])
    op = R.moe_stage(x, ids[:, perm], wa[:, perm], 6, bi.expert)
    np.testing.assert_allclose(op, oa, rtol=1e-12, atol=1e-13 * np.abs(oa).max())
    # duplicate (e, w1), (e, w2) equals (e, w1 + w2)
    dup = np.array([[ids[0, 0], ids[0, 0], ids[0, 1]], [ids[1, 0], ids[1, 1], ids[1, 2]]], np.int32)
    wd = np.array([[0.25, 0.5, 1.0], [1.0, 1.0, 1.0]], np.float32)
    one = np.array([[ids[0, 0], ids[0, 1], ids[0, 2]], [ids[1, 0], ids[1, 1], ids[1, 2]]], np.int32)
    wo = np.array([[0.75, 1.0, 0.0], [1.0, 1.0, 1.0]], np.float32)
    np.testing.assert_allclose(R.moe_stage(x, dup, wd, 6, bi.expert), R.moe_stage(x, one, wo, 6, bi.expert),
                               rtol=1e-12, atol=1e-12 * np.abs(oa).max())


def test_invalid_ids_contribute_nothing():
    bi, x, ids, w = _micro(seed=6, E=5, k=2, M=2)
    bad = ids.copy()
    bad[1, 0] = 5
    wz = w.copy()
    wz[1, 0] = 0.0
    np.testing.assert_array_equal(R.moe_stage(x, bad, w, 5, bi.expert), R.moe_stage(x, ids, wz, 5, bi.expert))


# ---------------------------------------------------------------------------
# router selection, gates
# ---------------------------------------------------------------------------

def test_topk_softmax_brute_force_and_ties():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((4, 40)).astype(np.float32)
    logits[0, [3, 9, 17]] = 5.0                    # a three-way tie at the top
    logits[1, :] = 0.0                             # everything tied
    ids, w = R.topk_softmax(logits, 10)
    for t in range(4):
        order = sorted(range(40), key=lambda e: (-float(logits[t, e]), e))[:10]
        assert ids[t].tolist() == order
        v = [float(logits[t, e]) for e in order]
        m = max(v)
        p = [math.exp(a - m) for a in v]
        np.testing.assert_allclose(w[t], [a / sum(p) for a in p], rtol=1e-15)
    assert ids[0, :3].tolist() == [3, 9, 17]
    assert ids[1].tolist() == list(range(10))


def test_higham_gamma_closed_form():
    """gamma_n = n u / (1 - n u): n = 1 gives u / (1 - u), and it exceeds n u."""
    u = 2.0 ** -24
    assert R.higham_gamma(1) == u / (1.0 - u)
    assert R.higham_gamma(1000) == 1000 * u / (1.0 - 1000 * u)
    assert R.higham_gamma(1000) > 1000 * u
    assert R.higham_gamma(0) == 0.0


def test_gate_helper():
    ref = np.array([1.0, -2.0, 4.0])
    ok, _ = R.within_gate(ref + np.array([0.0, 0.001, 0.0]), ref)
    assert ok
    ok, _ = R.within_gate(ref + np.array([0.0, 0.1, 0.0]), ref)
    assert not ok
    tiny = np.full(4, 1e-6)
    assert R.within_gate(tiny + 2.0 ** -25, tiny)[0]
    assert not R.within_gate(tiny + 2.0 ** -20, tiny)[0]


@pytest.mark.parametrize("mistake", ["drop_zero", "swap_gate_up", "group_index", "transpose_down"])
def test_planted_oracle_mistakes_are_caught(mistake, monkeypatch):
    """Plant a plausible slip in the oracle and check that the scalar-loop pin fails."""
    bi, x, ids, w = _micro(seed=9, E=4, H=64, I=32, M=2, k=2)
    orig_dequant, orig_dense = R.dequant, R.expert_dense
    if mistake == "drop_zero":
        monkeypatch.setattr(R, "dequant", lambda q, s, z: orig_dequant(q, s, np.zeros_like(z)))
    elif mistake == "group_index":
        def bad(q, s, z):
            K = q.shape[0]
            g = (np.arange(K) // 16) % s.shape[0]
            return (q.astype(np.float64) - z.astype(np.float64)[g]) * s.astype(np.float64)[g]
        monkeypatch.setattr(R, "dequant", bad)
    elif mistake == "swap_gate_up":
        monkeypatch.setattr(R, "expert_dense", lambda ew: (lambda a: (a[1], a[0], a[2]))(orig_dense(ew)))
    elif mistake == "transpose_down":
        def tr(ew):
            Wg, Wu, Wd = orig_dense(ew)
            return Wg, Wu, Wd[::-1, :]
        monkeypatch.setattr(R, "expert_dense", tr)
    got = R.moe_stage(x, ids, w, 4, bi.expert)
    want = np.array(LP.stage_loops(x.astype(np.float64).tolist(), ids.tolist(),
                                   w.astype(np.float64).tolist(), 4, bi.expert))
    assert np.abs(got - want).max() > 1e-6 * np.abs(want).max()


def test_rms_norm_worked_values_and_closed_forms():
    """[3, 4] has mean square 12.5: [3, 4] / sqrt(12.5) = [0.848528137..., 1.131370849...];
    a constant row c maps to sign(c) / sqrt(1 + eps / c^2); a positive scale of
    the row changes the result only through eps."""
    got = R.rms_norm(np.array([[3.0, 4.0]], np.float16), eps=0.0)
    np.testing.assert_allclose(got, [[0.8485281374238570, 1.1313708498984760]], rtol=1e-15)
    got = R.rms_norm(np.full((1, 8), -2.0), eps=1e-6)
    np.testing.assert_allclose(got, np.full((1, 8), -1.0 / np.sqrt(1.0 + 1e-6 / 4.0)), rtol=1e-15)
    rng = np.random.default_rng(3)
    r = rng.standard_normal((3, 64))
    np.testing.assert_allclose(R.rms_norm(r * 8.0, eps=0.0), R.rms_norm(r, eps=0.0), rtol=1e-13)
    # every row of the output has mean square ms / (ms + eps)
    out = R.rms_norm(r, eps=1e-2)
    ms = (r * r).mean(axis=1)
    np.testing.assert_allclose((out * out).mean(axis=1), ms / (ms + 1e-2), rtol=1e-13)


def test_w2_rounding_bound_covers_a_float32_evaluation():
    """A plain fp32 evaluation (sequential sums in NumPy float32, then fp16)
    must fall inside the bound; the bound must not be vacuous (it is below
    the output magnitude for most elements)."""
    E, H, I, M, k = 6, 64, 64, 3, 4
    bi = inputs.bank_inputs(9, E, H, I)
    rng = inputs.call_rng(9, 1)
    ids = inputs.ids_distinct(rng, M, k, E)
    wts = inputs.router_weights(rng, M, k)
    route = R.route_compact(ids, E)
    act = rng.standard_normal((M * k, I)).astype(np.float16)
    bound, exact = R.w2_rounding_bound(act, wts, route, k, bi.expert, M, H)
    f32 = np.zeros((M, H), np.float32)
    for a in range(route["num_active"]):
        e = int(route["active_ids"][a])
        Wd = R.expert_dense(bi.expert(e))[2].astype(np.float32)
        for r in range(route["offsets"][a], route["offsets"][a + 1]):
            slot = int(route["sorted_slots"][r])
            acc = np.zeros(H, np.float32)
            for i in range(I):
                acc = acc + np.float32(act[r, i]) * Wd[i]
            f32[slot // k] = f32[slot // k] + np.float32(wts.reshape(-1)[slot]) * acc
    got = f32.astype(np.float16).astype(np.float64)
    assert np.all(np.abs(got - exact) <= bound)
    assert np.mean(bound < np.abs(exact)) > 0.9
