"""GPU parity of the layer-stack support: the router (top-k + softmax), the
residual/RMS-norm step, and a teacher-forced check of a short stack of
512-expert layers built from banks drawn on the device."""

import numpy as np
import pytest

from awq_int4_mixture_amd import inputs
from oracle import layout as OL
from oracle import ref as R
from tests.gpu_helpers import f16_to_np, say, to_dev, torch_mod

pytestmark = pytest.mark.gpu

torch = torch_mod()
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from awq_int4_mixture_amd import abi  # noqa: E402


def router_check(logits, k):
    ids, w = abi.awq_moe_router_topk(to_dev(logits), k)
    torch.cuda.synchronize()
    want_ids, want_w = R.topk_softmax(logits, k)
    np.testing.assert_array_equal(ids.cpu().numpy(), want_ids)
    got_w = w.cpu().numpy().astype(np.float64)
    finite = np.isfinite(want_w)
    np.testing.assert_allclose(got_w[finite], want_w[finite], rtol=1e-5, atol=1e-7)
    assert np.array_equal(np.isnan(got_w), np.isnan(want_w))


@pytest.mark.parametrize("M", [1, 3, 8])
def test_router_matches_oracle(M):
    rng = inputs.call_rng(500, M)
    router_check(inputs.router_logits(rng, M, 512), 10)


@pytest.mark.parametrize("E,k", [(32, 1), (512, 10), (512, 32), (4096, 32), (16, 16), (100, 7)])
def test_router_ties_and_special_values(E, k):
    rng = inputs.call_rng(501, E + k)
    M = 8
    lg = rng.integers(-2, 3, size=(M, E)).astype(np.float32)      # many exact ties
    lg[0, ::3] = -0.0
    lg[1, 5:9] = 0.0
    lg[1, 9:11] = -0.0
    lg[2, :] = -np.inf
    lg[2, E // 2] = 1.0
    lg[3, ::5] = np.nan
    lg[4, :] = 3.0                                                  # all equal: ids 0..k-1
    lg[5, -1] = np.inf
    say("router ties", E, k)
    router_check(lg, k)


def test_router_nan_row_selected_last():
    """With fewer numbers than k, NaN logits fill the tail by ascending id."""
    lg = np.full((1, 16), np.nan, np.float32)
    lg[0, 3] = 1.0
    lg[0, 11] = 2.0
    ids, _ = abi.awq_moe_router_topk(to_dev(lg), 4)
    torch.cuda.synchronize()
    assert ids.cpu().numpy().tolist() == [[11, 3, 0, 1]]


def test_residual_rmsnorm():
    rng = inputs.call_rng(502, 0)
    M, H = 8, 2560
    r = (rng.standard_normal((M, H)) * 3).astype(np.float16)
    d = rng.standard_normal((M, H)).astype(np.float16)
    r_next, x = abi.awq_moe_residual_rmsnorm(to_dev(r), to_dev(d))
    torch.cuda.synchronize()
    want_r = (r.astype(np.float32) + d.astype(np.float32)).astype(np.float16)   # fp32 add, one rounding
    np.testing.assert_array_equal(f16_to_np(r_next).view(np.uint16), want_r.view(np.uint16))
    want_x = R.rms_norm(want_r)
    got_x = f16_to_np(x).astype(np.float64)
    assert np.max(np.abs(got_x - want_x) / np.maximum(np.abs(want_x), 2.0 ** -14)) <= 2.0 ** -10
    r2, x2 = abi.awq_moe_residual_rmsnorm(to_dev(r))                 # no delta: r_next = r
    torch.cuda.synchronize()
    np.testing.assert_array_equal(f16_to_np(r2).view(np.uint16), r.view(np.uint16))
    assert np.max(np.abs(f16_to_np(x2) - R.rms_norm(r)) / np.maximum(np.abs(R.rms_norm(r)), 2.0 ** -14)) <= 2.0 ** -10


@pytest.mark.parametrize("E,H,k", [(512, 2560, 10), (4096, 256, 32), (64, 8192, 4)])
def test_router_residual_equals_the_two_calls(E, H, k):
    rng = inputs.call_rng(504, E + H)
    M = 8
    logits = to_dev(inputs.router_logits(rng, M, E))
    r = to_dev((rng.standard_normal((M, H)) * 2).astype(np.float16))
    d = to_dev(rng.standard_normal((M, H)).astype(np.float16))
    ids1, w1 = abi.awq_moe_router_topk(logits, k)
    rn1, x1 = abi.awq_moe_residual_rmsnorm(r, d)
    ids2, w2, rn2, x2 = abi.awq_moe_router_residual(logits, k, r, d)
    torch.cuda.synchronize()
    for a, b in ((ids1, ids2), (w1, w2), (rn1, rn2), (x1, x2)):
        assert torch.equal(a.view(torch.uint8) if a.dtype != torch.int32 else a,
                           b.view(torch.uint8) if b.dtype != torch.int32 else b)


@pytest.mark.parametrize("M,H,E", [(8, 2560, 512), (3, 256, 64), (1, 4096, 130), (5, 8192, 37), (2, 6144, 9),
                                   (7, 560, 513)])
def test_router_gemv(M, H, E):
    """The residual step bit-identical to awq_moe_residual_rmsnorm; logits
    against float64 x . W^T on the GPU's own x. The fp32 sums form a tree of
    depth well under 100 (a chain over each thread's runs, then lane and wave
    sums), so |err| <= gamma_100 * sum |x w| < 1e-5 * sum |x w| (Higham's
    bound for a summation tree; fp16 products are exact in fp32). The top-k
    of the GPU's logits equals the oracle's top-k of them."""
    rng = inputs.call_rng(505, M * H + E)
    r = to_dev((rng.standard_normal((M, H)) * 2).astype(np.float16))
    d = to_dev(rng.standard_normal((M, H)).astype(np.float16))
    wr_np = (rng.standard_normal((E, H)) / np.sqrt(H)).astype(np.float16)
    rn, x, logits = abi.awq_moe_router_gemv(r, to_dev(wr_np), d)
    rn1, x1 = abi.awq_moe_residual_rmsnorm(r, d)
    torch.cuda.synchronize()
    assert torch.equal(rn.view(torch.int16), rn1.view(torch.int16)) and torch.equal(x.view(torch.int16), x1.view(torch.int16))
    x64 = f16_to_np(x).astype(np.float64)
    w64 = wr_np.astype(np.float64)
    want = x64 @ w64.T
    mag = np.abs(x64) @ np.abs(w64).T
    got = logits.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - want) <= 1e-5 * mag + 1e-30), np.max(np.abs(got - want) / mag)
    k = min(10, E)
    ids, w = abi.awq_moe_router_topk(logits, k)
    torch.cuda.synchronize()
    want_ids, want_w = R.topk_softmax(logits.cpu().numpy(), k)
    np.testing.assert_array_equal(ids.cpu().numpy(), want_ids)
    np.testing.assert_allclose(w.cpu().numpy().astype(np.float64), want_w, rtol=1e-5, atol=1e-7)


def experts_from_bank(d, bank_np):
    """weights_of(e) for the oracle, decoded by the oracle from the bank bytes."""
    cache = {}

    def weights_of(e):
        if e not in cache:
            de = OL.decode_expert(d, bank_np, e)
            cache[e] = inputs.ExpertWeights(de.q13[:, 0::2], de.q13[:, 1::2], de.q2, de.s13[:, 0::2],
                                            de.s13[:, 1::2], de.s2, de.z13[:, 0::2], de.z13[:, 1::2], de.z2)
        return cache[e]
    return weights_of


def test_stack_teacher_forced_four_layers():
    """Four 512-expert layers, M = 8, 3-byte records: the GPU chain (router,
    residual/norm, decode) is checked layer by layer against the oracle on
    the GPU's own layer input."""
    E, H, I, K, M, RB, layers = 512, 2560, 160, 10, 8, 3, 4
    dims = abi.make_dims(E, H, I, RB)
    Lq = abi.awq_moe_bank_layout_query(dims)
    G13, G2 = H // 32, I // 32
    sections = [(int(Lq.w13_meta_off), G13 * 2 * I), (int(Lq.w2_meta_off), G2 * H)]
    d = OL.Dims(E, H, I, RB)
    rng = inputs.call_rng(503, 0)
    r = to_dev(inputs.activations(rng, M, H))
    dec = None
    for layer in range(layers):
        bank = inputs.device_bank(7000 + layer, E, sections, int(Lq.expert_bytes), RB)
        if dec is None:
            dec = abi.Decoder(dims, bank, K, max_tokens=M)
        dec.bank = bank
        logits = inputs.router_logits(rng, M, E)
        ids, w, r_next, x = abi.awq_moe_router_residual(to_dev(logits), K, r, None if layer == 0 else out)
        out = dec(x, ids, w)
        torch.cuda.synchronize()
        want_ids, want_w = R.topk_softmax(logits, K)
        np.testing.assert_array_equal(ids.cpu().numpy(), want_ids)
        x_np = f16_to_np(x)
        want = R.moe_stage(x_np, want_ids, w.cpu().numpy(), E, experts_from_bank(d, bank.cpu().numpy()))
        ok, e = R.within_gate(f16_to_np(out), want)
        say("stack layer", layer, e)
        assert ok, (layer, e)
        r = r_next


@pytest.mark.parametrize("E,H,I,k,M,rb", [
    (64, 2560, 160, 10, 1, 3),     # W13 lane pairs with the norm, W2 slot segments with the residual
    (64, 2560, 160, 10, 8, 4),     # single-lane W13 with the norm
    (64, 2560, 160, 10, 3, 3),
    (6, 8192, 32, 3, 2, 3),        # hidden 8192: 16 waves of squares
    (8, 512, 2048, 4, 2, 3),       # the generic W2 kernel (inter > 1024) with the residual
    (12, 4096, 64, 2, 1, 4),       # lane pairs at their largest block (16 waves)
    (12, 1024, 320, 6, 3, 3),      # W2 with one slot per wave (inter 320) with the residual
    (8, 512, 768, 4, 2, 4),        # W2 with two groups per lane (inter 768) with the residual
])
def test_decode_rmsnorm_residual_against_oracle_and_separate_calls(E, H, I, k, M, rb):
    """awq_moe_decode_rmsnorm_residual(r): the update r_next - r is within
    the gate of the float64 oracle's moe_stage(r / rms(r)) (x unrounded, as
    the fused layer applies the norm to the fp32 column sums), and within
    the gate of the separate chain residual_rmsnorm -> decode -> residual
    (which rounds x to fp16); the stage on a scaled row (r * 2^k, the same x)
    gives the same update up to the fp16 rounding of r_next."""
    from tests.gpu_helpers import bank_case
    dims, bank, bi = bank_case(510 + H, E, H, I, rb)
    rng = inputs.call_rng(511, H + I + M)
    r = (rng.standard_normal((M, H)) * 3).astype(np.float16)
    ids = inputs.ids_shared_pool(rng, M, k, E) if k <= E else rng.integers(0, E, size=(M, k)).astype(np.int32)
    w = inputs.router_weights(rng, M, k)
    rd, idd, wd = to_dev(r), to_dev(ids), to_dev(w)
    say("fused layer", E, H, I, k, M, rb)
    _, x = abi.awq_moe_residual_rmsnorm(rd)
    out = abi.awq_moe_decode(dims, bank, x, idd, wd)
    sep_rn, _ = abi.awq_moe_residual_rmsnorm(rd, out)
    rn = abi.awq_moe_decode_rmsnorm_residual(dims, bank, rd, idd, wd)
    torch.cuda.synchronize()
    r64 = r.astype(np.float64)
    upd = f16_to_np(rn).astype(np.float64) - r64
    want = R.moe_stage(R.rms_norm(r), ids, w, E, bi.expert)
    ok, e = R.within_gate(upd, want)
    say("fused layer vs oracle (the update r_next - r)", e)
    assert ok, e
    ok, e = R.within_gate(upd, f16_to_np(sep_rn).astype(np.float64) - r64)
    say("fused layer vs the separate chain", e)
    assert ok, e
    # scale invariance of the norm: r * 4 gives the same stage output (eps aside)
    rn4 = abi.awq_moe_decode_rmsnorm_residual(dims, bank, to_dev((r.astype(np.float32) * 4).astype(np.float16)),
                                              idd, wd)
    torch.cuda.synchronize()
    upd4 = f16_to_np(rn4).astype(np.float64) - r64 * 4
    ok, e = R.within_gate(upd4, want)
    assert ok, ("scaled row", e)


def test_router_rows_of_many_layers_in_one_call():
    """The top-k of 48 layers x 8 tokens in one call (rows are independent)
    equals the per-layer calls and the oracle."""
    rng = inputs.call_rng(512, 0)
    lg = inputs.router_logits(rng, 48 * 8, 512)
    ids, w = abi.awq_moe_router_topk(to_dev(lg), 10)
    torch.cuda.synchronize()
    want_ids, want_w = R.topk_softmax(lg, 10)
    np.testing.assert_array_equal(ids.cpu().numpy(), want_ids)
    np.testing.assert_allclose(w.cpu().numpy().astype(np.float64), want_w, rtol=1e-5, atol=1e-7)
    for layer in (0, 17, 47):
        i1, w1 = abi.awq_moe_router_topk(to_dev(lg[8 * layer:8 * layer + 8]), 10)
        torch.cuda.synchronize()
        assert torch.equal(i1, ids[8 * layer:8 * layer + 8]) and torch.equal(w1, w[8 * layer:8 * layer + 8])


def test_stack_fused_layers_teacher_forced():
    """Four 512-expert layers, M = 8, 3-byte records, in the benchmark's
    chain: every layer's top-k in one router call, then one fused layer call
    per layer (norm in W13, residual in W2). Each layer is checked against
    the oracle on the GPU's own residual input."""
    E, H, I, K, M, RB, layers = 512, 2560, 160, 10, 8, 3, 4
    dims = abi.make_dims(E, H, I, RB)
    Lq = abi.awq_moe_bank_layout_query(dims)
    sections = [(int(Lq.w13_meta_off), (H // 32) * 2 * I), (int(Lq.w2_meta_off), (I // 32) * H)]
    d = OL.Dims(E, H, I, RB)
    rng = inputs.call_rng(513, 0)
    r = to_dev(inputs.activations(rng, M, H))
    logits = inputs.router_logits(rng, layers * M, E)
    ids_all, w_all = abi.awq_moe_router_topk(to_dev(logits), K)
    ws = abi.alloc_workspace(dims, M, K, "cuda")
    for layer in range(layers):
        bank = inputs.device_bank(7100 + layer, E, sections, int(Lq.expert_bytes), RB)
        ids, w = ids_all[layer * M:(layer + 1) * M], w_all[layer * M:(layer + 1) * M]
        rn = abi.awq_moe_decode_rmsnorm_residual(dims, bank, r, ids, w, workspace=ws)
        torch.cuda.synchronize()
        r_np = f16_to_np(r)
        want_ids, _ = R.topk_softmax(logits[layer * M:(layer + 1) * M], K)
        np.testing.assert_array_equal(ids.cpu().numpy(), want_ids)
        upd = R.moe_stage(R.rms_norm(r_np), want_ids, w.cpu().numpy(), E, experts_from_bank(d, bank.cpu().numpy()))
        ok, e = R.within_gate(f16_to_np(rn).astype(np.float64) - r_np.astype(np.float64), upd)
        say("fused stack layer", layer, e)
        assert ok, (layer, e)
        r = rn


@pytest.mark.parametrize("M", [1, 8])   # W13 lane pairs / single lanes with the norm
def test_norm_zero_row_at_the_smallest_eps(M):
    """eps = 2^-126, the smallest the entry points admit, on a row of zeros:
    1/rms comes from the hardware reciprocal square root of eps itself, so
    the row's update is exactly zero (no inf or NaN); the other rows match
    the oracle with the same eps, and awq_moe_residual_rmsnorm gives x = 0
    for the zero row."""
    from tests.gpu_helpers import bank_case
    E, H, I, k, rb = 64, 2560, 160, 10, 3
    eps = 2.0 ** -126
    dims, bank, bi = bank_case(530 + M, E, H, I, rb)
    rng = inputs.call_rng(531, M)
    r = (rng.standard_normal((M, H)) * 3).astype(np.float16)
    r[0] = 0
    ids = inputs.ids_shared_pool(rng, M, k, E)
    w = inputs.router_weights(rng, M, k)
    say("zero row, eps 2^-126", M)
    rn = abi.awq_moe_decode_rmsnorm_residual(dims, bank, to_dev(r), to_dev(ids), to_dev(w), eps=eps)
    r2, x = abi.awq_moe_residual_rmsnorm(to_dev(r), eps=eps)
    torch.cuda.synchronize()
    got = f16_to_np(rn)
    assert np.all(np.isfinite(got))
    assert not got[0].any()
    assert not f16_to_np(x)[0].any() and np.all(np.isfinite(f16_to_np(x)))
    if M > 1:
        upd = got[1:].astype(np.float64) - r[1:].astype(np.float64)
        want = R.moe_stage(R.rms_norm(r[1:], eps=eps), ids[1:], w[1:], E, bi.expert)
        ok, e = R.within_gate(upd, want)
        assert ok, e
