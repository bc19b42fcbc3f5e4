"""GPU parity over the whole record range the ABI admits, through the C ABI.

The records are {fp16 scale, u8 zero} (PR #522 "Coalesce AWQ QPN W13 compact
metadata loads...", Purpose); the ABI accepts any zero 0..255 and any finite
scale, including +-0, subnormals and negative values. Fork PR #12 "Add
opt-in native-g32 AWQ QPN M1 dispatch" (Numerical acceptance) checks kernels
against an independently decoded FP64 reference, with W2 checked on its own
intermediate. These cases drive every hot-path kernel form with such
records:

  * decode W13 + SwiGLU in both forms: lane pairs (M = 1 at the rank shape,
    one workgroup per CU) and single lanes (M = 8);
  * decode W2 + reduction in both forms: slot segments (inter 160) and the
    generic kernel (inter 2048);
  * prefill: the decode kernels (up to 64 tokens), the per-tile kernels
    (more than 1,024 slots at up to 64 tokens) and the wide kernels with
    both forms of the W13 weight ring;
  * 3-byte and 4-byte records (byte-identical outputs).

Two input families:
  "wide": zeros U{0..255}; scales with a random sign, 5 % +-0, 10 %
          subnormal, the rest |N(0,1)| * 0.002; three W13 K-groups carry
          scales in [32768, 65504], and the activations of exactly those
          groups are tiny subnormals (N(0,1) * 2^-22), so every result stays
          finite;
  "xmax": activations with |x| in [2^14, 65504] (the top of the fp16 range),
          W13 scales that are subnormal multiples 1..3 of 2^-24, zeros
          U{0..255}, W2 records "wide".
Gates: max|gpu - ref| <= 4e-3 max|ref| and ||gpu - ref|| / ||ref|| <= 2e-3.
"""

import numpy as np
import pytest

from awq_int4_mixture_amd import inputs
from oracle import ref as R
from tests.gpu_helpers import bank_case, f16_to_np, say, to_dev, torch_mod

pytestmark = pytest.mark.gpu

torch = torch_mod()
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from awq_int4_mixture_amd import abi  # noqa: E402  (fails loudly when the library is missing)

H, I = 2560, 160
BIG13 = (3, 40, 77)                      # W13 K-groups with scales near 65504
FAMILIES = {
    "wide": (("big_w13_groups", BIG13), ("kind", "wide")),
    "xmax": (("kind", "tiny"), ("kind_w2", "wide")),
}
FINITE_MARGIN = 60000.0                  # results of these inputs stay well inside fp16


def draw_x(family, rng, M, hidden, big=BIG13):
    if family == "wide":
        return inputs.activations_wide(rng, M, hidden, tiny_groups=big)
    return inputs.activations_near_max(rng, M, hidden)


def check(got, want, what):
    ok, e = R.within_gate(got, want)
    say(what, e)
    assert ok, (what, e)
    return e


def finite_inputs_precondition(act_ref, out_ref):
    assert np.abs(act_ref).max() < FINITE_MARGIN and np.abs(out_ref).max() < FINITE_MARGIN
    assert np.abs(out_ref).max() > 1.0


@pytest.mark.parametrize("family", ["wide", "xmax"])
@pytest.mark.parametrize("M", [1, 8])
@pytest.mark.parametrize("rb", [3, 4])
def test_decode_stages_wide_records(rb, M, family):
    """W13 + SwiGLU against the oracle (lane pairs at M = 1, single lanes at
    M = 8), W2 + reduction (slot segments, inter 160) on the GPU's own act,
    and the whole decode."""
    E, k = 64, 10
    dims, bank, bi = bank_case(301, E, H, I, rb, wide=FAMILIES[family])
    rng = inputs.call_rng(302, 10 * M + len(family))
    x = draw_x(family, rng, M, H)
    ids = inputs.ids_distinct(rng, 1, k, E) if M == 1 else inputs.ids_shared_pool(rng, M, k, E)
    w = inputs.router_weights(rng, M, k)
    say("decode wide records", family, "M", M, "rb", rb)
    route = R.route_compact(ids, E)
    V = route["num_valid"]
    act_ref = R.w13_swiglu_rows(x, route, k, bi.expert)
    out_ref = R.moe_stage(x, ids, w, E, bi.expert)
    finite_inputs_precondition(act_ref, out_ref)
    ws = abi.awq_moe_w13_swiglu(dims, bank, to_dev(x), to_dev(ids))
    torch.cuda.synchronize()
    act = f16_to_np(abi.workspace_act(ws, M, k, I))[route["sorted_slots"]]
    check(act[:V], act_ref[:V], f"w13 {family} M={M} rb={rb}")
    out = abi.awq_moe_w2_reduce(dims, bank, to_dev(ids), to_dev(w), ws)
    torch.cuda.synchronize()
    check(f16_to_np(out), R.w2_reduce(act, w, route, k, bi.expert, M, H), f"w2 own act {family} M={M} rb={rb}")
    bound, exact = R.w2_rounding_bound(act, w, route, k, bi.expert, M, H)
    frac = np.abs(f16_to_np(out).astype(np.float64) - exact) / np.maximum(bound, 1e-300)
    say(f"w2 rounding bound {family} M={M} rb={rb}: max |gpu - exact| / bound = {frac.max():.3f}")
    assert frac.max() <= 1.0
    full = abi.awq_moe_decode(dims, bank, to_dev(x), to_dev(ids), to_dev(w))
    torch.cuda.synchronize()
    check(f16_to_np(full), out_ref, f"decode {family} M={M} rb={rb}")


@pytest.mark.parametrize("family", ["wide", "xmax"])
def test_decode_wide_records_three_and_four_byte_identical(family):
    """PR #522 (Default switch): both record sizes give byte-identical outputs,
    here with records over the whole admitted range."""
    E, k = 64, 10
    d3, b3, _ = bank_case(301, E, H, I, 3, wide=FAMILIES[family])
    d4, b4, _ = bank_case(301, E, H, I, 4, wide=FAMILIES[family])
    for M in (1, 4, 8):
        rng = inputs.call_rng(303, M)
        x = to_dev(draw_x(family, rng, M, H))
        ids = to_dev(inputs.ids_shared_pool(rng, M, k, E))
        w = to_dev(inputs.router_weights(rng, M, k))
        a = f16_to_np(abi.awq_moe_decode(d3, b3, x, ids, w))
        b = f16_to_np(abi.awq_moe_decode(d4, b4, x, ids, w))
        torch.cuda.synchronize()
        assert a.view(np.uint16).tolist() == b.view(np.uint16).tolist(), (family, M)


@pytest.mark.parametrize("M", [1, 2])
def test_decode_wide_records_inter_2048(M):
    """The generic W2 kernel (inter > 1024: 64 K-groups, slots in passes) and
    the single-lane W13 kernel with wide records."""
    E, Hs, Is, k = 8, 512, 2048, 4
    big = (5,)
    dims, bank, bi = bank_case(304, E, Hs, Is, 3, wide=(("big_w13_groups", big), ("kind", "wide")))
    rng = inputs.call_rng(305, M)
    x = inputs.activations_wide(rng, M, Hs, tiny_groups=big)
    ids = inputs.ids_shared_pool(rng, M, k, E)
    w = inputs.router_weights(rng, M, k)
    say("decode wide records inter 2048 M", M)
    route = R.route_compact(ids, E)
    act_ref = R.w13_swiglu_rows(x, route, k, bi.expert)
    out_ref = R.moe_stage(x, ids, w, E, bi.expert)
    finite_inputs_precondition(act_ref, out_ref)
    ws = abi.awq_moe_w13_swiglu(dims, bank, to_dev(x), to_dev(ids))
    torch.cuda.synchronize()
    act = f16_to_np(abi.workspace_act(ws, M, k, Is))[route["sorted_slots"]]
    V = route["num_valid"]
    check(act[:V], act_ref[:V], f"w13 inter 2048 M={M}")
    out = abi.awq_moe_w2_reduce(dims, bank, to_dev(ids), to_dev(w), ws)
    torch.cuda.synchronize()
    check(f16_to_np(out), R.w2_reduce(act, w, route, k, bi.expert, M, Hs), f"w2 own act inter 2048 M={M}")
    full = abi.awq_moe_decode(dims, bank, to_dev(x), to_dev(ids), to_dev(w))
    torch.cuda.synchronize()
    check(f16_to_np(full), out_ref, f"decode inter 2048 M={M}")


@pytest.mark.parametrize("M", [1, 8])
@pytest.mark.parametrize("rb", [3, 4])
def test_w2_stage_scales_near_fp16_max_on_given_act(rb, M):
    """W2 records with scales in [32768, 65504] in K-group 2 (and wide
    records elsewhere), on an act the test writes: tiny subnormal values in
    that group's columns, fp16(4 N(0,1)) in the others."""
    E, k = 64, 10
    dims, bank, bi = bank_case(306, E, H, I, rb, wide=(("big_w2_groups", (2,)), ("kind", "wide")))
    rng = inputs.call_rng(307, M)
    ids = inputs.ids_distinct(rng, 1, k, E) if M == 1 else inputs.ids_shared_pool(rng, M, k, E)
    w = inputs.router_weights(rng, M, k)
    act = (rng.standard_normal((M * k, I)) * 4.0)
    act[:, 64:96] = rng.standard_normal((M * k, 32)) * 2.0 ** -22
    act = act.astype(np.float16)                                      # indexed by slot
    route = R.route_compact(ids, E)
    want = R.w2_reduce(act[route["sorted_slots"]], w, route, k, bi.expert, M, H)
    assert np.abs(want).max() < FINITE_MARGIN and np.abs(want).max() > 1.0
    ws = abi.awq_moe_w13_swiglu(dims, bank, to_dev(np.zeros((M, H), np.float16)), to_dev(ids))
    abi.workspace_act(ws, M, k, I).copy_(to_dev(act))
    out = abi.awq_moe_w2_reduce(dims, bank, to_dev(ids), to_dev(w), ws)
    torch.cuda.synchronize()
    say("w2 big scales on given act", M, rb)
    check(f16_to_np(out), want, f"w2 big scales M={M} rb={rb}")


@pytest.mark.parametrize("family", ["wide", "xmax"])
@pytest.mark.parametrize("M,k", [(40, 10), (40, 30), (128, 10), (300, 10)])
@pytest.mark.parametrize("rb", [3, 4])
def test_prefill_wide_records(rb, M, k, family):
    """Indexed prefill with wide records: the decode kernels at M = 40, the
    per-tile kernels at M = 40 with top-k 30 (1,200 slots, about 19 rows per
    expert), the wide kernels at M = 128 (about 20 rows: items of one or two
    row tiles, whose W13 weights take the unit ring) and M = 300 (about 47
    rows: three row tiles, the per-group ring), the matrix-core B operand
    (q - z) over zeros 0..255, and W2 with signed/zero/subnormal scales."""
    E = 64
    dims, bank, bi = bank_case(301, E, H, I, rb, wide=FAMILIES[family])
    rng = inputs.call_rng(308, M + len(family) + (1000 * k if k != 10 else 0))
    x = draw_x(family, rng, M, H)
    ids = inputs.ids_distinct(rng, M, k, E)
    w = inputs.router_weights(rng, M, k)
    say("prefill wide records", family, "M", M, "k", k, "rb", rb)
    out_ref = R.moe_stage(x, ids, w, E, bi.expert)
    assert np.abs(out_ref).max() < FINITE_MARGIN
    out = abi.awq_moe_prefill(dims, bank, to_dev(x), to_dev(ids), to_dev(w))
    torch.cuda.synchronize()
    check(f16_to_np(out), out_ref, f"prefill {family} M={M} k={k} rb={rb}")
