"""GPU parity of the HIP path against the float64 oracle, through the C ABI.

Integer work (routing arrays, dequantised fp32 weights) must match bit for
bit; floating outputs must satisfy max|gpu - ref| <= 4e-3 max|ref| and
||gpu - ref|| / ||ref|| <= 2e-3.
"""

import itertools

import numpy as np
import pytest

from awq_int4_mixture_amd import inputs
from oracle import ref as R
from tests.gpu_helpers import bank_case, exact_in_fp32, f16_to_np, say, to_dev, torch_mod

pytestmark = pytest.mark.gpu

torch = torch_mod()
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from awq_int4_mixture_amd import abi  # noqa: E402  (fails loudly when the library is missing)

RANK = (2560, 160)
TINY = (256, 32)


def oracle_route(ids, E):
    return R.route_compact(ids, E)


def gpu_route(ids, E):
    r = abi.awq_moe_route_compact(to_dev(ids), E)
    torch.cuda.synchronize()
    return {k: getattr(r, k).cpu().numpy() for k in
            ("active_expert_ids", "active_expert_offsets", "sorted_slots", "num_active", "status")}, r


def assert_route_equal(g, o):
    assert g["active_expert_ids"].tolist() == o["active_ids"].tolist()
    assert g["active_expert_offsets"].tolist() == o["offsets"].tolist()
    assert g["sorted_slots"].tolist() == o["sorted_slots"].tolist()
    assert int(g["num_active"][0]) == o["num_active"]
    assert int(g["status"][0]) == o["status"]


# ---------------------------------------------------------------------------
# integer work: dequantised weights and routing arrays, bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("rb", [3, 4])
@pytest.mark.parametrize("shape", [TINY, RANK])
def test_dequant_bit_exact(rb, shape):
    H, I = shape
    say("dequant", rb, shape)
    dims, bank, bi = bank_case(31, 6, H, I, rb, 256)
    for which in (0, 1):
        got = abi.awq_moe_dequant(dims, bank, 1, 4, which).cpu().numpy()
        for el in range(4):
            w = bi.expert(1 + el)
            want = R.w13_interleaved(w) if which == 0 else R.dequant(w.q_down, w.s_down, w.z_down)
            assert exact_in_fp32(want)
            np.testing.assert_array_equal(got[el], want.astype(np.float32))


def test_route_exhaustive_small():
    """Every id tensor with E=4, k=2, M=1..3."""
    say("route exhaustive")
    for M in (1, 2, 3):
        for flat in itertools.product(range(4), repeat=2 * M):
            ids = np.array(flat, np.int32).reshape(M, 2)
            g, _ = gpu_route(ids, 4)
            assert_route_equal(g, oracle_route(ids, 4))


def test_route_random_and_edges():
    rng = np.random.default_rng(4)
    cases = []
    for _ in range(150):
        M = int(rng.integers(1, 9))
        k = int(rng.integers(1, 33))
        E = int(rng.integers(1, 1024))
        cases.append((rng.integers(-3, E + 3, size=(M, k)).astype(np.int32), E))
    cases += [
        (np.full((8, 32), 7, np.int32), 512),                 # one expert takes every slot (256 rows)
        (np.full((8, 32), -1, np.int32), 512),                # every id invalid
        (np.arange(256, dtype=np.int32).reshape(8, 32), 256),  # all distinct, max slots
        (np.array([[511, 0, 255, 256, 1, 510, 2, 509, 3, 508]], np.int32), 512),
    ]
    for ids, E in cases:
        say("route", ids.shape, E)
        g, _ = gpu_route(ids, E)
        assert_route_equal(g, oracle_route(ids, E))


# ---------------------------------------------------------------------------
# stages and the whole decode
# ---------------------------------------------------------------------------

def run_decode(dims, bank, x, ids, w):
    out = abi.awq_moe_decode(dims, bank, to_dev(x), to_dev(ids), to_dev(w))
    torch.cuda.synchronize()
    return f16_to_np(out)


def check(got, want, what):
    ok, e = R.within_gate(got, want)
    say(what, e)
    assert ok, (what, e)
    return e


@pytest.mark.parametrize("rb", [3, 4])
@pytest.mark.parametrize("M", [1, 2, 8])
def test_w13_stage_and_w2_stage_pair(rb, M):
    """W13+SwiGLU against the oracle; W2+reduction checked on the GPU's own
    intermediate (fork PR #12, Numerical acceptance)."""
    H, I = RANK
    dims, bank, bi = bank_case(7, 64, H, I, rb)
    rng = inputs.call_rng(7, 100 + M)
    x = inputs.activations(rng, M, H)
    ids = inputs.ids_shared_pool(rng, M, 10, 64)
    w = inputs.router_weights(rng, M, 10)
    route_o = oracle_route(ids, 64)
    ws = abi.awq_moe_w13_swiglu(dims, bank, to_dev(x), to_dev(ids))
    torch.cuda.synchronize()
    V = route_o["num_valid"]
    act_sorted = f16_to_np(abi.workspace_act(ws, M, 10, I))[route_o["sorted_slots"]]   # by slot -> sorted rows
    act_ref = R.w13_swiglu_rows(x, route_o, 10, bi.expert)
    check(act_sorted[:V], act_ref[:V], f"w13 M={M} rb={rb}")
    out = abi.awq_moe_w2_reduce(dims, bank, to_dev(ids), to_dev(w), ws)
    torch.cuda.synchronize()
    out_ref = R.w2_reduce(act_sorted, w, route_o, 10, bi.expert, M, H)
    check(f16_to_np(out), out_ref, f"w2 on own act M={M} rb={rb}")
    # informational rounding bound of the W2 step on its own act
    bound, exact = R.w2_rounding_bound(act_sorted, w, route_o, 10, bi.expert, M, H)
    frac = np.abs(f16_to_np(out).astype(np.float64) - exact) / bound
    say(f"w2 rounding bound M={M} rb={rb}: max |gpu - exact| / bound = {frac.max():.3f}")
    assert frac.max() <= 1.0


@pytest.mark.parametrize("rb", [3, 4])
def test_tiny_config(rb):
    """E=16, top-k 2, hidden 256, inter 32, M=1."""
    dims, bank, bi = bank_case(1, 16, 256, 32, rb)
    for c in range(4):
        rng = inputs.call_rng(1, c)
        x = inputs.activations(rng, 1, 256)
        ids = inputs.ids_distinct(rng, 1, 2, 16)
        w = inputs.router_weights(rng, 1, 2)
        check(run_decode(dims, bank, x, ids, w), R.moe_stage(x, ids, w, 16, bi.expert), f"tiny rb={rb} c={c}")


@pytest.mark.parametrize("rb", [3, 4])
@pytest.mark.parametrize("M,mode", [(1, "distinct"), (2, "pool"), (4, "pool"), (8, "pool"), (8, "all"),
                                    (3, "pool"), (5, "distinct")])
def test_decode_rank_shape(rb, M, mode):
    H, I = RANK
    dims, bank, bi = bank_case(7, 128, H, I, rb)
    rng = inputs.call_rng(8, M * 10 + len(mode))
    x = inputs.activations(rng, M, H)
    draw = {"distinct": inputs.ids_distinct, "pool": inputs.ids_shared_pool, "all": inputs.ids_all_distinct}[mode]
    ids = draw(rng, M, 10, 128)
    w = inputs.router_weights(rng, M, 10)
    check(run_decode(dims, bank, x, ids, w), R.moe_stage(x, ids, w, 128, bi.expert), f"rank M={M} {mode} rb={rb}")


@pytest.mark.parametrize("E,H,I,k,M", [
    (8, 512, 2048, 10, 2),     # W2: 256 lanes per slot, 4 slots per pass -> 3 passes
    (16, 256, 32, 32, 8),      # top-k 32, 256 slots; 4 lanes per slot
    (6, 96, 64, 3, 5),         # hidden 96: 6 column tiles
    (12, 128, 96, 1, 3),       # top-k 1
    (10, 512, 128, 7, 3),      # W2: 16 lanes per slot, 4 slots per wave
    (9, 256, 256, 5, 2),       # W2: 32 lanes per slot, 2 slots per wave
    (7, 160, 224, 3, 4),       # W2: 28 lanes per slot, 2 slots per wave, hidden 160
    (6, 4096, 64, 2, 1),       # W13 lane pairs at their largest block: 1024 threads, 16 waves
    (5, 8192, 32, 3, 1),       # M = 1 but hidden 8192: pairs would need 2048 threads, single-lane W13
    (64, 2560, 160, 10, 8),    # a token whose ids are all invalid, next to valid ones
    (4096, 256, 32, 32, 8),    # 4096 experts, top-k 32, M = 8: 256 slots, expert offsets past 32 MB
    (24, 2560, 320, 10, 8),    # W2: 40 lanes per slot, one slot per wave (inter 320)
    (24, 2560, 320, 10, 1),
    (12, 512, 512, 16, 3),     # W2: 64 lanes per slot, one per wave, 16 waves (its largest block)
    (12, 512, 512, 17, 2),     # ... one slot more than 16 waves hold: the generic W2 kernel
    (10, 256, 288, 4, 5),      # W2: 36 lanes per slot (nine groups), one per wave
    (8, 512, 640, 6, 3),       # inter 640: one slot per wave, two groups on the first 16 lanes
    (6, 256, 544, 5, 3),       # inter 544: 17 groups, a second group on 4 lanes only
    (8, 512, 1024, 16, 2),     # inter 1024: two groups on every lane, 16 waves
    (8, 512, 1024, 17, 2),     # ... one slot more: the generic W2 kernel
])
def test_decode_other_shapes(E, H, I, k, M):
    dims, bank, bi = bank_case(40 + I, E, H, I, 3)
    rng = inputs.call_rng(41, H + k)
    x = inputs.activations(rng, M, H)
    ids = inputs.ids_shared_pool(rng, M, k, E) if k <= E else rng.integers(0, E, size=(M, k)).astype(np.int32)
    if E == 64:
        ids[3, :] = -7
    w = inputs.router_weights(rng, M, k)
    say("other shape", E, H, I, k, M)
    got = run_decode(dims, bank, x, ids, w)
    want = R.moe_stage(x, ids, w, E, bi.expert)
    if E == 64:
        assert not got[3].any()
    check(got, want, f"shape E={E} H={H} I={I} k={k} M={M}")


def test_decode_largest_hidden_and_inter_together():
    """Hidden 8192 with inter 2048, the admitted maxima together, top-k 32
    over 4 experts (each token routes to every expert several times), M = 2:
    the single-lane W13 kernel at its 16 waves and the W2 kernel for
    inter > 1024 at their largest strides."""
    E, H, I, k, M = 4, 8192, 2048, 32, 2
    dims, bank, bi = bank_case(90, E, H, I, 3)
    rng = inputs.call_rng(91, 0)
    x = inputs.activations(rng, M, H)
    ids = rng.integers(0, E, size=(M, k)).astype(np.int32)
    w = inputs.router_weights(rng, M, k)
    say("largest hidden and inter", E, H, I, k, M)
    check(run_decode(dims, bank, x, ids, w), R.moe_stage(x, ids, w, E, bi.expert), "largest hidden and inter")


def test_decode_full_bank_rank_shape_m1_and_m8():
    """The benchmark's layer: E=512, hidden 2560, inter 160, top-k 10, 3-byte records."""
    H, I = RANK
    dims, bank, bi = bank_case(2026, 512, H, I, 3)
    for M in (1, 8):
        rng = inputs.call_rng(2026, M)
        x = inputs.activations(rng, M, H)
        ids = inputs.ids_shared_pool(rng, M, 10, 512) if M > 1 else inputs.ids_distinct(rng, 1, 10, 512)
        w = inputs.router_weights(rng, M, 10)
        check(run_decode(dims, bank, x, ids, w), R.moe_stage(x, ids, w, 512, bi.expert), f"full E512 M={M}")


def test_duplicate_and_invalid_ids_and_status():
    H, I = RANK
    dims, bank, bi = bank_case(7, 64, H, I, 3)
    rng = inputs.call_rng(9, 0)
    M, k = 3, 10
    x = inputs.activations(rng, M, H)
    w = inputs.router_weights(rng, M, k)
    ids = inputs.ids_distinct(rng, M, k, 64)
    ids[0, 3] = ids[0, 1]          # duplicate inside one token
    ids[1, :] = 5                  # every slot of a token on one expert
    ids[2, 4] = 64                 # out of range
    ids[2, 7] = -1
    dec = abi.Decoder(dims, bank, k)
    out = dec(to_dev(x), to_dev(ids), to_dev(w))
    torch.cuda.synchronize()
    check(f16_to_np(out), R.moe_stage(x, ids, w, 64, bi.expert), "dup/invalid")
    assert dec.status() == abi.STATUS_BAD_ID
    ok_ids = inputs.ids_distinct(rng, M, k, 64)
    dec(to_dev(x), to_dev(ok_ids), to_dev(w))
    assert dec.status() == 0


def test_three_and_four_byte_records_give_identical_bytes():
    """PR #522 (Default switch): outputs of the two layouts are byte-identical."""
    H, I = RANK
    _, b3, _ = bank_case(7, 64, H, I, 3)
    d3 = abi.make_dims(64, H, I, 3)
    _, b4, _ = bank_case(7, 64, H, I, 4)
    d4 = abi.make_dims(64, H, I, 4)
    for M in (1, 4, 8):
        rng = inputs.call_rng(10, M)
        x = inputs.activations(rng, M, H)
        ids = inputs.ids_shared_pool(rng, M, 10, 64)
        w = inputs.router_weights(rng, M, 10)
        a = run_decode(d3, b3, x, ids, w)
        b = run_decode(d4, b4, x, ids, w)
        assert a.view(np.uint16).tolist() == b.view(np.uint16).tolist()


# ---------------------------------------------------------------------------
# exact cases and invariants (bit-exact on the GPU)
# ---------------------------------------------------------------------------

def test_w2_exact_integer_case_bit_exact():
    """s = 1, z = 8, act in {-1, 0, 1}, weights 1: every value is an integer with
    |y| <= 2048, so fp32 accumulation and the fp16 output are exact."""
    H, I, E = 2560, 160, 16
    bi = inputs.bank_inputs(12, E, H, I)
    bi.s_down[:] = np.float16(1.0)
    bi.z_down[:] = 8
    dims = abi.make_dims(E, H, I, 3)
    bank = to_dev(abi.prepare_from_inputs(dims, bi))
    rng = np.random.default_rng(5)
    M, k = 2, 10
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(M)]).astype(np.int32)
    w = np.zeros((M, k), np.float32)
    w[:, 0] = 1.0
    route_o = oracle_route(ids, E)
    act = rng.integers(-1, 2, size=(M * k, I)).astype(np.float16)      # indexed by slot
    ws = abi.awq_moe_w13_swiglu(dims, bank, to_dev(np.zeros((M, H), np.float16)), to_dev(ids))
    abi.workspace_act(ws, M, k, I).copy_(to_dev(act))                  # replace the intermediate
    out = abi.awq_moe_w2_reduce(dims, bank, to_dev(ids), to_dev(w), ws)
    torch.cuda.synchronize()
    want = R.w2_reduce(act[route_o["sorted_slots"]], w, route_o, k, bi.expert, M, H)
    assert np.abs(want).max() <= 2048 and np.array_equal(want, np.round(want))
    np.testing.assert_array_equal(f16_to_np(out).astype(np.float64), want)


def test_invariants_bit_exact():
    H, I = RANK
    dims, bank, bi = bank_case(7, 64, H, I, 3)
    rng = inputs.call_rng(11, 0)
    M, k = 4, 10
    x = inputs.activations(rng, M, H)
    ids = inputs.ids_shared_pool(rng, M, k, 64)
    w = inputs.router_weights(rng, M, k)
    base = run_decode(dims, bank, x, ids, w)
    # run to run (PR #520 addendum: same-arm teacher-forced A/A was exact)
    assert run_decode(dims, bank, x, ids, w).view(np.uint16).tolist() == base.view(np.uint16).tolist()
    # permuting a token's (id, weight) pairs
    perm = rng.permutation(k)
    p = run_decode(dims, bank, x, ids[:, perm], w[:, perm])
    assert p.view(np.uint16).tolist() == base.view(np.uint16).tolist()
    # power-of-two scaling of the router weights scales the output exactly
    s = run_decode(dims, bank, x, ids, (w * np.float32(0.25)).astype(np.float32))
    assert np.array_equal(s.astype(np.float64) * 4, base.astype(np.float64)) or \
        np.abs(s.astype(np.float64) * 4 - base).max() <= 2.0 ** -14 * 4
    # zero weights give +0, zero activations give 0
    z = run_decode(dims, bank, x, ids, np.zeros_like(w))
    assert not z.view(np.uint16).any()
    z2 = run_decode(dims, bank, np.zeros_like(x), ids, w)
    assert not (z2.astype(np.float64) != 0).any()


def test_linearity_in_router_weights_and_duplicate_merging():
    """out(w_a + w_b) ~ out(w_a) + out(w_b) within the gate, and a token that
    lists one expert twice, (e, w1) and (e, w2), matches (e, w1 + w2)."""
    H, I = RANK
    dims, bank, bi = bank_case(7, 64, H, I, 3)
    rng = inputs.call_rng(13, 0)
    M, k = 3, 10
    x = inputs.activations(rng, M, H)
    ids = inputs.ids_distinct(rng, M, k, 64)
    wa = inputs.router_weights(rng, M, k)
    wb = inputs.router_weights(rng, M, k)
    sum_out = run_decode(dims, bank, x, ids, (wa + wb).astype(np.float32))
    parts = run_decode(dims, bank, x, ids, wa).astype(np.float64) + run_decode(dims, bank, x, ids, wb)
    check(sum_out, parts, "linearity in w")
    dup = ids.copy()
    dup[:, 1] = dup[:, 0]                     # expert of slot 0 listed twice
    wd = wa.copy()
    merged = wa.copy()
    merged[:, 0] = wa[:, 0] + wa[:, 1]
    merged[:, 1] = 0.0                        # the second listing carries no weight
    check(run_decode(dims, bank, x, dup, wd), run_decode(dims, bank, x, dup, merged).astype(np.float64),
          "duplicate merging")


def test_batch_independence_within_tolerance():
    """A token alone and inside a batch: the pages record cross-batch sensitivity
    as a known property (PR #520, Precision); here report bit-equality and gate
    on the tolerance."""
    H, I = RANK
    dims, bank, bi = bank_case(7, 64, H, I, 3)
    rng = inputs.call_rng(12, 0)
    M, k = 8, 10
    x = inputs.activations(rng, M, H)
    ids = inputs.ids_shared_pool(rng, M, k, 64)
    w = inputs.router_weights(rng, M, k)
    batch = run_decode(dims, bank, x, ids, w)
    same = 0
    for t in range(M):
        alone = run_decode(dims, bank, x[t:t + 1], ids[t:t + 1], w[t:t + 1])
        same += int(alone.view(np.uint16).tolist() == batch[t:t + 1].view(np.uint16).tolist())
        ok, _ = R.within_gate(alone[0], batch[t])
        assert ok
    say("batch-independent tokens (bit-equal)", same, "of", M)


def test_decode_back_to_back_on_one_workspace_equals_stage_pair():
    """Calls in a row on one workspace with changing inputs (a stale act would
    show): each equals the two stage entry points bit for bit and the oracle
    within tolerance, with the status word set only by the call that has
    invalid ids."""
    H, I = RANK
    E, k = 64, 10
    dims, bank, bi = bank_case(7, E, H, I, 3)
    dec = abi.Decoder(dims, bank, k)
    for c in range(8):
        rng = inputs.call_rng(14, c)
        M = 1 if c % 2 == 0 else 3
        x = inputs.activations(rng, M, H)
        ids = inputs.ids_distinct(rng, M, k, E)
        if c == 4:
            ids[0, 2], ids[0, 6] = -1, E      # invalid ids: no row, status bit 0
        if c == 6:
            ids[0, :] = ids[0, 0]             # one expert in every slot
        w = inputs.router_weights(rng, M, k)
        say("back-to-back decode call", c, "M", M)
        got = f16_to_np(dec(to_dev(x), to_dev(ids), to_dev(w)))
        assert dec.status() == (abi.STATUS_BAD_ID if c == 4 else 0)
        ws = abi.awq_moe_w13_swiglu(dims, bank, to_dev(x), to_dev(ids))
        pair = abi.awq_moe_w2_reduce(dims, bank, to_dev(ids), to_dev(w), ws)
        torch.cuda.synchronize()
        assert got.view(np.uint16).tolist() == f16_to_np(pair).view(np.uint16).tolist(), c
        check(got, R.moe_stage(x, ids, w, E, bi.expert), f"back-to-back call {c}")


@pytest.mark.parametrize("M", [1, 2])
def test_graph_capture_replays_match_eager(M):
    H, I = RANK
    dims, bank, bi = bank_case(7, 64, H, I, 3)
    rng = inputs.call_rng(13, 0)
    k = 10
    x = to_dev(inputs.activations(rng, M, H))
    ids = to_dev(inputs.ids_shared_pool(rng, M, k, 64))
    w = to_dev(inputs.router_weights(rng, M, k))
    dec = abi.Decoder(dims, bank, k)
    eager = dec(x, ids, w).clone()
    torch.cuda.synchronize()
    out = torch.empty_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dec(x, ids, w, out=out)            # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dec(x, ids, w, out=out)
    for rep in range(4):
        out.fill_(float("nan"))
        _ = torch.randn(1000, device="cuda").sum()      # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep


# ---------------------------------------------------------------------------
# every kernel form of the tactic table
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("rb", [3, 4])
@pytest.mark.parametrize("M", [1, 2, 8])
def test_every_decode_form_against_oracle(rb, M):
    """Each W13 form (lane pairs, single lanes, single lanes with two tiles
    per workgroup) and each W2 form (most slots per wave, one step fewer) is
    within the gate of the oracle; two tiles per workgroup is bit-identical
    to one, and the W2 forms are bit-identical to each other (same per-lane
    work, same reduction order); the table's forms equal awq_moe_decode."""
    H, I, E, k = 2560, 160, 64, 10
    dims, bank, bi = bank_case(7, E, H, I, rb)
    rng = inputs.call_rng(70, M)
    x = inputs.activations(rng, M, H)
    ids = inputs.ids_shared_pool(rng, M, k, E) if M > 1 else inputs.ids_distinct(rng, 1, k, E)
    w = inputs.router_weights(rng, M, k)
    want = R.moe_stage(x, ids, w, E, bi.expert)
    xd, idd, wd = to_dev(x), to_dev(ids), to_dev(w)
    outs = {}
    for f13 in (abi.W13_PAIR, abi.W13_SINGLE, abi.W13_SINGLE_TWO_TILES):
        for f2 in (abi.W2_SEG_MOST, abi.W2_SEG_FEWER):
            say("decode forms", M, rb, f13, f2)
            out = abi.awq_moe_decode_forms(dims, bank, xd, idd, wd, f13, f2)
            torch.cuda.synchronize()
            outs[(f13, f2)] = f16_to_np(out)
            check(outs[(f13, f2)], want, f"forms w13={f13} w2={f2} M={M} rb={rb}")
    bits = {key: v.view(np.uint16).tolist() for key, v in outs.items()}
    for f2 in (abi.W2_SEG_MOST, abi.W2_SEG_FEWER):
        assert bits[(abi.W13_SINGLE, f2)] == bits[(abi.W13_SINGLE_TWO_TILES, f2)]
    for f13 in (abi.W13_PAIR, abi.W13_SINGLE, abi.W13_SINGLE_TWO_TILES):
        assert bits[(f13, abi.W2_SEG_MOST)] == bits[(f13, abi.W2_SEG_FEWER)]
    table = abi.awq_moe_decode_table(dims, M, k)
    assert run_decode(dims, bank, x, ids, w).view(np.uint16).tolist() == bits[table]


@pytest.mark.parametrize("I", [64, 96, 160, 192, 256])
def test_w2_fewer_slots_per_wave_lanes_past_the_segments(I):
    """The W2 form with one step fewer slots per wave leaves lanes past the
    wave's segments (at inter 64, 96 and 160 more than one segment's worth;
    at 192 and 256 it is one slot per wave): their loads are clamped into
    the tile, so the last expert's last tile reads nothing past its block.
    The form equals the most-slots form bit for bit, with every slot on the
    bank's last expert in one token, and is within the gate of the
    oracle."""
    E, H, k, M = 6, 512, 6, 2
    dims, bank, bi = bank_case(700 + I, E, H, I, 3)
    rng = inputs.call_rng(701, I)
    x = inputs.activations(rng, M, H)
    ids = inputs.ids_distinct(rng, M, k, E)
    ids[0, :] = E - 1                      # every slot of token 0 on the last expert
    w = inputs.router_weights(rng, M, k)
    xd, idd, wd = to_dev(x), to_dev(ids), to_dev(w)
    say("w2 fewer slots per wave", I)
    most = abi.awq_moe_decode_forms(dims, bank, xd, idd, wd, abi.W13_SINGLE, abi.W2_SEG_MOST)
    fewer = abi.awq_moe_decode_forms(dims, bank, xd, idd, wd, abi.W13_SINGLE, abi.W2_SEG_FEWER)
    torch.cuda.synchronize()
    assert f16_to_np(most).view(np.uint16).tolist() == f16_to_np(fewer).view(np.uint16).tolist()
    check(f16_to_np(fewer), R.moe_stage(x, ids, w, E, bi.expert), f"w2 fewer slots per wave I={I}")


@pytest.mark.parametrize("f13", ["single", "single_two_tiles"])
@pytest.mark.parametrize("rb", [3, 4])
def test_w13_plain_and_non_temporal_weight_loads_agree(f13, rb):
    """W13 reads its weights with non-temporal loads when its whole grid fits
    the chip at once and with plain loads otherwise. Eight tokens at top-k 32
    (20 tiles x 256 slots x 5 waves, past 8192 waves) take plain loads; the
    same tokens in calls of two (5 x 1,280 waves) take non-temporal ones.
    Rows are independent, so both give the same bytes, within the gate of
    the oracle."""
    form = abi.W13_SINGLE if f13 == "single" else abi.W13_SINGLE_TWO_TILES
    E, (H, I), k, M = 64, RANK, 32, 8
    dims, bank, bi = bank_case(90 + rb, E, H, I, rb)
    rng = inputs.call_rng(91, rb)
    x = inputs.activations(rng, M, H)
    ids = inputs.ids_distinct(rng, M, k, E)
    w = inputs.router_weights(rng, M, k)
    say("w13 plain vs non-temporal loads", f13, rb)
    full = abi.awq_moe_decode_forms(dims, bank, to_dev(x), to_dev(ids), to_dev(w), form, abi.W2_SEG_MOST)
    parts = [abi.awq_moe_decode_forms(dims, bank, to_dev(x[i:i + 2]), to_dev(ids[i:i + 2]), to_dev(w[i:i + 2]),
                                      form, abi.W2_SEG_MOST) for i in range(0, M, 2)]
    torch.cuda.synchronize()
    got = f16_to_np(full)
    assert got.view(np.uint16).tolist() == np.concatenate([f16_to_np(p) for p in parts]).view(np.uint16).tolist()
    check(got, R.moe_stage(x, ids, w, E, bi.expert), f"w13 {f13} rb={rb} top-k 32")


def test_forms_on_other_shapes_and_stage_split():
    """Forms at shapes that change their geometry (hidden 96: lanes past L;
    inter 32: 16 slots per wave; hidden 4096: 16-wave two-tile blocks), and
    the W13-only / W2-only stages of the forms composing to the full call."""
    for (E, H, I, k, M) in ((6, 96, 64, 3, 5), (16, 256, 32, 8, 3), (6, 4096, 64, 2, 2)):
        dims, bank, bi = bank_case(80 + H, E, H, I, 3)
        rng = inputs.call_rng(81, H)
        x = inputs.activations(rng, M, H)
        ids = inputs.ids_shared_pool(rng, M, k, E)
        w = inputs.router_weights(rng, M, k)
        want = R.moe_stage(x, ids, w, E, bi.expert)
        xd, idd, wd = to_dev(x), to_dev(ids), to_dev(w)
        for f13 in (abi.W13_PAIR, abi.W13_SINGLE, abi.W13_SINGLE_TWO_TILES):
            for f2 in (abi.W2_SEG_MOST, abi.W2_SEG_FEWER):
                say("forms other shape", E, H, I, k, M, f13, f2)
                full = abi.awq_moe_decode_forms(dims, bank, xd, idd, wd, f13, f2)
                ws = abi.awq_moe_decode_forms(dims, bank, xd, idd, wd, f13, 0, stages=1)
                split = abi.awq_moe_decode_forms(dims, bank, xd, idd, wd, 0, f2, stages=2, workspace=ws)
                torch.cuda.synchronize()
                check(f16_to_np(full), want, f"forms E={E} H={H} I={I} w13={f13} w2={f2}")
                assert f16_to_np(full).view(np.uint16).tolist() == f16_to_np(split).view(np.uint16).tolist()
