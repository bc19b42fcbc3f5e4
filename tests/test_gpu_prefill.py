"""GPU parity of the indexed prefill stage (M >= 9 tokens) against the
float64 oracle, through the C ABI, plus its bit-exact invariants.

The oracle is the same whole-stage definition as for decode (PR #520,
Tests: indexed prefill serves the token counts above the grouped decode's
1..8); the gates are max|gpu - ref| <= 4e-3 max|ref| and
||gpu - ref|| / ||ref|| <= 2e-3.
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


def run_prefill(dims, bank, x, ids, w, workspace=None):
    out = abi.awq_moe_prefill(dims, bank, to_dev(x), to_dev(ids), to_dev(w), workspace=workspace)
    torch.cuda.synchronize()
    return f16_to_np(out)


def check(got, want, what):
    ok, e = R.within_gate(got, want)
    say(what, e)
    assert ok, (what, e)
    return e


@pytest.mark.parametrize("E,H,I,k,M,rb", [
    (16, 256, 32, 2, 9, 3),        # the admission boundary, tiny shape (decode kernels)
    (16, 256, 32, 4, 128, 4),      # wide kernels, 32 rows per expert on average: items of two or three row tiles
    (6, 96, 64, 3, 17, 3),         # hidden 96 in the decode kernels
    (16, 512, 2048, 10, 40, 3),    # inter 2048 in the decode kernels (the generic W2 kernel)
    (12, 128, 96, 1, 33, 4),       # top-k 1
    (64, 2560, 160, 10, 64, 3),    # rank shape with 64 experts at the decode kernels' last token count
    (64, 2560, 160, 10, 65, 4),    # ... and one token more: the wide kernels in one launch
    (64, 2560, 160, 10, 127, 3),   # rank shape with 64 experts, ~20 rows each
    (4, 8192, 32, 2, 9, 3),        # hidden 8192: 256 W13 groups, 64 per wave
    (32, 256, 64, 32, 40, 3),      # top-k 32, 1,280 slots: the per-tile kernels (more slots than the decode form)
    (64, 2560, 160, 20, 60, 4),    # the per-tile kernels at the rank shape, 1,200 slots
    (32, 512, 2048, 17, 64, 3),    # the per-tile kernels with inter 2048, 1,088 slots
    (96, 256, 32, 24, 48, 3),      # 1,152 slots over 96 experts: per-tile items of one to three rows
    (64, 256, 32, 32, 32, 4),      # top-k 32 at 1,024 slots: the decode kernels' largest call (status over 1,024 ids)
    (4096, 256, 32, 8, 16, 3),     # 4096 experts in the decode kernels
    (16, 256, 32, 2, 4096, 3),     # the largest M: 8192 slots, ~512 rows per expert
    (16, 352, 64, 4, 600, 4),      # wide kernels: 11 groups (W13 chunks of 4, 4, 3), ~150 rows per expert
    (40, 2560, 160, 10, 512, 3),   # wide kernels at the rank shape, ~128 rows per expert: 64-row items
    (8, 8192, 32, 2, 520, 3),      # wide kernels, hidden 8192: 64 W13 chunks, ~130 rows per expert
    (4, 8192, 2048, 4, 9, 3),      # hidden 8192 with inter 2048 (the maxima together), decode kernels
    (6, 96, 64, 3, 300, 3),        # wide items with 3 groups: one chunk, shorter than the weight ring
    (6, 96, 64, 3, 300, 4),        # the same with 4-byte records
    (24, 96, 64, 3, 128, 3),       # wide items of one or two row tiles (the unit ring) with 3 groups: clamped units
    (44, 352, 64, 4, 160, 4),      # the unit ring over 11 groups (chunks of 4, 4, 3), ~15 rows per expert
    (32, 512, 96, 6, 256, 3),      # inter 96 in one launch: 3 act groups (2 zero groups), 12 W13 tiles
    (16, 1024, 128, 4, 384, 4),    # inter 128 in one launch: 4 act groups, 16 W13 tiles, 4 W2 column blocks
    (16, 512, 256, 4, 160, 3),     # inter 256: the two wide kernels (no single-launch form), W2 on 32-row items
    (16, 256, 192, 8, 2048, 4),    # inter 192 at 16,384 slots: the two wide kernels, W2 on the wide items
    (24, 1024, 320, 6, 200, 4),    # inter 320 on the two wide kernels: two W13 column blocks, 10 W2 K groups
    (12, 512, 352, 4, 300, 3),     # inter 352: 22 W13 tiles (a 2-tile second block), 11 W2 K groups
    (24, 1024, 320, 10, 40, 3),    # inter 320 in the decode kernels: W2 with one slot per wave
])
def test_prefill_shapes(E, H, I, k, M, rb):
    dims, bank, bi = bank_case(60 + I, E, H, I, rb)
    rng = inputs.call_rng(61, M + H + k)
    x = inputs.activations(rng, M, H)
    ids = inputs.ids_distinct(rng, M, k, E)
    w = inputs.router_weights(rng, M, k)
    say("prefill shape", E, H, I, k, M, rb)
    check(run_prefill(dims, bank, x, ids, w), R.moe_stage(x, ids, w, E, bi.expert),
          f"prefill E={E} H={H} I={I} k={k} M={M} rb={rb}")


def test_prefill_largest_hidden_and_inter_sampled():
    """Hidden 8192 with inter 2048 at M = 300 (four tiles per W13
    workgroup, ~300 rows per expert: ten items each, 26 chunks of groups):
    the oracle on 12 sampled tokens, the first and last among them (a
    token's result depends only on its own (id, weight) pairs)."""
    E, H, I, k, M = 4, 8192, 2048, 4, 300
    dims, bank, bi = bank_case(92, E, H, I, 4)
    rng = inputs.call_rng(93, 0)
    x = inputs.activations(rng, M, H)
    ids = inputs.ids_distinct(rng, M, k, E)
    w = inputs.router_weights(rng, M, k)
    say("prefill largest hidden and inter", E, H, I, k, M)
    got = run_prefill(dims, bank, x, ids, w)
    sel = np.unique(np.concatenate([[0, M - 1], rng.choice(np.arange(1, M - 1), 10, replace=False)]))
    check(got[sel], R.moe_stage(x[sel], ids[sel], w[sel], E, bi.expert), "prefill largest hidden and inter")


@pytest.mark.parametrize("rb", [3, 4])
def test_prefill_rank_shape_wide_items_sampled(rb):
    """Hidden 2560, inter 160, 64 experts, top-k 10, M = 2048 (20,480 slots,
    about 320 rows per expert): W2 takes the wide items (five 64-row items
    per expert), W13 the wide items throughout; the oracle on 16 sampled
    tokens, the first and last among them."""
    E, H, I, k, M = 64, 2560, 160, 10, 2048
    dims, bank, bi = bank_case(96, E, H, I, rb)
    rng = inputs.call_rng(97, rb)
    x = inputs.activations(rng, M, H)
    ids = inputs.ids_distinct(rng, M, k, E)
    w = inputs.router_weights(rng, M, k)
    say("prefill rank shape wide items", M, rb)
    got = run_prefill(dims, bank, x, ids, w)
    sel = np.unique(np.concatenate([[0, M - 1], rng.choice(np.arange(1, M - 1), 14, replace=False)]))
    check(got[sel], R.moe_stage(x[sel], ids[sel], w[sel], E, bi.expert), f"prefill rank shape wide items rb={rb}")


def test_prefill_maximum_experts_topk_tokens_sampled():
    """4096 experts, top-k 32 and 4096 tokens (131,072 slots, the admitted
    maxima), hidden 256, inter 32: the oracle on 16 sampled tokens, the
    first and last among them."""
    E, H, I, k, M = 4096, 256, 32, 32, 4096
    dims, bank, bi = bank_case(94, E, H, I, 3)
    rng = inputs.call_rng(95, 0)
    x = inputs.activations(rng, M, H)
    ids = inputs.ids_distinct(rng, M, k, E)
    w = inputs.router_weights(rng, M, k)
    say("prefill maximum experts, top-k and tokens", E, k, M)
    got = run_prefill(dims, bank, x, ids, w)
    sel = np.unique(np.concatenate([[0, M - 1], rng.choice(np.arange(1, M - 1), 14, replace=False)]))
    check(got[sel], R.moe_stage(x[sel], ids[sel], w[sel], E, bi.expert), "prefill maximum experts, top-k, tokens")


@pytest.mark.parametrize("rb", [3, 4])
@pytest.mark.parametrize("M", [9, 128, 512])
def test_prefill_rank_shape_full_bank(rb, M):
    """The decode benchmark's layer (512 experts, hidden 2560, inter 160,
    top-k 10) with M tokens that pick their experts independently."""
    H, I = 2560, 160
    dims, bank, bi = bank_case(2026, 512, H, I, rb)
    rng = inputs.call_rng(2027, M)
    x = inputs.activations(rng, M, H)
    ids = inputs.ids_distinct(rng, M, 10, 512)
    w = inputs.router_weights(rng, M, 10)
    say("prefill rank", M, rb)
    check(run_prefill(dims, bank, x, ids, w), R.moe_stage(x, ids, w, 512, bi.expert), f"prefill rank M={M} rb={rb}")


@pytest.mark.parametrize("M", [20, 130])  # the decode kernels, the wide kernels (routed)
def test_prefill_invalid_and_duplicate_ids(M):
    """Ids outside [0, E) set status bit 0 and contribute nothing; a token
    may route to one expert twice (two rows); a token with no valid id gives
    an all-zero row."""
    E, H, I, k = 16, 256, 32, 4
    dims, bank, bi = bank_case(62, E, H, I, 3)
    rng = inputs.call_rng(63, 0)
    x = inputs.activations(rng, M, H)
    ids = inputs.ids_distinct(rng, M, k, E)
    ids[2, 1] = -1
    ids[5, 3] = E
    ids[7, :] = [3, 3, 9, 3]
    ids[11, :] = -5
    w = inputs.router_weights(rng, M, k)
    ws = abi.alloc_prefill_workspace(dims, M, k)
    got = run_prefill(dims, bank, x, ids, w, workspace=ws)
    assert int(ws[:4].view(torch.int32).cpu()[0]) & 1 == 1
    assert not got[11].any()
    check(got, R.moe_stage(x, ids, w, E, bi.expert), "prefill invalid/duplicate ids")
    ok_ids = inputs.ids_distinct(rng, M, k, E)
    run_prefill(dims, bank, x, ok_ids, w, workspace=ws)
    assert int(ws[:4].view(torch.int32).cpu()[0]) == 0


@pytest.mark.parametrize("E,k,M,Msub", [(24, 6, 40, 9),      # the decode kernels
                                       (64, 32, 40, 36),    # the per-tile kernels (1,280 and 1,152 slots)
                                       (24, 6, 200, 130)])  # the wide kernels (one launch at inter 64)
def test_prefill_bit_exact_invariants(E, k, M, Msub):
    """Each token's result depends only on its own (id, weight) pairs: two
    calls give identical bytes; permuting a token's pairs gives identical
    bytes (ascending (expert, slot) summation); a token gives identical bytes
    inside a call of its first Msub tokens and inside the M-token call (a
    row's matrix-core result does not depend on the rows sharing its tile);
    router weights scaled by 2 give exactly twice the output."""
    H, I = 512, 64
    dims, bank, bi = bank_case(64, E, H, I, 3)
    rng = inputs.call_rng(65, M)
    x = inputs.activations(rng, M, H)
    ids = inputs.ids_shared_pool(rng, M, k, E, frac=0.3) if k < E // 2 else inputs.ids_distinct(rng, M, k, E)
    w = inputs.router_weights(rng, M, k)
    a = run_prefill(dims, bank, x, ids, w)
    b = run_prefill(dims, bank, x, ids, w)
    assert a.tobytes() == b.tobytes()
    perm = np.stack([rng.permutation(k) for _ in range(M)])
    ids_p = np.take_along_axis(ids, perm, 1)
    w_p = np.take_along_axis(w, perm, 1)
    c = run_prefill(dims, bank, x, ids_p, w_p)
    assert a.tobytes() == c.tobytes()
    sub = run_prefill(dims, bank, x[:Msub], ids[:Msub], w[:Msub])
    assert sub.tobytes() == a[:Msub].tobytes()
    d = run_prefill(dims, bank, x, ids, (w * 2).astype(np.float32))
    mag = np.abs(a.astype(np.float64))
    normal = (mag >= 2.0 ** -14) & (mag < 3e4)  # doubling is exact there, subnormals excluded
    assert np.array_equal(d[normal].astype(np.float64), 2.0 * a[normal].astype(np.float64))
    check(a, R.moe_stage(x, ids, w, E, bi.expert), f"prefill invariants M={M} k={k}")


@pytest.mark.parametrize("rb", [3, 4])
def test_prefill_rows_identical_across_cache_policies(rb):
    """At the rank layer the one-launch kernel picks its weight loads' cache
    policy from the mean rows per expert: 128 tokens (2.5 rows per expert)
    non-temporal W13 only, 1024 tokens (20) both, 4096 tokens (80) W2 only,
    and the items hold one, two or four row tiles. The first 128 tokens give
    the same bytes in all three calls, and the first 1024 in the last two,
    and 8 sampled tokens of the largest call are within the gate of the
    oracle."""
    E, H, I, k = 512, 2560, 160, 10
    dims, bank, bi = bank_case(2026, E, H, I, rb)
    rng = inputs.call_rng(2029, rb)
    M = 4096
    x = inputs.activations(rng, M, H)
    ids = inputs.ids_distinct(rng, M, k, E)
    w = inputs.router_weights(rng, M, k)
    say("prefill rows across cache policies", rb)
    outs = {m: run_prefill(dims, bank, x[:m], ids[:m], w[:m]) for m in (128, 1024, 4096)}
    assert outs[128].tobytes() == outs[1024][:128].tobytes() == outs[4096][:128].tobytes()
    assert outs[1024].tobytes() == outs[4096][:1024].tobytes()
    sel = np.unique(np.concatenate([[0, M - 1], rng.choice(np.arange(1, M - 1), 6, replace=False)]))
    check(outs[4096][sel], R.moe_stage(x[sel], ids[sel], w[sel], E, bi.expert), f"prefill rows across policies rb={rb}")


def test_prefill_decode_form_equals_decode_calls():
    """Up to 64 tokens (and 1,024 slots) the prefill runs the decode kernels
    on the whole call; each token's work is its own, so 24 tokens in one
    prefill call give the same bytes as three 8-token decode calls."""
    H, I = 2560, 160
    dims, bank, bi = bank_case(7, 128, H, I, 3)
    rng = inputs.call_rng(66, 0)
    x = inputs.activations(rng, 24, H)
    ids = inputs.ids_shared_pool(rng, 24, 10, 128)
    w = inputs.router_weights(rng, 24, 10)
    p = run_prefill(dims, bank, x, ids, w)
    d = np.concatenate([f16_to_np(abi.awq_moe_decode(dims, bank, to_dev(x[h:h + 8]), to_dev(ids[h:h + 8]),
                                                     to_dev(w[h:h + 8]))) for h in (0, 8, 16)])
    torch.cuda.synchronize()
    assert p.tobytes() == d.tobytes()
    check(p, R.moe_stage(x, ids, w, 128, bi.expert), "prefill decode form")


def test_prefill_close_to_decode():
    """The matrix-core path and the decode path compute the same stage: 96
    tokens in one prefill call (the wide kernels) against twelve 8-token
    decode calls, within the gate."""
    H, I = 2560, 160
    dims, bank, bi = bank_case(7, 128, H, I, 3)
    rng = inputs.call_rng(66, 1)
    x = inputs.activations(rng, 96, H)
    ids = inputs.ids_shared_pool(rng, 96, 10, 128)
    w = inputs.router_weights(rng, 96, 10)
    p = run_prefill(dims, bank, x, ids, w)
    d = np.concatenate([f16_to_np(abi.awq_moe_decode(dims, bank, to_dev(x[h:h + 8]), to_dev(ids[h:h + 8]),
                                                     to_dev(w[h:h + 8]))) for h in range(0, 96, 8)])
    torch.cuda.synchronize()
    check(p, d.astype(np.float64), "prefill vs decode")


@pytest.mark.parametrize("M", [64, 130])  # the decode kernels, the wide kernels
def test_prefill_graph_capture_replays_match_eager(M):
    E, H, I, k = 32, 256, 64, 4
    dims, bank, bi = bank_case(67, E, H, I, 4)
    rng = inputs.call_rng(68, 0)
    x = to_dev(inputs.activations(rng, M, H))
    ids = to_dev(inputs.ids_distinct(rng, M, k, E))
    w = to_dev(inputs.router_weights(rng, M, k))
    ws = abi.alloc_prefill_workspace(dims, M, k)
    out = torch.empty((M, H), dtype=torch.float16, device="cuda")
    abi.awq_moe_prefill(dims, bank, x, ids, w, out=out, workspace=ws)
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            abi.awq_moe_prefill(dims, bank, x, ids, w, out=out, workspace=ws)
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16))


def _pad256(b):
    return (b + 255) // 256 * 256


@pytest.mark.parametrize("E,k,M,hot", [(16, 4, 128, False), (512, 10, 128, False), (8, 2, 300, True),
                                       (64, 10, 65, False),  # the smallest routed call
                                       (4096, 32, 4096, False)])  # the admitted maxima: 131,072 slots
def test_prefill_routing_arrays(E, k, M, hot):
    """The routing arrays in the workspace (layout as documented in the
    header). Unique parts, bit-exact against the oracle's compaction: the
    number of work items and each item (expert, first row, rows), the status
    word, the segment of every slot. The rest checked for validity: slot ->
    row and row -> slot are inverse bijections on the valid slots, and every
    slot's row lies inside its expert's segment."""
    H, I = 256, 32
    dims, bank, bi = bank_case(70, E, H, I, 3)
    rng = inputs.call_rng(71, E + M)
    x = inputs.activations(rng, M, H)
    if hot:  # a few experts take most rows: several 32-row items per expert
        ids = np.stack([rng.choice(3, size=k, replace=False) for _ in range(M)]).astype(np.int32)
    else:
        ids = inputs.ids_distinct(rng, M, k, E)
    ids[M // 2, 0] = -3  # one invalid slot
    w = inputs.router_weights(rng, M, k)
    ws = abi.alloc_prefill_workspace(dims, M, k)
    run_prefill(dims, bank, x, ids, w, workspace=ws)
    raw = ws.cpu().numpy()
    n = M * k
    X = (n + 31) // 32 + min(E, n)
    W = (n + 63) // 64 + min(E, n)
    o_slot_row = 256
    o_row_slot = o_slot_row + _pad256(4 * n)
    o_items = o_row_slot + _pad256(4 * n)
    o_witems = o_items + _pad256(8 * X)
    status, n_items, n_witems = raw[:12].view(np.int32)
    slot_row = raw[o_slot_row:o_slot_row + 4 * n].view(np.int32)
    row_slot = raw[o_row_slot:o_row_slot + 4 * n].view(np.int32)
    items = raw[o_items:o_items + 8 * X].view(np.int32).reshape(X, 2)
    witems = raw[o_witems:o_witems + 8 * W].view(np.int32).reshape(W, 2)

    ro = R.route_compact(ids, E)
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    V = int(valid.sum())
    assert status == 1 and V == ro["num_valid"]
    # segments (unique): expert e owns rows [off, off + cnt) in ascending expert order
    seg = {int(e): (int(ro["offsets"][a]), int(ro["offsets"][a + 1])) for a, e in
           enumerate(ro["active_ids"][:ro["num_active"]])}
    want_items = []
    for e, (lo, hi) in sorted(seg.items()):
        for r0 in range(lo, hi, 32):
            want_items.append((e, r0 | (min(32, hi - r0) << 24)))
    assert n_items == len(want_items)
    assert [tuple(v) for v in items[:n_items].tolist()] == want_items
    # wide items: ceil(c / 64) per expert, rows shared out in multiples of 16
    want_witems = []
    for e, (lo, hi) in sorted(seg.items()):
        c = hi - lo
        nw = -(-c // 64)
        per = -(-(-(-c // nw)) // 16) * 16
        for p in range(nw):
            want_witems.append((e, (lo + per * p) | (min(per, c - per * p) << 24)))
    assert n_witems == len(want_witems) <= W
    assert [tuple(v) for v in witems[:n_witems].tolist()] == want_witems
    # rows (valid placement): bijection, each slot inside its expert's segment
    assert (slot_row[~valid] == -1).all()
    rows_of_valid = slot_row[valid]
    assert sorted(rows_of_valid.tolist()) == list(range(V))
    assert (row_slot[rows_of_valid] == np.flatnonzero(valid)).all()
    for s in np.flatnonzero(valid):
        lo, hi = seg[int(flat[s])]
        assert lo <= slot_row[s] < hi
