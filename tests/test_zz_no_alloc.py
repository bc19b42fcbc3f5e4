"""The no-allocation decode entry point against awq_moe_decode, through the C ABI.

awq_moe_decode_noalloc runs the same kernels as awq_moe_decode on the
library's fixed scratch, so its outputs must be bit-identical to those of
awq_moe_decode with a caller-owned workspace, and the status word must agree.
Two calls in a row, the second with a smaller input (fewer tokens and a
smaller top-k), check that the scratch left by the first call changes
nothing; a third call repeats the first. Each result is also within the gate
of the float64 oracle.
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


def _call_case(dims, bank, bi, E, M, k, seed, bad_id):
    H = dims.hidden
    rng = inputs.call_rng(seed, M * 100 + k)
    x = inputs.activations(rng, M, H)
    ids = inputs.ids_shared_pool(rng, M, k, E) if M > 1 else inputs.ids_distinct(rng, 1, k, E)
    if bad_id:
        ids[0, 1] = E + 3                      # outside [0, E): status bit 0, row contributes 0
    w = inputs.router_weights(rng, M, k)
    xd, idd, wd = to_dev(x), to_dev(ids), to_dev(w)
    ws = abi.alloc_workspace(dims, M, k, xd.device)
    ref = abi.awq_moe_decode(dims, bank, xd, idd, wd, workspace=ws)
    status = torch.full((1,), -1, dtype=torch.int32, device=xd.device)
    got = abi.awq_moe_decode_noalloc(dims, bank, xd, idd, wd, status=status)
    torch.cuda.synchronize()
    ref_status = int(ws[:4].view(torch.int32).item())
    return f16_to_np(got), f16_to_np(ref), int(status.item()), ref_status, R.moe_stage(x, ids, w, E, bi.expert)


@pytest.mark.parametrize("rb", [3, 4])
def test_noalloc_equals_decode_on_calls_in_a_row(rb):
    H, I, E = 2560, 160, 64
    dims, bank, bi = bank_case(7, E, H, I, rb)
    for c, (M, k, bad) in enumerate([(8, 10, True), (1, 4, False), (8, 10, False)]):
        say("noalloc call", c, "M", M, "k", k, "rb", rb)
        got, ref, st, ref_st, want = _call_case(dims, bank, bi, E, M, k, 50 + c, bad)
        assert got.view(np.uint16).tolist() == ref.view(np.uint16).tolist(), c
        assert st == ref_st == (abi.STATUS_BAD_ID if bad else 0), (c, st, ref_st)
        ok, err = R.within_gate(got, want)
        say("noalloc vs oracle", c, err)
        assert ok, err


def test_noalloc_largest_admitted_scratch():
    """M*topk*inter*2 = 512 KiB exactly: hidden 256, inter 2048, top-k 32,
    M = 4 over 6 experts (the generic W2 kernel), then a smaller call."""
    E, H, I = 6, 256, 2048
    dims, bank, bi = bank_case(8, E, H, I, 3)
    assert abi.awq_moe_workspace_bytes(dims, 4, 32) == abi.NOALLOC_SCRATCH_BYTES
    for c, (M, k) in enumerate([(4, 32), (2, 3)]):
        rng = inputs.call_rng(60, c)
        x = inputs.activations(rng, M, H)
        ids = rng.integers(0, E, size=(M, k)).astype(np.int32)
        w = inputs.router_weights(rng, M, k)
        say("noalloc largest scratch call", c, "M", M, "k", k)
        ref = abi.awq_moe_decode(dims, bank, to_dev(x), to_dev(ids), to_dev(w))
        got = abi.awq_moe_decode_noalloc(dims, bank, to_dev(x), to_dev(ids), to_dev(w))
        torch.cuda.synchronize()
        assert f16_to_np(got).view(np.uint16).tolist() == f16_to_np(ref).view(np.uint16).tolist(), c
        ok, err = R.within_gate(f16_to_np(got), R.moe_stage(x, ids, w, E, bi.expert))
        assert ok, err
    with pytest.raises(abi.AwqMoeError) as ei:
        abi.awq_moe_decode_noalloc(dims, bank, to_dev(np.zeros((5, H), np.float16)),
                                   to_dev(np.zeros((5, 32), np.int32)), to_dev(np.zeros((5, 32), np.float32)))
    assert ei.value.code == abi.ENOSPC
