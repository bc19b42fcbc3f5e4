"""C-ABI checks that need no GPU: the library loads and exports every declared
symbol; the host packer matches the oracle packer byte for byte; invalid
arguments are rejected before anything is written or launched."""

import ctypes
import os
import re

import numpy as np
import pytest

from awq_int4_mixture_amd import inputs
from oracle import layout as OL

abi = pytest.importorskip("awq_int4_mixture_amd.abi", reason="libawq_moe.so not built")

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "awq_moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(awq_moe_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == set(abi.EXPORTED), names
    lib = ctypes.CDLL(abi.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


@pytest.mark.parametrize("E,H,I,rb", [(512, 2560, 160, 3), (512, 2560, 160, 4), (16, 256, 32, 4), (3, 96, 64, 3)])
def test_layout_query_matches_oracle(E, H, I, rb):
    L = abi.awq_moe_bank_layout_query(abi.make_dims(E, H, I, rb))
    O = OL.layout(OL.Dims(E, H, I, rb))
    assert (L.w13_off, L.w13_meta_off, L.w2_off, L.w2_meta_off, L.expert_bytes, L.total_bytes) == \
           (O.w13_off, O.w13_meta_off, O.w2_off, O.w2_meta_off, O.expert_bytes, O.total_bytes)


@pytest.mark.parametrize("rb", [3, 4])
@pytest.mark.parametrize("E,H,I", [(4, 256, 32), (2, 96, 64), (2, 2560, 160)])
def test_prepare_bytes_equal_oracle_pack(rb, E, H, I):
    bi = inputs.bank_inputs(21, E, H, I, zero_hi=256)
    got = abi.prepare_from_inputs(abi.make_dims(E, H, I, rb), bi)
    want = OL.pack_bank(OL.Dims(E, H, I, rb), bi)
    assert got.tobytes() == want.tobytes()


@pytest.mark.parametrize("rb", [3, 4])
def test_prepare_bytes_equal_oracle_pack_wide_records(rb):
    """Zeros 0..255 and scales of both signs (+-0, subnormal, near 65504)."""
    bi = inputs.bank_inputs(22, 3, 96, 64, draw=inputs.expert_weights_wide, big_w13_groups=(2,),
                            big_w2_groups=(1,))
    got = abi.prepare_from_inputs(abi.make_dims(3, 96, 64, rb), bi)
    want = OL.pack_bank(OL.Dims(3, 96, 64, rb), bi)
    assert got.tobytes() == want.tobytes()


@pytest.mark.parametrize("rb", [3, 4])
def test_prepare_worked_example(rb):
    from tests.test_oracle_layout import golden_entries, worked_example_weights
    w = worked_example_weights()
    bank = abi.awq_moe_prepare(abi.make_dims(1, 64, 32, rb), *(a[None] for a in (
        w.q_gate, w.q_up, w.q_down, w.s_gate, w.s_up, w.s_down, w.z_gate, w.z_up, w.z_down)))
    for r, off, want in golden_entries():
        if r == rb:
            assert bytes(bank[off:off + len(want)]) == want


def _small_inputs():
    return inputs.bank_inputs(2, 2, 64, 32)


def test_prepare_rejects_bad_values_and_writes_nothing():
    dims = abi.make_dims(2, 64, 32, 3)
    total = abi.awq_moe_bank_layout_query(dims).total_bytes
    bi = _small_inputs()
    bad_q = bi.q_up.copy()
    bad_q[1, 5, 7] = 16
    bank = np.full(total, 0xAB, np.uint8)
    with pytest.raises(abi.AwqMoeError) as ei:
        abi.awq_moe_prepare(dims, bi.q_gate, bad_q, bi.q_down, bi.s_gate, bi.s_up, bi.s_down,
                            bi.z_gate, bi.z_up, bi.z_down, bank=bank)
    assert ei.value.code == abi.EINVAL and (bank == 0xAB).all()
    for bits in (0x7C00, 0xFC00, 0x7E00):          # +inf, -inf, NaN
        s = bi.s_down.copy().view(np.uint16)
        s[0, 0, 3] = bits
        with pytest.raises(abi.AwqMoeError) as ei:
            abi.awq_moe_prepare(dims, bi.q_gate, bi.q_up, bi.q_down, bi.s_gate, bi.s_up, s.view(np.float16),
                                bi.z_gate, bi.z_up, bi.z_down, bank=bank)
        assert ei.value.code == abi.EINVAL and (bank == 0xAB).all()
    small = np.zeros(total - 1, np.uint8)
    with pytest.raises(abi.AwqMoeError) as ei:
        abi.awq_moe_prepare(dims, bi.q_gate, bi.q_up, bi.q_down, bi.s_gate, bi.s_up, bi.s_down,
                            bi.z_gate, bi.z_up, bi.z_down, bank=small)
    assert ei.value.code == abi.ENOSPC and not small.any()


@pytest.mark.parametrize("dims,code", [
    ((512, 2560, 160, 32, 5), abi.EUNSUPPORTED),
    ((512, 2560, 160, 64, 4), abi.EUNSUPPORTED),
    ((512, 2560, 160, 16, 3), abi.EUNSUPPORTED),
    ((512, 2570, 160, 32, 3), abi.EUNSUPPORTED),
    ((512, 2560, 150, 32, 3), abi.EUNSUPPORTED),
    ((512, 16384, 160, 32, 3), abi.EUNSUPPORTED),
    ((512, 2560, 4096, 32, 3), abi.EUNSUPPORTED),
    ((0, 2560, 160, 32, 3), abi.EINVAL),
])
def test_unsupported_dims_fail_closed(dims, code):
    d = abi.awq_moe_dims(dims[0], dims[1], dims[2], dims[3], dims[4])
    with pytest.raises(abi.AwqMoeError) as ei:
        abi.awq_moe_bank_layout_query(d)
    assert ei.value.code == code


@pytest.mark.parametrize("M,k", [(0, 10), (9, 10), (1, 0), (1, 33), (-1, 2), (127, 10), (128, 10)])
def test_token_and_topk_bounds(M, k):
    """PR #520 (Tests) checks 1/2/8/9/127/128-token boundaries: only M in 1..8 is served."""
    d = abi.make_dims(512, 2560, 160, 3)
    with pytest.raises(abi.AwqMoeError) as ei:
        abi.awq_moe_workspace_bytes(d, M, k)
    assert ei.value.code == abi.EINVAL


def test_device_calls_reject_bad_arguments_before_launch():
    """Host validation returns before any HIP call, so these run without a GPU."""
    lib = abi._lib
    d = abi.make_dims(512, 2560, 160, 3)
    buf = (ctypes.c_uint8 * 4096)()
    base = (ctypes.addressof(buf) + 255) // 256 * 256
    p = ctypes.c_void_p(base)
    mis = ctypes.c_void_p(base + 2)
    q1 = ctypes.c_void_p(base + 1024)       # two disjoint 1 KiB row buffers
    q2 = ctypes.c_void_p(base + 2048)
    ws_need = abi.awq_moe_workspace_bytes(d, 1, 10)
    pws_need = abi.awq_moe_prefill_workspace_bytes(d, 9, 10)
    d_big = abi.make_dims(4097, 256, 32, 3)
    bb = abi.awq_moe_bank_layout_query(d).total_bytes          # the bank size the dims need
    bb_big = abi.awq_moe_bank_layout_query(d_big).total_bytes
    d_wide = abi.make_dims(4, 256, 2048, 3)                    # 8 x 32 x 2048 fp16 act: above the fixed scratch
    bb_wide = abi.awq_moe_bank_layout_query(d_wide).total_bytes
    d8k = abi.make_dims(4, 8192, 32, 3)                        # hidden 8192: no lane pairs (2048 threads)
    bb8k = abi.awq_moe_bank_layout_query(d8k).total_bytes
    cases = [
        (lambda: lib.awq_moe_decode(ctypes.byref(d), p, bb, p, p, p, 9, 10, p, p, ws_need, None), abi.EINVAL),
        (lambda: lib.awq_moe_decode(ctypes.byref(d), p, bb, p, p, p, 1, 10, p, p, ws_need - 1, None), abi.ENOSPC),
        (lambda: lib.awq_moe_decode(ctypes.byref(d), mis, bb, p, p, p, 1, 10, p, p, ws_need, None), abi.EINVAL),
        (lambda: lib.awq_moe_decode(ctypes.byref(d), p, bb, mis, p, p, 1, 10, p, p, ws_need, None), abi.EINVAL),
        (lambda: lib.awq_moe_decode(ctypes.byref(d), p, bb, p, None, p, 1, 10, p, p, ws_need, None), abi.EINVAL),
        (lambda: lib.awq_moe_decode(ctypes.byref(d), p, bb, p, p, p, 1, 10, mis, p, ws_need, None), abi.EINVAL),
        (lambda: lib.awq_moe_decode(None, p, bb, p, p, p, 1, 10, p, p, ws_need, None), abi.EINVAL),
        (lambda: lib.awq_moe_route_compact(p, 0, 10, 512, p, p, p, p, p, None), abi.EINVAL),
        (lambda: lib.awq_moe_route_compact(p, 1, 10, 0, p, p, p, p, p, None), abi.EINVAL),
        (lambda: lib.awq_moe_route_compact(p, 1, 10, 512, p, p, None, p, p, None), abi.EINVAL),
        (lambda: lib.awq_moe_w13_swiglu(ctypes.byref(d), p, bb, p, p, 1, 10, mis, ws_need, None), abi.EINVAL),
        (lambda: lib.awq_moe_w13_swiglu(ctypes.byref(d), p, bb, p, None, 1, 10, p, ws_need, None), abi.EINVAL),
        (lambda: lib.awq_moe_w13_swiglu(ctypes.byref(d), p, bb, p, p, 1, 10, p, ws_need - 1, None), abi.ENOSPC),
        (lambda: lib.awq_moe_w2_reduce(ctypes.byref(d), p, bb, p, p, 1, 10, p, ws_need, mis, None), abi.EINVAL),
        (lambda: lib.awq_moe_w2_reduce(ctypes.byref(d), p, bb, p, p, 9, 10, p, ws_need, p, None), abi.EINVAL),
        (lambda: lib.awq_moe_w2_reduce(ctypes.byref(d), p, bb, None, p, 1, 10, p, ws_need, p, None), abi.EINVAL),
        (lambda: lib.awq_moe_w2_reduce(ctypes.byref(d), p, bb, p, p, 1, 10, p, ws_need - 1, p, None), abi.ENOSPC),
        (lambda: lib.awq_moe_w2_reduce(ctypes.byref(d), p, bb, p, None, 1, 10, p, ws_need, p, None), abi.EINVAL),
        (lambda: lib.awq_moe_dequant(ctypes.byref(d), p, bb, 510, 3, 0, p, None), abi.EINVAL),
        (lambda: lib.awq_moe_dequant(ctypes.byref(d), p, bb, 0, 1, 2, p, None), abi.EINVAL),
        (lambda: lib.awq_moe_router_topk(p, 0, 512, 10, p, p, None), abi.EINVAL),
        (lambda: lib.awq_moe_router_topk(p, 4097, 512, 10, p, p, None), abi.EINVAL),
        (lambda: lib.awq_moe_router_topk(p, 1, 4097, 10, p, p, None), abi.EINVAL),
        (lambda: lib.awq_moe_router_topk(p, 1, 8, 9, p, p, None), abi.EINVAL),
        (lambda: lib.awq_moe_router_topk(p, 1, 512, 33, p, p, None), abi.EINVAL),
        (lambda: lib.awq_moe_router_topk(None, 1, 512, 10, p, p, None), abi.EINVAL),
        (lambda: lib.awq_moe_router_topk(mis, 1, 512, 10, p, p, None), abi.EINVAL),
        (lambda: lib.awq_moe_residual_rmsnorm(p, None, 1, 2560, 0.0, q1, q2, None), abi.EINVAL),
        (lambda: lib.awq_moe_residual_rmsnorm(p, None, 1, 2560, 1e-40, q1, q2, None), abi.EINVAL),  # subnormal eps
        (lambda: lib.awq_moe_residual_rmsnorm(p, None, 9, 256, 1e-6, q1, q2, None), abi.EINVAL),
        (lambda: lib.awq_moe_residual_rmsnorm(p, None, 1, 256, 1e-6, p, q2, None), abi.EINVAL),
        (lambda: lib.awq_moe_residual_rmsnorm(p, q2, 1, 256, 1e-6, q1, q2, None), abi.EINVAL),
        (lambda: lib.awq_moe_residual_rmsnorm(p, None, 1, 256, 1e-6, q1, q1, None), abi.EINVAL),
        (lambda: lib.awq_moe_residual_rmsnorm(p, None, 1, 8193, 1e-6, q1, q2, None), abi.EINVAL),
        (lambda: lib.awq_moe_residual_rmsnorm(p, None, 1, 100, 1e-6, q1, q2, None), abi.EINVAL),
        (lambda: lib.awq_moe_residual_rmsnorm(mis, None, 1, 256, 1e-6, q1, q2, None), abi.EINVAL),
        (lambda: lib.awq_moe_router_residual(p, 1, 512, 33, p, p, p, None, 256, 1e-6, q1, q2, None), abi.EINVAL),
        (lambda: lib.awq_moe_router_residual(p, 1, 512, 10, p, p, p, None, 256, 1e-6, p, q2, None), abi.EINVAL),
        (lambda: lib.awq_moe_router_residual(p, 9, 512, 10, p, p, p, None, 256, 1e-6, q1, q2, None), abi.EINVAL),
        (lambda: lib.awq_moe_router_gemv(p, None, 9, 256, 1e-6, p, 512, q1, q2, p, None), abi.EINVAL),
        (lambda: lib.awq_moe_router_gemv(p, None, 1, 256, 1e-6, None, 512, q1, q2, p, None), abi.EINVAL),
        (lambda: lib.awq_moe_router_gemv(p, None, 1, 256, 1e-6, p, 0, q1, q2, p, None), abi.EINVAL),
        (lambda: lib.awq_moe_router_gemv(p, None, 1, 256, 1e-6, p, 512, q1, q2, None, None), abi.EINVAL),
        (lambda: lib.awq_moe_prefill(ctypes.byref(d), p, bb, p, p, p, 8, 10, p, p, pws_need, None), abi.EINVAL),
        (lambda: lib.awq_moe_prefill(ctypes.byref(d), p, bb, p, p, p, 4097, 10, p, p, 1 << 62, None), abi.EINVAL),
        (lambda: lib.awq_moe_prefill(ctypes.byref(d), p, bb, p, p, p, 9, 33, p, p, 1 << 62, None), abi.EINVAL),
        (lambda: lib.awq_moe_prefill(ctypes.byref(d), p, bb, p, p, p, 9, 10, p, p, pws_need - 1, None), abi.ENOSPC),
        (lambda: lib.awq_moe_prefill(ctypes.byref(d), mis, bb, p, p, p, 9, 10, p, p, pws_need, None), abi.EINVAL),
        (lambda: lib.awq_moe_prefill(ctypes.byref(d), p, bb, mis, p, p, 9, 10, p, p, pws_need, None), abi.EINVAL),
        (lambda: lib.awq_moe_prefill(ctypes.byref(d), p, bb, p, None, p, 9, 10, p, p, pws_need, None), abi.EINVAL),
        (lambda: lib.awq_moe_prefill(ctypes.byref(d), p, bb, p, p, None, 9, 10, p, p, pws_need, None), abi.EINVAL),
        (lambda: lib.awq_moe_prefill(ctypes.byref(d), p, bb, p, p, p, 9, 10, mis, p, pws_need, None), abi.EINVAL),
        (lambda: lib.awq_moe_prefill(ctypes.byref(d), p, bb, p, p, p, 9, 10, p, mis, pws_need, None), abi.EINVAL),
        (lambda: lib.awq_moe_prefill(ctypes.byref(d_big), p, bb_big, p, p, p, 9, 10, p, p, 1 << 62, None),
         abi.EUNSUPPORTED),
        (lambda: lib.awq_moe_prefill(None, p, bb, p, p, p, 9, 10, p, p, pws_need, None), abi.EINVAL),
        # a bank smaller than the layout of dims (e.g. packed for fewer experts or 3-byte records)
        (lambda: lib.awq_moe_decode(ctypes.byref(d), p, bb - 1, p, p, p, 1, 10, p, p, ws_need, None), abi.ENOSPC),
        (lambda: lib.awq_moe_w13_swiglu(ctypes.byref(d), p, bb - 256, p, p, 1, 10, p, ws_need, None), abi.ENOSPC),
        (lambda: lib.awq_moe_w2_reduce(ctypes.byref(d), p, 0, p, p, 1, 10, p, ws_need, p, None), abi.ENOSPC),
        (lambda: lib.awq_moe_prefill(ctypes.byref(d), p, bb - 1, p, p, p, 9, 10, p, p, pws_need, None), abi.ENOSPC),
        (lambda: lib.awq_moe_dequant(ctypes.byref(d), p, bb - 1, 0, 1, 0, p, None), abi.ENOSPC),
        (lambda: lib.awq_moe_decode(ctypes.byref(abi.make_dims(512, 2560, 160, 4)), p, bb, p, p, p, 1, 10, p, p,
                                    1 << 40, None), abi.ENOSPC),
        # the fused stacked layer: the stage's checks plus eps and the two rows
        (lambda: lib.awq_moe_decode_rmsnorm_residual(ctypes.byref(d), p, bb, q1, 0.0, p, p, 1, 10, q2, p, ws_need,
                                                     None), abi.EINVAL),
        (lambda: lib.awq_moe_decode_rmsnorm_residual(ctypes.byref(d), p, bb, q1, 1e-40, p, p, 1, 10, q2, p, ws_need,
                                                     None), abi.EINVAL),
        (lambda: lib.awq_moe_decode_rmsnorm_residual(ctypes.byref(d), p, bb, q1, 1e-6, p, p, 1, 10, q1, p, ws_need,
                                                     None), abi.EINVAL),
        (lambda: lib.awq_moe_decode_rmsnorm_residual(ctypes.byref(d), p, bb, mis, 1e-6, p, p, 1, 10, q2, p, ws_need,
                                                     None), abi.EINVAL),
        (lambda: lib.awq_moe_decode_rmsnorm_residual(ctypes.byref(d), p, bb, q1, 1e-6, p, p, 9, 10, q2, p, ws_need,
                                                     None), abi.EINVAL),
        (lambda: lib.awq_moe_decode_rmsnorm_residual(ctypes.byref(d), p, bb - 1, q1, 1e-6, p, p, 1, 10, q2, p,
                                                     ws_need, None), abi.ENOSPC),
        (lambda: lib.awq_moe_decode_rmsnorm_residual(ctypes.byref(d), p, bb, q1, 1e-6, p, p, 1, 10, q2, p,
                                                     ws_need - 1, None), abi.ENOSPC),
        # forced kernel forms: the stage's checks, then the forms and stages
        (lambda: lib.awq_moe_decode_forms(ctypes.byref(d), p, bb, p, p, p, 1, 10, p, p, ws_need, 4, 0, 3, None),
         abi.EINVAL),
        (lambda: lib.awq_moe_decode_forms(ctypes.byref(d), p, bb, p, p, p, 1, 10, p, p, ws_need, 0, 3, 3, None),
         abi.EINVAL),
        (lambda: lib.awq_moe_decode_forms(ctypes.byref(d), p, bb, p, p, p, 1, 10, p, p, ws_need, 0, 0, 0, None),
         abi.EINVAL),
        (lambda: lib.awq_moe_decode_forms(ctypes.byref(d), p, bb, p, p, p, 9, 10, p, p, ws_need, 0, 0, 3, None),
         abi.EINVAL),
        (lambda: lib.awq_moe_decode_forms(ctypes.byref(d8k), p, bb8k, p, p, p, 1, 2, p, p, 1 << 30, 1, 0, 3, None),
         abi.EUNSUPPORTED),
        (lambda: lib.awq_moe_decode_forms(ctypes.byref(d_wide), p, bb_wide, p, p, p, 1, 2, p, p, 1 << 30, 0, 2, 3,
                                          None), abi.EUNSUPPORTED),
        # the no-allocation entry point: same checks, and a fixed scratch maximum
        (lambda: lib.awq_moe_decode_noalloc(ctypes.byref(d), p, bb, p, p, p, 9, 10, p, None, None), abi.EINVAL),
        (lambda: lib.awq_moe_decode_noalloc(ctypes.byref(d), p, bb - 1, p, p, p, 1, 10, p, None, None), abi.ENOSPC),
        (lambda: lib.awq_moe_decode_noalloc(ctypes.byref(d), p, bb, mis, p, p, 1, 10, p, None, None), abi.EINVAL),
        (lambda: lib.awq_moe_decode_noalloc(ctypes.byref(d), p, bb, p, p, p, 1, 10, mis, None, None), abi.EINVAL),
        (lambda: lib.awq_moe_decode_noalloc(ctypes.byref(d), p, bb, p, p, p, 1, 10, p, mis, None), abi.EINVAL),
        (lambda: lib.awq_moe_decode_noalloc(None, p, bb, p, p, p, 1, 10, p, None, None), abi.EINVAL),
        (lambda: lib.awq_moe_decode_noalloc(ctypes.byref(d_wide), p, bb_wide, p, p, p, 8, 32, p, None, None),
         abi.ENOSPC),
    ]
    for i, (call, code) in enumerate(cases):
        assert call() == code, (i, abi.awq_moe_last_error())
        assert abi.awq_moe_last_error() != ""
    assert bytes(buf) == bytes(4096)


def test_tactic_table_forms_are_valid_for_every_admitted_token_count():
    """The table answers for every M and record size, and only with forms
    that fit the shape (lane pairs need hidden <= 4096; the generic W2
    kernel, past inter 1024, has one form)."""
    for dims in (abi.make_dims(512, 2560, 160, 3), abi.make_dims(512, 2560, 160, 4), abi.make_dims(4, 8192, 32, 3),
                 abi.make_dims(8, 512, 2048, 3), abi.make_dims(16, 96, 64, 4), abi.make_dims(64, 2560, 320, 3),
                 abi.make_dims(64, 2560, 640, 4)):
        for M in range(1, 9):
            f13, f2 = abi.awq_moe_decode_table(dims, M, 10)
            assert f13 in (abi.W13_PAIR, abi.W13_SINGLE, abi.W13_SINGLE_TWO_TILES)
            assert f2 in (abi.W2_SEG_MOST, abi.W2_SEG_FEWER)
            if dims.hidden > 4096:
                assert f13 == abi.W13_SINGLE
            if dims.inter > 1024:
                assert f2 == abi.W2_SEG_MOST


def test_noalloc_scratch_covers_the_rank_shape():
    """The fixed scratch of the no-allocation entry point holds the decode
    workspace of the rank shape at M = 8 and of every shape with
    M * topk * inter <= 262144; one element more does not fit."""
    assert abi.awq_moe_workspace_bytes(abi.make_dims(512, 2560, 160, 3), 8, 10) <= abi.NOALLOC_SCRATCH_BYTES
    assert abi.awq_moe_workspace_bytes(abi.make_dims(4, 256, 2048, 3), 4, 32) == abi.NOALLOC_SCRATCH_BYTES
    assert abi.awq_moe_workspace_bytes(abi.make_dims(4, 256, 2048, 3), 5, 32) > abi.NOALLOC_SCRATCH_BYTES


def test_workspace_grows_with_tokens():
    d = abi.make_dims(512, 2560, 160, 3)
    sizes = [abi.awq_moe_workspace_bytes(d, M, 10) for M in range(1, 9)]
    assert all(b > a for a, b in zip(sizes, sizes[1:]))
    assert sizes[-1] >= 80 * 160 * 2


def test_prefill_workspace_bounds():
    """The prefill workspace holds the row maps, the work items, fp16 act and
    fp32 y for every slot; admission is M in [9, 4096] (1..8 go to decode)."""
    d = abi.make_dims(512, 2560, 160, 3)
    for M in (9, 128, 4096):
        n = M * 10
        need = abi.awq_moe_prefill_workspace_bytes(d, M, 10)
        assert need >= 256 + 8 * n + n * 160 * 2 + n * 2560 * 4
        assert need % 256 == 0
    for M in (8, 4097):
        with pytest.raises(abi.AwqMoeError):
            abi.awq_moe_prefill_workspace_bytes(d, M, 10)
    with pytest.raises(abi.AwqMoeError):
        abi.awq_moe_workspace_bytes(d, 9, 10)
