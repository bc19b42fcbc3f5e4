"""Exhaustive bit-exact check of the on-the-fly dequantisation on the GPU.

Every 4-bit value q (16) x every zero z (256) x every finite fp16 scale
(63,488 bit patterns) is packed into W13 records and read back through
awq_moe_dequant; the result must equal NumPy's fp32 (q - z) * s bit for bit.
That product is exact in fp32 (q - z is an integer in [-255, 15] and s an
fp16, at most 19 significant bits), so the closed form is the reference.
Eight banks of 32 experts (hidden 512, inter 2048) hold one zero value per
expert and all finite scales in each expert's 65,536 W13 records; banks
alternate 3- and 4-byte records. W2 is checked the same way on one bank.
"""

import numpy as np
import pytest

from tests.gpu_helpers import say, to_dev, torch_mod

pytestmark = pytest.mark.gpu

torch = torch_mod()
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from awq_int4_mixture_amd import abi  # noqa: E402

H, I, EC = 512, 2048, 32
G13, G2 = H // 32, I // 32


def finite_fp16_bits() -> np.ndarray:
    b = np.arange(65536, dtype=np.uint32)
    return b[(b & 0x7C00) != 0x7C00].astype(np.uint16)


def chunk_inputs(z0: int):
    fin = finite_fp16_bits()
    assert fin.size == 63488
    k = np.arange(H)[:, None]
    n = np.arange(2 * I)[None, :]
    q13 = ((k + n) % 16).astype(np.uint8)                                  # every q twice per group
    s13 = fin[np.arange(G13 * 2 * I) % fin.size].reshape(G13, 2 * I).view(np.float16)
    kd = np.arange(I)[:, None]
    nd = np.arange(H)[None, :]
    q2 = ((kd + 3 * nd) % 16).astype(np.uint8)
    s2 = fin[(np.arange(G2 * H) * 7) % fin.size].reshape(G2, H).view(np.float16)
    qg = np.ascontiguousarray(np.broadcast_to(q13[:, 0::2], (EC, H, I)))
    qu = np.ascontiguousarray(np.broadcast_to(q13[:, 1::2], (EC, H, I)))
    qd = np.ascontiguousarray(np.broadcast_to(q2, (EC, I, H)))
    sg = np.ascontiguousarray(np.broadcast_to(s13[:, 0::2], (EC, G13, I)))
    su = np.ascontiguousarray(np.broadcast_to(s13[:, 1::2], (EC, G13, I)))
    sd = np.ascontiguousarray(np.broadcast_to(s2, (EC, G2, H)))
    zz = (z0 + np.arange(EC)).astype(np.uint8)
    zg = np.ascontiguousarray(np.broadcast_to(zz[:, None, None], (EC, G13, I)))
    zd = np.ascontiguousarray(np.broadcast_to(zz[:, None, None], (EC, G2, H)))
    return (qg, qu, qd, sg, su, sd, zg, zg.copy(), zd), q13, s13, q2, s2, zz


@pytest.mark.parametrize("chunk", range(8))
def test_dequant_exhaustive(chunk):
    rb = 3 if chunk % 2 == 0 else 4
    z0 = EC * chunk
    say("dequant exhaustive chunk", chunk, "zeros", z0, z0 + EC - 1, "rb", rb)
    arrays, q13, s13, q2, s2, zz = chunk_inputs(z0)
    dims = abi.make_dims(EC, H, I, rb)
    bank = to_dev(abi.awq_moe_prepare(dims, *arrays))
    got = abi.awq_moe_dequant(dims, bank, 0, EC, 0)                        # [EC][H][2I]
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    qf = q13.astype(np.float32)
    sf = np.repeat(s13.astype(np.float32), 32, axis=0)                     # [H][2I]
    for e in range(EC):
        want = (qf - np.float32(zz[e])) * sf
        if not np.array_equal(got[e].view(np.uint32), want.view(np.uint32)):
            bad = np.argwhere(got[e].view(np.uint32) != want.view(np.uint32))[0]
            raise AssertionError(f"W13 expert {e} (z={zz[e]}) at {tuple(bad)}: {got[e][tuple(bad)]} vs {want[tuple(bad)]}")
    if chunk == 0:
        got2 = abi.awq_moe_dequant(dims, bank, 0, EC, 1).cpu().numpy()    # [EC][I][H]
        sf2 = np.repeat(s2.astype(np.float32), 32, axis=0)
        for e in range(EC):
            want2 = (q2.astype(np.float32) - np.float32(zz[e])) * sf2
            assert np.array_equal(got2[e].view(np.uint32), want2.view(np.uint32)), e
