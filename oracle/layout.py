"""Oracle packer and decoder of the prepared AWQ weight bank (test infrastructure).

Only tests, the smoke check and the benchmark's CPU baseline may use this.

What the pages fix, and what this layout adds
---------------------------------------------
* Weights are 4-bit values with one {fp16 scale, u8 zero} record per group of
  32 (PR #520, Purpose: "native or effective group 32"; PR #522, Purpose:
  the 3-byte {FP16 scale, u8 zero} metadata).
* Records are stored either padded to 4 bytes or as compact 3-byte records,
  and both decode to identical weights (PR #522, Default switch section).
* A 3-byte record tile is 96 bytes = 24 aligned dwords = 32 records, the last
  record starting at byte 93 (PR #522, Purpose, first bullet).
* W13 is gate and up interleaved (fork PR #12, Purpose and stack: "W13
  interleaving").

Everything else (the order of units and records) is this bank's own layout,
chosen for 64-lane wavefronts; the byte-level specification is:

Dims: E experts, H hidden, I inter, group G = 32, record bytes RB in {3, 4};
H and I multiples of 32. Each expert block has four sections, each padded
to a multiple of 256 bytes, in this order: W13 units, W13 records, W2 units,
W2 records.

A *unit* is 16 bytes: the 32 packed values of one group g (k = 32g .. 32g+31)
of one output column n. Dword d (0..3, little endian) holds k = 32g + 8d + p
for p = 0..7, value p at bit 4*(p >> 1) + 16*(p & 1).

A *record* is RB bytes: bytes 0-1 the fp16 scale (little endian), byte 2
the zero; for RB = 4, byte 3 is 0.

Both matrices use one tiled placement, for a matrix with K rows (K = H for
W13, K = I for W2), G = K/32 groups and N columns. For W13 (N = 2I) column
n = 2i is gate column i and n = 2i + 1 is up column i; for W2, N = H.
Columns form tiles of 16; with L = 4*G:
  nt = n // 16, c = n % 16, quad = c // 4, j = c % 4, t = 4*g + quad
  unit offset   = nt*256*G + (j*L + t)*16
  record offset = nt*16*G*RB + (4*t + j)*RB

Lane t of a tile owns units j = 0..3 (four adjacent columns of one group),
its four unit loads are each contiguous across the tile's lanes, and its
four records are one aligned 12- or 16-byte run. One tile is one contiguous
run of 256*G unit bytes and one of 16*G*RB record bytes.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

GROUP = 32
SECTION_ALIGN = 256
# Bit position of value p (0..7) inside its dword.
_NIBBLE_SHIFT = [4 * (p >> 1) + 16 * (p & 1) for p in range(8)]


def _pad(n: int) -> int:
    return (n + SECTION_ALIGN - 1) // SECTION_ALIGN * SECTION_ALIGN


@dataclass(frozen=True)
class Dims:
    num_experts: int
    hidden: int
    inter: int
    meta_bytes: int
    group_size: int = GROUP

    def check(self) -> None:
        if self.group_size != GROUP:
            raise ValueError("group size must be 32")
        if self.meta_bytes not in (3, 4):
            raise ValueError("meta_bytes must be 3 or 4")
        if self.hidden <= 0 or self.hidden % 32 or self.inter <= 0 or self.inter % 32:
            raise ValueError("hidden and inter must be positive multiples of 32")
        if self.num_experts <= 0:
            raise ValueError("num_experts must be positive")


@dataclass(frozen=True)
class Layout:
    w13_units: int      # bytes of W13 units (unpadded)
    w13_meta: int       # bytes of W13 records (unpadded)
    w2_units: int
    w2_meta: int
    w13_off: int        # section offsets inside one expert block
    w13_meta_off: int
    w2_off: int
    w2_meta_off: int
    expert_bytes: int
    total_bytes: int


def layout(d: Dims) -> Layout:
    d.check()
    H, I, RB = d.hidden, d.inter, d.meta_bytes
    w13_units = (H // GROUP) * (2 * I) * 16
    w13_meta = (H // GROUP) * (2 * I) * RB
    w2_units = (I // GROUP) * H * 16
    w2_meta = (I // GROUP) * H * RB
    o0 = 0
    o1 = o0 + _pad(w13_units)
    o2 = o1 + _pad(w13_meta)
    o3 = o2 + _pad(w2_units)
    eb = o3 + _pad(w2_meta)
    return Layout(w13_units, w13_meta, w2_units, w2_meta, o0, o1, o2, o3, eb, eb * d.num_experts)


# ---------------------------------------------------------------------------
# unit / record placement
# ---------------------------------------------------------------------------

def tile_unit_offset(K: int, g, n):
    """Byte offset of the unit of (group g, column n) in a section whose
    matrix has K rows."""
    G = K // GROUP
    L = 4 * G
    nt, c = n // 16, n % 16
    quad, j = c // 4, c % 4
    t = 4 * g + quad
    return nt * 256 * G + (j * L + t) * 16


def tile_record_offset(K: int, RB: int, g, n):
    G = K // GROUP
    nt, c = n // 16, n % 16
    quad, j = c // 4, c % 4
    t = 4 * g + quad
    return nt * 16 * G * RB + (4 * t + j) * RB


def w13_unit_offset(H: int, g, n):
    return tile_unit_offset(H, g, n)


def w13_record_offset(H: int, RB: int, g, n):
    return tile_record_offset(H, RB, g, n)


def w2_unit_offset(I: int, g, n):
    return tile_unit_offset(I, g, n)


def w2_record_offset(I: int, RB: int, g, n):
    return tile_record_offset(I, RB, g, n)


# ---------------------------------------------------------------------------
# packing
# ---------------------------------------------------------------------------

def _unit_dwords(q: np.ndarray) -> np.ndarray:
    """q uint8 [K][N] -> uint32 [K/32][N][4] unit dwords (value p at its shift)."""
    K, N = q.shape
    qk = q.reshape(K // GROUP, 4, 8, N).astype(np.uint32)   # [g][d][p][n]
    dw = np.zeros((K // GROUP, 4, N), np.uint32)
    for p in range(8):
        dw |= qk[:, :, p, :] << np.uint32(_NIBBLE_SHIFT[p])
    return np.ascontiguousarray(dw.transpose(0, 2, 1))     # [g][n][d]


def _records(s: np.ndarray, z: np.ndarray, RB: int) -> np.ndarray:
    """s fp16 [G][N], z uint8 [G][N] -> uint8 [G][N][RB]."""
    sb = np.ascontiguousarray(s.astype(np.float16)).view(np.uint16)
    rec = np.zeros(s.shape + (RB,), np.uint8)
    rec[..., 0] = (sb & 0xFF).astype(np.uint8)
    rec[..., 1] = (sb >> 8).astype(np.uint8)
    rec[..., 2] = z.astype(np.uint8)
    return rec


def _scatter_units(dst: np.ndarray, base: int, dw: np.ndarray, offs: np.ndarray) -> None:
    # dw [G][N][4] uint32, offs [G][N] byte offsets
    b = dw.astype("<u4").view(np.uint8).reshape(dw.shape[0], dw.shape[1], 16)
    idx = (base + offs)[..., None] + np.arange(16)
    dst[idx] = b


def _scatter_records(dst: np.ndarray, base: int, rec: np.ndarray, offs: np.ndarray) -> None:
    RB = rec.shape[-1]
    idx = (base + offs)[..., None] + np.arange(RB)
    dst[idx] = rec


def interleave_w13(a_gate: np.ndarray, a_up: np.ndarray) -> np.ndarray:
    """[..][I] gate and up -> [..][2I] with column 2i = gate i, 2i+1 = up i."""
    out = np.empty(a_gate.shape[:-1] + (2 * a_gate.shape[-1],), a_gate.dtype)
    out[..., 0::2] = a_gate
    out[..., 1::2] = a_up
    return out


def pack_expert(d: Dims, w, out: np.ndarray | None = None) -> np.ndarray:
    """Pack one expert's logical weights (``inputs.ExpertWeights``) into its block."""
    L = layout(d)
    H, I, RB = d.hidden, d.inter, d.meta_bytes
    blk = np.zeros(L.expert_bytes, np.uint8) if out is None else out
    # W13
    q13 = interleave_w13(w.q_gate, w.q_up)
    s13 = interleave_w13(w.s_gate, w.s_up)
    z13 = interleave_w13(w.z_gate, w.z_up)
    g = np.arange(H // GROUP)[:, None]
    n = np.arange(2 * I)[None, :]
    _scatter_units(blk, L.w13_off, _unit_dwords(q13), w13_unit_offset(H, g, n))
    _scatter_records(blk, L.w13_meta_off, _records(s13, z13, RB), w13_record_offset(H, RB, g, n))
    # W2
    g = np.arange(I // GROUP)[:, None]
    n = np.arange(H)[None, :]
    _scatter_units(blk, L.w2_off, _unit_dwords(w.q_down), w2_unit_offset(I, g, n))
    _scatter_records(blk, L.w2_meta_off, _records(w.s_down, w.z_down, RB), w2_record_offset(I, RB, g, n))
    return blk


def pack_bank(d: Dims, bank_inputs) -> np.ndarray:
    """Pack all experts (``inputs.BankInputs``) into one bank byte array."""
    L = layout(d)
    out = np.zeros(L.total_bytes, np.uint8)
    for e in range(d.num_experts):
        pack_expert(d, bank_inputs.expert(e), out[e * L.expert_bytes:(e + 1) * L.expert_bytes])
    return out


# ---------------------------------------------------------------------------
# decoding
# ---------------------------------------------------------------------------

def _gather_units(src: np.ndarray, base: int, offs: np.ndarray) -> np.ndarray:
    idx = (base + offs)[..., None] + np.arange(16)
    b = src[idx]                                         # [G][N][16]
    dw = b.reshape(b.shape[0], b.shape[1], 16).copy().view("<u4")  # [G][N][4]
    G, N = offs.shape
    q = np.empty((G, 4, 8, N), np.uint8)
    for p in range(8):
        q[:, :, p, :] = ((dw >> np.uint32(_NIBBLE_SHIFT[p])) & 0xF).transpose(0, 2, 1)
    return q.reshape(G * GROUP, N)


def _gather_records(src: np.ndarray, base: int, offs: np.ndarray, RB: int):
    idx = (base + offs)[..., None] + np.arange(RB)
    r = src[idx]
    sbits = r[..., 0].astype(np.uint16) | (r[..., 1].astype(np.uint16) << 8)
    s = sbits.view(np.float16)
    z = r[..., 2].copy()
    pad = r[..., 3].copy() if RB == 4 else None
    return s, z, pad


@dataclass
class DecodedExpert:
    q13: np.ndarray   # uint8 [H][2I] interleaved
    s13: np.ndarray   # fp16 [H/32][2I]
    z13: np.ndarray   # uint8 [H/32][2I]
    q2: np.ndarray    # uint8 [I][H]
    s2: np.ndarray    # fp16 [I/32][H]
    z2: np.ndarray    # uint8 [I/32][H]
    pad_ok: bool      # 4-byte records: every pad byte is zero


def decode_expert(d: Dims, bank: np.ndarray, e: int) -> DecodedExpert:
    """Read expert ``e``'s block back into logical (q, s, z) arrays."""
    L = layout(d)
    H, I, RB = d.hidden, d.inter, d.meta_bytes
    blk = bank[e * L.expert_bytes:(e + 1) * L.expert_bytes]
    g = np.arange(H // GROUP)[:, None]
    n = np.arange(2 * I)[None, :]
    q13 = _gather_units(blk, L.w13_off, w13_unit_offset(H, g, n))
    s13, z13, p13 = _gather_records(blk, L.w13_meta_off, w13_record_offset(H, RB, g, n), RB)
    g = np.arange(I // GROUP)[:, None]
    n = np.arange(H)[None, :]
    q2 = _gather_units(blk, L.w2_off, w2_unit_offset(I, g, n))
    s2, z2, p2 = _gather_records(blk, L.w2_meta_off, w2_record_offset(I, RB, g, n), RB)
    pad_ok = RB == 3 or (not p13.any() and not p2.any())
    return DecodedExpert(q13, s13, z13, q2, s2, z2, pad_ok)
