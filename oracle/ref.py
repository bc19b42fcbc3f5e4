"""Float64 reference of the AWQ int4 MoE expert stage (test infrastructure).

Only tests, the smoke check and the benchmark's CPU baseline may use this.

The stage, as the pages describe it (PR #520 "Narrow Qwen3.8 AWQ active
grouped decode", Purpose and Implementation; fork PR #12 "Add opt-in
native-g32 AWQ QPN M1 dispatch", Purpose and stack): for each decode token,
take its top-k routed experts, compact them into active-expert ids and
offsets, run W13 (gate/up interleaved, K = hidden, N = 2*inter) with SwiGLU,
then W2 (K = inter, N = hidden), and sum the expert outputs weighted by the
router weights. Weights are AWQ int4 with one {fp16 scale, u8 zero} per
group of 32 along K.

Fork PR #12 (Numerical acceptance) evaluates kernels against an
independently decoded-weight FP64 reference, with W2 checked on its own
intermediate; that is what this module is. Everything is float64 from
exactly converted inputs; no blocking, fusion or reordering is applied.

Readings where the pages are silent (each also listed in the design notes):
  * dequantised weight  w = (q - z) * s, group along K (AWQ convention);
  * SwiGLU              act = silu(gate) * up, silu(g) = g / (1 + e^-g);
  * compaction order    active experts in ascending id, rows inside a
                        segment in ascending flat slot s = t*k + j;
  * invalid ids         ids outside [0, E) set status bit 0 and contribute 0;
  * weights             router weights are used as given (no renormalising).
"""

from __future__ import annotations

import numpy as np

GROUP = 32
STATUS_BAD_ID = 1


# ---------------------------------------------------------------------------
# dequantisation
# ---------------------------------------------------------------------------

def dequant(q: np.ndarray, s: np.ndarray, z: np.ndarray) -> np.ndarray:
    """W[k][n] = (q[k][n] - z[k//32][n]) * s[k//32][n], in float64.

    q uint8 [K][N] (0..15), s fp16 [K/32][N], z uint8 [K/32][N].
    """
    K, N = q.shape
    g = np.arange(K) // GROUP
    qf = q.astype(np.float64)
    zf = z.astype(np.float64)[g, :]
    sf = s.astype(np.float64)[g, :]
    return (qf - zf) * sf


def expert_dense(w):
    """(Wg [H][I], Wu [H][I], Wd [I][H]) float64 of one ``ExpertWeights``."""
    return (dequant(w.q_gate, w.s_gate, w.z_gate),
            dequant(w.q_up, w.s_up, w.z_up),
            dequant(w.q_down, w.s_down, w.z_down))


def w13_interleaved(w) -> np.ndarray:
    """Dense W13 [H][2I] with column 2i = gate i and 2i+1 = up i (fork PR #12: W13 interleaving)."""
    Wg, Wu, _ = expert_dense(w)
    out = np.empty((Wg.shape[0], 2 * Wg.shape[1]))
    out[:, 0::2] = Wg
    out[:, 1::2] = Wu
    return out


# ---------------------------------------------------------------------------
# routing compaction
# ---------------------------------------------------------------------------

def route_compact(topk_ids: np.ndarray, num_experts: int) -> dict:
    """Compact a [M][k] id tensor into active-expert segments.

    PR #520 (Purpose and Implementation) keeps multi-row active-expert
    segments with offsets-based scheduling and has the op write
    active_expert_ids and active_expert_offsets. The order is this build's
    reading: experts ascending, rows in a segment by ascending flat slot,
    invalid slots (id outside [0, E)) after all valid ones in slot order.

    Returns n = M*k sized arrays:
      active_ids[n]     segment -> expert id, -1 past num_active
      offsets[n+1]      segment row ranges; entries past num_active equal V
      sorted_slots[n]   row -> flat slot
      num_active, num_valid (V), status (bit 0: some id was out of range)
    """
    flat = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    n = flat.size
    slots = np.arange(n)
    valid = (flat >= 0) & (flat < num_experts)
    vs = slots[valid]
    order = vs[np.lexsort((vs, flat[vs]))]          # by id, then slot
    sorted_slots = np.concatenate([order, slots[~valid]]).astype(np.int32)
    uniq, counts = np.unique(flat[vs], return_counts=True)
    A, V = uniq.size, int(valid.sum())
    active_ids = np.full(n, -1, np.int32)
    active_ids[:A] = uniq
    offsets = np.full(n + 1, V, np.int32)
    offsets[0] = 0
    offsets[1:A + 1] = np.cumsum(counts)
    status = 0 if valid.all() else STATUS_BAD_ID
    return dict(active_ids=active_ids, offsets=offsets, sorted_slots=sorted_slots,
                num_active=A, num_valid=V, status=status)


# ---------------------------------------------------------------------------
# stage pieces
# ---------------------------------------------------------------------------

def silu(g: np.ndarray) -> np.ndarray:
    """g * sigmoid(g), evaluated without overflow for either sign."""
    g = np.asarray(g, dtype=np.float64)
    e = np.exp(-np.abs(g))
    sig = np.where(g >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return g * sig


def w13_swiglu_rows(x: np.ndarray, route: dict, topk: int, weights_of) -> np.ndarray:
    """act rows in sorted order: act[r] = silu(x_t Wg_e) * (x_t Wu_e).

    x fp16 [M][H]; ``weights_of(e)`` returns an ``ExpertWeights``. Rows past
    the valid count are left at zero. Result float64 [n][I].
    """
    xs = np.asarray(x).astype(np.float64)
    n = route["sorted_slots"].size
    act = None
    for a in range(route["num_active"]):
        e = int(route["active_ids"][a])
        Wg, Wu, _ = expert_dense(weights_of(e))
        if act is None:
            act = np.zeros((n, Wg.shape[1]))
        for r in range(route["offsets"][a], route["offsets"][a + 1]):
            t = int(route["sorted_slots"][r]) // topk
            act[r] = silu(xs[t] @ Wg) * (xs[t] @ Wu)
    if act is None:
        I = weights_of(0).q_gate.shape[1]
        act = np.zeros((n, I))
    return act


def w2_reduce(act_rows: np.ndarray, topk_w: np.ndarray, route: dict, topk: int,
              weights_of, M: int, H: int) -> np.ndarray:
    """out[t] = sum over rows r of token t of w[t][j] * (act[r] @ Wd_e), float64 [M][H].

    ``act_rows`` [n][I] in sorted row order (any dtype; converted exactly).
    Rows of invalid slots contribute nothing.
    """
    a64 = np.asarray(act_rows).astype(np.float64)
    w64 = np.asarray(topk_w).astype(np.float64).reshape(-1)
    out = np.zeros((M, H))
    for a in range(route["num_active"]):
        e = int(route["active_ids"][a])
        _, _, Wd = expert_dense(weights_of(e))
        for r in range(route["offsets"][a], route["offsets"][a + 1]):
            slot = int(route["sorted_slots"][r])
            out[slot // topk] += w64[slot] * (a64[r] @ Wd)
    return out


def w2_rounding_bound(act_rows: np.ndarray, topk_w: np.ndarray, route: dict, topk: int,
                      weights_of, M: int, H: int):
    """Informational bound on |fp16 out - exact out| for W2 + reduction from a
    given act (the pages print no bound formula; this is the standard one).

    An fp32 evaluation that accumulates the n products w * act[i] * Wd[i][c]
    of token t in any order errs by at most gamma_n * sum of their magnitudes
    (Higham's dot-product bound), and the final rounding to fp16 adds at most
    half an fp16 ulp, 2^-11 * |out|. Here n = (valid rows of the token) * I,
    plus one per row for the weighting. Returns (bound [M][H], exact out).
    """
    a64 = np.asarray(act_rows).astype(np.float64)
    w64 = np.asarray(topk_w).astype(np.float64).reshape(-1)
    out = np.zeros((M, H))
    mag = np.zeros((M, H))
    nterms = np.zeros(M, dtype=np.int64)
    for a in range(route["num_active"]):
        e = int(route["active_ids"][a])
        _, _, Wd = expert_dense(weights_of(e))
        for r in range(route["offsets"][a], route["offsets"][a + 1]):
            slot = int(route["sorted_slots"][r])
            t = slot // topk
            out[t] += w64[slot] * (a64[r] @ Wd)
            mag[t] += abs(w64[slot]) * (np.abs(a64[r]) @ np.abs(Wd))
            nterms[t] += Wd.shape[0] + 1
    gam = np.array([higham_gamma(int(n)) for n in nterms])
    return gam[:, None] * mag + 2.0 ** -11 * np.abs(out), out


def moe_stage(x: np.ndarray, topk_ids: np.ndarray, topk_w: np.ndarray, num_experts: int,
              weights_of) -> np.ndarray:
    """The whole stage for M tokens, float64 [M][H] (no intermediate rounding)."""
    M, k = np.asarray(topk_ids).shape
    route = route_compact(topk_ids, num_experts)
    act = w13_swiglu_rows(x, route, k, weights_of)
    return w2_reduce(act, topk_w, route, k, weights_of, M, np.asarray(x).shape[1])


# ---------------------------------------------------------------------------
# router selection (48-layer stack workload)
# ---------------------------------------------------------------------------

def topk_softmax(logits: np.ndarray, k: int):
    """Top-k of fp32 logits per token, then softmax over the k selected.

    Selection compares the fp32 values exactly; ties go to the lower expert
    id; ids are listed by descending logit. The pages leave the router
    unchanged (fork PR #12, Purpose and stack), so this form is this
    build's reading. Returns (ids int32 [M][k], w float64 [M][k]).
    """
    lg = np.asarray(logits, dtype=np.float32)
    M, E = lg.shape
    ids = np.empty((M, k), np.int32)
    w = np.empty((M, k))
    for t in range(M):
        order = np.lexsort((np.arange(E), -lg[t].astype(np.float64)))
        sel = order[:k]
        ids[t] = sel
        v = lg[t, sel].astype(np.float64)
        with np.errstate(invalid="ignore"):      # inf - inf and NaN give NaN weights, as in fp32
            p = np.exp(v - v.max())
            w[t] = p / p.sum()
    return ids, w


def rms_norm(r: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """Parameter-free RMS normalisation of each row, float64."""
    r64 = np.asarray(r).astype(np.float64)
    return r64 / np.sqrt((r64 * r64).mean(axis=-1, keepdims=True) + eps)


# ---------------------------------------------------------------------------
# comparison helpers
# ---------------------------------------------------------------------------

def errors(gpu: np.ndarray, ref: np.ndarray) -> dict:
    """max-abs, max|ref|, relative L2 of a result against the reference."""
    g = np.asarray(gpu).astype(np.float64)
    r = np.asarray(ref).astype(np.float64)
    d = g - r
    mx = float(np.abs(r).max()) if r.size else 0.0
    nr = float(np.linalg.norm(r))
    return dict(max_abs=float(np.abs(d).max()) if d.size else 0.0, max_ref=mx,
                rel_l2=float(np.linalg.norm(d) / nr) if nr > 0 else float(np.linalg.norm(d)))


def within_gate(gpu: np.ndarray, ref: np.ndarray, max_rel: float = 4e-3, l2: float = 2e-3) -> tuple[bool, dict]:
    """max|gpu - ref| <= 4e-3 max|ref| and ||gpu - ref|| / ||ref|| <= 2e-3.

    When max|ref| < 2^-14 the relative gates are replaced by an absolute
    bound of 2^-24 (PR #522 addendum, Reader-level evidence, records a
    relative-only gate failing on a tiny value of that size).
    """
    e = errors(gpu, ref)
    if e["max_ref"] < 2.0 ** -14:
        ok = e["max_abs"] <= 2.0 ** -24
    else:
        ok = e["max_abs"] <= max_rel * e["max_ref"] and e["rel_l2"] <= l2
    return ok, e


def higham_gamma(n: int, u: float = 2.0 ** -24) -> float:
    """gamma_n = n u / (1 - n u), the standard bound for an n-term fp32 dot product."""
    return n * u / (1.0 - n * u)
