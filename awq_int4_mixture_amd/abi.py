"""Thin Python binding of libawq_moe.so (include/awq_moe.h), same names as the C ABI.

The binding only marshals arguments: it checks dtypes, devices and
contiguity of torch tensors, passes raw pointers and the current HIP stream
to the library, and turns error codes into exceptions. Every step of the
stage runs in the library's gfx950 kernels; PyTorch supplies device memory
and streams. Importing this module fails when the library is not built.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libawq_moe.so")

OK, EINVAL, EUNSUPPORTED, ENOSPC, EHIP = 0, -1, -2, -3, -4
MAX_TOKENS, MAX_TOPK = 8, 32
STATUS_BAD_ID = 1
W13_TABLE, W13_PAIR, W13_SINGLE, W13_SINGLE_TWO_TILES = 0, 1, 2, 3
W2_TABLE, W2_SEG_MOST, W2_SEG_FEWER = 0, 1, 2
NOALLOC_SCRATCH_BYTES = 256 + 512 * 1024
WS_STATUS_OFFSET = 0
WS_ACT_OFFSET = 256

EXPORTED = (
    "awq_moe_bank_layout_query", "awq_moe_prepare", "awq_moe_workspace_bytes",
    "awq_moe_route_compact", "awq_moe_decode", "awq_moe_decode_noalloc", "awq_moe_decode_rmsnorm_residual",
    "awq_moe_decode_table", "awq_moe_decode_forms",
    "awq_moe_w13_swiglu", "awq_moe_w2_reduce",
    "awq_moe_dequant", "awq_moe_router_topk", "awq_moe_residual_rmsnorm", "awq_moe_router_residual",
    "awq_moe_router_gemv", "awq_moe_prefill_workspace_bytes", "awq_moe_prefill", "awq_moe_last_error",
)


class AwqMoeError(RuntimeError):
    def __init__(self, code: int, func: str, msg: str):
        super().__init__(f"{func} failed with {code}: {msg}")
        self.code = code


class awq_moe_dims(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("meta_bytes", ctypes.c_int32)]


class awq_moe_bank_layout(ctypes.Structure):
    _fields_ = [("w13_off", ctypes.c_uint64), ("w13_meta_off", ctypes.c_uint64),
                ("w2_off", ctypes.c_uint64), ("w2_meta_off", ctypes.c_uint64),
                ("expert_bytes", ctypes.c_uint64), ("total_bytes", ctypes.c_uint64)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m awq_int4_mixture_amd.build`")
    # PyTorch-ROCm ships its own HIP runtime (same soname, libamdhip64.so.7).
    # Load torch first so the library binds to that runtime instead of
    # bringing a second HIP/HSA runtime into the process; two runtimes
    # cannot share the device or each other's memory and streams.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, U64, V = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_void_p
    D = ctypes.POINTER(awq_moe_dims)
    sig = {
        "awq_moe_bank_layout_query": [D, ctypes.POINTER(awq_moe_bank_layout)],
        "awq_moe_prepare": [D, P, P, P, P, P, P, P, P, P, P, U64],
        "awq_moe_workspace_bytes": [D, I32, I32, ctypes.POINTER(ctypes.c_uint64)],
        "awq_moe_route_compact": [P, I32, I32, I32, P, P, P, P, P, V],
        "awq_moe_decode": [D, P, U64, P, P, P, I32, I32, P, P, U64, V],
        "awq_moe_decode_noalloc": [D, P, U64, P, P, P, I32, I32, P, P, V],
        "awq_moe_decode_rmsnorm_residual": [D, P, U64, P, ctypes.c_float, P, P, I32, I32, P, P, U64, V],
        "awq_moe_decode_table": [D, I32, I32, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)],
        "awq_moe_decode_forms": [D, P, U64, P, P, P, I32, I32, P, P, U64, I32, I32, I32, V],
        "awq_moe_prefill_workspace_bytes": [D, I32, I32, ctypes.POINTER(ctypes.c_uint64)],
        "awq_moe_prefill": [D, P, U64, P, P, P, I32, I32, P, P, U64, V],
        "awq_moe_w13_swiglu": [D, P, U64, P, P, I32, I32, P, U64, V],
        "awq_moe_w2_reduce": [D, P, U64, P, P, I32, I32, P, U64, P, V],
        "awq_moe_dequant": [D, P, U64, I32, I32, I32, P, V],
        "awq_moe_router_topk": [P, I32, I32, I32, P, P, V],
        "awq_moe_residual_rmsnorm": [P, P, I32, I32, ctypes.c_float, P, P, V],
        "awq_moe_router_residual": [P, I32, I32, I32, P, P, P, P, I32, ctypes.c_float, P, P, V],
        "awq_moe_router_gemv": [P, P, I32, I32, ctypes.c_float, P, I32, P, P, P, V],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.awq_moe_last_error.argtypes = []
    lib.awq_moe_last_error.restype = ctypes.c_char_p
    return lib


_lib = _load()


def _check(rc: int, func: str) -> None:
    if rc != OK:
        raise AwqMoeError(rc, func, _lib.awq_moe_last_error().decode())


def make_dims(num_experts: int, hidden: int, inter: int, meta_bytes: int, group_size: int = 32) -> awq_moe_dims:
    return awq_moe_dims(num_experts, hidden, inter, group_size, meta_bytes)


# ---------------------------------------------------------------------------
# host-only entry points
# ---------------------------------------------------------------------------

def awq_moe_bank_layout_query(dims: awq_moe_dims) -> awq_moe_bank_layout:
    out = awq_moe_bank_layout()
    _check(_lib.awq_moe_bank_layout_query(ctypes.byref(dims), ctypes.byref(out)), "awq_moe_bank_layout_query")
    return out


def awq_moe_workspace_bytes(dims: awq_moe_dims, max_tokens: int, topk: int) -> int:
    out = ctypes.c_uint64()
    _check(_lib.awq_moe_workspace_bytes(ctypes.byref(dims), max_tokens, topk, ctypes.byref(out)),
           "awq_moe_workspace_bytes")
    return out.value


def _host(a: np.ndarray, dtype, shape) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.dtype(dtype):
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    if tuple(a.shape) != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {a.shape}")
    return a


def awq_moe_prepare(dims: awq_moe_dims, q_gate, q_up, q_down, s_gate, s_up, s_down, z_gate, z_up, z_down,
                    bank: np.ndarray | None = None) -> np.ndarray:
    """Pack logical weights (host numpy) into a host bank array (uint8)."""
    E, H, I = dims.num_experts, dims.hidden, dims.inter
    G13, G2 = H // 32, I // 32
    arrs = [
        _host(q_gate, np.uint8, (E, H, I)), _host(q_up, np.uint8, (E, H, I)), _host(q_down, np.uint8, (E, I, H)),
        _host(np.asarray(s_gate).view(np.uint16), np.uint16, (E, G13, I)),
        _host(np.asarray(s_up).view(np.uint16), np.uint16, (E, G13, I)),
        _host(np.asarray(s_down).view(np.uint16), np.uint16, (E, G2, H)),
        _host(z_gate, np.uint8, (E, G13, I)), _host(z_up, np.uint8, (E, G13, I)), _host(z_down, np.uint8, (E, G2, H)),
    ]
    total = awq_moe_bank_layout_query(dims).total_bytes
    if bank is None:
        bank = np.empty(total, np.uint8)
    ptrs = [a.ctypes.data for a in arrs]
    _check(_lib.awq_moe_prepare(ctypes.byref(dims), *ptrs, bank.ctypes.data, bank.nbytes), "awq_moe_prepare")
    return bank


def prepare_from_inputs(dims: awq_moe_dims, bi) -> np.ndarray:
    """awq_moe_prepare on an ``inputs.BankInputs``."""
    return awq_moe_prepare(dims, bi.q_gate, bi.q_up, bi.q_down, bi.s_gate, bi.s_up, bi.s_down,
                           bi.z_gate, bi.z_up, bi.z_down)


# ---------------------------------------------------------------------------
# device entry points (torch tensors)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dev(t, dtype, shape=None, name="tensor"):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


@dataclass
class Route:
    active_expert_ids: object
    active_expert_offsets: object
    sorted_slots: object
    num_active: object
    status: object


def alloc_route(n: int, device) -> Route:
    torch = _torch()
    return Route(torch.empty(n, dtype=torch.int32, device=device), torch.empty(n + 1, dtype=torch.int32, device=device),
                 torch.empty(n, dtype=torch.int32, device=device), torch.empty(1, dtype=torch.int32, device=device),
                 torch.empty(1, dtype=torch.int32, device=device))


def awq_moe_route_compact(topk_ids, num_experts: int, out: Route | None = None, stream=None) -> Route:
    torch = _torch()
    M, k = topk_ids.shape
    _dev(topk_ids, torch.int32, name="topk_ids")
    if out is None:
        out = alloc_route(M * k, topk_ids.device)
    _check(_lib.awq_moe_route_compact(
        topk_ids.data_ptr(), M, k, num_experts, _dev(out.active_expert_ids, torch.int32, (M * k,)),
        _dev(out.active_expert_offsets, torch.int32, (M * k + 1,)), _dev(out.sorted_slots, torch.int32, (M * k,)),
        _dev(out.num_active, torch.int32, (1,)), _dev(out.status, torch.int32, (1,)), _stream(stream)),
        "awq_moe_route_compact")
    return out


def awq_moe_decode(dims: awq_moe_dims, bank, x, topk_ids, topk_w, out=None, workspace=None, stream=None):
    torch = _torch()
    M, H = x.shape
    k = topk_ids.shape[1]
    if out is None:
        out = torch.empty((M, H), dtype=torch.float16, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(dims, M, k, x.device)
    _check(_lib.awq_moe_decode(
        ctypes.byref(dims), _dev(bank, torch.uint8, name="bank"), bank.numel(),
        _dev(x, torch.float16, (M, dims.hidden), "x"),
        _dev(topk_ids, torch.int32, (M, k), "topk_ids"), _dev(topk_w, torch.float32, (M, k), "topk_w"), M, k,
        _dev(out, torch.float16, (M, dims.hidden), "out"), _dev(workspace, torch.uint8, name="workspace"),
        workspace.numel(), _stream(stream)), "awq_moe_decode")
    return out


def awq_moe_decode_noalloc(dims: awq_moe_dims, bank, x, topk_ids, topk_w, out=None, status=None, stream=None):
    """awq_moe_decode on the library's fixed scratch (no workspace argument).
    ``status``: an int32 device tensor of one element, or None."""
    torch = _torch()
    M, H = x.shape
    k = topk_ids.shape[1]
    if out is None:
        out = torch.empty((M, H), dtype=torch.float16, device=x.device)
    sp = None if status is None else _dev(status, torch.int32, (1,), "status")
    _check(_lib.awq_moe_decode_noalloc(
        ctypes.byref(dims), _dev(bank, torch.uint8, name="bank"), bank.numel(),
        _dev(x, torch.float16, (M, dims.hidden), "x"),
        _dev(topk_ids, torch.int32, (M, k), "topk_ids"), _dev(topk_w, torch.float32, (M, k), "topk_w"), M, k,
        _dev(out, torch.float16, (M, dims.hidden), "out"), sp, _stream(stream)), "awq_moe_decode_noalloc")
    return out


def awq_moe_decode_rmsnorm_residual(dims: awq_moe_dims, bank, r, topk_ids, topk_w, eps: float = 1e-6, r_next=None,
                                    workspace=None, stream=None):
    """One stacked layer: r_next = fp16(r + stage(fp16(rms_norm(r)))). Returns r_next."""
    torch = _torch()
    M, H = r.shape
    k = topk_ids.shape[1]
    if r_next is None:
        r_next = torch.empty_like(r)
    if workspace is None:
        workspace = alloc_workspace(dims, M, k, r.device)
    _check(_lib.awq_moe_decode_rmsnorm_residual(
        ctypes.byref(dims), _dev(bank, torch.uint8, name="bank"), bank.numel(),
        _dev(r, torch.float16, (M, dims.hidden), "r"), eps,
        _dev(topk_ids, torch.int32, (M, k), "topk_ids"), _dev(topk_w, torch.float32, (M, k), "topk_w"), M, k,
        _dev(r_next, torch.float16, (M, dims.hidden), "r_next"), _dev(workspace, torch.uint8, name="workspace"),
        workspace.numel(), _stream(stream)), "awq_moe_decode_rmsnorm_residual")
    return r_next


def awq_moe_decode_table(dims: awq_moe_dims, M: int, topk: int) -> tuple[int, int]:
    """(W13 form, W2 form) the tactic table picks for (dims, M, topk)."""
    a, b = ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.awq_moe_decode_table(ctypes.byref(dims), M, topk, ctypes.byref(a), ctypes.byref(b)),
           "awq_moe_decode_table")
    return a.value, b.value


def awq_moe_decode_forms(dims: awq_moe_dims, bank, x, topk_ids, topk_w, w13_form: int, w2_form: int, stages: int = 3,
                         out=None, workspace=None, stream=None):
    """awq_moe_decode with forced kernel forms (0 = the table's). stages: 1 W13, 2 W2, 3 both."""
    torch = _torch()
    M, k = topk_ids.shape
    H = dims.hidden
    if out is None and stages & 2:
        out = torch.empty((M, H), dtype=torch.float16, device=topk_ids.device)
    if workspace is None:
        workspace = alloc_workspace(dims, M, k, topk_ids.device)
    xp = _dev(x, torch.float16, (M, H), "x") if stages & 1 else None
    wp = _dev(topk_w, torch.float32, (M, k), "topk_w") if stages & 2 else None
    op = _dev(out, torch.float16, (M, H), "out") if stages & 2 else None
    _check(_lib.awq_moe_decode_forms(
        ctypes.byref(dims), _dev(bank, torch.uint8, name="bank"), bank.numel(), xp,
        _dev(topk_ids, torch.int32, (M, k), "topk_ids"), wp, M, k, op,
        _dev(workspace, torch.uint8, name="workspace"), workspace.numel(), w13_form, w2_form, stages,
        _stream(stream)), "awq_moe_decode_forms")
    return out if stages & 2 else workspace


def awq_moe_prefill_workspace_bytes(dims: awq_moe_dims, max_tokens: int, topk: int) -> int:
    out = ctypes.c_uint64()
    _check(_lib.awq_moe_prefill_workspace_bytes(ctypes.byref(dims), max_tokens, topk, ctypes.byref(out)),
           "awq_moe_prefill_workspace_bytes")
    return out.value


def alloc_prefill_workspace(dims: awq_moe_dims, max_tokens: int, topk: int, device="cuda"):
    """An indexed-prefill workspace (needs no initialisation)."""
    torch = _torch()
    return torch.empty(awq_moe_prefill_workspace_bytes(dims, max_tokens, topk), dtype=torch.uint8, device=device)


def awq_moe_prefill(dims: awq_moe_dims, bank, x, topk_ids, topk_w, out=None, workspace=None, stream=None):
    """The stage for M in [9, 4096] tokens (expert-major, matrix cores)."""
    torch = _torch()
    M, H = x.shape
    k = topk_ids.shape[1]
    if out is None:
        out = torch.empty((M, H), dtype=torch.float16, device=x.device)
    if workspace is None:
        workspace = alloc_prefill_workspace(dims, M, k, x.device)
    _check(_lib.awq_moe_prefill(
        ctypes.byref(dims), _dev(bank, torch.uint8, name="bank"), bank.numel(),
        _dev(x, torch.float16, (M, dims.hidden), "x"),
        _dev(topk_ids, torch.int32, (M, k), "topk_ids"), _dev(topk_w, torch.float32, (M, k), "topk_w"), M, k,
        _dev(out, torch.float16, (M, dims.hidden), "out"), _dev(workspace, torch.uint8, name="workspace"),
        workspace.numel(), _stream(stream)), "awq_moe_prefill")
    return out


def alloc_workspace(dims: awq_moe_dims, max_tokens: int, topk: int, device="cuda"):
    """A decode workspace (zero-filled so that unused rows read as zero)."""
    torch = _torch()
    return torch.zeros(awq_moe_workspace_bytes(dims, max_tokens, topk), dtype=torch.uint8, device=device)


def workspace_act(workspace, M: int, topk: int, inter: int):
    """View of the fp16 intermediate act[M*topk][inter] (indexed by slot) inside a workspace."""
    torch = _torch()
    nbytes = M * topk * inter * 2
    return workspace[WS_ACT_OFFSET:WS_ACT_OFFSET + nbytes].view(torch.float16).view(M * topk, inter)


def awq_moe_w13_swiglu(dims: awq_moe_dims, bank, x, topk_ids, workspace=None, stream=None):
    """Runs W13 + SwiGLU; returns the workspace holding act and the status."""
    torch = _torch()
    M, k = topk_ids.shape
    if workspace is None:
        workspace = alloc_workspace(dims, M, k, x.device)
    _check(_lib.awq_moe_w13_swiglu(
        ctypes.byref(dims), _dev(bank, torch.uint8, name="bank"), bank.numel(),
        _dev(x, torch.float16, (M, dims.hidden), "x"), _dev(topk_ids, torch.int32, (M, k), "topk_ids"), M, k,
        _dev(workspace, torch.uint8, name="workspace"), workspace.numel(), _stream(stream)), "awq_moe_w13_swiglu")
    return workspace


def awq_moe_w2_reduce(dims: awq_moe_dims, bank, topk_ids, topk_w, workspace, out=None, stream=None):
    """W2 + reduction from the act in ``workspace`` (as awq_moe_w13_swiglu left it)."""
    torch = _torch()
    M, k = topk_w.shape
    if out is None:
        out = torch.empty((M, dims.hidden), dtype=torch.float16, device=topk_w.device)
    _check(_lib.awq_moe_w2_reduce(
        ctypes.byref(dims), _dev(bank, torch.uint8, name="bank"), bank.numel(),
        _dev(topk_ids, torch.int32, (M, k), "topk_ids"),
        _dev(topk_w, torch.float32, (M, k), "topk_w"), M, k, _dev(workspace, torch.uint8, name="workspace"),
        workspace.numel(), _dev(out, torch.float16, (M, dims.hidden), "out"), _stream(stream)), "awq_moe_w2_reduce")
    return out


def awq_moe_dequant(dims: awq_moe_dims, bank, expert_begin: int, expert_count: int, which: int, out=None, stream=None):
    torch = _torch()
    K, N = (dims.hidden, 2 * dims.inter) if which == 0 else (dims.inter, dims.hidden)
    if out is None:
        out = torch.empty((expert_count, K, N), dtype=torch.float32, device=bank.device)
    _check(_lib.awq_moe_dequant(ctypes.byref(dims), _dev(bank, torch.uint8, name="bank"), bank.numel(), expert_begin,
                                expert_count, which, _dev(out, torch.float32, (expert_count, K, N), "out"),
                                _stream(stream)), "awq_moe_dequant")
    return out


def awq_moe_router_topk(logits, topk: int, ids=None, w=None, stream=None):
    """Top-k + softmax of fp32 logits [M][E] -> (ids int32 [M][k], w fp32 [M][k])."""
    torch = _torch()
    M, E = logits.shape
    if ids is None:
        ids = torch.empty((M, topk), dtype=torch.int32, device=logits.device)
    if w is None:
        w = torch.empty((M, topk), dtype=torch.float32, device=logits.device)
    _check(_lib.awq_moe_router_topk(_dev(logits, torch.float32, (M, E), "logits"), M, E, topk,
                                    _dev(ids, torch.int32, (M, topk), "ids"), _dev(w, torch.float32, (M, topk), "w"),
                                    _stream(stream)), "awq_moe_router_topk")
    return ids, w


def awq_moe_residual_rmsnorm(r, delta=None, eps: float = 1e-6, r_next=None, x=None, stream=None):
    """r_next = fp16(r + delta); x = fp16(rms_norm(r_next)). Returns (r_next, x)."""
    torch = _torch()
    M, H = r.shape
    if r_next is None:
        r_next = torch.empty_like(r)
    if x is None:
        x = torch.empty_like(r)
    dp = None if delta is None else _dev(delta, torch.float16, (M, H), "delta")
    _check(_lib.awq_moe_residual_rmsnorm(_dev(r, torch.float16, (M, H), "r"), dp, M, H, eps,
                                         _dev(r_next, torch.float16, (M, H), "r_next"),
                                         _dev(x, torch.float16, (M, H), "x"), _stream(stream)),
           "awq_moe_residual_rmsnorm")
    return r_next, x


def awq_moe_router_residual(logits, topk: int, r, delta=None, eps: float = 1e-6, ids=None, w=None, r_next=None,
                            x=None, stream=None):
    """Router top-k + softmax and the residual/RMS-norm step in one launch.
    Returns (ids, w, r_next, x)."""
    torch = _torch()
    M, E = logits.shape
    H = r.shape[1]
    if ids is None:
        ids = torch.empty((M, topk), dtype=torch.int32, device=logits.device)
    if w is None:
        w = torch.empty((M, topk), dtype=torch.float32, device=logits.device)
    if r_next is None:
        r_next = torch.empty_like(r)
    if x is None:
        x = torch.empty_like(r)
    dp = None if delta is None else _dev(delta, torch.float16, (M, H), "delta")
    _check(_lib.awq_moe_router_residual(
        _dev(logits, torch.float32, (M, E), "logits"), M, E, topk, _dev(ids, torch.int32, (M, topk), "ids"),
        _dev(w, torch.float32, (M, topk), "w"), _dev(r, torch.float16, (M, H), "r"), dp, H, eps,
        _dev(r_next, torch.float16, (M, H), "r_next"), _dev(x, torch.float16, (M, H), "x"), _stream(stream)),
        "awq_moe_router_residual")
    return ids, w, r_next, x


def awq_moe_router_gemv(r, router_w, delta=None, eps: float = 1e-6, r_next=None, x=None, logits=None, stream=None):
    """Residual + RMS norm, then fp32 logits = x . router_w^T (router_w fp16 [E][H]).
    Returns (r_next, x, logits)."""
    torch = _torch()
    M, H = r.shape
    E = router_w.shape[0]
    if r_next is None:
        r_next = torch.empty_like(r)
    if x is None:
        x = torch.empty_like(r)
    if logits is None:
        logits = torch.empty((M, E), dtype=torch.float32, device=r.device)
    dp = None if delta is None else _dev(delta, torch.float16, (M, H), "delta")
    _check(_lib.awq_moe_router_gemv(
        _dev(r, torch.float16, (M, H), "r"), dp, M, H, eps, _dev(router_w, torch.float16, (E, H), "router_w"), E,
        _dev(r_next, torch.float16, (M, H), "r_next"), _dev(x, torch.float16, (M, H), "x"),
        _dev(logits, torch.float32, (M, E), "logits"), _stream(stream)), "awq_moe_router_gemv")
    return r_next, x, logits


def awq_moe_last_error() -> str:
    return _lib.awq_moe_last_error().decode()


# ---------------------------------------------------------------------------
# convenience: a decoder that owns its workspace (no allocation per call)
# ---------------------------------------------------------------------------

class Decoder:
    """Holds a device bank and a workspace sized for up to ``max_tokens`` x ``topk``."""

    def __init__(self, dims: awq_moe_dims, bank, topk: int, max_tokens: int = MAX_TOKENS):
        torch = _torch()
        self.dims, self.bank, self.topk = dims, bank, topk
        self.workspace = alloc_workspace(dims, max_tokens, topk, bank.device)

    def __call__(self, x, topk_ids, topk_w, out=None, stream=None):
        return awq_moe_decode(self.dims, self.bank, x, topk_ids, topk_w, out=out, workspace=self.workspace,
                              stream=stream)

    def status(self) -> int:
        """The status word of the last decode (reads the device: synchronises)."""
        return int(self.workspace[WS_STATUS_OFFSET:WS_STATUS_OFFSET + 4].view(_torch().int32).item())
