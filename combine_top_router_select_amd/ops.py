"""Python binding of the C ABI (include/moe_route.h), entry point for entry point.

Each function checks the dtype, shape, device and contiguity of every tensor
argument, outputs passed in included, and that the sizes agree with each other
(so that no kernel can write past a buffer the binding was handed), allocates
any output that was not passed in (torch is used for device memory and streams
only), passes raw pointers and the current HIP stream to the library, and
raises MoeError on a non-zero status.  No step of the computation runs here.
Device-side contents (expert ids in range, placement values, slot_row entries
below the row count) are preconditions the kernels clamp but do not check;
check_placement() checks a placement table on the host, on request.
"""
from __future__ import annotations

from typing import Optional

import torch

from ._lib import MoeError, check, lib, status_string  # noqa: F401

__all__ = ["MoeError", "check_placement", "moe_status_string", "moe_workspace_bytes",
           "moe_route_topk", "moe_route_plan",
           "moe_send_counts", "moe_dispatch_permute", "moe_dispatch_permute_dedup",
           "moe_dispatch_permute_noalloc", "moe_route_dispatch",
           "moe_combine", "moe_coselect_counts", "workspace", "moe_expand_workspace_bytes",
           "expand_workspace", "moe_expand_counts", "moe_expand_permute", "moe_expand_reduce",
           "moe_placement_search", "moe_shuffle_fit", "moe_shuffle_predict",
           "moe_shuffle_assign"]


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr() or None


def _dev(t: torch.Tensor, name: str, dtype=None, ndim=None, shape=None, itemsize=None,
         device=None) -> torch.Tensor:
    """Checks that `t` is a contiguous GPU tensor with the given dtype (or one of
    a tuple), number of dimensions, exact shape, element size and device."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other arguments on {device}")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if itemsize is not None and t.element_size() != itemsize:
        raise TypeError(f"{name} must have {itemsize}-byte elements, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got shape {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _out(o: dict, key: str, shape, dtype, device, itemsize=None) -> torch.Tensor:
    """The caller's output buffer `o[key]`, checked against the exact shape and
    type the library will write, or a new one."""
    t = o.get(key)
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if itemsize is not None:
        return _dev(t, key, shape=shape, itemsize=itemsize, device=device)
    return _dev(t, key, dtype, shape=shape, device=device)


def _ws(ws, device) -> torch.Tensor:
    """A workspace: a contiguous 1-D byte tensor on the device (the library
    checks its size)."""
    return _dev(ws, "ws", torch.uint8, ndim=1, device=device)


def _placement(placement, n_experts, device):
    if placement is None:
        return None
    return _dev(placement, "placement", torch.int32, shape=(n_experts,), device=device)


def check_placement(placement, n_experts: int, n_ranks: int) -> None:
    """Opt-in debug helper: checks on the host that an expert -> rank table has
    n_experts entries in [0, n_ranks) and gives every rank exactly
    n_experts / n_ranks experts (each GPU holds E/EP experts), which the
    kernels take as a precondition and do not check.  A GPU tensor is copied
    to the host, so the call synchronises.  Raises ValueError."""
    if n_ranks < 1 or n_experts % n_ranks != 0:
        raise ValueError(f"n_experts {n_experts} is not a multiple of n_ranks {n_ranks}")
    p = torch.as_tensor(placement).detach().to("cpu", torch.int64).reshape(-1)
    if p.numel() != n_experts:
        raise ValueError(f"placement has {p.numel()} entries, expected {n_experts}")
    if p.numel() and (int(p.min()) < 0 or int(p.max()) >= n_ranks):
        raise ValueError(f"placement values must lie in [0, {n_ranks})")
    per = torch.bincount(p, minlength=n_ranks)
    bad = (per != n_experts // n_ranks).nonzero().reshape(-1).tolist()
    if bad:
        raise ValueError(f"ranks {bad[:8]} do not hold exactly {n_experts // n_ranks} experts "
                         f"(counts {per[bad[:8]].tolist()})")


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def moe_status_string(code: int) -> str:
    return status_string(code)


def moe_workspace_bytes(tokens: int, n_experts: int, top_k: int, n_ranks: int,
                        dedup: bool) -> int:
    return int(lib().moe_workspace_bytes(tokens, n_experts, top_k, n_ranks, int(bool(dedup))))


def workspace(tokens, n_experts, top_k, n_ranks, dedup, device) -> torch.Tensor:
    n = moe_workspace_bytes(tokens, n_experts, top_k, n_ranks, dedup)
    if n == 0:
        raise MoeError(1, "moe_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def moe_route_topk(logits, top_k, topk_idx=None, topk_gate=None, stream=None,
                   softmax_all=False):
    """Top-k experts per token and their gates: softmax over the k selected
    logits, or (softmax_all) the softmax over all E logits at the selected
    experts (moe_route_topk_softmax_all)."""
    _dev(logits, "logits", torch.float32, 2)
    T, E = logits.shape
    dev = logits.device
    o = {"topk_idx": topk_idx, "topk_gate": topk_gate}
    topk_idx = _out(o, "topk_idx", (T, top_k), torch.int32, dev)
    topk_gate = _out(o, "topk_gate", (T, top_k), torch.float32, dev)
    fn = lib().moe_route_topk_softmax_all if softmax_all else lib().moe_route_topk
    check(fn(_ptr(logits), T, E, top_k, _ptr(topk_idx), _ptr(topk_gate), _stream(stream)),
          "moe_route_topk_softmax_all" if softmax_all else "moe_route_topk")
    return topk_idx, topk_gate


def _count_outputs(o, E, R, dedup, dev):
    ec = _out(o, "expert_counts", (E,), torch.int32, dev)
    rc = _out(o, "rank_counts", (R,), torch.int32, dev)
    ro = _out(o, "rank_offsets", (R + 1,), torch.int32, dev)
    eo = None if dedup else _out(o, "expert_offsets", (E,), torch.int32, dev)
    return ec, rc, ro, eo


def moe_send_counts(topk_idx, n_experts, n_ranks, placement=None, dedup=False, ws=None,
                    out=None, stream=None):
    """Returns a dict with expert_counts, rank_counts, rank_offsets, expert_offsets
    (None in dedup mode) and the workspace `ws` that the dispatch call needs."""
    _dev(topk_idx, "topk_idx", torch.int32, 2)
    T, k = topk_idx.shape
    dev = topk_idx.device
    placement = _placement(placement, n_experts, dev)
    ws = workspace(T, n_experts, k, n_ranks, dedup, dev) if ws is None else _ws(ws, dev)
    ec, rc, ro, eo = _count_outputs(dict(out or {}), n_experts, n_ranks, dedup, dev)
    check(lib().moe_send_counts(_ptr(topk_idx), T, n_experts, k, n_ranks, _ptr(placement),
                                int(bool(dedup)), _ptr(ec), _ptr(rc), _ptr(ro), _ptr(eo),
                                _ptr(ws), ws.numel(), _stream(stream)), "moe_send_counts")
    return {"expert_counts": ec, "rank_counts": rc, "rank_offsets": ro,
            "expert_offsets": eo, "ws": ws}


def moe_route_plan(logits, top_k, n_ranks, placement=None, dedup=False, softmax_all=False,
                   topk_idx=None, topk_gate=None, ws=None, out=None, coselect=None,
                   coselect_tokens=None, stream=None):
    """moe_route_topk, moe_send_counts and (with `coselect`, an [E][E] int32
    matrix that is accumulated into) moe_coselect_counts over the first
    `coselect_tokens` tokens (default all) in one call.  Returns (topk_idx,
    topk_gate, counts) with counts as moe_send_counts returns them."""
    _dev(logits, "logits", torch.float32, 2)
    T, E = logits.shape
    dev = logits.device
    o = {"topk_idx": topk_idx, "topk_gate": topk_gate}
    topk_idx = _out(o, "topk_idx", (T, top_k), torch.int32, dev)
    topk_gate = _out(o, "topk_gate", (T, top_k), torch.float32, dev)
    placement = _placement(placement, E, dev)
    ws = workspace(T, E, top_k, n_ranks, dedup, dev) if ws is None else _ws(ws, dev)
    ec, rc, ro, eo = _count_outputs(dict(out or {}), E, n_ranks, dedup, dev)
    ncs = 0
    if coselect is not None:
        _dev(coselect, "coselect", torch.int32, shape=(E, E), device=dev)
        ncs = T if coselect_tokens is None else int(coselect_tokens)
    check(lib().moe_route_plan(_ptr(logits), T, E, top_k, int(bool(softmax_all)), n_ranks,
                               _ptr(placement), int(bool(dedup)), _ptr(topk_idx),
                               _ptr(topk_gate), _ptr(ec), _ptr(rc), _ptr(ro), _ptr(eo), ncs,
                               _ptr(coselect), _ptr(ws), ws.numel(), _stream(stream)),
          "moe_route_plan")
    return topk_idx, topk_gate, {"expert_counts": ec, "rank_counts": rc, "rank_offsets": ro,
                                 "expert_offsets": eo, "ws": ws}


def _x_bpe(x, name="x"):
    _dev(x, name, None, 2)
    if x.element_size() not in (1, 2, 4):
        raise TypeError(f"{name} must have 1-, 2- or 4-byte elements")
    return x.element_size()


def _routed(x, topk_idx, topk_gate):
    """Checks the dispatch inputs against each other: ids and gates [T][k] for
    the T rows of x, on x's device.  Returns (T, H, k, bpe, device)."""
    bpe = _x_bpe(x)
    T, H = x.shape
    dev = x.device
    _dev(topk_idx, "topk_idx", torch.int32, 2, device=dev)
    if topk_idx.shape[0] != T:
        raise ValueError(f"topk_idx has {topk_idx.shape[0]} rows, x has {T}")
    k = topk_idx.shape[1]
    _dev(topk_gate, "topk_gate", torch.float32, shape=(T, k), device=dev)
    return T, H, k, bpe, dev


def _coselect_arg(coselect, coselect_tokens, n_experts, T, dev):
    """(tokens, matrix) for the optional co-selection counts of a dispatch."""
    if coselect is None:
        return 0, None
    _dev(coselect, "coselect", torch.int32, shape=(n_experts, n_experts), device=dev)
    n = T if coselect_tokens is None else int(coselect_tokens)
    if not 0 <= n <= T:
        raise ValueError(f"coselect_tokens must be in [0, {T}], got {n}")
    return n, coselect


def moe_dispatch_permute(x, topk_idx, topk_gate, n_experts, n_ranks, ws, out=None, stream=None,
                         coselect=None, coselect_tokens=None):
    """Plain dispatch of the plan in `ws` (from moe_send_counts or
    moe_route_plan with dedup False, same topk_idx).  With `coselect` (an
    [E][E] int32 matrix, accumulated into) the same launch also adds the
    co-selection counts of the first `coselect_tokens` tokens (default all)."""
    T, H, k, bpe, dev = _routed(x, topk_idx, topk_gate)
    _ws(ws, dev)
    ncs, W = _coselect_arg(coselect, coselect_tokens, n_experts, T, dev)
    o = dict(out or {})
    N = T * k
    send = _out(o, "send", (N, H), x.dtype, dev, itemsize=bpe)
    rt = _out(o, "row_token", (N,), torch.int32, dev)
    re = _out(o, "row_expert", (N,), torch.int32, dev)
    rw = _out(o, "row_weight", (N,), torch.float32, dev)
    sr = _out(o, "slot_row", (T, k), torch.int32, dev)
    check(lib().moe_dispatch_permute(_ptr(x), _ptr(topk_idx), _ptr(topk_gate), T, H, n_experts,
                                     k, n_ranks, bpe, _ptr(ws), ws.numel(), _ptr(send),
                                     _ptr(rt), _ptr(re), _ptr(rw), _ptr(sr), ncs, _ptr(W),
                                     _stream(stream)),
          "moe_dispatch_permute")
    return {"send": send, "row_token": rt, "row_expert": re, "row_weight": rw, "slot_row": sr}


def moe_dispatch_permute_dedup(x, topk_idx, topk_gate, n_experts, n_ranks, ws, out=None,
                               stream=None, coselect=None, coselect_tokens=None):
    """Deduplicating dispatch of the plan in `ws` (from moe_send_counts or
    moe_route_plan with dedup True, same topk_idx).  Buffers hold T*k rows.
    `coselect`, `coselect_tokens`: as moe_dispatch_permute."""
    T, H, k, bpe, dev = _routed(x, topk_idx, topk_gate)
    _ws(ws, dev)
    ncs, W = _coselect_arg(coselect, coselect_tokens, n_experts, T, dev)
    o = dict(out or {})
    N = T * k
    send = _out(o, "send", (N, H), x.dtype, dev, itemsize=bpe)
    rt = _out(o, "row_token", (N,), torch.int32, dev)
    rx = _out(o, "row_experts", (N, k), torch.int32, dev)
    rg = _out(o, "row_gates", (N, k), torch.float32, dev)
    rw = _out(o, "row_weight", (N,), torch.float32, dev)
    sr = _out(o, "slot_row", (T, k), torch.int32, dev)
    nr = _out(o, "n_rows", (1,), torch.int32, dev)
    check(lib().moe_dispatch_permute_dedup(_ptr(x), _ptr(topk_idx), _ptr(topk_gate), T, H,
                                           n_experts, k, n_ranks, bpe, _ptr(ws), ws.numel(),
                                           _ptr(send), _ptr(rt), _ptr(rx), _ptr(rg), _ptr(rw),
                                           _ptr(sr), _ptr(nr), ncs, _ptr(W), _stream(stream)),
          "moe_dispatch_permute_dedup")
    return {"send": send, "row_token": rt, "row_experts": rx, "row_gates": rg,
            "row_weight": rw, "slot_row": sr, "n_rows": nr}


def moe_route_dispatch(logits, x, top_k, n_ranks, placement=None, dedup=False, softmax_all=False,
                       ws=None, out=None, coselect=None, coselect_tokens=None, stream=None):
    """moe_route_plan followed by moe_dispatch_permute (dedup: _dedup) in one C
    call, with the same outputs; for small plans two launches instead of three.
    `out` may hold any of the routing, count and dispatch outputs.  With
    `coselect` (an [E][E] int32 matrix, accumulated into) the co-selection
    counts of the first `coselect_tokens` tokens (default all) are added too.
    Returns (topk_idx, topk_gate, counts, rows): counts as moe_route_plan
    returns them (with "ws"), rows as the dispatch call returns them."""
    _dev(logits, "logits", torch.float32, 2)
    T, E = logits.shape
    dev = logits.device
    bpe = _x_bpe(x)
    if x.shape[0] != T or x.device != dev:
        raise ValueError(f"x has {x.shape[0]} rows on {x.device}, logits {T} on {dev}")
    H = x.shape[1]
    k = int(top_k)
    o = dict(out or {})
    idx = _out(o, "topk_idx", (T, k), torch.int32, dev)
    gate = _out(o, "topk_gate", (T, k), torch.float32, dev)
    placement = _placement(placement, E, dev)
    ws = workspace(T, E, k, n_ranks, dedup, dev) if ws is None else _ws(ws, dev)
    ec, rc, ro, eo = _count_outputs(o, E, n_ranks, dedup, dev)
    ncs, W = _coselect_arg(coselect, coselect_tokens, E, T, dev)
    N = T * k
    send = _out(o, "send", (N, H), x.dtype, dev, itemsize=bpe)
    rt = _out(o, "row_token", (N,), torch.int32, dev)
    rw = _out(o, "row_weight", (N,), torch.float32, dev)
    sr = _out(o, "slot_row", (T, k), torch.int32, dev)
    if dedup:
        rx = _out(o, "row_experts", (N, k), torch.int32, dev)
        rg = _out(o, "row_gates", (N, k), torch.float32, dev)
        nr = _out(o, "n_rows", (1,), torch.int32, dev)
    else:
        rx = _out(o, "row_expert", (N,), torch.int32, dev)
        rg = nr = None
    check(lib().moe_route_dispatch(_ptr(logits), _ptr(x), T, H, E, k, int(bool(softmax_all)),
                                   n_ranks, _ptr(placement), int(bool(dedup)), bpe, _ptr(idx),
                                   _ptr(gate), _ptr(ec), _ptr(rc), _ptr(ro), _ptr(eo),
                                   _ptr(send), _ptr(rt), _ptr(rx), _ptr(rg), _ptr(rw), _ptr(sr),
                                   _ptr(nr), ncs, _ptr(W), _ptr(ws), ws.numel(),
                                   _stream(stream)), "moe_route_dispatch")
    counts = {"expert_counts": ec, "rank_counts": rc, "rank_offsets": ro, "expert_offsets": eo,
              "ws": ws}
    rows = {"send": send, "row_token": rt, "row_weight": rw, "slot_row": sr}
    if dedup:
        rows.update(row_experts=rx, row_gates=rg, n_rows=nr)
    else:
        rows["row_expert"] = rx
    return idx, gate, counts, rows


def moe_combine_route(rows, row_weight, slot_row, next_logits, top_k, n_ranks, placement=None,
                      dedup=False, softmax_all=False, out=None, next_out=None, stream=None):
    """moe_combine of this batch (rows None: no combine) and the routing of the
    next batch (next_logits [Tn][E] fp32) into its plan without the scan, in one
    launch (moe_combine_route).  `next_out` may hold the next batch's
    "topk_idx", "topk_gate" and "ws".  Returns (out, routed): the combine's
    [T][H] bf16 output (None without rows) and a dict of the next batch's ids,
    gates, workspace and routing parameters, for moe_dispatch_routed."""
    _dev(next_logits, "next_logits", torch.float32, 2)
    Tn, E = next_logits.shape
    dev = next_logits.device
    k = int(top_k)
    if rows is None:
        T, H, kc, bpe, W, sr = 0, 8, 1, 2, None, None
    else:
        bpe = _row_bpe(rows, "rows")
        n_rows, H = rows.shape
        _dev(slot_row, "slot_row", torch.int32, 2, device=dev)
        if rows.device != dev:
            raise ValueError(f"rows are on {rows.device}, next_logits on {dev}")
        if row_weight is not None:
            _dev(row_weight, "row_weight", torch.float32, shape=(n_rows,), device=dev)
        W, sr = row_weight, slot_row
        T, kc = slot_row.shape
        out = _out({"out": out}, "out", (T, H), torch.bfloat16, dev, itemsize=2)
    o = dict(next_out or {})
    idx = _out(o, "topk_idx", (Tn, k), torch.int32, dev)
    gate = _out(o, "topk_gate", (Tn, k), torch.float32, dev)
    placement = _placement(placement, E, dev)
    ws = o.get("ws")
    ws = workspace(Tn, E, k, n_ranks, dedup, dev) if ws is None else _ws(ws, dev)
    check(lib().moe_combine_route(_ptr(rows), _ptr(W), _ptr(sr), T, H, kc, bpe,
                                  _ptr(out if rows is not None else None), _ptr(next_logits), Tn,
                                  E, k, int(bool(softmax_all)), n_ranks, _ptr(placement),
                                  int(bool(dedup)), _ptr(idx), _ptr(gate), _ptr(ws), ws.numel(),
                                  _stream(stream)), "moe_combine_route")
    routed = {"topk_idx": idx, "topk_gate": gate, "ws": ws, "n_experts": E, "n_ranks": n_ranks,
              "placement": placement, "dedup": bool(dedup)}
    return (out if rows is not None else None), routed


def moe_dispatch_routed(x, routed, out=None, coselect=None, coselect_tokens=None, stream=None):
    """The dispatch of a batch routed by moe_combine_route (`routed` is the dict
    it returned): the plan's scan and the dispatch (moe_dispatch_routed), with
    the outputs of the second half of moe_route_dispatch.  `out` may hold any
    count or dispatch output.  Returns (counts, rows) as moe_route_dispatch."""
    idx, gate, ws = routed["topk_idx"], routed["topk_gate"], routed["ws"]
    T, H, k, bpe, dev = _routed(x, idx, gate)
    E, R, dedup = routed["n_experts"], routed["n_ranks"], routed["dedup"]
    placement = routed["placement"]
    ws = _ws(ws, dev)
    o = dict(out or {})
    ec, rc, ro, eo = _count_outputs(o, E, R, dedup, dev)
    ncs, W = _coselect_arg(coselect, coselect_tokens, E, T, dev)
    N = T * k
    send = _out(o, "send", (N, H), x.dtype, dev, itemsize=bpe)
    rt = _out(o, "row_token", (N,), torch.int32, dev)
    rw = _out(o, "row_weight", (N,), torch.float32, dev)
    sr = _out(o, "slot_row", (T, k), torch.int32, dev)
    if dedup:
        rx = _out(o, "row_experts", (N, k), torch.int32, dev)
        rg = _out(o, "row_gates", (N, k), torch.float32, dev)
        nr = _out(o, "n_rows", (1,), torch.int32, dev)
    else:
        rx = _out(o, "row_expert", (N,), torch.int32, dev)
        rg = nr = None
    check(lib().moe_dispatch_routed(_ptr(x), _ptr(idx), _ptr(gate), T, H, E, k, R,
                                    _ptr(placement), int(dedup), bpe, _ptr(ec), _ptr(rc),
                                    _ptr(ro), _ptr(eo), _ptr(send), _ptr(rt), _ptr(rx), _ptr(rg),
                                    _ptr(rw), _ptr(sr), _ptr(nr), ncs, _ptr(W), _ptr(ws),
                                    ws.numel(), _stream(stream)), "moe_dispatch_routed")
    counts = {"expert_counts": ec, "rank_counts": rc, "rank_offsets": ro, "expert_offsets": eo,
              "ws": ws}
    rows = {"send": send, "row_token": rt, "row_weight": rw, "slot_row": sr}
    if dedup:
        rows.update(row_experts=rx, row_gates=rg, n_rows=nr)
    else:
        rows["row_expert"] = rx
    return counts, rows


def moe_dispatch_permute_noalloc(x, topk_idx, topk_gate, n_experts, n_ranks, placement=None,
                                 out=None, stream=None):
    """moe_send_counts (plain) and moe_dispatch_permute in one call whose plan
    lives in the library's static per-device scratch: the C entry point
    allocates nothing (outputs not passed in are allocated here, by torch).
    Returns the counts and the dispatch outputs in one dict."""
    T, H, k, bpe, dev = _routed(x, topk_idx, topk_gate)
    placement = _placement(placement, n_experts, dev)
    o = dict(out or {})
    ec, rc, ro, eo = _count_outputs(o, n_experts, n_ranks, False, dev)
    N = T * k
    send = _out(o, "send", (N, H), x.dtype, dev, itemsize=bpe)
    rt = _out(o, "row_token", (N,), torch.int32, dev)
    re = _out(o, "row_expert", (N,), torch.int32, dev)
    rw = _out(o, "row_weight", (N,), torch.float32, dev)
    sr = _out(o, "slot_row", (T, k), torch.int32, dev)
    check(lib().moe_dispatch_permute_noalloc(_ptr(x), _ptr(topk_idx), _ptr(topk_gate), T, H,
                                             n_experts, k, n_ranks, _ptr(placement), bpe,
                                             _ptr(ec), _ptr(rc), _ptr(ro), _ptr(eo), _ptr(send),
                                             _ptr(rt), _ptr(re), _ptr(rw), _ptr(sr),
                                             _stream(stream)), "moe_dispatch_permute_noalloc")
    return {"expert_counts": ec, "rank_counts": rc, "rank_offsets": ro, "expert_offsets": eo,
            "send": send, "row_token": rt, "row_expert": re, "row_weight": rw, "slot_row": sr}


_FP8 = tuple(t for t in (getattr(torch, "float8_e4m3fn", None), torch.uint8) if t is not None)
_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _row_bpe(rows, name):
    """Row element size: bf16 (2 bytes) or fp8 E4M3 (1 byte)."""
    _dev(rows, name, _BF16 + _FP8, 2)
    return 1 if rows.dtype in _FP8 else 2


def moe_combine(rows, row_weight, slot_row, out=None, stream=None):
    """out[T][H] bf16; rows bf16, or fp8 E4M3 (torch.float8_e4m3fn or uint8).
    row_weight: one fp32 weight per row of `rows`, or None (weight 1).  The
    entries of slot_row must be below rows.shape[0] (a device precondition)."""
    bpe = _row_bpe(rows, "rows")
    dev = rows.device
    n_rows, H = rows.shape
    _dev(slot_row, "slot_row", torch.int32, 2, device=dev)
    if row_weight is not None:
        _dev(row_weight, "row_weight", torch.float32, shape=(n_rows,), device=dev)
    T, k = slot_row.shape
    out = _out({"out": out}, "out", (T, H), torch.bfloat16, dev, itemsize=2)
    check(lib().moe_combine(_ptr(rows), _ptr(row_weight), _ptr(slot_row), T, H, k, bpe,
                            _ptr(out), _stream(stream)), "moe_combine")
    return out


def moe_coselect_counts(topk_idx, n_experts, tokens=None, coselect=None, stream=None):
    _dev(topk_idx, "topk_idx", torch.int32, 2)
    T, k = topk_idx.shape
    dev = topk_idx.device
    n = T if tokens is None else min(int(tokens), T)
    if coselect is None:
        coselect = torch.zeros((n_experts, n_experts), dtype=torch.int32, device=dev)
    _dev(coselect, "coselect", torch.int32, shape=(n_experts, n_experts), device=dev)
    if n == 0:
        return coselect
    check(lib().moe_coselect_counts(_ptr(topk_idx), n, n_experts, k, _ptr(coselect),
                                    _stream(stream)), "moe_coselect_counts")
    return coselect


# ------------------------------------------------------------- receive side --

def moe_expand_workspace_bytes(capacity: int, n_experts: int, top_k: int, n_ranks: int) -> int:
    return int(lib().moe_expand_workspace_bytes(capacity, n_experts, top_k, n_ranks))


def expand_workspace(capacity, n_experts, top_k, n_ranks, device) -> torch.Tensor:
    n = moe_expand_workspace_bytes(capacity, n_experts, top_k, n_ranks)
    if n == 0:
        raise MoeError(1, "moe_expand_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _n_rows(n_rows, device):
    return _dev(n_rows, "n_rows", torch.int32, shape=(1,), device=device)


def moe_expand_counts(row_experts, n_rows, n_experts, n_ranks, placement=None, ws=None,
                      out=None, stream=None):
    """Receive-side counts and plan for received dedup rows.  `row_experts`
    [C][k] int32, `n_rows` a 1-element device int32 tensor.  Returns a dict with
    expert_counts, rank_counts, rank_offsets, expert_offsets and `ws`."""
    _dev(row_experts, "row_experts", torch.int32, 2)
    C, k = row_experts.shape
    dev = row_experts.device
    _n_rows(n_rows, dev)
    placement = _placement(placement, n_experts, dev)
    ws = expand_workspace(C, n_experts, k, n_ranks, dev) if ws is None else _ws(ws, dev)
    ec, rc, ro, eo = _count_outputs(dict(out or {}), n_experts, n_ranks, False, dev)
    check(lib().moe_expand_counts(_ptr(row_experts), _ptr(n_rows), C, n_experts, k, n_ranks,
                                  _ptr(placement), _ptr(ec), _ptr(rc), _ptr(ro), _ptr(eo),
                                  _ptr(ws), ws.numel(), _stream(stream)), "moe_expand_counts")
    return {"expert_counts": ec, "rank_counts": rc, "rank_offsets": ro, "expert_offsets": eo,
            "ws": ws}


def moe_expand_permute(rows, row_gates, n_rows, n_experts, n_ranks, ws,
                       expanded_capacity=None, out=None, stream=None):
    """Receive-side expansion of the plan in `ws` (from moe_expand_counts over
    the same received rows).  expanded_capacity defaults to C rows, which
    holds every entry when the received buffers have the dedup dispatch's
    capacity T*k (the expansion has exactly T*k rows).  Returns expanded,
    exp_row, exp_expert, exp_gate, row_slot."""
    bpe = _x_bpe(rows, "rows")
    C, H = rows.shape
    dev = rows.device
    _dev(row_gates, "row_gates", torch.float32, 2, device=dev)
    if row_gates.shape[0] != C:
        raise ValueError(f"row_gates has {row_gates.shape[0]} rows, rows has {C}")
    k = row_gates.shape[1]
    _n_rows(n_rows, dev)
    _ws(ws, dev)
    cap = C if expanded_capacity is None else int(expanded_capacity)
    o = dict(out or {})
    ex = _out(o, "expanded", (cap, H), rows.dtype, dev, itemsize=bpe)
    er = _out(o, "exp_row", (cap,), torch.int32, dev)
    ee = _out(o, "exp_expert", (cap,), torch.int32, dev)
    eg = _out(o, "exp_gate", (cap,), torch.float32, dev)
    rs = _out(o, "row_slot", (C, k), torch.int32, dev)
    check(lib().moe_expand_permute(_ptr(rows), _ptr(row_gates), _ptr(n_rows), C, H, n_experts,
                                   k, n_ranks, bpe, _ptr(ws), ws.numel(), _ptr(ex), cap,
                                   _ptr(er), _ptr(ee), _ptr(eg), _ptr(rs), _stream(stream)),
          "moe_expand_permute")
    return {"expanded": ex, "exp_row": er, "exp_expert": ee, "exp_gate": eg, "row_slot": rs}


def moe_expand_reduce(expert_out, exp_gate, row_slot, n_rows, out=None, stream=None):
    """Receive-side reduction of the experts' outputs (bf16, or fp8 E4M3) back
    to one bf16 row per received row (rows past n_rows are not written)."""
    bpe = _row_bpe(expert_out, "expert_out")
    dev = expert_out.device
    n_exp, H = expert_out.shape
    _dev(row_slot, "row_slot", torch.int32, 2, device=dev)
    _n_rows(n_rows, dev)
    if exp_gate is not None:
        _dev(exp_gate, "exp_gate", torch.float32, shape=(n_exp,), device=dev)
    C, k = row_slot.shape
    out = _out({"out": out}, "out", (C, H), torch.bfloat16, dev, itemsize=2)
    check(lib().moe_expand_reduce(_ptr(expert_out), _ptr(exp_gate), _ptr(row_slot),
                                  _ptr(n_rows), C, H, k, bpe, _ptr(out), _stream(stream)),
          "moe_expand_reduce")
    return out


# -------------------------------------------------------- placement search --

def moe_placement_search(coselect, n_ranks, initial=None, max_swaps=None):
    """Correlated placement from a co-selection matrix (host computation).
    `coselect` [E][E] int32 (a GPU tensor is copied to the host first),
    `initial` [E] int32 or None (contiguous).  Returns (placement, objective,
    swaps) with placement a host int32 tensor."""
    import ctypes
    W = coselect.detach().to("cpu", torch.int32).contiguous()
    if W.dim() != 2 or W.shape[0] != W.shape[1]:
        raise ValueError("coselect must be [E][E]")
    E = W.shape[0]
    init = None
    if initial is not None:
        init = initial.detach().to("cpu", torch.int32).contiguous()
        if init.numel() != E:
            raise ValueError("initial must have E entries")
    place = torch.empty(E, dtype=torch.int32)
    obj = ctypes.c_int64(0)
    sw = ctypes.c_int(0)
    ms = E * E if max_swaps is None else int(max_swaps)
    check(lib().moe_placement_search(W.data_ptr(), E, n_ranks,
                                     None if init is None else init.data_ptr(), ms,
                                     place.data_ptr(), ctypes.byref(obj), ctypes.byref(sw)),
          "moe_placement_search")
    return place, int(obj.value), int(sw.value)


# ---------------------------------------------------- token shuffle planner --

def moe_shuffle_fit(prev_idx, cur_idx, next_idx, n_experts, n_ranks, placement_next=None,
                    pair_counts=None, single_counts=None, stream=None):
    """Accumulate the planner's count tables from one calibration batch."""
    _dev(cur_idx, "cur_idx", torch.int32, 2)
    T, k = cur_idx.shape
    dev = cur_idx.device
    _dev(prev_idx, "prev_idx", torch.int32, shape=(T, k), device=dev)
    _dev(next_idx, "next_idx", torch.int32, shape=(T, k), device=dev)
    placement_next = _placement(placement_next, n_experts, dev)
    E, R = n_experts, n_ranks
    if pair_counts is None:
        pair_counts = torch.zeros((E, E, R), dtype=torch.int32, device=dev)
    if single_counts is None:
        single_counts = torch.zeros((E, R), dtype=torch.int32, device=dev)
    _dev(pair_counts, "pair_counts", torch.int32, shape=(E, E, R), device=dev)
    _dev(single_counts, "single_counts", torch.int32, shape=(E, R), device=dev)
    check(lib().moe_shuffle_fit(_ptr(prev_idx), _ptr(cur_idx), _ptr(next_idx), T, n_experts, k,
                                n_ranks, _ptr(placement_next), _ptr(pair_counts),
                                _ptr(single_counts), _stream(stream)), "moe_shuffle_fit")
    return pair_counts, single_counts


def moe_shuffle_predict(prev_idx, cur_idx, pair_counts, single_counts, min_obs, scores=None,
                        stream=None):
    _dev(cur_idx, "cur_idx", torch.int32, 2)
    T, k = cur_idx.shape
    dev = cur_idx.device
    _dev(prev_idx, "prev_idx", torch.int32, shape=(T, k), device=dev)
    _dev(single_counts, "single_counts", torch.int32, 2, device=dev)
    E, R = single_counts.shape
    _dev(pair_counts, "pair_counts", torch.int32, shape=(E, E, R), device=dev)
    scores = _out({"scores": scores}, "scores", (T, R), torch.float32, dev)
    check(lib().moe_shuffle_predict(_ptr(prev_idx), _ptr(cur_idx), T, E, k, R, _ptr(pair_counts),
                                    _ptr(single_counts), int(min_obs), _ptr(scores),
                                    _stream(stream)), "moe_shuffle_predict")
    return scores


def moe_shuffle_assign(scores):
    """Host assignment of owner ranks from [T][R] scores (a GPU tensor is
    copied to the host first).  Returns a host int32 tensor [T]."""
    S = scores.detach().to("cpu", torch.float32).contiguous()
    T, R = S.shape
    owner = torch.empty(T, dtype=torch.int32)
    check(lib().moe_shuffle_assign(S.data_ptr() if T else None, T, R,
                                   owner.data_ptr() if T else None), "moe_shuffle_assign")
    return owner
