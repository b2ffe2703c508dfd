"""Python binding of the C ABI (include/moe_route.h), entry point for entry point.

Each function checks dtype/device/contiguity, allocates any output that was not
passed in (torch is used for device memory and streams only), passes raw
pointers and the current HIP stream to the library, and raises MoeError on a
non-zero status.  No step of the computation runs here.
"""
from __future__ import annotations

from typing import Optional

import torch

from ._lib import MoeError, check, lib, status_string  # noqa: F401

__all__ = ["MoeError", "moe_status_string", "moe_workspace_bytes", "moe_route_topk",
           "moe_send_counts", "moe_dispatch_permute", "moe_dispatch_permute_dedup",
           "moe_combine", "moe_coselect_counts", "workspace", "moe_expand_workspace_bytes",
           "expand_workspace", "moe_expand_counts", "moe_expand_permute", "moe_expand_reduce",
           "moe_placement_search", "moe_shuffle_fit", "moe_shuffle_predict",
           "moe_shuffle_assign"]


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr() or None


def _dev(t: torch.Tensor, name: str, dtype=None, ndim=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


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
    if topk_idx is None:
        topk_idx = torch.empty((T, top_k), dtype=torch.int32, device=logits.device)
    if topk_gate is None:
        topk_gate = torch.empty((T, top_k), dtype=torch.float32, device=logits.device)
    _dev(topk_idx, "topk_idx", torch.int32)
    _dev(topk_gate, "topk_gate", torch.float32)
    fn = lib().moe_route_topk_softmax_all if softmax_all else lib().moe_route_topk
    check(fn(_ptr(logits), T, E, top_k, _ptr(topk_idx), _ptr(topk_gate), _stream(stream)),
          "moe_route_topk_softmax_all" if softmax_all else "moe_route_topk")
    return topk_idx, topk_gate


def moe_send_counts(topk_idx, n_experts, n_ranks, placement=None, dedup=False, ws=None,
                    out=None, stream=None):
    """Returns a dict with expert_counts, rank_counts, rank_offsets, expert_offsets
    (None in dedup mode) and the workspace `ws` that the dispatch call needs."""
    _dev(topk_idx, "topk_idx", torch.int32, 2)
    T, k = topk_idx.shape
    dev = topk_idx.device
    if placement is not None:
        _dev(placement, "placement", torch.int32, 1)
    if ws is None:
        ws = workspace(T, n_experts, k, n_ranks, dedup, dev)
    o = dict(out or {})
    ec = o.get("expert_counts")
    ec = torch.empty(n_experts, dtype=torch.int32, device=dev) if ec is None else ec
    rc = o.get("rank_counts")
    rc = torch.empty(n_ranks, dtype=torch.int32, device=dev) if rc is None else rc
    ro = o.get("rank_offsets")
    ro = torch.empty(n_ranks + 1, dtype=torch.int32, device=dev) if ro is None else ro
    eo = None
    if not dedup:
        eo = o.get("expert_offsets")
        eo = torch.empty(n_experts, dtype=torch.int32, device=dev) if eo is None else eo
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
    if topk_idx is None:
        topk_idx = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    if topk_gate is None:
        topk_gate = torch.empty((T, top_k), dtype=torch.float32, device=dev)
    _dev(topk_idx, "topk_idx", torch.int32)
    _dev(topk_gate, "topk_gate", torch.float32)
    if placement is not None:
        _dev(placement, "placement", torch.int32, 1)
    if ws is None:
        ws = workspace(T, E, top_k, n_ranks, dedup, dev)
    o = dict(out or {})
    ec = o.get("expert_counts")
    ec = torch.empty(E, dtype=torch.int32, device=dev) if ec is None else ec
    rc = o.get("rank_counts")
    rc = torch.empty(n_ranks, dtype=torch.int32, device=dev) if rc is None else rc
    ro = o.get("rank_offsets")
    ro = torch.empty(n_ranks + 1, dtype=torch.int32, device=dev) if ro is None else ro
    eo = None
    if not dedup:
        eo = o.get("expert_offsets")
        eo = torch.empty(E, dtype=torch.int32, device=dev) if eo is None else eo
    ncs = 0
    if coselect is not None:
        _dev(coselect, "coselect", torch.int32, 2)
        ncs = T if coselect_tokens is None else int(coselect_tokens)
    check(lib().moe_route_plan(_ptr(logits), T, E, top_k, int(bool(softmax_all)), n_ranks,
                               _ptr(placement), int(bool(dedup)), _ptr(topk_idx),
                               _ptr(topk_gate), _ptr(ec), _ptr(rc), _ptr(ro), _ptr(eo), ncs,
                               _ptr(coselect), _ptr(ws), ws.numel(), _stream(stream)),
          "moe_route_plan")
    return topk_idx, topk_gate, {"expert_counts": ec, "rank_counts": rc, "rank_offsets": ro,
                                 "expert_offsets": eo, "ws": ws}


def _x_bpe(x):
    _dev(x, "x", None, 2)
    if x.element_size() not in (1, 2, 4):
        raise TypeError("x must have 1-, 2- or 4-byte elements")
    return x.element_size()


def moe_dispatch_permute(x, topk_idx, topk_gate, n_experts, n_ranks, ws, placement=None,
                         out=None, stream=None):
    bpe = _x_bpe(x)
    _dev(topk_idx, "topk_idx", torch.int32, 2)
    _dev(topk_gate, "topk_gate", torch.float32, 2)
    T, H = x.shape
    k = topk_idx.shape[1]
    dev = x.device
    o = dict(out or {})
    N = T * k
    send = o.get("send")
    send = torch.empty((N, H), dtype=x.dtype, device=dev) if send is None else send
    rt = o.get("row_token")
    rt = torch.empty(N, dtype=torch.int32, device=dev) if rt is None else rt
    re = o.get("row_expert")
    re = torch.empty(N, dtype=torch.int32, device=dev) if re is None else re
    rw = o.get("row_weight")
    rw = torch.empty(N, dtype=torch.float32, device=dev) if rw is None else rw
    sr = o.get("slot_row")
    sr = torch.empty((T, k), dtype=torch.int32, device=dev) if sr is None else sr
    if send.numel() < N * H or rt.numel() < N or re.numel() < N or rw.numel() < N:
        raise ValueError("output buffers are smaller than tokens*top_k rows")
    check(lib().moe_dispatch_permute(_ptr(x), _ptr(topk_idx), _ptr(topk_gate), T, H, n_experts,
                                     k, n_ranks, _ptr(placement), bpe, _ptr(ws), ws.numel(),
                                     _ptr(send), _ptr(rt), _ptr(re), _ptr(rw), _ptr(sr),
                                     _stream(stream)), "moe_dispatch_permute")
    return {"send": send, "row_token": rt, "row_expert": re, "row_weight": rw, "slot_row": sr}


def moe_dispatch_permute_dedup(x, topk_idx, topk_gate, n_experts, n_ranks, ws, placement=None,
                               out=None, stream=None):
    bpe = _x_bpe(x)
    _dev(topk_idx, "topk_idx", torch.int32, 2)
    _dev(topk_gate, "topk_gate", torch.float32, 2)
    T, H = x.shape
    k = topk_idx.shape[1]
    dev = x.device
    o = dict(out or {})
    N = T * k
    send = o.get("send")
    send = torch.empty((N, H), dtype=x.dtype, device=dev) if send is None else send
    rt = o.get("row_token")
    rt = torch.empty(N, dtype=torch.int32, device=dev) if rt is None else rt
    rx = o.get("row_experts")
    rx = torch.empty((N, k), dtype=torch.int32, device=dev) if rx is None else rx
    rg = o.get("row_gates")
    rg = torch.empty((N, k), dtype=torch.float32, device=dev) if rg is None else rg
    rw = o.get("row_weight")
    rw = torch.empty(N, dtype=torch.float32, device=dev) if rw is None else rw
    sr = o.get("slot_row")
    sr = torch.empty((T, k), dtype=torch.int32, device=dev) if sr is None else sr
    nr = o.get("n_rows")
    nr = torch.empty(1, dtype=torch.int32, device=dev) if nr is None else nr
    if send.numel() < N * H or rx.numel() < N * k or rg.numel() < N * k or rw.numel() < N:
        raise ValueError("output buffers are smaller than tokens*top_k rows")
    check(lib().moe_dispatch_permute_dedup(_ptr(x), _ptr(topk_idx), _ptr(topk_gate), T, H,
                                           n_experts, k, n_ranks, _ptr(placement), bpe,
                                           _ptr(ws), ws.numel(), _ptr(send), _ptr(rt),
                                           _ptr(rx), _ptr(rg), _ptr(rw), _ptr(sr), _ptr(nr),
                                           _stream(stream)), "moe_dispatch_permute_dedup")
    return {"send": send, "row_token": rt, "row_experts": rx, "row_gates": rg,
            "row_weight": rw, "slot_row": sr, "n_rows": nr}


_FP8 = tuple(t for t in (getattr(torch, "float8_e4m3fn", None), torch.uint8) if t is not None)
_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _row_bpe(rows, name):
    """Row element size: bf16 (2 bytes) or fp8 E4M3 (1 byte)."""
    _dev(rows, name, _BF16 + _FP8, 2)
    return 1 if rows.dtype in _FP8 else 2


def moe_combine(rows, row_weight, slot_row, out=None, stream=None):
    """out[T][H] bf16; rows bf16, or fp8 E4M3 (torch.float8_e4m3fn or uint8)."""
    bpe = _row_bpe(rows, "rows")
    _dev(slot_row, "slot_row", torch.int32, 2)
    if row_weight is not None:
        _dev(row_weight, "row_weight", torch.float32)
    T, k = slot_row.shape
    H = rows.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=rows.device)
    _dev(out, "out", _BF16, 2)
    check(lib().moe_combine(_ptr(rows), _ptr(row_weight), _ptr(slot_row), T, H, k, bpe,
                            _ptr(out), _stream(stream)), "moe_combine")
    return out


def moe_coselect_counts(topk_idx, n_experts, tokens=None, coselect=None, stream=None):
    _dev(topk_idx, "topk_idx", torch.int32, 2)
    T, k = topk_idx.shape
    n = T if tokens is None else min(int(tokens), T)
    if coselect is None:
        coselect = torch.zeros((n_experts, n_experts), dtype=torch.int32,
                               device=topk_idx.device)
    _dev(coselect, "coselect", torch.int32, 2)
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


def moe_expand_counts(row_experts, n_rows, n_experts, n_ranks, placement=None, ws=None,
                      out=None, stream=None):
    """Receive-side counts and plan for received dedup rows.  `row_experts`
    [C][k] int32, `n_rows` a 1-element device int32 tensor.  Returns a dict with
    expert_counts, rank_counts, rank_offsets, expert_offsets and `ws`."""
    _dev(row_experts, "row_experts", torch.int32, 2)
    _dev(n_rows, "n_rows", torch.int32)
    C, k = row_experts.shape
    dev = row_experts.device
    if placement is not None:
        _dev(placement, "placement", torch.int32, 1)
    if ws is None:
        ws = expand_workspace(C, n_experts, k, n_ranks, dev)
    o = dict(out or {})
    i32 = torch.int32
    ec = o.get("expert_counts")
    ec = torch.empty(n_experts, dtype=i32, device=dev) if ec is None else ec
    rc = o.get("rank_counts")
    rc = torch.empty(n_ranks, dtype=i32, device=dev) if rc is None else rc
    ro = o.get("rank_offsets")
    ro = torch.empty(n_ranks + 1, dtype=i32, device=dev) if ro is None else ro
    eo = o.get("expert_offsets")
    eo = torch.empty(n_experts, dtype=i32, device=dev) if eo is None else eo
    check(lib().moe_expand_counts(_ptr(row_experts), _ptr(n_rows), C, n_experts, k, n_ranks,
                                  _ptr(placement), _ptr(ec), _ptr(rc), _ptr(ro), _ptr(eo),
                                  _ptr(ws), ws.numel(), _stream(stream)), "moe_expand_counts")
    return {"expert_counts": ec, "rank_counts": rc, "rank_offsets": ro, "expert_offsets": eo,
            "ws": ws}


def moe_expand_permute(rows, row_experts, row_gates, n_rows, n_experts, n_ranks, ws,
                       expanded_capacity=None, out=None, stream=None):
    """Receive-side expansion.  expanded_capacity defaults to C rows, which
    holds every entry when the received buffers have the dedup dispatch's
    capacity T*k (the expansion has exactly T*k rows).  Returns expanded,
    exp_row, exp_expert, exp_gate, row_slot."""
    bpe = _x_bpe(rows)
    _dev(row_experts, "row_experts", torch.int32, 2)
    _dev(row_gates, "row_gates", torch.float32, 2)
    _dev(n_rows, "n_rows", torch.int32)
    C, H = rows.shape
    k = row_experts.shape[1]
    dev = rows.device
    cap = C if expanded_capacity is None else int(expanded_capacity)
    o = dict(out or {})
    ex = o.get("expanded")
    ex = torch.empty((cap, H), dtype=rows.dtype, device=dev) if ex is None else ex
    er = o.get("exp_row")
    er = torch.empty(cap, dtype=torch.int32, device=dev) if er is None else er
    ee = o.get("exp_expert")
    ee = torch.empty(cap, dtype=torch.int32, device=dev) if ee is None else ee
    eg = o.get("exp_gate")
    eg = torch.empty(cap, dtype=torch.float32, device=dev) if eg is None else eg
    rs = o.get("row_slot")
    rs = torch.empty((C, k), dtype=torch.int32, device=dev) if rs is None else rs
    if ex.numel() < cap * H or er.numel() < cap or ee.numel() < cap or eg.numel() < cap:
        raise ValueError("expanded buffers are smaller than expanded_capacity rows")
    check(lib().moe_expand_permute(_ptr(rows), _ptr(row_experts), _ptr(row_gates), _ptr(n_rows),
                                   C, H, n_experts, k, n_ranks, bpe, _ptr(ws), ws.numel(),
                                   _ptr(ex), cap, _ptr(er), _ptr(ee), _ptr(eg), _ptr(rs),
                                   _stream(stream)), "moe_expand_permute")
    return {"expanded": ex, "exp_row": er, "exp_expert": ee, "exp_gate": eg, "row_slot": rs}


def moe_expand_reduce(expert_out, exp_gate, row_slot, n_rows, out=None, stream=None):
    """Receive-side reduction of the experts' outputs (bf16, or fp8 E4M3) back
    to one bf16 row per received row (rows past n_rows are not written)."""
    bpe = _row_bpe(expert_out, "expert_out")
    _dev(row_slot, "row_slot", torch.int32, 2)
    _dev(n_rows, "n_rows", torch.int32)
    if exp_gate is not None:
        _dev(exp_gate, "exp_gate", torch.float32)
    C, k = row_slot.shape
    H = expert_out.shape[1]
    if out is None:
        out = torch.empty((C, H), dtype=torch.bfloat16, device=expert_out.device)
    _dev(out, "out", _BF16, 2)
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
    for name, t in (("prev_idx", prev_idx), ("cur_idx", cur_idx), ("next_idx", next_idx)):
        _dev(t, name, torch.int32, 2)
    T, k = cur_idx.shape
    dev = cur_idx.device
    if placement_next is not None:
        _dev(placement_next, "placement_next", torch.int32, 1)
    if pair_counts is None:
        pair_counts = torch.zeros((n_experts, n_experts, n_ranks), dtype=torch.int32, device=dev)
    if single_counts is None:
        single_counts = torch.zeros((n_experts, n_ranks), dtype=torch.int32, device=dev)
    _dev(pair_counts, "pair_counts", torch.int32, 3)
    _dev(single_counts, "single_counts", torch.int32, 2)
    check(lib().moe_shuffle_fit(_ptr(prev_idx), _ptr(cur_idx), _ptr(next_idx), T, n_experts, k,
                                n_ranks, _ptr(placement_next), _ptr(pair_counts),
                                _ptr(single_counts), _stream(stream)), "moe_shuffle_fit")
    return pair_counts, single_counts


def moe_shuffle_predict(prev_idx, cur_idx, pair_counts, single_counts, min_obs, scores=None,
                        stream=None):
    _dev(prev_idx, "prev_idx", torch.int32, 2)
    _dev(cur_idx, "cur_idx", torch.int32, 2)
    _dev(pair_counts, "pair_counts", torch.int32, 3)
    _dev(single_counts, "single_counts", torch.int32, 2)
    T, k = cur_idx.shape
    E, R = single_counts.shape
    if scores is None:
        scores = torch.empty((T, R), dtype=torch.float32, device=cur_idx.device)
    _dev(scores, "scores", torch.float32, 2)
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
