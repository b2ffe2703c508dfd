"""numpy front end of the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product path.  It does not import
the HIP package and the HIP package does not import it.

Every function takes and returns numpy arrays on the host and runs the plain C
loops of oracle.c on one host thread.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# Plain IEEE double arithmetic: no fast-math, no contraction into FMA.
GCC_CMD = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", _LIB, _SRC, "-lm"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (gcc, host only)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        subprocess.run(GCC_CMD, check=True)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int
        L.oracle_route_topk.argtypes = [P, i64, i32, i32, P, P]
        L.oracle_route_topk_softmax_all.argtypes = [P, i64, i32, i32, P, P]
        L.oracle_send_counts.argtypes = [P, i64, i32, i32, i32, P, i32, P, P, P, P]
        L.oracle_dispatch.argtypes = [P, P, P, i64, i32, i32, i32, P, P, P, P, P, P]
        L.oracle_dispatch_dedup.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, P,
                                            P, P, P, P, P, P, P]
        L.oracle_expand_dedup.argtypes = [P, P, P, i64, i64, i32, i32, i32, i32, P, P, P, P,
                                          P, P, P, P, P, P]
        L.oracle_combine.argtypes = [P, P, P, i64, i32, i32, P]
        L.oracle_combine_fp8.argtypes = [P, P, P, i64, i32, i32, P]
        L.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_to_double.restype = ctypes.c_double
        L.oracle_coselect.argtypes = [P, i64, i32, i32, P]
        L.oracle_placement_search.argtypes = [P, i32, i32, P, i32, P, P, P]
        L.oracle_placement_search.restype = ctypes.c_int
        L.oracle_placement_objective.argtypes = [P, i32, P]
        L.oracle_placement_objective.restype = ctypes.c_int64
        L.oracle_shuffle_fit.argtypes = [P, P, P, i64, i32, i32, i32, P, P, P]
        L.oracle_shuffle_predict.argtypes = [P, P, i64, i32, i32, i32, P, P, i32, P]
        L.oracle_shuffle_assign.argtypes = [P, i64, i32, P]
        for f in ("oracle_shuffle_fit", "oracle_shuffle_predict", "oracle_shuffle_assign"):
            getattr(L, f).restype = ctypes.c_int
        L.oracle_bf16_from_double.argtypes = [ctypes.c_double]
        L.oracle_bf16_from_double.restype = ctypes.c_uint16
        L.oracle_bf16_from_float.argtypes = [ctypes.c_float]
        L.oracle_bf16_from_float.restype = ctypes.c_uint16
        for f in ("oracle_route_topk", "oracle_route_topk_softmax_all", "oracle_send_counts",
                  "oracle_dispatch",
                  "oracle_dispatch_dedup", "oracle_expand_dedup", "oracle_combine",
                  "oracle_combine_fp8", "oracle_coselect"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, name):
    if rc != 0:
        raise RuntimeError(f"{name} returned {rc}")


def contiguous(n_experts, n_ranks):
    return (np.arange(n_experts, dtype=np.int32) // (n_experts // n_ranks)).astype(np.int32)


def route_topk(logits, top_k):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    idx = np.empty((T, top_k), np.int32)
    gate = np.empty((T, top_k), np.float32)
    _check(lib().oracle_route_topk(_p(logits), T, E, top_k, _p(idx), _p(gate)), "route")
    return idx, gate


def route_topk_softmax_all(logits, top_k):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    idx = np.empty((T, top_k), np.int32)
    gate = np.empty((T, top_k), np.float32)
    _check(lib().oracle_route_topk_softmax_all(_p(logits), T, E, top_k, _p(idx), _p(gate)),
           "route_softmax_all")
    return idx, gate


def send_counts(idx, n_experts, n_ranks, placement=None, dedup=False):
    idx = _c(idx, np.int32)
    T, k = idx.shape
    place = contiguous(n_experts, n_ranks) if placement is None else _c(placement, np.int32)
    ec = np.empty(n_experts, np.int32)
    rc = np.empty(n_ranks, np.int32)
    ro = np.empty(n_ranks + 1, np.int32)
    eo = np.empty(n_experts, np.int32)
    _check(lib().oracle_send_counts(_p(idx), T, n_experts, k, n_ranks, _p(place),
                                    int(bool(dedup)), _p(ec), _p(rc), _p(ro), _p(eo)),
           "send_counts")
    return {"expert_counts": ec, "rank_counts": rc, "rank_offsets": ro,
            "expert_offsets": eo}


def dispatch(x_bits, idx, gate, n_experts, n_ranks, placement=None, with_rows=True):
    """Non-dedup pack.  x_bits: [T][H] of any 1/2/4-byte dtype (copied bitwise)."""
    idx = _c(idx, np.int32)
    gate = _c(gate, np.float32)
    T, k = idx.shape
    x = np.ascontiguousarray(x_bits)
    row_bytes = x.shape[1] * x.itemsize
    cnt = send_counts(idx, n_experts, n_ranks, placement, dedup=False)
    N = T * k
    send = np.empty((N,) + x.shape[1:], x.dtype) if with_rows else None
    row_token = np.empty(N, np.int32)
    row_expert = np.empty(N, np.int32)
    row_weight = np.empty(N, np.float32)
    slot_row = np.empty((T, k), np.int32)
    _check(lib().oracle_dispatch(_p(x), _p(idx), _p(gate), T, row_bytes, n_experts, k,
                                 _p(cnt["expert_offsets"]), _p(send), _p(row_token),
                                 _p(row_expert), _p(row_weight), _p(slot_row)), "dispatch")
    return dict(cnt, send=send, row_token=row_token, row_expert=row_expert,
                row_weight=row_weight, slot_row=slot_row, n_rows=N)


def dispatch_dedup(x_bits, idx, gate, n_experts, n_ranks, placement=None, with_rows=True):
    idx = _c(idx, np.int32)
    gate = _c(gate, np.float32)
    T, k = idx.shape
    x = np.ascontiguousarray(x_bits)
    row_bytes = x.shape[1] * x.itemsize
    place = contiguous(n_experts, n_ranks) if placement is None else _c(placement, np.int32)
    cnt = send_counts(idx, n_experts, n_ranks, place, dedup=True)
    D = int(cnt["rank_offsets"][-1])
    send = np.empty((D,) + x.shape[1:], x.dtype) if with_rows else None
    row_token = np.empty(D, np.int32)
    row_experts = np.empty((D, k), np.int32)
    row_gates = np.empty((D, k), np.float32)
    row_weight = np.empty(D, np.float32)
    slot_row = np.empty((T, k), np.int32)
    n_rows = np.zeros(1, np.int32)
    _check(lib().oracle_dispatch_dedup(_p(x), _p(idx), _p(gate), T, row_bytes, n_experts,
                                       k, n_ranks, _p(place), _p(cnt["rank_offsets"]),
                                       _p(send), _p(row_token), _p(row_experts),
                                       _p(row_gates), _p(row_weight), _p(slot_row),
                                       _p(n_rows)), "dispatch_dedup")
    return dict(cnt, send=send, row_token=row_token, row_experts=row_experts,
                row_gates=row_gates, row_weight=row_weight, slot_row=slot_row,
                n_rows=int(n_rows[0]))


def expand_dedup(rows_bits, row_experts, row_gates, n_rows, n_experts, n_ranks,
                 placement=None, capacity=None, with_rows=True):
    """Receive-side expansion of deduplicated rows into per-expert segments.
    rows_bits: [>= n_rows][H] of any 1/2/4-byte dtype (copied bitwise) or None."""
    row_experts = _c(row_experts, np.int32)
    row_gates = _c(row_gates, np.float32)
    k = row_experts.shape[1]
    cap = row_experts.shape[0] if capacity is None else int(capacity)
    assert n_rows <= cap <= row_experts.shape[0]
    place = contiguous(n_experts, n_ranks) if placement is None else _c(placement, np.int32)
    ec = np.empty(n_experts, np.int32)
    rc = np.empty(n_ranks, np.int32)
    ro = np.empty(n_ranks + 1, np.int32)
    eo = np.empty(n_experts, np.int32)
    n_exp = int((row_experts[:n_rows] >= 0).sum())
    if rows_bits is not None and with_rows:
        x = np.ascontiguousarray(rows_bits)
        row_bytes = x.shape[1] * x.itemsize
        expanded = np.empty((n_exp,) + x.shape[1:], x.dtype)
    else:
        x, row_bytes, expanded = None, 0, None
    exp_row = np.empty(n_exp, np.int32)
    exp_expert = np.empty(n_exp, np.int32)
    exp_gate = np.empty(n_exp, np.float32)
    row_slot = np.empty((cap, k), np.int32)
    _check(lib().oracle_expand_dedup(_p(x), _p(row_experts), _p(row_gates), int(n_rows), cap,
                                     row_bytes, n_experts, k, n_ranks, _p(place), _p(ec),
                                     _p(rc), _p(ro), _p(eo), _p(expanded), _p(exp_row),
                                     _p(exp_expert), _p(exp_gate), _p(row_slot)),
           "expand_dedup")
    return {"expert_counts": ec, "rank_counts": rc, "rank_offsets": ro, "expert_offsets": eo,
            "expanded": expanded, "exp_row": exp_row, "exp_expert": exp_expert,
            "exp_gate": exp_gate, "row_slot": row_slot, "n_expanded": n_exp}


def reduce_rows(expert_out_bits, exp_gate, row_slot, n_rows):
    """Receive-side reduction: row p < n_rows becomes the gate-weighted sum of
    its experts' outputs (the combine definition over the received rows)."""
    return combine(expert_out_bits, exp_gate, _c(row_slot, np.int32)[:n_rows])


def e4m3_to_double(b: int) -> float:
    return float(lib().oracle_e4m3_to_double(int(b) & 0xFF))


def combine_fp8(rows_u8, row_weight, slot_row):
    """Combine of fp8 E4M3 rows (uint8 bit patterns) into bf16 bits."""
    rows = _c(rows_u8, np.uint8)
    slot_row = _c(slot_row, np.int32)
    T, k = slot_row.shape
    H = rows.shape[1]
    w = None if row_weight is None else _c(row_weight, np.float32)
    out = np.empty((T, H), np.uint16)
    _check(lib().oracle_combine_fp8(_p(rows), _p(w), _p(slot_row), T, H, k, _p(out)),
           "combine_fp8")
    return out


def combine(rows_bits, row_weight, slot_row):
    rows = _c(rows_bits, np.uint16)
    slot_row = _c(slot_row, np.int32)
    T, k = slot_row.shape
    H = rows.shape[1]
    w = None if row_weight is None else _c(row_weight, np.float32)
    out = np.empty((T, H), np.uint16)
    _check(lib().oracle_combine(_p(rows), _p(w), _p(slot_row), T, H, k, _p(out)), "combine")
    return out


def coselect(idx, n_experts, tokens=None, W=None):
    idx = _c(idx, np.int32)
    T, k = idx.shape
    n = T if tokens is None else min(int(tokens), T)
    if W is None:
        W = np.zeros((n_experts, n_experts), np.int32)
    else:
        assert W.dtype == np.int32 and W.flags.c_contiguous
    _check(lib().oracle_coselect(_p(idx), n, n_experts, k, _p(W)), "coselect")
    return W


def bf16_from_double(d: float) -> int:
    return int(lib().oracle_bf16_from_double(float(d)))


def bf16_from_float(f) -> int:
    """bf16 bits of the fp32 value f (round to nearest even)."""
    return int(lib().oracle_bf16_from_float(ctypes.c_float(np.float32(f))))


def placement_objective(W, placement):
    W = _c(W, np.int32)
    place = _c(placement, np.int32)
    return int(lib().oracle_placement_objective(_p(W), W.shape[0], _p(place)))


def placement_search(W, n_ranks, initial=None, max_swaps=None):
    """Best-gain swap search from `initial` (contiguous if None).  Returns
    (placement, objective, swaps)."""
    W = _c(W, np.int32)
    E = W.shape[0]
    init = None if initial is None else _c(initial, np.int32)
    place = np.empty(E, np.int32)
    obj = np.zeros(1, np.int64)
    sw = np.zeros(1, np.int32)
    ms = E * E if max_swaps is None else int(max_swaps)
    _check(lib().oracle_placement_search(_p(W), E, n_ranks, _p(init), ms, _p(place), _p(obj),
                                         _p(sw)), "placement_search")
    return place, int(obj[0]), int(sw[0])


def shuffle_fit(prev, cur, nxt, n_experts, n_ranks, place_next=None, pair=None, single=None):
    prev, cur, nxt = (_c(a, np.int32) for a in (prev, cur, nxt))
    T, k = cur.shape
    E, R = n_experts, n_ranks
    place = contiguous(E, R) if place_next is None else _c(place_next, np.int32)
    if pair is None:
        pair = np.zeros((E, E, R), np.int32)
    if single is None:
        single = np.zeros((E, R), np.int32)
    _check(lib().oracle_shuffle_fit(_p(prev), _p(cur), _p(nxt), T, E, k, R, _p(place),
                                    _p(pair), _p(single)), "shuffle_fit")
    return pair, single


def shuffle_predict(prev, cur, pair, single, min_obs):
    prev, cur = _c(prev, np.int32), _c(cur, np.int32)
    pair, single = _c(pair, np.int32), _c(single, np.int32)
    T, k = cur.shape
    E, R = single.shape
    scores = np.empty((T, R), np.float32)
    _check(lib().oracle_shuffle_predict(_p(prev), _p(cur), T, E, k, R, _p(pair), _p(single),
                                        int(min_obs), _p(scores)), "shuffle_predict")
    return scores


def shuffle_assign(scores):
    scores = _c(scores, np.float32)
    T, R = scores.shape
    owner = np.empty(T, np.int32)
    _check(lib().oracle_shuffle_assign(_p(scores), T, R, _p(owner)), "shuffle_assign")
    return owner
