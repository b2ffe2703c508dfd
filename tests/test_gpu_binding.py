"""The Python binding rejects a wrong argument before anything is launched.

Every entry point checks the dtype (or element size), exact shape, device and
contiguity of each tensor it is given - inputs, output buffers passed through
`out=`, the co-selection matrix, the shuffle planner's tables - and that the
sizes agree with each other, so that no kernel can be handed a buffer too small
for what it writes.  Each case passes one wrong argument next to valid,
sentinel-filled outputs and checks that the call raises ValueError or TypeError
and that the sentinels are untouched (nothing ran).
"""
import pytest
import torch

from combine_top_router_select_amd import ops
from gpu_util import say

pytestmark = pytest.mark.gpu

T, H, E, K, R = 64, 128, 16, 4, 4
DEV = torch.device("cuda:0")


def _full(shape, dtype, v):
    return torch.full(shape, v, dtype=dtype, device=DEV)


def _inputs():
    g = torch.Generator(device=DEV).manual_seed(5)
    logits = torch.randn((T, E), generator=g, device=DEV)
    x = torch.randn((T, H), generator=g, device=DEV).to(torch.bfloat16)
    idx, gate = ops.moe_route_topk(logits, K)
    torch.cuda.synchronize()
    return logits, x, idx, gate


def _sentinels():
    return {"expert_counts": _full((E,), torch.int32, 7), "rank_counts": _full((R,), torch.int32, 7),
            "rank_offsets": _full((R + 1,), torch.int32, 7),
            "expert_offsets": _full((E,), torch.int32, 7)}


def _untouched(d):
    torch.cuda.synchronize()
    for key, t in d.items():
        assert (t == 7).all(), key


def _raises(exc, fn, *a, **kw):
    with pytest.raises(exc):
        fn(*a, **kw)


def test_routing_and_counts_reject_bad_buffers():
    logits, x, idx, gate = _inputs()
    say("[binding] routing and counts")
    s = _sentinels()
    _raises(TypeError, ops.moe_route_topk, logits.double(), K)
    _raises(ValueError, ops.moe_route_topk, logits, K, topk_idx=_full((T, K + 1), torch.int32, 7))
    _raises(TypeError, ops.moe_route_topk, logits, K, topk_idx=_full((T, K), torch.int64, 7))
    _raises(ValueError, ops.moe_route_topk, logits.t(), K)              # not contiguous
    bad = dict(s, expert_counts=_full((E - 1,), torch.int32, 7))
    _raises(ValueError, ops.moe_send_counts, idx, E, R, out=bad)
    _raises(ValueError, ops.moe_route_plan, logits, K, R, out=bad)
    _raises(TypeError, ops.moe_send_counts, idx.long(), E, R, out=s)
    _raises(ValueError, ops.moe_send_counts, idx, E, R, ws=_full((64, 64), torch.uint8, 7), out=s)
    _raises(ValueError, ops.moe_send_counts, idx, E, R,
            placement=_full((E - 1,), torch.int32, 0), out=s)
    # the co-selection matrix must be exactly [E][E] int32
    _raises(ValueError, ops.moe_route_plan, logits, K, R, out=s,
            coselect=_full((8, 8), torch.int32, 7))
    _raises(ValueError, ops.moe_coselect_counts, idx, E, coselect=_full((8, 8), torch.int32, 7))
    _raises(TypeError, ops.moe_coselect_counts, idx, E, coselect=_full((E, E), torch.int64, 7))
    _untouched(s)


def test_dispatch_and_combine_reject_bad_buffers():
    logits, x, idx, gate = _inputs()
    say("[binding] dispatch and combine")
    c = ops.moe_send_counts(idx, E, R)
    torch.cuda.synchronize()
    N = T * K
    out = {"send": _full((N, H), torch.bfloat16, 7), "row_token": _full((N,), torch.int32, 7),
           "row_expert": _full((N,), torch.int32, 7), "row_weight": _full((N,), torch.float32, 7),
           "slot_row": _full((T, K), torch.int32, 7)}
    # a send buffer of bytes sized for one byte per element: too small for bf16 rows
    _raises(TypeError, ops.moe_dispatch_permute, x, idx, gate, E, R, c["ws"],
            out=dict(out, send=_full((N, H), torch.uint8, 7)))
    _raises(ValueError, ops.moe_dispatch_permute, x, idx, gate, E, R, c["ws"],
            out=dict(out, slot_row=_full((T, K - 1), torch.int32, 7)))
    _raises(ValueError, ops.moe_dispatch_permute, x, idx[:T - 1], gate[:T - 1], E, R, c["ws"],
            out=out)                                              # ids for fewer tokens than x
    _raises(ValueError, ops.moe_dispatch_permute, x, idx, gate[:, :K - 1], E, R, c["ws"], out=out)
    _raises(TypeError, ops.moe_dispatch_permute, x, idx, gate.double(), E, R, c["ws"], out=out)
    _raises(ValueError, ops.moe_dispatch_permute, x, idx, gate, E, R, c["ws"], out=out,
            coselect=_full((8, 8), torch.int32, 7))
    _raises(ValueError, ops.moe_dispatch_permute, x, idx, gate, E, R, c["ws"], out=out,
            coselect=_full((E, E), torch.int32, 7), coselect_tokens=T + 1)
    _untouched(out)
    rows = torch.zeros((N, H), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros(N, dtype=torch.float32, device=DEV)
    slot = torch.zeros((T, K), dtype=torch.int32, device=DEV)
    o = {"o": _full((T, H), torch.bfloat16, 7)}
    _raises(ValueError, ops.moe_combine, rows, w, slot, out=_full((T, H // 2), torch.bfloat16, 7))
    _raises(TypeError, ops.moe_combine, rows, w, slot, out=_full((T, H), torch.float32, 7))
    _raises(ValueError, ops.moe_combine, rows, w[:N - 1], slot, out=o["o"])
    _raises(TypeError, ops.moe_combine, rows.float(), w, slot, out=o["o"])
    _raises(TypeError, ops.moe_combine, rows, w, slot.long(), out=o["o"])
    _untouched(o)


def test_one_call_and_pipelined_reject_bad_buffers():
    logits, x, idx, gate = _inputs()
    say("[binding] one-call and pipelined")
    s = _sentinels()
    _raises(ValueError, ops.moe_route_dispatch, logits, x[:T - 1], K, R, out=s)
    _raises(ValueError, ops.moe_route_dispatch, logits, x, K, R,
            out=dict(s, send=_full((T * K - 1, H), torch.bfloat16, 7)))
    nxt = {"topk_idx": _full((T, K), torch.int32, 7), "topk_gate": _full((T, K), torch.float32, 7)}
    _raises(ValueError, ops.moe_combine_route, None, None, None, logits, K, R,
            next_out=dict(nxt, topk_idx=_full((T, K + 1), torch.int32, 7)))
    _raises(TypeError, ops.moe_combine_route, None, None, None, logits.double(), K, R,
            next_out=nxt)
    _raises(ValueError, ops.moe_combine_route, None, None, None, logits, K, R, next_out=nxt,
            placement=_full((E + 1,), torch.int32, 0))
    rows = torch.zeros((T * K, H), dtype=torch.bfloat16, device=DEV)
    slot = torch.zeros((T, K), dtype=torch.int32, device=DEV)
    _raises(ValueError, ops.moe_combine_route, rows, torch.zeros(T, device=DEV), slot, logits, K, R,
            next_out=nxt)                                        # one weight per row
    _raises(ValueError, ops.moe_combine_route, rows, None, slot, logits, K, R, next_out=nxt,
            out=_full((T + 1, H), torch.bfloat16, 7))
    _untouched(nxt)
    _, routed = ops.moe_combine_route(None, None, None, logits, K, R)
    torch.cuda.synchronize()
    _raises(ValueError, ops.moe_dispatch_routed, x[:T - 1], routed, out=s)
    _raises(ValueError, ops.moe_dispatch_routed, x, routed,
            out=dict(s, slot_row=_full((T, K + 1), torch.int32, 7)))
    _raises(ValueError, ops.moe_dispatch_routed, x, routed, out=s,
            coselect=_full((E + 1, E + 1), torch.int32, 7))
    _untouched(s)


def test_receive_side_and_planner_reject_bad_buffers():
    logits, x, idx, gate = _inputs()
    say("[binding] receive side and shuffle planner")
    c = ops.moe_send_counts(idx, E, R, dedup=True)
    d = ops.moe_dispatch_permute_dedup(x, idx, gate, E, R, c["ws"])
    torch.cuda.synchronize()
    C = T * K
    s = _sentinels()
    _raises(ValueError, ops.moe_expand_counts, d["row_experts"][:, :K - 1], d["n_rows"], E, R,
            out=s)
    _raises(TypeError, ops.moe_expand_counts, d["row_experts"], d["n_rows"].long(), E, R, out=s)
    ews = ops.expand_workspace(C, E, K, R, DEV)
    _raises(ValueError, ops.moe_expand_permute, d["send"], d["row_gates"][:C - 1], d["n_rows"], E,
            R, ews)
    _raises(ValueError, ops.moe_expand_reduce, d["send"], torch.zeros(C - 1, device=DEV),
            torch.zeros((C, K), dtype=torch.int32, device=DEV), d["n_rows"])
    _untouched(s)
    prev = cur = nxt = idx
    pc = _full((E, E, R), torch.int32, 7)
    sc = _full((E, R), torch.int32, 7)
    _raises(ValueError, ops.moe_shuffle_fit, prev, cur, nxt[:T - 1], E, R, pair_counts=pc,
            single_counts=sc)
    _raises(ValueError, ops.moe_shuffle_fit, prev, cur, nxt, E, R,
            pair_counts=_full((E, E, R + 1), torch.int32, 7), single_counts=sc)
    _raises(TypeError, ops.moe_shuffle_fit, prev, cur, nxt, E, R, pair_counts=pc,
            single_counts=_full((E, R), torch.int64, 7))
    _raises(ValueError, ops.moe_shuffle_predict, prev, cur, _full((E, E + 1, R), torch.int32, 7),
            sc, 8)
    _raises(ValueError, ops.moe_shuffle_predict, prev, cur, pc, sc, 8,
            scores=_full((T, R + 1), torch.float32, 7))
    _untouched({"pair": pc, "single": sc})
