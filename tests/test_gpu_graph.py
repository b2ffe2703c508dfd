"""The hot path captured in a HIP graph replays correctly.

The chain (route -> counts -> dispatch -> combine -> co-selection; in dedup
mode also the receive side: expansion -> reduction -> weight-1 combine) is
captured once, then replayed several times with eager GPU work and
synchronisations in between; every replay must reproduce the eager result bit
for bit.
"""
import numpy as np
import pytest
import torch

from combine_top_router_select_amd import ops
from combine_top_router_select_amd import workloads as WL
from gpu_util import bf16_dev, bf16_host, host, say, to_dev

pytestmark = pytest.mark.gpu


def _buffers(w, dedup, dev):
    T, H, E, k, R = w.tokens, w.hidden_dim, w.n_experts, w.top_k, w.n_ranks
    N = T * k
    i32, f32 = torch.int32, torch.float32
    b = {"idx": torch.empty((T, k), dtype=i32, device=dev),
         "gate": torch.empty((T, k), dtype=f32, device=dev),
         "ws": ops.workspace(T, E, k, R, dedup, dev),
         "cnt": {"expert_counts": torch.empty(E, dtype=i32, device=dev),
                 "rank_counts": torch.empty(R, dtype=i32, device=dev),
                 "rank_offsets": torch.empty(R + 1, dtype=i32, device=dev)},
         "disp": {"send": torch.empty((N, H), dtype=torch.bfloat16, device=dev),
                  "row_token": torch.empty(N, dtype=i32, device=dev),
                  "row_weight": torch.empty(N, dtype=f32, device=dev),
                  "slot_row": torch.empty((T, k), dtype=i32, device=dev)},
         "out": torch.empty((T, H), dtype=torch.bfloat16, device=dev),
         "W": torch.zeros((E, E), dtype=i32, device=dev)}
    if dedup:
        b["disp"].update(row_experts=torch.empty((N, k), dtype=i32, device=dev),
                         row_gates=torch.empty((N, k), dtype=f32, device=dev),
                         n_rows=torch.empty(1, dtype=i32, device=dev))
        b["ews"] = ops.expand_workspace(N, E, k, R, dev)
        b["ecnt"] = {"expert_counts": torch.empty(E, dtype=i32, device=dev),
                     "rank_counts": torch.empty(R, dtype=i32, device=dev),
                     "rank_offsets": torch.empty(R + 1, dtype=i32, device=dev),
                     "expert_offsets": torch.empty(E, dtype=i32, device=dev)}
        b["exp"] = {"expanded": torch.empty((N, H), dtype=torch.bfloat16, device=dev),
                    "exp_row": torch.empty(N, dtype=i32, device=dev),
                    "exp_expert": torch.empty(N, dtype=i32, device=dev),
                    "exp_gate": torch.empty(N, dtype=f32, device=dev),
                    "row_slot": torch.empty((N, k), dtype=i32, device=dev)}
        b["red"] = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
        b["out2"] = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    else:
        b["cnt"]["expert_offsets"] = torch.empty(E, dtype=i32, device=dev)
        b["disp"]["row_expert"] = torch.empty(N, dtype=i32, device=dev)
    return b


def _routed(w, dedup, place, b):
    return {"topk_idx": b["idx"], "topk_gate": b["gate"], "ws": b["ws"], "n_experts": w.n_experts,
            "n_ranks": w.n_ranks, "placement": place, "dedup": dedup}


def _step(w, dedup, logits, x, place, b, mode="separate"):
    """mode: "separate" calls; "plan": moe_route_plan (with the co-selection
    counts) then the dispatch; "one": moe_route_dispatch (with them); "pipe":
    moe_dispatch_routed (with them) on the batch that the previous step's
    combine launch routed, and a combine launch (moe_combine_route) that routes
    the same inputs again for the next step."""
    E, k, R = w.n_experts, w.top_k, w.n_ranks
    if mode == "pipe":
        d = ops.moe_dispatch_routed(x, _routed(w, dedup, place, b), out={**b["cnt"], **b["disp"]},
                                    coselect=b["W"], coselect_tokens=w.coselect_tokens)[1]
    elif mode == "one":   # routing, plan, rows and co-selection counts in one call
        d = ops.moe_route_dispatch(logits, x, k, R, place, dedup,
                                   out={"topk_idx": b["idx"], "topk_gate": b["gate"], **b["cnt"],
                                        **b["disp"]},
                                   ws=b["ws"], coselect=b["W"],
                                   coselect_tokens=w.coselect_tokens)[3]
    else:
        if mode == "plan":   # routing, plan and co-selection counts in one call
            c = ops.moe_route_plan(logits, k, R, place, dedup, topk_idx=b["idx"],
                                   topk_gate=b["gate"], ws=b["ws"], out=b["cnt"], coselect=b["W"],
                                   coselect_tokens=w.coselect_tokens)[2]
        else:
            ops.moe_route_topk(logits, k, b["idx"], b["gate"])
            c = ops.moe_send_counts(b["idx"], E, R, place, dedup, ws=b["ws"], out=b["cnt"])
        f = ops.moe_dispatch_permute_dedup if dedup else ops.moe_dispatch_permute
        d = f(x, b["idx"], b["gate"], E, R, c["ws"], out=b["disp"])
    if mode == "pipe":
        ops.moe_combine_route(d["send"], d["row_weight"], d["slot_row"], logits, k, R, place, dedup,
                              out=b["out"], next_out={"topk_idx": b["idx"], "topk_gate": b["gate"],
                                                      "ws": b["ws"]})
    else:
        ops.moe_combine(d["send"], d["row_weight"], d["slot_row"], out=b["out"])
    if dedup:
        ops.moe_expand_counts(d["row_experts"], d["n_rows"], E, R, place, ws=b["ews"],
                              out=b["ecnt"])
        ex = ops.moe_expand_permute(d["send"], d["row_gates"], d["n_rows"], E, R, b["ews"],
                                    out=b["exp"])
        red = ops.moe_expand_reduce(ex["expanded"], ex["exp_gate"], ex["row_slot"], d["n_rows"],
                                    out=b["red"])
        ops.moe_combine(red, None, d["slot_row"], out=b["out2"])
    if mode == "separate":
        ops.moe_coselect_counts(b["idx"], E, tokens=w.coselect_tokens, coselect=b["W"])


def _snapshot(b):
    snap = {"idx": host(b["idx"]), "gate": host(b["gate"]).view(np.uint32),
            "out": bf16_host(b["out"]), "W": host(b["W"])}
    if "ecnt" in b:
        for key, v in b["ecnt"].items():
            snap["e_" + key] = host(v)
        ne = int(snap["e_rank_offsets"][-1])
        D = int(host(b["disp"]["n_rows"])[0])
        snap["expanded"] = bf16_host(b["exp"]["expanded"][:ne])
        for key in ("exp_row", "exp_expert", "exp_gate"):
            snap[key] = host(b["exp"][key][:ne]).copy()
        snap["row_slot"] = host(b["exp"]["row_slot"][:D]).copy()
        snap["red"] = bf16_host(b["red"][:D])
        snap["out2"] = bf16_host(b["out2"])
    for key, v in b["cnt"].items():
        snap[key] = host(v)
    n = int(snap["rank_offsets"][-1])
    for key, v in b["disp"].items():
        if key == "send":
            snap[key] = bf16_host(v[:n])
        elif key in ("row_token", "row_expert", "row_experts", "row_gates", "row_weight"):
            snap[key] = host(v[:n]).copy()
        else:
            snap[key] = host(v)
    return snap


@pytest.mark.parametrize("name,dedup,mode", [
    ("deepseek_moe_16b", False, "separate"), ("zyphra_top6_ep32", True, "separate"),
    ("deepseek_moe_16b", False, "plan"), ("e256_top8_h2048", False, "plan"),
    ("zyphra_top2_ep8", True, "plan"),
    ("deepseek_moe_16b", False, "one"), ("qwen3_30b_a3b", True, "one"),
    ("e256_top8_h2048", False, "one"), ("zyphra_top2_ep8", True, "one"),
    ("zyphra_top6_ep32", True, "one"),
    ("deepseek_moe_16b", False, "pipe"), ("qwen3_30b_a3b", True, "pipe"),
    ("e256_top8_h2048", False, "pipe"), ("zyphra_top2_ep8", True, "pipe"),
    ("zyphra_top6_ep32", True, "pipe")])
def test_graph_replays_match_eager(name, dedup, mode):
    """mode "plan": moe_route_plan in place of the routing, counting and
    co-selection calls; "one": moe_route_dispatch in place of those and the
    dispatch (the dispatch scanning the plan itself at 4096 tokens and for the
    16384-token batch over 8 ranks, the scan kernel for the one over 32);
    "pipe": each replay dispatches the batch that the previous replay's combine
    launch routed (the first one routed before the warm-up) and routes it again.
    The eager reference uses the separate calls, so the replays also check the
    paths against each other."""
    w = WL.get(name)
    say(f"[graph] {name} dedup={dedup} mode={mode}")
    dev = torch.device("cuda:0")
    inp = WL.make_inputs(w)
    logits = to_dev(inp["logits"])
    x = bf16_dev(inp["x_bits"])
    place = to_dev(inp["placement"]) if inp["placement"] is not None else None

    eager = _buffers(w, dedup, dev)
    _step(w, dedup, logits, x, place, eager)
    torch.cuda.synchronize()
    ref = _snapshot(eager)

    gb = _buffers(w, dedup, dev)
    if mode == "pipe":   # the first batch: a routing-only combine launch
        ops.moe_combine_route(None, None, None, logits, w.top_k, w.n_ranks, place, dedup,
                              next_out={"topk_idx": gb["idx"], "topk_gate": gb["gate"],
                                        "ws": gb["ws"]})
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _step(w, dedup, logits, x, place, gb, mode)   # warm up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(w, dedup, logits, x, place, gb, mode)
    torch.cuda.synchronize()
    for rep in range(4):
        # scramble the outputs with eager work, then replay
        for v in list(gb["cnt"].values()) + list(gb["disp"].values()):
            v.view(torch.uint8).fill_(0xA5)
        gb["out"].view(torch.uint8).fill_(0x5A)
        if dedup:
            for v in list(gb["ecnt"].values()) + list(gb["exp"].values()):
                v.view(torch.uint8).fill_(0xA5)
            gb["red"].view(torch.uint8).fill_(0x5A)
            gb["out2"].view(torch.uint8).fill_(0x5A)
        if mode != "pipe":   # (pipelined: the previous replay routed this one's batch)
            gb["idx"].fill_(-1)
            gb["ws"].fill_(0xA5)   # the plan is rebuilt by every replay
        gb["W"].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(gb)
        for key, v in ref.items():
            assert (got[key] == v).all(), (rep, key)
