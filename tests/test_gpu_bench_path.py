"""The benchmark's timed calls compute the path: bench.py's C-ABI call lists
(raw_step_calls, every argument marshalled once per buffer set), run the way
its timed loop runs them - each batch routed inside the combine launch of the
step before it on the same stream, consecutive steps alternating between the
streams with no waits - leave every buffer set's ids, gates, counts, rows,
combined output and co-selection counts equal to the oracle's."""
import importlib.util
import os

import numpy as np
import pytest
import torch

from combine_top_router_select_amd import ops
from combine_top_router_select_amd import workloads as WL
from gpu_util import bf16_host, f32_ulp_diff, host, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_path", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name,dedup,n_streams", [
    ("deepseek_moe_16b", False, 2), ("qwen3_30b_a3b", True, 2), ("e256_top8_h2048", False, 2),
    ("zyphra_top2_ep8", True, 1)])
def test_bench_pipelined_calls(oracle_mod, name, dedup, n_streams):
    bench = _bench()
    w = WL.get(name)
    T, E, k, R = w.tokens, w.n_experts, w.top_k, w.n_ranks
    say(f"[bench path] {name} dedup={dedup} streams={n_streams}")
    dev = torch.device("cuda:0")
    inp = WL.make_inputs(w)
    nsets = 2 * n_streams
    sets = [bench.BufferSet(torch, ops, inp, w, dedup, dev) for _ in range(nsets)]
    streams = [torch.cuda.current_stream()] + [torch.cuda.Stream() for _ in range(n_streams - 1)]
    for b in sets:   # every set routed before its first dispatch, as the bench does
        ops.moe_combine_route(None, None, None, b.logits, k, R, b.place, dedup,
                              next_out={"topk_idx": b.idx, "topk_gate": b.gate, "ws": b.ws})
    torch.cuda.synchronize()
    raw = [bench.raw_step_calls(torch, ops, b, w, dedup, False, 2, None, True,
                                streams[i % n_streams], "dispatch", False,
                                sets[(i + n_streams) % nsets])
           for i, b in enumerate(sets)]
    steps = 3 * nsets
    for i in range(steps):
        for fn, args in raw[i % nsets]:
            rc = fn(*args)
            assert rc == 0, (i, getattr(fn, "__name__", fn))
    torch.cuda.synchronize()
    idx_o, gate_o = oracle_mod.route_topk(inp["logits"], k)
    W_o = oracle_mod.coselect(idx_o, E, tokens=w.coselect_tokens)
    f = oracle_mod.dispatch_dedup if dedup else oracle_mod.dispatch
    o = None
    for b in sets:
        assert (host(b.idx) == idx_o).all()
        assert f32_ulp_diff(host(b.gate), gate_o).max() <= 1
        if o is None:
            o = f(inp["x_bits"], idx_o, host(b.gate), E, R, inp["placement"])
        n = o["n_rows"]
        assert (host(b.cnt["rank_offsets"]) == o["rank_offsets"]).all()
        assert (host(b.cnt["expert_counts"]) == o["expert_counts"]).all()
        assert (host(b.disp["slot_row"]) == o["slot_row"]).all()
        assert (bf16_host(b.disp["send"][:n]) == o["send"]).all()
        assert (host(b.disp["row_weight"][:n]).view(np.uint32) ==
                o["row_weight"].view(np.uint32)).all()
        assert (bf16_host(b.out) == inp["x_bits"]).all()     # identity experts
        assert (host(b.W) == (steps // nsets) * W_o).all()   # accumulated once per use


@pytest.mark.parametrize("name,dedup,receive,fp8", [
    ("deepseek_moe_16b", False, False, True), ("qwen3_30b_a3b", True, True, False)])
def test_prepared_sets_hold_whole_steps(oracle_mod, name, dedup, receive, fp8):
    """Before timing, every buffer set holds a whole step's plan, positions and
    rows (bench.prepare_sets): the per-kernel runs and the reference kernels
    read any set, also sets that no timed step of a short run dispatches."""
    import torch as _t
    bench = _bench()
    w = WL.get(name)
    T, k, R = w.tokens, w.top_k, w.n_ranks
    say(f"[bench prepare] {name} dedup={dedup} receive={receive} fp8={fp8}")
    dev = _t.device("cuda:0")
    inp = WL.make_inputs(w)
    if fp8:
        xb = _t.from_numpy(inp["x_bits"].view(np.int16)).view(_t.bfloat16)
        inp["x_fp8"] = xb.float().to(_t.float8_e4m3fn).view(_t.uint8).numpy()
    sets = [bench.BufferSet(_t, ops, inp, w, dedup, dev, receive, fp8) for _ in range(3)]
    bench.prepare_sets(_t, ops, sets, w, dedup, receive)
    idx_o, _ = oracle_mod.route_topk(inp["logits"], k)
    f = oracle_mod.dispatch_dedup if dedup else oracle_mod.dispatch
    o = f(inp["x_bits"], idx_o, host(sets[0].gate), w.n_experts, R, inp["placement"])
    n = o["n_rows"]
    for b in sets:
        assert (host(b.idx) == idx_o).all()
        assert (host(b.cnt["rank_offsets"]) == o["rank_offsets"]).all()
        assert (host(b.disp["slot_row"]) == o["slot_row"]).all()
        if fp8:
            assert (host(b.disp["send"][:n].view(_t.uint8)) == inp["x_fp8"][o["row_token"]]).all()
        else:
            assert (bf16_host(b.disp["send"][:n]) == o["send"]).all()
        if receive:
            assert (host(b.ecnt["rank_offsets"]) == host(sets[0].ecnt["rank_offsets"])).all()
        assert (bf16_host(b.out) == bf16_host(sets[0].out)).all()


def test_calls_allocate_nothing():
    """The entry points keep no device memory (the header's rule that they
    allocate nothing): with every buffer allocated beforehand, the free device
    memory reported by the runtime is the same before and after repeated whole
    steps - pipelined, one-call, separate calls, and dedup with the receive
    side.  (An allocation freed within the same call would not show here; the
    graph-capture tests run the same calls under capture.)"""
    import torch as _t
    bench = _bench()
    dev = _t.device("cuda:0")
    cases = [("deepseek_moe_16b", False, False, "pipe"), ("deepseek_moe_16b", False, False, "one"),
             ("qwen3_30b_a3b", False, False, "separate"), ("zyphra_top2_ep8", True, True, "pipe")]
    say("[allocate nothing] " + ", ".join(f"{c[0]}:{c[3]}" for c in cases))
    runs = []
    for name, dedup, receive, mode in cases:
        w = WL.get(name)
        inp = WL.make_inputs(w)
        sets = [bench.BufferSet(_t, ops, inp, w, dedup, dev, receive) for _ in range(2)]
        bench.prepare_sets(_t, ops, sets, w, dedup, receive)
        pipe = mode == "pipe"
        calls = [bench.raw_step_calls(_t, ops, b, w, dedup, receive, 2, None, mode != "separate",
                                      None, "dispatch", mode == "one",
                                      sets[(i + 1) % 2] if pipe else None)
                 for i, b in enumerate(sets)]
        runs.append((sets, calls))   # the sets stay alive: the calls hold their raw pointers

    def steps(n):
        for _, calls in runs:
            for i in range(n):
                for fn, args in calls[i % 2]:
                    assert fn(*args) == 0
        _t.cuda.synchronize()

    steps(2)   # first launches: code objects and runtime resources
    free0 = _t.cuda.mem_get_info()[0]
    steps(6)
    free1 = _t.cuda.mem_get_info()[0]
    assert free1 == free0, (free0, free1)
