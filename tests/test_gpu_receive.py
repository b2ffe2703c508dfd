"""GPU parity of the receive side of the deduplicating dispatcher.

Received rows come from the GPU's own dedup dispatch (capacity T*k rows, of
which only n_rows are valid; the rest holds whatever the buffer held), are
expanded per expert, reduced back to one row per received row, and combined.
Every output is compared with the CPU oracle on every row: plans, rows and
metadata bit for bit, and reductions bit for bit too (both sides take the same
fixed chain of fp32 fused multiply-adds in ascending row order, then one bf16
rounding).
"""
import numpy as np
import pytest
import torch

from combine_top_router_select_amd import ops
from combine_top_router_select_amd import workloads as WL
from gpu_util import (assert_bf16_equal, bf16_dev, bf16_host, bf16_to_f64, host, say,
                      to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.lib()
    yield
    torch.cuda.synchronize()


def sync():
    torch.cuda.synchronize()


def received(oracle_mod, x_bits, logits, k, E, R, placement, garbage=True):
    """GPU dedup dispatch of the inputs (the rows a rank receives) and the
    oracle's version of the same."""
    idx_o, gate_o = oracle_mod.route_topk(logits, k)
    place_dev = to_dev(placement) if placement is not None else None
    idx, gate = to_dev(idx_o), to_dev(gate_o)
    c = ops.moe_send_counts(idx, E, R, place_dev, dedup=True)
    T = idx_o.shape[0]
    N = T * k
    out = None
    if garbage:
        # rows past n_rows hold plausible-looking ids and gates: they must be ignored
        H = x_bits.shape[1]
        out = {"send": torch.zeros((N, H), dtype=torch.bfloat16, device="cuda:0"),
               "row_experts": torch.zeros((N, k), dtype=torch.int32, device="cuda:0"),
               "row_gates": torch.full((N, k), 0.5, dtype=torch.float32, device="cuda:0")}
    d = ops.moe_dispatch_permute_dedup(bf16_dev(x_bits), idx, gate, E, R, c["ws"],
                                       out=out)
    o = oracle_mod.dispatch_dedup(x_bits, idx_o, gate_o, E, R, placement)
    return idx_o, gate_o, d, o


def check_expand(oracle_mod, d, o, E, R, placement, k, exp_cap=None):
    """Expand the GPU's received rows; compare with the oracle's expansion of
    the oracle's rows (which equal the GPU's bit for bit)."""
    place_dev = to_dev(placement) if placement is not None else None
    C = d["row_experts"].shape[0]
    ec = ops.moe_expand_counts(d["row_experts"], d["n_rows"], E, R, place_dev)
    ex = ops.moe_expand_permute(d["send"], d["row_gates"], d["n_rows"], E, R, ec["ws"],
                                expanded_capacity=exp_cap)
    D = o["n_rows"]
    rx = np.concatenate([o["row_experts"], np.zeros((C - D, k), np.int32)])
    rg = np.concatenate([o["row_gates"], np.full((C - D, k), 0.5, np.float32)])
    ref = oracle_mod.expand_dedup(o["send"], rx, rg, D, E, R, placement, capacity=C)
    sync()
    for key in ("expert_counts", "rank_counts", "rank_offsets", "expert_offsets"):
        assert (host(ec[key]) == ref[key]).all(), key
    n = ref["n_expanded"]
    cap = n if exp_cap is None else min(n, exp_cap)
    assert (bf16_host(ex["expanded"][:cap]) == ref["expanded"][:cap]).all()
    assert (host(ex["exp_row"][:cap]) == ref["exp_row"][:cap]).all()
    assert (host(ex["exp_expert"][:cap]) == ref["exp_expert"][:cap]).all()
    assert (host(ex["exp_gate"][:cap]).view(np.uint32)
            == ref["exp_gate"][:cap].view(np.uint32)).all()
    rs_ref = ref["row_slot"].copy()
    rs_ref[rs_ref >= cap] = -1            # entries past the expanded capacity are dropped
    assert (host(ex["row_slot"]) == rs_ref).all()
    return ec, ex, ref


SMALL = [  # T, H, E, k, R
    (1, 64, 8, 2, 4), (65, 64, 8, 2, 4), (1000, 256, 64, 6, 16), (777, 512, 128, 8, 16),
    (300, 128, 8, 8, 8), (129, 2048, 64, 6, 1), (200, 64, 64, 6, 64), (130, 192, 1024, 16, 64),
    (257, 8, 16, 1, 4),
]


@pytest.mark.parametrize("T,H,E,k,R", SMALL)
@pytest.mark.parametrize("pl", ["contiguous", "random"])
def test_expand_parity(oracle_mod, T, H, E, k, R, pl):
    say(f"[expand] T={T} H={H} E={E} k={k} R={R} placement={pl}")
    inp = WL.make_custom_inputs(T, H, E, seed=T + 3 * E + k)
    place = None if pl == "contiguous" else WL.random_placement(E, R, seed=T + k)
    _, _, d, o = received(oracle_mod, inp["x_bits"], inp["logits"], k, E, R, place)
    check_expand(oracle_mod, d, o, E, R, place, k)


def test_expand_capacity_limit(oracle_mod):
    """An expanded buffer too small for every entry: entries past it are not
    written (canary) and their row_slot is -1; rank_offsets[R] still reports the
    rows the expansion needs."""
    T, H, E, k, R = 500, 128, 32, 4, 8
    inp = WL.make_custom_inputs(T, H, E, seed=3)
    _, _, d, o = received(oracle_mod, inp["x_bits"], inp["logits"], k, E, R, None)
    cap = T * k - 333
    PAD = 1024
    buf = torch.empty(((cap + PAD) * H,), dtype=torch.bfloat16, device="cuda:0")
    buf.view(torch.uint8).fill_(0x5A)
    place_dev = None
    ec = ops.moe_expand_counts(d["row_experts"], d["n_rows"], E, R, place_dev)
    out = {"expanded": buf[:cap * H].view(cap, H)}
    ops.moe_expand_permute(d["send"], d["row_gates"], d["n_rows"], E, R, ec["ws"],
                           expanded_capacity=cap, out=out)
    sync()
    assert int(host(ec["rank_offsets"])[R]) == T * k
    assert bool((buf.view(torch.uint8)[cap * H * 2:] == 0x5A).all())
    check_expand(oracle_mod, d, o, E, R, None, k, exp_cap=cap)


def test_expand_no_rows(oracle_mod):
    """n_rows = 0: nothing is counted or expanded, every row_slot is -1, and the
    reduction writes nothing."""
    C, H, E, k, R = 300, 64, 16, 4, 4
    dv = "cuda:0"
    rows = torch.ones((C, H), dtype=torch.bfloat16, device=dv)
    rx = torch.zeros((C, k), dtype=torch.int32, device=dv)
    rg = torch.ones((C, k), dtype=torch.float32, device=dv)
    n0 = torch.zeros(1, dtype=torch.int32, device=dv)
    ec = ops.moe_expand_counts(rx, n0, E, R)
    ex = ops.moe_expand_permute(rows, rg, n0, E, R, ec["ws"])
    out = torch.empty((C, H), dtype=torch.bfloat16, device=dv)
    out.view(torch.uint8).fill_(0x5A)
    ops.moe_expand_reduce(ex["expanded"], ex["exp_gate"], ex["row_slot"], n0, out=out)
    sync()
    assert (host(ec["expert_counts"]) == 0).all() and (host(ec["rank_offsets"]) == 0).all()
    assert (host(ex["row_slot"]) == -1).all()
    assert bool((out.view(torch.uint8) == 0x5A).all())


@pytest.mark.parametrize("T,H,E,k,R", [(1000, 512, 64, 6, 16), (777, 256, 128, 8, 16),
                                       (300, 128, 8, 8, 2)])
def test_expand_reduce_random_experts(oracle_mod, T, H, E, k, R):
    """Non-identity experts: random expert outputs in the expanded layout,
    gate weights and NULL weights; rows past n_rows are left untouched."""
    say(f"[reduce] T={T} H={H} E={E} k={k} R={R}")
    inp = WL.make_custom_inputs(T, H, E, seed=T + E)
    _, _, d, o = received(oracle_mod, inp["x_bits"], inp["logits"], k, E, R, None)
    ec, ex, ref = check_expand(oracle_mod, d, o, E, R, None, k)
    D, n = o["n_rows"], ref["n_expanded"]
    C = T * k
    rng = np.random.default_rng(T)
    Y = WL.bf16_bits_from_f32(rng.standard_normal((n, H)).astype(np.float32) * 2)
    Yd = torch.zeros((C, H), dtype=torch.bfloat16, device="cuda:0")
    Yd[:n] = bf16_dev(Y)
    for wname, w in (("gate", ref["exp_gate"]), ("none", None)):
        out = torch.empty((C, H), dtype=torch.bfloat16, device="cuda:0")
        out.view(torch.uint8).fill_(0x5A)
        wd = None if w is None else ex["exp_gate"]
        ops.moe_expand_reduce(Yd, wd, ex["row_slot"], d["n_rows"], out=out)
        rr = oracle_mod.reduce_rows(Y, w, ref["row_slot"], D)
        sync()
        assert_bf16_equal(bf16_host(out[:D]), rr, f"reduce weights={wname}")
        assert bool((out[D:].view(torch.uint8) == 0x5A).all())


@pytest.mark.parametrize("name", [n for n in WL.ORDER if "dedup" in WL.get(n).dispatch])
def test_receive_chain_workload(oracle_mod, name):
    """The whole receive side at the workload's full size, identity experts:
    expansion, the reduction of every received row and the weight-1 combine
    bit-exact against the oracle, and the combined output within 2 bf16 ulps of
    x (two bf16 roundings)."""
    w = WL.get(name)
    say(f"[receive] {name}")
    inp = WL.make_inputs(w)
    E, k, R = w.n_experts, w.top_k, w.n_ranks
    idx_o, gate_o, d, o = received(oracle_mod, inp["x_bits"], inp["logits"], k, E, R,
                                   inp["placement"], garbage=False)
    ec, ex, ref = check_expand(oracle_mod, d, o, E, R, inp["placement"], k)
    D = o["n_rows"]
    red = ops.moe_expand_reduce(ex["expanded"], ex["exp_gate"], ex["row_slot"], d["n_rows"])
    out = ops.moe_combine(red, None, d["slot_row"])
    red_o = oracle_mod.reduce_rows(ref["expanded"], ref["exp_gate"], ref["row_slot"], D)
    sync()
    red_g = bf16_host(red[:D])
    assert_bf16_equal(red_g, red_o, f"{name} reduce, all {D} rows")
    # combine of the reduced rows, weight 1: the oracle on the same rows
    out_o = oracle_mod.combine(red_o, None, o["slot_row"])
    got = bf16_host(out)
    assert_bf16_equal(got, out_o, f"{name} combine of the reduced rows")
    xf, of = bf16_to_f64(inp["x_bits"]), bf16_to_f64(got)
    ulp = np.maximum(np.abs(xf), 2.0 ** -126) * 2.0 ** -7
    assert (np.abs(of - xf) <= 2 * ulp).all()


def _random_receive_case(i):
    rng = np.random.default_rng(2000 + i)
    R = int(rng.choice([1, 2, 4, 8, 16, 32]))
    m = int(rng.choice([1, 2, 3, 4, 8]))
    E = R * m
    k = int(rng.integers(1, min(E, 16) + 1))
    T = int(rng.integers(1, 2000))
    H = int(rng.choice([8, 24, 64, 256, 2056]))
    pl = bool(rng.integers(0, 2))
    return T, H, E, k, R, pl


@pytest.mark.parametrize("i", range(50))
def test_random_receive(oracle_mod, i):
    """Fifty seeded random shapes through the receive side (garbage past the
    received rows): expansion and the gate-weighted reduction of random expert
    outputs bit-exact."""
    T, H, E, k, R, pl = _random_receive_case(i)
    placement = WL.random_placement(E, R, seed=i) if pl else None
    say(f"[receive random {i}] T={T} H={H} E={E} k={k} R={R} random placement={pl}")
    inp = WL.make_custom_inputs(T, H, E, seed=50 + i)
    _, _, d, o = received(oracle_mod, inp["x_bits"], inp["logits"], k, E, R, placement)
    ec, ex, ref = check_expand(oracle_mod, d, o, E, R, placement, k)
    D, n = o["n_rows"], ref["n_expanded"]
    C = T * k
    rng = np.random.default_rng(i)
    Y = WL.bf16_bits_from_f32(rng.standard_normal((max(n, 1), H)).astype(np.float32))[:n]
    Yd = torch.zeros((C, H), dtype=torch.bfloat16, device="cuda:0")
    Yd[:n] = bf16_dev(Y)
    out = ops.moe_expand_reduce(Yd, ex["exp_gate"], ex["row_slot"], d["n_rows"])
    rr = oracle_mod.reduce_rows(Y, ref["exp_gate"], ref["row_slot"], D)
    sync()
    assert_bf16_equal(bf16_host(out[:D]), rr, f"receive random {i}")
