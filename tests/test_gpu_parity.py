"""GPU parity: every C-ABI entry point against the CPU oracle on identical
seeded inputs.

Bars: bit-exact for indices, counts, offsets, row positions, copied rows and
integer metadata; gates within 1 fp32 ulp (both sides evaluate the same fp64
formula, only the exp implementations differ); dedup row weights bit-exact
(same fp64 additions in the same order); combine within 1 bf16 ulp of the
oracle's exactly rounded fp64 sum (plus the fp32 accumulation bound where the
terms can cancel); co-selection counts bit-exact.
"""
import numpy as np
import pytest
import torch

from combine_top_router_select_amd import ops
from combine_top_router_select_amd import workloads as WL
from gpu_util import (bf16_dev, bf16_host, bf16_to_f64, bf16_ulp_diff, f32_ulp_diff, host,
                      say, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.lib()
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def sync():
    torch.cuda.synchronize()


# ------------------------------------------------------------------- route --

ROUTE_CASES = [(1, 8, 2), (1000, 64, 6), (777, 128, 8), (300, 8, 8), (257, 3, 2), (129, 1, 1),
               (200, 100, 16), (500, 256, 8), (130, 1024, 16), (64, 2, 1), (100, 33, 5),
               (65, 512, 3)]


@pytest.mark.parametrize("T,E,k", ROUTE_CASES)
@pytest.mark.parametrize("tied", [False, True])
def test_route_parity(oracle_mod, T, E, k, tied):
    say(f"[route] T={T} E={E} k={k} tied={tied}")
    inp = WL.make_custom_inputs(T, 8, E, seed=T * 7 + E + k,
                                logit_values=[-1.0, -0.0, 0.0, 1.0] if tied else None)
    idx_o, gate_o = oracle_mod.route_topk(inp["logits"], k)
    idx, gate = ops.moe_route_topk(to_dev(inp["logits"]), k)
    sync()
    assert (host(idx) == idx_o).all()
    assert f32_ulp_diff(host(gate), gate_o).max() <= 1


@pytest.mark.parametrize("name", WL.ORDER)
def test_route_parity_workloads(oracle_mod, name):
    w = WL.get(name)
    say(f"[route] workload {name}")
    inp = WL.make_inputs(w, with_x=False)
    idx_o, gate_o = oracle_mod.route_topk(inp["logits"], w.top_k)
    idx, gate = ops.moe_route_topk(to_dev(inp["logits"]), w.top_k)
    sync()
    assert (host(idx) == idx_o).all()
    d = f32_ulp_diff(host(gate), gate_o)
    say(f"  gate max ulp {d.max()}, non-exact {(d > 0).mean():.2e}")
    assert d.max() <= 1


# ------------------------------------------------ fused routing + plan --

ROUTE_PLAN_CASES = [  # T, E, k, R
    (1, 8, 2, 4), (63, 8, 2, 4), (64, 64, 6, 16), (1000, 64, 6, 16), (777, 128, 8, 16),
    (300, 8, 8, 8), (257, 3, 1, 1), (129, 1, 1, 1), (500, 256, 8, 32), (200, 100, 16, 4),
    (4100, 16, 4, 16), (130, 512, 16, 64), (70, 1024, 3, 8),
    (5000, 256, 8, 16),   # tile bitmaps of 79 tiles: two chunks, atomic adds into W
    (100, 33, 5, 11),     # scalar logit loads (E % 4 != 0) in the fused kernel
    (90, 96, 7, 12),      # 16-byte loads with a partial last chunk
]


@pytest.mark.parametrize("T,E,k,R", ROUTE_PLAN_CASES)
@pytest.mark.parametrize("dedup", [False, True])
@pytest.mark.parametrize("pl", ["contiguous", "random"])
@pytest.mark.parametrize("softmax_all", [False, True])
def test_route_plan_parity(oracle_mod, T, E, k, R, dedup, pl, softmax_all):
    """moe_route_plan against the oracle (ids, gates, counts, offsets,
    co-selection counts accumulated onto a nonzero matrix) and against
    moe_route_topk + moe_send_counts (every byte of the plan, and the dispatch
    that consumes it).  E > 128 takes the unfused path."""
    say(f"[route_plan] T={T} E={E} k={k} R={R} dedup={dedup} placement={pl} "
        f"softmax_all={softmax_all}")
    inp = WL.make_custom_inputs(T, 64, E, seed=T * 5 + E + k + R)
    route = oracle_mod.route_topk_softmax_all if softmax_all else oracle_mod.route_topk
    idx_o, gate_o = route(inp["logits"], k)
    placement = WL.random_placement(E, R, seed=T) if pl == "random" else None
    place_dev = to_dev(placement) if placement is not None else None
    logits = to_dev(inp["logits"])
    rng = np.random.default_rng(T + E)
    W0 = rng.integers(0, 1000, size=(E, E)).astype(np.int32)
    cs = T if dedup else (T * 2) // 3          # all tokens, or a prefix ending inside a tile
    W = to_dev(W0.copy())
    idx, gate, c = ops.moe_route_plan(logits, k, R, place_dev, dedup, softmax_all, coselect=W,
                                      coselect_tokens=cs)
    idx2, gate2 = ops.moe_route_topk(logits, k, softmax_all=softmax_all)
    c2 = ops.moe_send_counts(idx2, E, R, place_dev, dedup=dedup)
    sync()
    assert (host(idx) == idx_o).all()
    assert f32_ulp_diff(host(gate), gate_o).max() <= 1
    assert (host(gate).view(np.uint32) == host(gate2).view(np.uint32)).all()
    co = oracle_mod.send_counts(idx_o, E, R, placement, dedup)
    _check_counts(c, co, dedup)
    W_o = oracle_mod.coselect(idx_o, E, tokens=cs, W=W0.copy())
    assert (host(W) == W_o).all()
    # the plan in the workspace: header, group bases, tile counts, slot codes
    assert _plan_equal(c["ws"], c2["ws"], T, E, k, R, dedup)
    f = ops.moe_dispatch_permute_dedup if dedup else ops.moe_dispatch_permute
    x = bf16_dev(inp["x_bits"])
    d = f(x, idx, gate, E, R, c["ws"], place_dev)
    o = (oracle_mod.dispatch_dedup if dedup else oracle_mod.dispatch)(inp["x_bits"], idx_o, gate_o,
                                                                     E, R, placement)
    sync()
    assert (host(d["slot_row"]) == o["slot_row"]).all()
    assert (bf16_host(d["send"][:o["n_rows"]]) == o["send"]).all()


def _plan_equal(ws_a, ws_b, T, E, k, R, dedup):
    """Plan regions compared field by field (the tile-count padding bytes past
    the last tile are never read and may differ)."""
    tiles = (T + 63) // 64
    tp = (tiles + 15) // 16 * 16
    groups = tp // 16
    cols = E + (R if dedup else 0)
    pos = R if dedup else E
    al = lambda v: (v + 255) // 256 * 256
    base_off = 256
    tcnt_off = al(base_off + pos * groups * 4)
    lslot_off = al(tcnt_off + cols * tp)
    a, b = host(ws_a), host(ws_b)
    if not (a[:4] == b[:4]).all():
        return False
    if not (a[base_off:base_off + pos * groups * 4] == b[base_off:base_off + pos * groups * 4]).all():
        return False
    ta = a[tcnt_off:tcnt_off + cols * tp].reshape(cols, tp)[:, :tiles]
    tb = b[tcnt_off:tcnt_off + cols * tp].reshape(cols, tp)[:, :tiles]
    if not (ta == tb).all():
        return False
    return bool((a[lslot_off:lslot_off + T * k * 4] == b[lslot_off:lslot_off + T * k * 4]).all())


# ------------------------------------------------------ counts + dispatch --

def _check_counts(c, co, dedup):
    assert (host(c["expert_counts"]) == co["expert_counts"]).all()
    assert (host(c["rank_counts"]) == co["rank_counts"]).all()
    assert (host(c["rank_offsets"]) == co["rank_offsets"]).all()
    if not dedup:
        assert (host(c["expert_offsets"]) == co["expert_offsets"]).all()


def run_dispatch_parity(oracle_mod, x_bits, idx_o, gate_o, E, R, placement, dedup,
                        explicit_place=False):
    T, k = idx_o.shape
    place_arr = placement if placement is not None else WL.contiguous_placement(E, R)
    place_dev = to_dev(place_arr) if (placement is not None or explicit_place) else None
    idx = to_dev(idx_o)
    gate = to_dev(gate_o)
    x = bf16_dev(x_bits)
    c = ops.moe_send_counts(idx, E, R, place_dev, dedup=dedup)
    if dedup:
        d = ops.moe_dispatch_permute_dedup(x, idx, gate, E, R, c["ws"], place_dev)
        o = oracle_mod.dispatch_dedup(x_bits, idx_o, gate_o, E, R, placement)
    else:
        d = ops.moe_dispatch_permute(x, idx, gate, E, R, c["ws"], place_dev)
        o = oracle_mod.dispatch(x_bits, idx_o, gate_o, E, R, placement)
    sync()
    _check_counts(c, o, dedup)
    n = o["n_rows"]
    assert (host(d["slot_row"]) == o["slot_row"]).all()
    assert (host(d["row_token"][:n]) == o["row_token"]).all()
    assert (host(d["row_weight"][:n]).view(np.uint32) == o["row_weight"].view(np.uint32)).all()
    if dedup:
        assert int(host(d["n_rows"])[0]) == n
        assert (host(d["row_experts"][:n]) == o["row_experts"]).all()
        assert (host(d["row_gates"][:n]).view(np.uint32) == o["row_gates"].view(np.uint32)).all()
    else:
        assert (host(d["row_expert"][:n]) == o["row_expert"]).all()
    assert (bf16_host(d["send"][:n]) == o["send"]).all()
    return c, d, o


SMALL = [  # T, H, E, k, R
    (1, 64, 8, 2, 4), (63, 64, 8, 2, 4), (65, 64, 8, 2, 4), (1000, 256, 64, 6, 16),
    (777, 512, 128, 8, 16), (300, 128, 8, 8, 8), (129, 2048, 64, 6, 1), (200, 64, 64, 6, 64),
    (500, 1024, 128, 2, 8), (130, 192, 1024, 16, 64), (257, 8, 16, 1, 4), (100, 4096, 32, 4, 32),
]


@pytest.mark.parametrize("T,H,E,k,R", SMALL)
@pytest.mark.parametrize("dedup", [False, True])
@pytest.mark.parametrize("pl", ["contiguous", "explicit", "random"])
def test_dispatch_parity_small(oracle_mod, T, H, E, k, R, dedup, pl):
    say(f"[dispatch] T={T} H={H} E={E} k={k} R={R} dedup={dedup} placement={pl}")
    inp = WL.make_custom_inputs(T, H, E, seed=T + H + E + k + R)
    idx_o, gate_o = oracle_mod.route_topk(inp["logits"], k)
    placement = WL.random_placement(E, R, seed=T) if pl == "random" else None
    run_dispatch_parity(oracle_mod, inp["x_bits"], idx_o, gate_o, E, R, placement, dedup,
                        explicit_place=(pl == "explicit"))


@pytest.mark.parametrize("dedup", [False, True])
def test_dispatch_parity_large_plan(oracle_mod, dedup):
    """70000 tokens, explicit placement: 1094 tiles, 69 tile-count vectors per
    column dealt to 16 lanes each (5 per lane) in the scan."""
    T, H, E, k, R = 70000, 32, 64, 4, 16
    say(f"[dispatch] large plan T={T} dedup={dedup}")
    inp = WL.make_custom_inputs(T, H, E, seed=99)
    idx_o, gate_o = oracle_mod.route_topk(inp["logits"], k)
    placement = WL.random_placement(E, R, seed=5)
    run_dispatch_parity(oracle_mod, inp["x_bits"], idx_o, gate_o, E, R, placement, dedup)


@pytest.mark.parametrize("dedup,pl", [(False, "contiguous"), (False, "random"), (True, "random")])
def test_dispatch_parity_huge_plan(oracle_mod, dedup, pl):
    """300000 tokens: 4688 tiles, 293 vectors per column, more than the scan
    keeps in registers, so it takes the looping variant (one lane per column)."""
    T, H, E, k, R = 300000, 16, 8, 2, 4
    say(f"[dispatch] huge plan T={T} dedup={dedup} placement={pl}")
    inp = WL.make_custom_inputs(T, H, E, seed=101)
    idx_o, gate_o = oracle_mod.route_topk(inp["logits"], k)
    placement = None if pl == "contiguous" else WL.random_placement(E, R, seed=6)
    run_dispatch_parity(oracle_mod, inp["x_bits"], idx_o, gate_o, E, R, placement, dedup)


@pytest.mark.parametrize("dedup", [False, True])
def test_route_plan_huge(oracle_mod, dedup):
    """The combined routing call at 300000 tokens (4688 tiles: the looping scan)
    against the oracle's ids, counts and co-selection counts, and its plan
    against the separate calls byte for byte."""
    T, E, k, R = 300000, 64, 6, 16
    say(f"[route_plan] huge T={T} E={E} k={k} R={R} dedup={dedup}")
    inp = WL.make_custom_inputs(T, 16, E, seed=303)
    logits = to_dev(inp["logits"])
    W = torch.zeros((E, E), dtype=torch.int32, device=logits.device)
    idx, gate, c = ops.moe_route_plan(logits, k, R, None, dedup, coselect=W)
    idx2, _ = ops.moe_route_topk(logits, k)
    c2 = ops.moe_send_counts(idx2, E, R, None, dedup=dedup)
    sync()
    idx_o, _ = oracle_mod.route_topk(inp["logits"], k)
    assert (host(idx) == idx_o).all()
    _check_counts(c, oracle_mod.send_counts(idx_o, E, R, None, dedup), dedup)
    assert (host(W) == oracle_mod.coselect(idx_o, E)).all()
    assert _plan_equal(c["ws"], c2["ws"], T, E, k, R, dedup)


def _random_case(i):
    """Seeded shape draw for the randomized parity sweep (same cases every run)."""
    rng = np.random.default_rng(1000 + i)
    R = int(rng.choice([1, 2, 3, 4, 8, 16, 32, 64]))
    m = int(rng.choice([1, 2, 3, 4, 8]))
    E = min(R * m, 1024)
    k = int(rng.integers(1, min(E, 16) + 1))
    T = int(rng.integers(1, 3000))
    H = int(rng.choice([8, 16, 24, 64, 200, 1024, 2056]))
    dedup = bool(rng.integers(0, 2))
    pl = str(rng.choice(["contiguous", "random"]))
    ties = bool(rng.integers(0, 4) == 0)
    return T, H, E, k, R, dedup, pl, ties


@pytest.mark.parametrize("i", range(100))
def test_random_shapes(oracle_mod, i):
    """A hundred seeded random shapes (T, H, E, k, R, mode, placement, tied
    logits) through the combined routing call, dispatch and combine, against
    the oracle."""
    T, H, E, k, R, dedup, pl, ties = _random_case(i)
    say(f"[random {i}] T={T} H={H} E={E} k={k} R={R} dedup={dedup} placement={pl} ties={ties}")
    inp = WL.make_custom_inputs(T, H, E, seed=i,
                                logit_values=[-1.0, -0.0, 0.0, 1.0] if ties else None)
    placement = WL.random_placement(E, R, seed=i) if pl == "random" else None
    place_dev = to_dev(placement) if placement is not None else None
    W = torch.zeros((E, E), dtype=torch.int32, device=torch.device("cuda:0"))
    idx, gate, c = ops.moe_route_plan(to_dev(inp["logits"]), k, R, place_dev, dedup, coselect=W)
    f = ops.moe_dispatch_permute_dedup if dedup else ops.moe_dispatch_permute
    d = f(bf16_dev(inp["x_bits"]), idx, gate, E, R, c["ws"], place_dev)
    out = ops.moe_combine(d["send"], d["row_weight"], d["slot_row"])
    sync()
    idx_o, gate_o = oracle_mod.route_topk(inp["logits"], k)
    assert (host(idx) == idx_o).all()
    assert f32_ulp_diff(host(gate), gate_o).max() <= 1
    gate_h = host(gate)
    o = (oracle_mod.dispatch_dedup if dedup else oracle_mod.dispatch)(
        inp["x_bits"], idx_o, gate_h, E, R, placement)
    _check_counts(c, o, dedup)
    n = o["n_rows"]
    assert (host(d["slot_row"]) == o["slot_row"]).all()
    assert (bf16_host(d["send"][:n]) == o["send"]).all()
    assert (host(d["row_weight"][:n]).view(np.uint32) == o["row_weight"].view(np.uint32)).all()
    ref = oracle_mod.combine(o["send"], o["row_weight"], o["slot_row"])
    assert bf16_ulp_diff(bf16_host(out), ref).max() <= 1
    assert (host(W) == oracle_mod.coselect(idx_o, E)).all()


@pytest.mark.parametrize("T", [2044, 2048, 2049, 4097])
@pytest.mark.parametrize("dedup", [False, True])
def test_dispatch_metadata_order_boundary(oracle_mod, T, dedup):
    """Token counts around the grid size (512 workgroups of four one-chunk
    tokens) from which each token's metadata is written in the XCD-contiguous
    order, on grids padded to a multiple of 8 workgroups: 511, 512, 513 and
    1025 workgroups.  Rows, metadata and slots against the oracle."""
    H, E, k, R = 64, 64, 6, 16
    say(f"[metadata order] T={T} dedup={dedup}")
    inp = WL.make_custom_inputs(T, H, E, seed=T)
    placement = WL.random_placement(E, R, seed=T)
    place_dev = to_dev(placement)
    idx, gate, c = ops.moe_route_plan(to_dev(inp["logits"]), k, R, place_dev, dedup)
    f = ops.moe_dispatch_permute_dedup if dedup else ops.moe_dispatch_permute
    d = f(bf16_dev(inp["x_bits"]), idx, gate, E, R, c["ws"], place_dev)
    sync()
    idx_h, gate_h = host(idx), host(gate)
    o = (oracle_mod.dispatch_dedup if dedup else oracle_mod.dispatch)(
        inp["x_bits"], idx_h, gate_h, E, R, placement)
    n = o["n_rows"]
    assert (host(d["slot_row"]) == o["slot_row"]).all()
    assert (bf16_host(d["send"][:n]) == o["send"]).all()
    assert (host(d["row_token"][:n]) == o["row_token"]).all()
    assert (host(d["row_weight"][:n]).view(np.uint32) == o["row_weight"].view(np.uint32)).all()
    if dedup:
        assert int(host(d["n_rows"])[0]) == n
        assert (host(d["row_experts"][:n]) == o["row_experts"]).all()
        assert (host(d["row_gates"][:n]).view(np.uint32) == o["row_gates"].view(np.uint32)).all()
    else:
        assert (host(d["row_expert"][:n]) == o["row_expert"]).all()


def test_dispatch_empty_ranks(oracle_mod):
    """Tokens that only ever pick experts of ranks 0 and 2: ranks 1 and 3 are
    empty segments."""
    T, H, E, k, R = 500, 128, 16, 3, 4
    inp = WL.make_custom_inputs(T, H, E, seed=3)
    lg = inp["logits"].copy()
    lg[:, 4:8] -= 100.0
    lg[:, 12:16] -= 100.0
    idx_o, gate_o = oracle_mod.route_topk(lg, k)
    for dedup in (False, True):
        c, d, o = run_dispatch_parity(oracle_mod, inp["x_bits"], idx_o, gate_o, E, R, None,
                                      dedup)
        rc = host(c["rank_counts"])
        assert rc[1] == 0 and rc[3] == 0


def test_bytes_per_element_1_and_4(oracle_mod):
    """The pack is a byte copy: fp8-sized and fp32-sized rows move bit for bit."""
    T, E, k, R = 300, 16, 4, 4
    inp = WL.make_custom_inputs(T, 8, E, seed=11)
    idx_o, gate_o = oracle_mod.route_topk(inp["logits"], k)
    rng = np.random.default_rng(0)
    for dt, H in ((np.uint8, 48), (np.uint32, 20)):
        xb = rng.integers(0, np.iinfo(dt).max, size=(T, H), dtype=dt)
        x = to_dev(xb)
        idx, gate = to_dev(idx_o), to_dev(gate_o)
        for dedup in (False, True):
            c = ops.moe_send_counts(idx, E, R, None, dedup=dedup)
            f = ops.moe_dispatch_permute_dedup if dedup else ops.moe_dispatch_permute
            d = f(x, idx, gate, E, R, c["ws"])
            o = (oracle_mod.dispatch_dedup if dedup else oracle_mod.dispatch)(
                xb, idx_o, gate_o, E, R)
            sync()
            n = o["n_rows"]
            assert (host(d["send"][:n]) == o["send"]).all()
            assert (host(d["slot_row"]) == o["slot_row"]).all()


# ------------------------------------------------------------------ combine --

@pytest.mark.parametrize("dedup", [False, True])
def test_combine_random_rows(oracle_mod, dedup):
    """Non-identity experts: random signed rows, random weights (both signs),
    NULL weights, and slots marked -1 (skipped)."""
    T, H, E, k, R = 1000, 512, 64, 8, 8
    say(f"[combine] random rows dedup={dedup}")
    inp = WL.make_custom_inputs(T, 8, E, seed=21)
    idx_o, gate_o = oracle_mod.route_topk(inp["logits"], k)
    o = (oracle_mod.dispatch_dedup if dedup else oracle_mod.dispatch)(
        inp["x_bits"], idx_o, gate_o, E, R)
    n = o["n_rows"]
    rng = np.random.default_rng(5)
    Y = WL.bf16_bits_from_f32(rng.standard_normal((n, H)).astype(np.float32) * 3)
    slot = o["slot_row"].copy()
    slot[rng.random(slot.shape) < 0.05] = -1
    for wname, w in (("gate", o["row_weight"]), ("none", None),
                     ("signed", rng.standard_normal(n).astype(np.float32))):
        ref = oracle_mod.combine(Y, w, slot)
        got = bf16_host(ops.moe_combine(bf16_dev(Y), to_dev(w), to_dev(slot)))
        sync()
        # bound: 1 bf16 ulp + fp32 accumulation error gamma_k * sum |w*y|
        yv = bf16_to_f64(Y)
        wv = np.ones(n) if w is None else w.astype(np.float64)
        absum = np.zeros((T, H))
        for t in range(T):
            for r in sorted({int(v) for v in slot[t] if v >= 0}):
                absum[t] += np.abs(wv[r] * yv[r])
        gam = k * 2.0 ** -24 / (1 - k * 2.0 ** -24)
        g64, r64 = bf16_to_f64(got), bf16_to_f64(ref)
        ulp = np.maximum(np.abs(r64), np.abs(g64)) * 2.0 ** -7
        ulp = np.maximum(ulp, 2.0 ** -133)
        ok = np.abs(g64 - r64) <= ulp + gam * absum
        exact = (got == ref).mean()
        say(f"  weights={wname}: bit-exact {exact:.6f}, max ulp {bf16_ulp_diff(got, ref).max()}")
        assert ok.all()


# -------------------------------------------------------------- co-selection --

@pytest.mark.parametrize("T,E,k,n", [(4096, 64, 6, 4096), (16384, 128, 6, 4096),
                                     (16384, 128, 2, 16384), (300, 8, 8, 300),
                                     (1000, 256, 8, 1000), (20000, 128, 4, 20000),
                                     (5, 3, 3, 5), (600, 1024, 16, 600),
                                     (4100, 64, 16, 4100), (64, 17, 1, 64)])
def test_coselect_parity(oracle_mod, T, E, k, n):
    say(f"[coselect] T={T} E={E} k={k} n={n}")
    inp = WL.make_custom_inputs(T, 1, E, seed=E + k + n)
    idx_o, _ = oracle_mod.route_topk(inp["logits"], k)
    W_o = oracle_mod.coselect(idx_o, E, tokens=n)
    idx = to_dev(idx_o)
    W = ops.moe_coselect_counts(idx, E, tokens=n)
    sync()
    assert (host(W) == W_o).all()
    ops.moe_coselect_counts(idx, E, tokens=n, coselect=W)   # accumulates
    sync()
    assert (host(W) == 2 * W_o).all()


# ------------------------------------------------------- full workloads --

def gpu_chain(inp, w, dedup, stream=None, fused=False):
    """The whole hot path on the GPU, through the C ABI: the separate routing,
    counting and co-selection calls, or (fused) the combined routing call the
    benchmark times."""
    E, k, R = w.n_experts, w.top_k, w.n_ranks
    place = to_dev(inp["placement"]) if inp["placement"] is not None else None
    logits = to_dev(inp["logits"])
    x = bf16_dev(inp["x_bits"])
    if fused:
        W = torch.zeros((E, E), dtype=torch.int32, device=logits.device)
        idx, gate, c = ops.moe_route_plan(logits, k, R, place, dedup, coselect=W,
                                          coselect_tokens=w.coselect_tokens, stream=stream)
    else:
        idx, gate = ops.moe_route_topk(logits, k, stream=stream)
        c = ops.moe_send_counts(idx, E, R, place, dedup=dedup, stream=stream)
    f = ops.moe_dispatch_permute_dedup if dedup else ops.moe_dispatch_permute
    d = f(x, idx, gate, E, R, c["ws"], place, stream=stream)
    out = ops.moe_combine(d["send"], d["row_weight"], d["slot_row"], stream=stream)
    if not fused:
        W = ops.moe_coselect_counts(idx, E, tokens=w.coselect_tokens, stream=stream)
    return idx, gate, c, d, out, W


def _cases():
    for name in WL.ORDER:
        for mode in WL.get(name).dispatch:
            yield name, mode == "dedup", True
    yield "deepseek_moe_16b", False, False
    yield "zyphra_top6_ep32", True, False


@pytest.mark.parametrize("name,dedup,fused", list(_cases()))
def test_workload_end_to_end(oracle_mod, name, dedup, fused):
    """Full sizes, the launch configuration the benchmark times (fused: the
    combined routing call; two cases also with the separate calls): logits ->
    route, counts, co-selection -> dispatch -> combine (identity experts), all on
    the GPU, against the oracle chain on the same inputs."""
    w = WL.get(name)
    say(f"[e2e] {name} dedup={dedup} fused={fused} T={w.tokens} H={w.hidden_dim} "
        f"E={w.n_experts} k={w.top_k} R={w.n_ranks}")
    inp = WL.make_inputs(w)
    idx, gate, c, d, out, W = gpu_chain(inp, w, dedup, fused=fused)
    sync()
    idx_o, gate_o = oracle_mod.route_topk(inp["logits"], w.top_k)
    assert (host(idx) == idx_o).all()
    assert f32_ulp_diff(host(gate), gate_o).max() <= 1
    # downstream of routing the oracle consumes the GPU's gates, so that fp32
    # gate ulps do not blur the bit-exact comparisons
    gate_h = host(gate)
    f = oracle_mod.dispatch_dedup if dedup else oracle_mod.dispatch
    o = f(inp["x_bits"], idx_o, gate_h, w.n_experts, w.n_ranks, inp["placement"])
    _check_counts(c, o, dedup)
    n = o["n_rows"]
    say(f"  rows {n} of {w.tokens * w.top_k} ({100 * (1 - n / (w.tokens * w.top_k)):.1f}% "
        f"removed)")
    assert (host(d["slot_row"]) == o["slot_row"]).all()
    assert (host(d["row_token"][:n]) == o["row_token"]).all()
    assert (host(d["row_weight"][:n]).view(np.uint32) == o["row_weight"].view(np.uint32)).all()
    if dedup:
        assert int(host(d["n_rows"])[0]) == n
        assert (host(d["row_experts"][:n]) == o["row_experts"]).all()
        assert (host(d["row_gates"][:n]).view(np.uint32) == o["row_gates"].view(np.uint32)).all()
    else:
        assert (host(d["row_expert"][:n]) == o["row_expert"]).all()
    send_h = bf16_host(d["send"][:n])
    assert (send_h == o["send"]).all()
    del send_h
    out_h = bf16_host(out)
    ref = oracle_mod.combine(o["send"], o["row_weight"], o["slot_row"])
    diff = bf16_ulp_diff(out_h, ref)
    say(f"  combine max ulp {diff.max()}, non-exact {(diff > 0).mean():.2e}")
    assert diff.max() <= 1
    # identity experts with gates summing to 1 return the input
    assert (out_h == inp["x_bits"]).all()
    W_o = oracle_mod.coselect(idx_o, w.n_experts, tokens=w.coselect_tokens)
    assert (host(W) == W_o).all()


# ------------------------------------------------ determinism, streams, edges --

@pytest.mark.parametrize("name", ["deepseek_moe_16b", "qwen3_30b_a3b"])
def test_two_streams_of_batches(oracle_mod, name):
    """The benchmark's launch configuration: independent batches alternate
    between two streams with no waits between them (four batches, two per
    stream, each on its own buffers and workspace), every call through the
    combined routing call, dispatch and combine; every batch matches the
    oracle."""
    w = WL.get(name)
    E, k, R = w.n_experts, w.top_k, w.n_ranks
    say(f"[two streams] {name}: 4 batches")
    streams = [torch.cuda.current_stream(), torch.cuda.Stream()]
    batches = [WL.make_inputs(w, seed=s) for s in (0, 1, 2, 3)]
    sync()
    res = []
    for i, inp in enumerate(batches):
        st = streams[i % 2]
        with torch.cuda.stream(st):
            logits = to_dev(inp["logits"])
            x = bf16_dev(inp["x_bits"])
            W = torch.zeros((E, E), dtype=torch.int32, device=logits.device)
            idx, gate, c = ops.moe_route_plan(logits, k, R, None, False, coselect=W,
                                              coselect_tokens=w.coselect_tokens, stream=st)
            d = ops.moe_dispatch_permute(x, idx, gate, E, R, c["ws"], stream=st)
            out = ops.moe_combine(d["send"], d["row_weight"], d["slot_row"], stream=st)
        res.append((idx, gate, c, d, out, W))
    sync()
    for inp, (idx, gate, c, d, out, W) in zip(batches, res):
        idx_o, gate_o = oracle_mod.route_topk(inp["logits"], k)
        assert (host(idx) == idx_o).all()
        assert f32_ulp_diff(host(gate), gate_o).max() <= 1
        o = oracle_mod.dispatch(inp["x_bits"], idx_o, host(gate), E, R)
        _check_counts(c, o, False)
        assert (host(d["slot_row"]) == o["slot_row"]).all()
        assert (bf16_host(d["send"]) == o["send"]).all()
        assert (bf16_host(out) == inp["x_bits"]).all()
        assert (host(W) == oracle_mod.coselect(idx_o, E, tokens=w.coselect_tokens)).all()

def test_determinism_and_nondefault_stream():
    w = WL.get("qwen3_30b_a3b")
    inp = WL.make_inputs(w)
    say("[determinism] qwen3_30b_a3b dedup, separate calls on the default stream vs the "
        "combined routing call on a side stream")
    a = gpu_chain(inp, w, True)
    sync()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = gpu_chain(inp, w, True, stream=s, fused=True)
    s.synchronize()
    n = int(host(a[3]["n_rows"])[0])
    assert (host(a[0]) == host(b[0])).all()
    assert (host(a[1]).view(np.uint32) == host(b[1]).view(np.uint32)).all()
    for key in ("slot_row", "row_token", "row_weight"):
        assert (host(a[3][key][:n]) == host(b[3][key][:n])).all()
    assert (bf16_host(a[3]["send"][:n]) == bf16_host(b[3]["send"][:n])).all()
    assert (bf16_host(a[4]) == bf16_host(b[4])).all()
    assert (host(a[5]) == host(b[5])).all()


def test_canary_padding_untouched(oracle_mod):
    """Outputs are views at the front of larger buffers filled with a canary;
    nothing past the documented extents is written."""
    T, H, E, k, R = 333, 256, 32, 4, 8
    inp = WL.make_custom_inputs(T, H, E, seed=77)
    dv = torch.device("cuda:0")
    PAD = 4096

    def canary(n, dtype):
        t = torch.empty(n + PAD, dtype=dtype, device=dv)
        t.view(torch.uint8).fill_(0x5A)
        return t

    def untouched(buf, n):
        return bool((buf.view(torch.uint8)[n * buf.element_size():] == 0x5A).all())

    idx_b, gate_b = canary(T * k, torch.int32), canary(T * k, torch.float32)
    idx, gate = ops.moe_route_topk(to_dev(inp["logits"]), k, idx_b[:T * k].view(T, k),
                                   gate_b[:T * k].view(T, k))
    for dedup in (False, True):
        bufs = {"expert_counts": canary(E, torch.int32), "rank_counts": canary(R, torch.int32),
                "rank_offsets": canary(R + 1, torch.int32)}
        sizes = {"expert_counts": E, "rank_counts": R, "rank_offsets": R + 1}
        if not dedup:
            bufs["expert_offsets"] = canary(E, torch.int32)
            sizes["expert_offsets"] = E
        c = ops.moe_send_counts(idx, E, R, None, dedup,
                                out={kk: v[:sizes[kk]] for kk, v in bufs.items()})
        N = T * k
        ob = {"send": canary(N * H, torch.bfloat16), "row_token": canary(N, torch.int32),
              "row_weight": canary(N, torch.float32), "slot_row": canary(N, torch.int32)}
        osz = {"send": N * H, "row_token": N, "row_weight": N, "slot_row": N}
        if dedup:
            ob.update(row_experts=canary(N * k, torch.int32), row_gates=canary(N * k, torch.float32),
                      n_rows=canary(1, torch.int32))
            osz.update(row_experts=N * k, row_gates=N * k, n_rows=1)
        else:
            ob["row_expert"] = canary(N, torch.int32)
            osz["row_expert"] = N
        views = {}
        for kk, v in ob.items():
            vv = v[:osz[kk]]
            if kk == "send":
                vv = vv.view(N, H)
            elif kk in ("slot_row", "row_experts", "row_gates"):
                vv = vv.view(-1, k)
            views[kk] = vv
        f = ops.moe_dispatch_permute_dedup if dedup else ops.moe_dispatch_permute
        d = f(bf16_dev(inp["x_bits"]), idx, gate, E, R, c["ws"], None, out=views)
        out_b = canary(T * H, torch.bfloat16)
        ops.moe_combine(d["send"], d["row_weight"], d["slot_row"], out=out_b[:T * H].view(T, H))
        W_b = canary(E * E, torch.int32)
        W_b[:E * E].zero_()
        ops.moe_coselect_counts(idx, E, coselect=W_b[:E * E].view(E, E))
        sync()
        for kk, v in bufs.items():
            assert untouched(v, sizes[kk]), kk
        for kk, v in ob.items():
            assert untouched(v, osz[kk]), kk
        assert untouched(out_b, T * H) and untouched(W_b, E * E)
        assert untouched(idx_b, T * k) and untouched(gate_b, T * k)


def test_zero_tokens():
    dv = torch.device("cuda:0")
    E, k, R, H = 16, 2, 4, 64
    idx = torch.empty((0, k), dtype=torch.int32, device=dv)
    gate = torch.empty((0, k), dtype=torch.float32, device=dv)
    ops.moe_route_topk(torch.empty((0, E), dtype=torch.float32, device=dv), k, idx, gate)
    for dedup in (False, True):
        c = ops.moe_send_counts(idx, E, R, None, dedup)
        x = torch.empty((0, H), dtype=torch.bfloat16, device=dv)
        f = ops.moe_dispatch_permute_dedup if dedup else ops.moe_dispatch_permute
        nr = torch.full((1,), 7, dtype=torch.int32, device=dv)
        out = {"n_rows": nr} if dedup else None
        d = f(x, idx, gate, E, R, c["ws"], out=out)
        sync()
        assert (host(c["rank_counts"]) == 0).all() and (host(c["rank_offsets"]) == 0).all()
        assert (host(c["expert_counts"]) == 0).all()
        if dedup:
            assert int(host(d["n_rows"])[0]) == 0
    out = ops.moe_combine(torch.empty((0, H), dtype=torch.bfloat16, device=dv), None,
                          torch.empty((0, k), dtype=torch.int32, device=dv))
    sync()
    assert out.shape == (0, H)
    for dedup in (False, True):    # the combined routing call: zeros, W untouched
        W = torch.full((E, E), 3, dtype=torch.int32, device=dv)
        _, _, c = ops.moe_route_plan(torch.empty((0, E), dtype=torch.float32, device=dv), k, R,
                                     None, dedup, coselect=W)
        sync()
        assert (host(c["rank_counts"]) == 0).all() and (host(c["rank_offsets"]) == 0).all()
        assert (host(c["expert_counts"]) == 0).all() and (host(W) == 3).all()


def test_k_equals_e_and_k1(oracle_mod):
    """Every expert selected (k = E: one rank per token per rank, dedup rows =
    T*R) and k = 1 (combine returns x)."""
    T, H = 200, 128
    for E, k, R in ((8, 8, 4), (16, 16, 16), (64, 1, 16)):
        inp = WL.make_custom_inputs(T, H, E, seed=E + k)
        idx_o, gate_o = oracle_mod.route_topk(inp["logits"], k)
        for dedup in (False, True):
            c, d, o = run_dispatch_parity(oracle_mod, inp["x_bits"], idx_o, gate_o, E, R, None,
                                          dedup)
            if dedup and k == E:
                assert o["n_rows"] == T * R
            out = ops.moe_combine(d["send"], d["row_weight"], d["slot_row"])
            sync()
            assert (bf16_host(out) == inp["x_bits"]).all()


# ------------------------------------------------------------- fp8 rows --

def _fp8_dev(u8):
    return torch.from_numpy(np.ascontiguousarray(u8)).to("cuda:0").view(torch.float8_e4m3fn)


def _bound_ok(got, ref, Y_f64, w, slot, k):
    n = Y_f64.shape[0]
    wv = np.ones(n) if w is None else w.astype(np.float64)
    absum = np.zeros((slot.shape[0], Y_f64.shape[1]))
    for t in range(slot.shape[0]):
        for r in sorted({int(v) for v in slot[t] if v >= 0}):
            absum[t] += np.abs(wv[r] * Y_f64[r])
    gam = k * 2.0 ** -24 / (1 - k * 2.0 ** -24)
    g64, r64 = bf16_to_f64(got), bf16_to_f64(ref)
    ulp = np.maximum(np.maximum(np.abs(r64), np.abs(g64)) * 2.0 ** -7, 2.0 ** -133)
    return bool((np.abs(g64 - r64) <= ulp + gam * absum).all())


@pytest.mark.parametrize("dedup", [False, True])
@pytest.mark.parametrize("H", [1024, 2048, 4096, 272, 2064, 16])
def test_combine_fp8_rows(oracle_mod, dedup, H):
    """fp8 E4M3 rows (random bytes, no NaN, some -0) into bf16, for gate, NULL
    and signed weights, against the oracle's exact decode and sum."""
    T, E, k, R = 600, 64, 6, 8
    say(f"[combine fp8] H={H} dedup={dedup}")
    inp = WL.make_custom_inputs(T, 8, E, seed=H + dedup)
    idx_o, gate_o = oracle_mod.route_topk(inp["logits"], k)
    o = (oracle_mod.dispatch_dedup if dedup else oracle_mod.dispatch)(
        inp["x_bits"], idx_o, gate_o, E, R)
    n = o["n_rows"]
    rng = np.random.default_rng(H)
    Y = rng.integers(0, 256, (n, H)).astype(np.uint8)
    Y[(Y & 0x7F) == 0x7F] = 0x80
    Yf = torch.from_numpy(Y).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    slot = o["slot_row"]
    for w in (o["row_weight"], None, rng.standard_normal(n).astype(np.float32)):
        ref = oracle_mod.combine_fp8(Y, w, slot)
        got = bf16_host(ops.moe_combine(_fp8_dev(Y), to_dev(w), to_dev(slot)))
        sync()
        assert _bound_ok(got, ref, Yf, w, slot, k)


def test_fp8_dispatch_combine_chain(oracle_mod):
    """x in fp8: dispatch moves the bytes bit for bit (bytes_per_element 1),
    combine decodes them; identity experts with gates summing to 1 return x
    converted to bf16 within the fp32 rounding of the gate sum (1 bf16 ulp)."""
    T, H, E, k, R = 1000, 2048, 64, 6, 16
    inp = WL.make_custom_inputs(T, H, E, seed=8)
    xf = torch.from_numpy(inp["x_bits"].view(np.int16)).view(torch.bfloat16).float()
    x8 = xf.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    idx_o, gate_o = oracle_mod.route_topk(inp["logits"], k)
    for dedup in (False, True):
        idx, gate = to_dev(idx_o), to_dev(gate_o)
        c = ops.moe_send_counts(idx, E, R, None, dedup=dedup)
        f = ops.moe_dispatch_permute_dedup if dedup else ops.moe_dispatch_permute
        d = f(_fp8_dev(x8), idx, gate, E, R, c["ws"])
        o = (oracle_mod.dispatch_dedup if dedup else oracle_mod.dispatch)(x8, idx_o, gate_o, E, R)
        n = o["n_rows"]
        sync()
        assert (host(d["send"][:n].view(torch.uint8)) == o["send"]).all()
        out = bf16_host(ops.moe_combine(d["send"], d["row_weight"], d["slot_row"]))
        ref = oracle_mod.combine_fp8(o["send"], o["row_weight"], o["slot_row"])
        sync()
        assert bf16_ulp_diff(out, ref).max() <= 1
        x_bf = (torch.from_numpy(x8).view(torch.float8_e4m3fn).to(torch.bfloat16)
                .view(torch.int16).numpy().view(np.uint16))
        assert bf16_ulp_diff(out, x_bf).max() <= 1


def test_fp8_reduce(oracle_mod):
    """The receive-side reduction with fp8 expert outputs."""
    T, H, E, k, R = 500, 512, 32, 4, 8
    inp = WL.make_custom_inputs(T, H, E, seed=12)
    idx_o, gate_o = oracle_mod.route_topk(inp["logits"], k)
    o = oracle_mod.dispatch_dedup(inp["x_bits"], idx_o, gate_o, E, R)
    D = o["n_rows"]
    ref_ex = oracle_mod.expand_dedup(None, o["row_experts"], o["row_gates"], D, E, R,
                                     with_rows=False)
    n = ref_ex["n_expanded"]
    rng = np.random.default_rng(4)
    Y = rng.integers(0, 256, (n, H)).astype(np.uint8)
    Y[(Y & 0x7F) == 0x7F] = 0x00
    nr = torch.tensor([D], dtype=torch.int32, device="cuda:0")
    out = ops.moe_expand_reduce(_fp8_dev(Y), to_dev(ref_ex["exp_gate"]),
                                to_dev(ref_ex["row_slot"]), nr)
    ref = oracle_mod.combine_fp8(Y, ref_ex["exp_gate"], ref_ex["row_slot"][:D])
    sync()
    Yf = torch.from_numpy(Y).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _bound_ok(bf16_host(out[:D]), ref, Yf, ref_ex["exp_gate"], ref_ex["row_slot"][:D], k)


@pytest.mark.parametrize("T,E,k", [(1000, 64, 6), (777, 128, 8), (300, 8, 8), (130, 1024, 16),
                                   (129, 1, 1), (257, 3, 2)])
def test_route_softmax_all_parity(oracle_mod, T, E, k):
    say(f"[route softmax_all] T={T} E={E} k={k}")
    inp = WL.make_custom_inputs(T, 8, E, seed=T + 5 * E + k)
    idx_o, gate_o = oracle_mod.route_topk_softmax_all(inp["logits"], k)
    idx, gate = ops.moe_route_topk(to_dev(inp["logits"]), k, softmax_all=True)
    sync()
    assert (host(idx) == idx_o).all()
    assert f32_ulp_diff(host(gate), gate_o).max() <= 1


@pytest.mark.parametrize("i", range(32))
def test_random_fp8_chain(oracle_mod, i):
    """Thirty-two seeded random shapes with fp8 rows: the combined routing call,
    dispatch of E4M3 bytes (bit for bit) and the decoding combine against the
    oracle's exact decode and sum."""
    rng = np.random.default_rng(3000 + i)
    R = int(rng.choice([1, 2, 4, 8, 16]))
    E = R * int(rng.choice([1, 2, 4, 8]))
    k = int(rng.integers(1, min(E, 16) + 1))
    T = int(rng.integers(1, 2000))
    H = int(rng.choice([16, 48, 272, 1024, 4096]))
    dedup = bool(rng.integers(0, 2))
    say(f"[fp8 random {i}] T={T} H={H} E={E} k={k} R={R} dedup={dedup}")
    inp = WL.make_custom_inputs(T, H, E, seed=70 + i)
    x8 = rng.integers(0, 256, (T, H)).astype(np.uint8)
    x8[(x8 & 0x7F) == 0x7F] = 0x80                 # no NaN; those become -0
    idx, gate, c = ops.moe_route_plan(to_dev(inp["logits"]), k, R, None, dedup)
    f = ops.moe_dispatch_permute_dedup if dedup else ops.moe_dispatch_permute
    d = f(_fp8_dev(x8), idx, gate, E, R, c["ws"])
    out = ops.moe_combine(d["send"], d["row_weight"], d["slot_row"])
    sync()
    idx_o, _ = oracle_mod.route_topk(inp["logits"], k)
    assert (host(idx) == idx_o).all()
    o = (oracle_mod.dispatch_dedup if dedup else oracle_mod.dispatch)(x8, idx_o, host(gate), E, R)
    n = o["n_rows"]
    assert (host(d["send"][:n].view(torch.uint8)) == o["send"]).all()
    ref = oracle_mod.combine_fp8(o["send"], o["row_weight"], o["slot_row"])
    Y = np.array([[oracle_mod.e4m3_to_double(int(b)) for b in row] for row in o["send"]]) \
        if n * H <= 200000 else None
    got = bf16_host(out)
    if Y is not None:
        assert _bound_ok(got, ref, Y, o["row_weight"], o["slot_row"], k)
    else:
        assert bf16_ulp_diff(got, ref).max() <= 1
