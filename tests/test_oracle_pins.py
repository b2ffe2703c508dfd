"""Pins of the CPU oracle against things other than itself (no GPU).

* the hand-worked example in golden/hand_example.json;
* brute-force enumeration on tiny inputs with dense ties and signed zeros;
* library routines for special cases (lexsort for top-k, full softmax at k=E,
  torch's fp32->bf16 cast for the rounding rule);
* the invariants the pages state (row sums, block sums, coarsening, dedup row
  count, Table I identities, co-selection symmetry and sums);
* closed forms (uniform-routing distinct-rank expectation).
"""
import json
import math
import os
import struct

from fractions import Fraction

import numpy as np
import pytest
import torch

import bruteforce as BF
from combine_top_router_select_amd import workloads as WL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32_ulp_diff(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    a = np.where(a < 0, -(a & 0x7FFFFFFF), a)
    b = np.where(b < 0, -(b & 0x7FFFFFFF), b)
    return np.abs(a - b)


def _float(v):
    return -0.0 if v == "-0.0" else float(v)


# ------------------------------------------------------------ hand example --

@pytest.fixture(scope="module")
def hand():
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        return json.load(f)


def test_hand_route(oracle_mod, hand):
    logits = np.array([[_float(v) for v in row] for row in hand["logits"]], np.float32)
    assert np.signbit(logits[2, 0]) and not np.signbit(logits[2, 1])
    idx, gate = oracle_mod.route_topk(logits, hand["k"])
    assert idx.tolist() == hand["topk_idx"]
    assert f32_ulp_diff(gate, np.array(hand["topk_gate"], np.float32)).max() <= 1


def test_hand_counts_and_nondedup(oracle_mod, hand):
    T, E, k, R = hand["T"], hand["E"], hand["k"], hand["R"]
    idx = np.array(hand["topk_idx"], np.int32)
    gate = np.array(hand["topk_gate"], np.float32)
    x = np.arange(T * 8, dtype=np.uint16).reshape(T, 8)
    d = oracle_mod.dispatch(x, idx, gate, E, R)
    nd = hand["nondedup"]
    assert d["expert_counts"].tolist() == hand["expert_counts"]
    for key in ("rank_counts", "rank_offsets", "expert_offsets", "row_token",
                "row_expert", "slot_row"):
        assert np.asarray(d[key]).tolist() == nd[key], key
    for p, (t, j) in enumerate(nd["row_weight_from_slot"]):
        assert d["row_weight"][p] == gate[t, j]
    for p, t in enumerate(nd["row_token"]):
        assert (d["send"][p] == x[t]).all()


def test_hand_dedup(oracle_mod, hand):
    T, E, k, R = hand["T"], hand["E"], hand["k"], hand["R"]
    idx = np.array(hand["topk_idx"], np.int32)
    gate = np.array(hand["topk_gate"], np.float32)
    x = np.arange(T * 8, dtype=np.uint16).reshape(T, 8)
    d = oracle_mod.dispatch_dedup(x, idx, gate, E, R)
    dd = hand["dedup"]
    for key in ("rank_counts", "rank_offsets", "row_token", "row_experts", "slot_row"):
        assert np.asarray(d[key]).tolist() == dd[key], key
    assert d["n_rows"] == dd["n_rows"]
    for p, srcs in enumerate(dd["row_gates_from_slot"]):
        for c, s in enumerate(srcs):
            want = 0.0 if s is None else gate[s[0], s[1]]
            assert d["row_gates"][p, c] == np.float32(want)
    assert d["row_weight"][2] == 1.0 and d["row_weight"][5] == 1.0
    assert d["row_weight"][0] == gate[0, 0] and d["row_weight"][4] == gate[1, 0]


def test_hand_coselect(oracle_mod, hand):
    idx = np.array(hand["topk_idx"], np.int32)
    W = oracle_mod.coselect(idx, hand["E"])
    assert W.tolist() == hand["coselect_W"]


def _bf16_bits(vals):
    return WL.bf16_bits_from_f32(np.array(vals, np.float32))


def test_hand_combine(oracle_mod, hand):
    cu = hand["combine_unweighted"]
    Y = _bf16_bits([[_float(v) for v in r] for r in cu["Y"]])
    out = oracle_mod.combine(Y, None, np.array(hand["nondedup"]["slot_row"], np.int32))
    assert out.tolist() == _bf16_bits(cu["out"]).tolist()
    cr = hand["combine_rounding"]
    Y = _bf16_bits(cr["Y"])
    # the inputs must be exact bf16 values for the example to mean anything
    assert [BF._bf16_value(int(b)) for b in Y[:, 0]] == [float(v[0]) for v in cr["Y"]]
    out = oracle_mod.combine(Y, None, np.array(cr["slot_row"], np.int32))
    assert out.tolist() == _bf16_bits(cr["out"]).tolist()


# -------------------------------------------------------------- brute force --

TINY = [(1, 1, 1, 1), (5, 4, 2, 2), (7, 8, 3, 4), (16, 8, 8, 2), (33, 6, 2, 3),
        (64, 8, 2, 4), (40, 8, 5, 8), (23, 12, 4, 1)]


def _tiny_logits(T, E, seed, tied):
    vals = [-1.0, -0.0, 0.0, 1.0] if tied else None
    return WL.make_custom_inputs(T, 4, E, seed=seed, logit_values=vals)


@pytest.mark.parametrize("T,E,k,R", TINY)
@pytest.mark.parametrize("tied", [True, False])
def test_bruteforce_route(oracle_mod, T, E, k, R, tied):
    inp = _tiny_logits(T, E, 100 + T + E + k, tied)
    idx, gate = oracle_mod.route_topk(inp["logits"], k)
    for t in range(T):
        assert idx[t].tolist() == BF.topk(inp["logits"][t].tolist(), k)
    # gates: positive, non-increasing along slots, sum to 1
    assert (gate > 0).all()
    assert (np.diff(gate, axis=1) <= 0).all()
    assert np.abs(gate.astype(np.float64).sum(1) - 1.0).max() <= k * 2.0 ** -24


@pytest.mark.parametrize("T,E,k,R", TINY)
@pytest.mark.parametrize("placement_kind", ["contiguous", "random"])
def test_bruteforce_layouts(oracle_mod, T, E, k, R, placement_kind):
    inp = _tiny_logits(T, E, 7 + T * E + k, tied=True)
    place = (WL.contiguous_placement(E, R) if placement_kind == "contiguous"
             else WL.random_placement(E, R, seed=T + E))
    idx, gate = oracle_mod.route_topk(inp["logits"], k)
    x = inp["x_bits"]
    # non-dedup: position = index in the sorted (rank, expert, token) key list
    d = oracle_mod.dispatch(x, idx, gate, E, R, place)
    keys, pos = BF.nondedup_layout(idx.tolist(), place.tolist())
    for (t, j), p in pos.items():
        assert d["slot_row"][t, j] == p
        assert d["row_token"][p] == t and d["row_expert"][p] == idx[t, j]
        assert d["row_weight"][p] == gate[t, j]
        assert (d["send"][p] == x[t]).all()
    cnt = np.bincount(idx.ravel(), minlength=E)
    assert d["expert_counts"].tolist() == cnt.tolist()
    # dedup: rows = sorted set of (rank, token)
    dd = oracle_mod.dispatch_dedup(x, idx, gate, E, R, place)
    pairs = BF.dedup_layout(idx.tolist(), place.tolist())
    assert dd["n_rows"] == len(pairs) == dd["rank_offsets"][-1]
    for p, (r, t) in enumerate(pairs):
        assert dd["row_token"][p] == t
        mine = sorted(int(e) for e in idx[t] if place[e] == r)
        assert dd["row_experts"][p].tolist() == mine + [-1] * (k - len(mine))
        g = [float(gate[t, list(idx[t]).index(e)]) for e in mine]
        assert dd["row_gates"][p].tolist() == [np.float32(v) for v in g] + [0.0] * (k - len(mine))
        assert dd["row_weight"][p] == np.float32(math.fsum(g))
        for j in range(k):
            if place[idx[t, j]] == r:
                assert dd["slot_row"][t, j] == p
        assert (dd["send"][p] == x[t]).all()
    assert dd["expert_counts"].tolist() == cnt.tolist()
    # co-selection by counting
    W = oracle_mod.coselect(idx, E)
    assert W.tolist() == BF.coselect(idx.tolist(), E, T)


def _within_chain_bound(out_bits, rows_bits, weights, slot_row, fp8=False):
    """The fp32 chain against the exact sum S: with n rows every fused
    multiply-add rounds once, so the chain's fp32 result lies within
    gamma_n * sum |w y| of S (gamma_n = n u / (1 - n u), u = 2^-24), and bf16
    rounding is monotone, so the output lies between the bf16 roundings of the
    two ends of that interval.  Returns the number of outputs checked."""
    u = Fraction(1, 2 ** 24)
    checked = 0
    for t, slots in enumerate(slot_row):
        rs = sorted({int(r) for r in slots if r >= 0})
        n = len(rs)
        gam = n * u / (1 - n * u)
        for h in range(len(rows_bits[0])):
            terms = []
            for r in rs:
                w = Fraction(1) if weights is None else Fraction(float(weights[r]))
                y = (BF.e4m3_to_fraction(rows_bits[r][h]) if fp8
                     else BF.bf16_to_fraction(rows_bits[r][h]))
                terms.append(w * y)
            S = sum(terms, Fraction(0))
            B = gam * sum((abs(v) for v in terms), Fraction(0))
            lo = BF._bf16_value(BF.nearest_bf16(S - B))
            hi = BF._bf16_value(BF.nearest_bf16(S + B))
            got = BF._bf16_value(int(out_bits[t][h]))
            assert lo <= got <= hi, (t, h, lo, got, hi)
            checked += 1
    return checked


@pytest.mark.parametrize("T,E,k,R", TINY)
def test_bruteforce_combine_random_rows(oracle_mod, T, E, k, R):
    """Random rows (signed, non-identity experts) and random weights: the
    oracle equals the fp32 chain emulated step by step with exact rationals,
    and lies within the chain's error bound of the exact rational sum."""
    rng = np.random.default_rng(T * 31 + k)
    H = 6
    inp = _tiny_logits(T, E, 3 + T, tied=False)
    idx, gate = oracle_mod.route_topk(inp["logits"], k)
    for dedup in (False, True):
        f = oracle_mod.dispatch_dedup if dedup else oracle_mod.dispatch
        d = f(inp["x_bits"][:, :1], idx, gate, E, R)
        n = d["n_rows"]
        Y = WL.bf16_bits_from_f32(rng.standard_normal((n, H)).astype(np.float32) * 4)
        Y[rng.random((n, H)) < 0.1] = 0x8000      # some -0.0
        slot = d["slot_row"].copy()
        slot[rng.random(slot.shape) < 0.1] = -1   # some skipped slots
        for w in (None, d["row_weight"], rng.standard_normal(n).astype(np.float32)):
            out = oracle_mod.combine(Y, w, slot)
            wl = None if w is None else w.tolist()
            assert out.tolist() == BF.combine_chain(Y.tolist(), wl, slot.tolist())
            assert _within_chain_bound(out.tolist(), Y.tolist(), wl, slot.tolist()) == T * H


def test_combine_order_matters_and_is_ascending(oracle_mod):
    """Rows whose fp32 sum depends on the order: the oracle takes the rows in
    ascending index whatever the slot order, so permuting a token's slots
    changes nothing, while renumbering the rows changes the result."""
    one, big, nbig = 0x3F80, 0x4E80, 0xCE80            # 1, 2^30, -2^30
    Y = np.array([[one], [big], [nbig]], np.uint16)
    for perm in ([0, 1, 2], [2, 1, 0], [1, 2, 0], [2, 0, 1]):
        out = oracle_mod.combine(Y, None, np.array([perm], np.int32))
        assert int(out[0, 0]) == 0x0000, perm          # (1 + 2^30) - 2^30 = 0 in fp32
    Y2 = np.array([[big], [nbig], [one]], np.uint16)    # same values, 1 added last
    out = oracle_mod.combine(Y2, None, np.array([[2, 0, 1]], np.int32))
    assert int(out[0, 0]) == 0x3F80


def _hex_bits(v):
    return int(v, 16)


@pytest.fixture(scope="module")
def chain_cases():
    with open(os.path.join(GOLDEN, "combine_fp32_chain.json")) as f:
        return json.load(f)["cases"]


def test_hand_combine_fp32_chain(oracle_mod, chain_cases):
    """Hand-worked cases of the combine reading (ascending rows, fp32 fused
    multiply-adds from -0.0, one bf16 rounding): order, accumulation
    precision, fusion, signed zeros, repeated and skipped slots, overflow,
    infinities, NaN and subnormals."""
    for c in chain_cases:
        Y = np.array([[_hex_bits(b)] for b in c["rows"]], np.uint16)
        w = None if c["weights"] is None else np.array(
            [float.fromhex(v) for v in c["weights"]], np.float32)
        if w is not None:   # the weights must be exact fp32 values
            assert [float(v) for v in w] == [float.fromhex(v) for v in c["weights"]], c["name"]
        out = int(oracle_mod.combine(Y, w, np.array([c["slot_row"]], np.int32))[0, 0])
        if c["out"] == "nan":
            assert (out & 0x7F80) == 0x7F80 and (out & 0x7F) != 0, c["name"]
        else:
            assert out == _hex_bits(c["out"]), (c["name"], hex(out))


def test_hand_combine_fp32_chain_matches_bruteforce(chain_cases):
    """The finite hand-worked cases, replayed through the step-by-step
    rational emulation of the chain (a second, independent check of the hand
    arithmetic)."""
    for c in chain_cases:
        if c["out"] == "nan" or c["out"] == "0x7F80":
            continue
        Y = [[_hex_bits(b)] for b in c["rows"]]
        w = None if c["weights"] is None else [float.fromhex(v) for v in c["weights"]]
        got = BF.combine_chain(Y, w, [c["slot_row"]])[0][0]
        assert got == _hex_bits(c["out"]), (c["name"], hex(got))


def test_bf16_from_float_nan_and_rounding(oracle_mod):
    """fp32 -> bf16 of the combine output: torch's cast for finite values and
    infinities; NaN stays NaN with its sign."""
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, size=5000, dtype=np.uint64).astype(np.uint32)
    bits[:1000] = (bits[:1000] & 0xFFFF0000) | 0x8000
    f = bits.view(np.float32)
    f = f[~np.isnan(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle_mod.bf16_from_float(v) for v in f], np.uint16)
    assert (got == ref).all()
    for v in (float("nan"), -float("nan")):
        b = oracle_mod.bf16_from_float(v)
        assert (b & 0x7F80) == 0x7F80 and (b & 0x7F) != 0
        assert bool(b & 0x8000) == bool(np.signbit(np.float32(v)))


# ------------------------------------------------------------ library pins --

def test_route_matches_lexsort_all_workloads(oracle_mod):
    for name in WL.ORDER:
        w = WL.get(name)
        inp = WL.make_inputs(w, with_x=False)
        lg = inp["logits"]
        idx, gate = oracle_mod.route_topk(lg, w.top_k)
        E = w.n_experts
        order = np.lexsort((np.broadcast_to(np.arange(E), lg.shape), -lg), axis=1)
        assert (idx == order[:, :w.top_k]).all(), name


def test_gates_k1_and_full_softmax(oracle_mod):
    inp = WL.make_custom_inputs(200, 4, 16, seed=5)
    idx, gate = oracle_mod.route_topk(inp["logits"], 1)
    assert (gate == 1.0).all()
    idx, gate = oracle_mod.route_topk(inp["logits"], 16)
    for t in range(200):
        ref = np.array(BF.softmax_desc([float(v) for v in inp["logits"][t]]), np.float32)
        assert f32_ulp_diff(gate[t], ref).max() <= 1


def test_bf16_rounding_matches_torch_cast(oracle_mod):
    """For inputs that are fp32 values, rounding the double to bf16 must equal
    torch's fp32->bf16 cast (round to nearest even)."""
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    # force many exact ties and near-ties in the dropped 16 bits
    bits[:5000] = (bits[:5000] & 0xFFFF0000) | 0x8000
    bits[5000:7000] = (bits[5000:7000] & 0xFFFF0000) | 0x7FFF
    bits[7000:9000] = (bits[7000:9000] & 0xFFFF0000) | 0x8001
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle_mod.bf16_from_double(float(v)) for v in f], np.uint16)
    assert (got == ref).all()
    for v, want in [(0.0, 0x0000), (-0.0, 0x8000), (1.0, 0x3F80), (-2.0, 0xC000),
                    (1.0 + 2 ** -8, 0x3F80), (1.0 + 3 * 2 ** -8, 0x3F82),
                    (float(np.finfo(np.float32).max), 0x7F80), (2.0 ** -140, 0x0000),
                    (-(2.0 ** -133), 0x8001)]:
        assert oracle_mod.bf16_from_double(v) == want, v


# ---------------------------------------------------------- page invariants --

@pytest.mark.parametrize("name", WL.ORDER)
def test_counts_invariants(oracle_mod, name):
    """DODOCO "Reading the counts": rows sum to tokens x top-k; each rank's expert
    block sums to its receive total; coarsening by summing contiguous rank blocks
    gives the traffic at half the ranks.  Dedup rows (Expert Coupling, Method 1)
    number the distinct (token, rank) pairs, between T and T*k."""
    w = WL.get(name)
    inp = WL.make_inputs(w, with_x=False)
    T, E, k, R = w.tokens, w.n_experts, w.top_k, w.n_ranks
    idx, gate = oracle_mod.route_topk(inp["logits"], k)
    place = inp["placement_array"]
    c = oracle_mod.send_counts(idx, E, R, inp["placement"], dedup=False)
    assert c["rank_counts"].sum() == T * k
    for r in range(R):
        assert c["rank_counts"][r] == c["expert_counts"][place == r].sum()
    assert (c["rank_offsets"] == np.concatenate([[0], np.cumsum(c["rank_counts"])])).all()
    if w.placement == "contiguous" and R % 2 == 0:
        c2 = oracle_mod.send_counts(idx, E, R // 2, None, dedup=False)
        assert (c2["rank_counts"] == c["rank_counts"].reshape(R // 2, 2).sum(1)).all()
    cd = oracle_mod.send_counts(idx, E, R, inp["placement"], dedup=True)
    D = cd["rank_counts"].sum()
    assert D == len({(int(place[e]), t) for t in range(T) for e in idx[t]})
    assert T <= D <= T * k
    assert (cd["expert_counts"] == c["expert_counts"]).all()
    if k == 2:
        same = int((place[idx[:, 0]] == place[idx[:, 1]]).sum())
        assert D == 2 * T - same     # Table I: Dedup = Same/2, GPUs = 2 - Same


def test_table1_identities_on_page():
    """Our reading of Table I: for top-2, dedup% = same%/2 and GPUs/token =
    2 - same%/100 on every printed row (within the table's rounding)."""
    rows = []
    with open(os.path.join(GOLDEN, "zyphra_table1.txt")) as f:
        for line in f:
            s = line.split()
            if not s or s[0].startswith("#") or s[0] == "top6":
                continue
            rows.append((int(s[0]), s[1], float(s[2]), float(s[3]), float(s[4])))
    assert len(rows) == 6
    # same% and dedup% are printed as integers (+-0.5), GPUs to 2 places (+-0.005)
    for ep, pl, same, gpus, dedup in rows:
        assert abs(dedup - same / 2) <= 0.5 + 0.25 + 1e-9, (ep, pl)
        assert abs(gpus - (2 - same / 100)) <= 0.005 + 0.005 + 1e-9, (ep, pl)


def _uniform_expect(E, k, R):
    m = E // R
    return R * (1.0 - math.comb(E - m, k) / math.comb(E, k))


@pytest.mark.parametrize("E,k,R", [(128, 2, 8), (128, 2, 32), (128, 6, 8), (128, 6, 32),
                                   (64, 6, 16)])
def test_dedup_rows_uniform_closed_form(oracle_mod, E, k, R):
    """Uniform routing, contiguous placement: E[D/T] = R(1 - C(E-m,k)/C(E,k)).
    Checked within 5 standard errors on 20000 uniform tokens."""
    T = 20000
    inp = WL.make_custom_inputs(T, 1, E, seed=E * k + R)
    idx, _ = oracle_mod.route_topk(inp["logits"], k)
    cd = oracle_mod.send_counts(idx, E, R, None, dedup=True)
    place = WL.contiguous_placement(E, R)
    per_tok = np.array([len(set(place[idx[t]].tolist())) for t in range(T)])
    assert per_tok.sum() == cd["rank_counts"].sum()
    mean = per_tok.mean()
    se = per_tok.std() / math.sqrt(T)
    assert abs(mean - _uniform_expect(E, k, R)) < 5 * se + 1e-9


def test_closed_form_against_table1_contiguous():
    """Context check of the reading: the uniform closed form lands within a point
    of Table I's contiguous rows (printed as rounded percentages)."""
    for ep, same_printed, dedup_printed in [(8, 12, 6), (16, 6, 3), (32, 2, 1)]:
        g = _uniform_expect(128, 2, ep)
        assert abs(100 * (2 - g) - same_printed) <= 1.0
        assert abs(100 * (1 - g / 2) - dedup_printed) <= 1.0
    assert abs(100 * (1 - _uniform_expect(128, 6, 8) / 6) - 25) <= 1.0
    assert abs(100 * (1 - _uniform_expect(128, 6, 32) / 6) - 5.5) <= 1.0


def test_dodoco_row_sums_and_payload(oracle_mod):
    """DODOCO: 4096 tokens per rank, rows sum to 4096 x top-k, payload bytes =
    count x hidden x 2 (bf16), for each model shape of the card."""
    with open(os.path.join(GOLDEN, "dodoco_models.txt")) as f:
        models = [l.split() for l in f if l.strip() and not l.startswith("#")]
    assert len(models) == 5
    for name, E, k, H in models:
        E, k, H = int(E), int(k), int(H)
        inp = WL.make_custom_inputs(4096, 1, E, seed=E + k)
        idx, gate = oracle_mod.route_topk(inp["logits"], k)
        c = oracle_mod.send_counts(idx, E, 16, None, dedup=False)
        assert c["rank_counts"].sum() == 4096 * k, name
        x = np.zeros((4096, 8), np.uint16)
        d = oracle_mod.dispatch(x, idx, gate, E, 16, with_rows=False)
        payload = d["rank_counts"].astype(np.int64) * H * 2
        assert payload.sum() == 4096 * k * H * 2


@pytest.mark.parametrize("name", WL.ORDER)
def test_identity_experts_return_input(oracle_mod, name):
    """Identity experts with gates summing to 1 give back x exactly, for the
    non-dedup rows (weight = gate) and the dedup rows (weight = gate sum)."""
    w = WL.get(name)
    if w.tokens * w.hidden_dim > 4096 * 2048:
        pytest.skip("full-size identity check runs in the GPU parity tests")
    inp = WL.make_inputs(w)
    idx, gate = oracle_mod.route_topk(inp["logits"], w.top_k)
    x = inp["x_bits"]
    for dedup in (False, True):
        f = oracle_mod.dispatch_dedup if dedup else oracle_mod.dispatch
        d = f(x, idx, gate, w.n_experts, w.n_ranks, inp["placement"])
        out = oracle_mod.combine(d["send"], d["row_weight"], d["slot_row"])
        assert (out == x).all(), (name, dedup)


def test_k1_combine_returns_input(oracle_mod):
    inp = WL.make_custom_inputs(300, 64, 8, seed=9)
    idx, gate = oracle_mod.route_topk(inp["logits"], 1)
    d = oracle_mod.dispatch(inp["x_bits"], idx, gate, 8, 4)
    assert (oracle_mod.combine(d["send"], d["row_weight"], d["slot_row"]) == inp["x_bits"]).all()
    assert (oracle_mod.combine(d["send"], None, d["slot_row"]) == inp["x_bits"]).all()


@pytest.mark.parametrize("name", ["deepseek_moe_16b", "zyphra_top6_ep32"])
def test_coselect_invariants(oracle_mod, name):
    w = WL.get(name)
    inp = WL.make_inputs(w, with_x=False)
    idx, _ = oracle_mod.route_topk(inp["logits"], w.top_k)
    n = w.coselect_tokens
    W = oracle_mod.coselect(idx, w.n_experts, tokens=n)
    assert (W == W.T).all()
    diag = np.diag(W)
    assert diag.sum() == n * w.top_k
    assert (diag == np.bincount(idx[:n].ravel(), minlength=w.n_experts)).all()
    assert ((W.sum(1) - diag) == (w.top_k - 1) * diag).all()
    # accumulation: a second call adds the same counts again
    W2 = oracle_mod.coselect(idx, w.n_experts, tokens=n, W=W.copy())
    assert (W2 == 2 * W).all()


# ------------------------------------------------ receive-side expansion --

@pytest.mark.parametrize("T,E,k,R", TINY)
@pytest.mark.parametrize("placement_kind", ["contiguous", "random"])
def test_bruteforce_expand(oracle_mod, T, E, k, R, placement_kind):
    """Expanded positions = index in the sorted (rank, expert, row) key list of
    the listed entries; padding and rows past n_rows map to -1."""
    inp = _tiny_logits(T, E, 11 + T * E + k, tied=True)
    place = (WL.contiguous_placement(E, R) if placement_kind == "contiguous"
             else WL.random_placement(E, R, seed=T + 2 * E))
    idx, gate = oracle_mod.route_topk(inp["logits"], k)
    dd = oracle_mod.dispatch_dedup(inp["x_bits"], idx, gate, E, R, place)
    D = dd["n_rows"]
    cap = D + 5   # rows past n_rows hold garbage ids that must be ignored
    rx = np.concatenate([dd["row_experts"], np.full((5, k), 3 % E, np.int32)])
    rg = np.concatenate([dd["row_gates"], np.ones((5, k), np.float32)])
    rows = np.concatenate([dd["send"], np.zeros((5, 4), np.uint16)])
    ex = oracle_mod.expand_dedup(rows, rx, rg, D, E, R, place, capacity=cap)
    pos = BF.expand_layout(rx.tolist(), D, place.tolist())
    assert ex["n_expanded"] == len(pos) == T * k
    for (p, c), q in pos.items():
        assert ex["row_slot"][p, c] == q
        assert ex["exp_row"][q] == p and ex["exp_expert"][q] == rx[p, c]
        assert ex["exp_gate"][q] == rg[p, c]
        assert (ex["expanded"][q] == rows[p]).all()
    listed = {pc for pc in pos}
    for p in range(cap):
        for c in range(k):
            if (p, c) not in listed:
                assert ex["row_slot"][p, c] == -1
    assert ex["expert_counts"].tolist() == np.bincount(idx.ravel(), minlength=E).tolist()


@pytest.mark.parametrize("name", [n for n in WL.ORDER if "dedup" in WL.get(n).dispatch])
def test_expand_of_dedup_rows_is_the_plain_dispatch(oracle_mod, name):
    """Expert Coupling, Method 1: the deduplicating dispatcher delivers the same
    (token, expert) work as the conventional one.  Expanding the dedup rows per
    expert must give back the conventional dispatcher's buffer exactly: same
    rows, same segment offsets, same experts and gates per row."""
    w = WL.get(name)
    inp = WL.make_inputs(w, with_x=False)
    T = min(w.tokens, 2048)
    logits = inp["logits"][:T]
    x = WL.make_custom_inputs(T, 16, 1, seed=5)["x_bits"]
    idx, gate = oracle_mod.route_topk(logits, w.top_k)
    place = inp["placement"]
    E, R = w.n_experts, w.n_ranks
    dd = oracle_mod.dispatch_dedup(x, idx, gate, E, R, place)
    pl = oracle_mod.dispatch(x, idx, gate, E, R, place)
    ex = oracle_mod.expand_dedup(dd["send"], dd["row_experts"], dd["row_gates"], dd["n_rows"],
                                 E, R, place)
    assert ex["n_expanded"] == pl["n_rows"] == T * w.top_k
    assert (ex["expanded"] == pl["send"]).all()
    assert (ex["expert_offsets"] == pl["expert_offsets"]).all()
    assert (ex["rank_offsets"] == pl["rank_offsets"]).all()
    assert (ex["exp_expert"] == pl["row_expert"]).all()
    assert (ex["exp_gate"].view(np.uint32) == pl["row_weight"].view(np.uint32)).all()
    assert (dd["row_token"][ex["exp_row"]] == pl["row_token"]).all()
    # every expanded row is reached from exactly one (row, column)
    rs = ex["row_slot"][: dd["n_rows"]]
    got = np.sort(rs[rs >= 0])
    assert (got == np.arange(T * w.top_k)).all()


@pytest.mark.parametrize("name", ["deepseek_moe_16b", "zyphra_top2_ep8", "zyphra_top6_ep32"])
def test_receive_round_trip_with_identity_experts(oracle_mod, name):
    """Identity experts: each received row reduces to (sum of its gates) * x,
    and combining those rows with weight 1 returns x (gates sum to 1), up to
    the two bf16 roundings: within 2 bf16 ulps of x, and exactly x where the
    token's experts all live on one rank (half the tokens of the top-2 EP8
    workload)."""
    w = WL.get(name)
    inp = WL.make_inputs(w, with_x=False)
    T = 1024
    x = WL.make_custom_inputs(T, 64, 1, seed=9)["x_bits"]
    idx, gate = oracle_mod.route_topk(inp["logits"][:T], w.top_k)
    E, R, place = w.n_experts, w.n_ranks, inp["placement"]
    dd = oracle_mod.dispatch_dedup(x, idx, gate, E, R, place)
    ex = oracle_mod.expand_dedup(dd["send"], dd["row_experts"], dd["row_gates"], dd["n_rows"],
                                 E, R, place)
    red = oracle_mod.reduce_rows(ex["expanded"], ex["exp_gate"], ex["row_slot"], dd["n_rows"])
    out = oracle_mod.combine(red, None, dd["slot_row"])
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    of = (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ulp = np.maximum(np.abs(xf), 2.0 ** -126) * 2.0 ** -7
    assert (np.abs(of - xf) <= 2 * ulp).all()
    pl = inp["placement_array"]
    one_rank = np.array([len({int(pl[e]) for e in row}) == 1 for row in idx])
    # one rank: x * sum(g) with |sum(g) - 1| <= k 2^-24 rounds back to x, and a
    # weight-1 combine of one row is exact
    if one_rank.any():
        g1 = gate[one_rank].astype(np.float64).sum(1)
        assert np.abs(g1 - 1).max() <= w.top_k * 2.0 ** -24
        assert (out[one_rank] == x[one_rank]).all()


# -------------------------------------------------------- placement search --

def _objective(W, place):
    """Co-location objective by brute force: sum of W[x][y] over ordered pairs
    x != y on one rank (Expert Coupling, Method 1)."""
    same = place[:, None] == place[None, :]
    np.fill_diagonal(same, False)
    return int((W.astype(np.int64) * same).sum())


def _swapped(place, e, f):
    p = place.copy()
    p[e], p[f] = place[f], place[e]
    return p


@pytest.mark.parametrize("E,R,sym", [(8, 2, True), (8, 4, False), (12, 3, True), (16, 8, True),
                                     (16, 4, False)])
def test_placement_search_bruteforce(oracle_mod, E, R, sym):
    """Every step takes the best swap (ties to the lowest pair) found by
    recomputing the objective for every swap; the end is a local optimum; the
    objective never decreases; every rank keeps E/R experts."""
    rng = np.random.default_rng(E * 7 + R)
    W = rng.integers(0, 9, (E, E)).astype(np.int32)
    if sym:
        W = (W + W.T).astype(np.int32)
    place = WL.contiguous_placement(E, R)
    prev = _objective(W, place)
    for step in range(1, 40):
        got, obj, sw = oracle_mod.placement_search(W, R, max_swaps=step)
        assert obj == _objective(W, got)
        assert (np.bincount(got, minlength=R) == E // R).all()
        # the expected next swap from the previous placement, by brute force
        best, pair = 0, None
        for e in range(E):
            for f in range(e + 1, E):
                if place[e] != place[f]:
                    d = _objective(W, _swapped(place, e, f)) - prev
                    if d > best:
                        best, pair = d, (e, f)
        if pair is None:
            assert sw == step - 1 and (got == place).all()
            break
        assert sw == step and (got == _swapped(place, *pair)).all()
        assert obj == prev + best
        place, prev = got, obj
    else:
        pytest.fail("no local optimum within 40 swaps")
    # local optimum: no single swap improves
    for e in range(E):
        for f in range(e + 1, E):
            if place[e] != place[f]:
                assert _objective(W, _swapped(place, e, f)) <= prev


def test_placement_search_recovers_planted_pairs(oracle_mod):
    """A co-selection matrix made of strongly coupled expert pairs (plus weak
    noise): the search puts every pair on one rank."""
    E, R = 64, 16
    rng = np.random.default_rng(3)
    perm = rng.permutation(E)
    W = rng.integers(0, 3, (E, E)).astype(np.int32)
    W = W + W.T
    for i in range(0, E, 2):
        a, b = perm[i], perm[i + 1]
        W[a, b] += 100
        W[b, a] += 100
    np.fill_diagonal(W, 0)
    place, obj, _ = oracle_mod.placement_search(W, R)
    for i in range(0, E, 2):
        assert place[perm[i]] == place[perm[i + 1]]
    assert obj >= _objective(W, WL.contiguous_placement(E, R))


# ------------------------------------------------------------ fp8 rows --

def test_e4m3_decode_matches_torch(oracle_mod):
    """The oracle's E4M3 decode equals torch's float8_e4m3fn -> float32 cast for
    all 256 byte values (NaN for S.1111.111), and the brute-force decode."""
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = np.array([oracle_mod.e4m3_to_double(int(v)) for v in b])
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all() and nan.sum() == 2
    assert (got[~nan] == ref[~nan].astype(np.float64)).all()
    assert (np.signbit(got[~nan]) == np.signbit(ref[~nan])).all()
    for v in b[~nan]:
        assert float(BF.e4m3_to_fraction(v)) == got[v]


@pytest.mark.parametrize("T,E,k,R", TINY[:5])
def test_bruteforce_combine_fp8_rows(oracle_mod, T, E, k, R):
    """fp8 rows (random bytes, NaN excluded, some -0): the oracle equals the
    fp32 chain emulated with exact rationals over the exactly decoded bytes,
    within the chain's bound of the exact sum, for NULL, gate and signed
    weights."""
    rng = np.random.default_rng(T * 13 + k)
    H = 5
    inp = _tiny_logits(T, E, 5 + T, tied=False)
    idx, gate = oracle_mod.route_topk(inp["logits"], k)
    d = oracle_mod.dispatch(inp["x_bits"][:, :1], idx, gate, E, R)
    n = d["n_rows"]
    Y = rng.integers(0, 256, (n, H)).astype(np.uint8)
    Y[(Y & 0x7F) == 0x7F] = 0x80                  # no NaN; those become -0
    for w in (None, d["row_weight"], rng.standard_normal(n).astype(np.float32)):
        out = oracle_mod.combine_fp8(Y, w, d["slot_row"])
        wl = None if w is None else w.tolist()
        assert out.tolist() == BF.combine_chain(Y.tolist(), wl, d["slot_row"].tolist(), fp8=True)
        _within_chain_bound(out.tolist(), Y.tolist(), wl, d["slot_row"].tolist(), fp8=True)


def test_fp8_single_row_is_exact(oracle_mod):
    """k = 1, weight 1: every E4M3 value is a bf16 value, so the output is the
    row itself converted exactly (torch's cast as the reference)."""
    b = np.arange(256, dtype=np.uint8)
    b = b[(b & 0x7F) != 0x7F].reshape(1, -1)
    out = oracle_mod.combine_fp8(b, None, np.zeros((1, 1), np.int32))
    ref = (torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float32)
           .to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    assert (out == ref).all()


# ------------------------------------------------- softmax over all experts --

def test_softmax_all_gates(oracle_mod):
    """Same selection as the k-softmax; gates equal torch's float64 softmax over
    all logits at the selected experts (within 1 fp32 ulp: summation order);
    at k = E they are the k-softmax gates."""
    for T, E, k in ((300, 64, 6), (200, 128, 8), (50, 8, 8), (40, 3, 1)):
        inp = WL.make_custom_inputs(T, 1, E, seed=T + E)
        idx, gate = oracle_mod.route_topk_softmax_all(inp["logits"], k)
        idx_k, gate_k = oracle_mod.route_topk(inp["logits"], k)
        assert (idx == idx_k).all()
        p = torch.softmax(torch.from_numpy(inp["logits"]).double(), dim=1).numpy()
        ref = np.take_along_axis(p, idx.astype(np.int64), axis=1).astype(np.float32)
        assert f32_ulp_diff(gate, ref).max() <= 1
        assert (gate.astype(np.float64).sum(1) <= 1 + k * 2.0 ** -24).all()
        if k == E:
            assert f32_ulp_diff(gate, gate_k).max() <= 1


# ---------------------------------------------------- token shuffle planner --

def _routes(rng, T, E, k, n=3):
    return [np.array([rng.choice(E, k, replace=False) for _ in range(T)], np.int32)
            for _ in range(n)]


@pytest.mark.parametrize("T,E,k,R", [(40, 8, 2, 4), (33, 6, 3, 3), (64, 16, 1, 8), (20, 4, 4, 2)])
def test_shuffle_fit_counts(oracle_mod, T, E, k, R):
    """Fit tables by enumeration: every (a at l-1, b at l, rank of c at l+1)
    triple counted once per token; single[b][r] = sum over a of pair / k."""
    from collections import Counter
    rng = np.random.default_rng(T + E)
    prev, cur, nxt = _routes(rng, T, E, k)
    place = WL.random_placement(E, R, seed=T)
    pair, single = oracle_mod.shuffle_fit(prev, cur, nxt, E, R, place)
    cnt = Counter((a, b, int(place[c])) for t in range(T) for a in prev[t] for b in cur[t]
                  for c in nxt[t])
    ref = np.zeros((E, E, R), np.int64)
    for (a, b, r), v in cnt.items():
        ref[a, b, r] = v
    assert (pair == ref).all()
    assert (pair.sum(axis=0) == k * single).all()
    assert pair.sum() == T * k ** 3 and single.sum() == T * k ** 2


def test_shuffle_predict_properties(oracle_mod):
    """Each (a, b) pair adds one probability distribution: scores sum to k^2
    when every pair or its fallback was seen; with min_obs above every count
    the scores are the single-expert fallback alone; a rank that took every
    calibration token of a pair is that pair's only rank."""
    T, E, k, R = 200, 8, 2, 4
    rng = np.random.default_rng(1)
    prev, cur, nxt = _routes(rng, T, E, k)
    pair, single = oracle_mod.shuffle_fit(prev, cur, nxt, E, R)
    s = oracle_mod.shuffle_predict(prev, cur, pair, single, 1)
    assert np.abs(s.astype(np.float64).sum(1) - k * k).max() < 1e-5
    fb = oracle_mod.shuffle_predict(prev, cur, pair, single, 10 ** 9)
    sd = single / single.sum(1, keepdims=True)
    ref = np.stack([k * sd[cur[t]].sum(0) for t in range(T)])
    assert np.abs(fb - ref).max() < 1e-5
    # a planted route: every calibration token goes to rank 3 at l+1
    place = np.full(E, 3, np.int32)
    place[:6] = [0, 0, 1, 1, 2, 2]
    nxt3 = np.tile(np.array([6, 7], np.int32), (T, 1))
    pair3, single3 = oracle_mod.shuffle_fit(prev, cur, nxt3, E, R, np.array(place))
    s3 = oracle_mod.shuffle_predict(prev, cur, pair3, single3, 1)
    assert (s3.argmax(1) == 3).all() and (s3[:, :3] == 0).all()


def load_shuffle_hand():
    """The hand-worked prediction fixture as numpy tables and token groups."""
    with open(os.path.join(GOLDEN, "shuffle_predict_hand.json")) as f:
        h = json.load(f)
    E, R = h["E"], h["R"]
    pair = np.zeros((E, E, R), np.int32)
    for p in h["pair"]:
        pair[p["a"], p["b"]] = p["counts"]
    single = np.array(h["single"], np.int32)
    groups = []
    for g in h["groups"]:
        prev = np.array([t["prev"] for t in g["tokens"]], np.int32)
        cur = np.array([t["cur"] for t in g["tokens"]], np.int32)
        want = np.array([[float(Fraction(v)) for v in t["scores"]] for t in g["tokens"]],
                        np.float32)
        groups.append((prev, cur, want))
    return h, pair, single, groups


def test_shuffle_predict_hand(oracle_mod):
    """Hand-worked scores: an asymmetric pair table (pair[a][b] != pair[b][a]),
    a pair seen exactly min_obs times (used) and one seen min_obs - 1 times
    (single-expert fallback), an expert never seen at layer l (no
    contribution), and the sum over a token's k*k pairs at k = 2.  Reading
    pair[b][a], or comparing with > instead of >=, changes these scores."""
    h, pair, single, groups = load_shuffle_hand()
    for prev, cur, want in groups:
        got = oracle_mod.shuffle_predict(prev, cur, pair, single, h["min_obs"])
        assert (got == want).all(), (prev.tolist(), cur.tolist(), got.tolist())


def test_shuffle_assign_properties(oracle_mod):
    """Every rank owns exactly T/R tokens; when each rank is the top choice of
    exactly T/R tokens every token gets its top choice; a token never gets a
    lower-scoring rank while a higher-scoring one of its ranks had room when
    it was placed (checked by replaying the confidence order)."""
    rng = np.random.default_rng(2)
    T, R = 96, 4
    s = rng.random((T, R)).astype(np.float32)
    own = oracle_mod.shuffle_assign(s)
    assert (np.bincount(own, minlength=R) == T // R).all()
    top = np.repeat(np.arange(R), T // R)
    rng.shuffle(top)
    s2 = rng.random((T, R)).astype(np.float32) * 0.5
    s2[np.arange(T), top] = 1.0
    assert (oracle_mod.shuffle_assign(s2) == top).all()
    conf = s.astype(np.float64).max(1) / s.astype(np.float64).sum(1)
    order = sorted(range(T), key=lambda t: (-conf[t], t))
    room = [T // R] * R
    for t in order:
        better = [r for r in range(R) if s[t, r] > s[t, own[t]]]
        assert all(room[r] == 0 for r in better)
        room[own[t]] -= 1
