"""The seeded generators produce the statistics the pages describe (no GPU).

Routing is computed with the oracle; these tests check the generators, not the
oracle.
"""
import numpy as np
import pytest

from combine_top_router_select_amd import workloads as WL


def test_shapes_and_determinism():
    for name in WL.ORDER:
        w = WL.get(name)
        a = WL.make_inputs(w, with_x=False)
        b = WL.make_inputs(w, with_x=False)
        assert a["logits"].shape == (w.tokens, w.n_experts)
        assert a["logits"].dtype == np.float32
        assert (a["logits"] == b["logits"]).all()
        pl = a["placement_array"]
        assert pl.shape == (w.n_experts,)
        # each rank holds exactly E/R experts (Expert Coupling, Method 1)
        assert (np.bincount(pl, minlength=w.n_ranks) == w.n_experts // w.n_ranks).all()
        if w.placement == "contiguous":
            assert a["placement"] is None
            assert (pl == np.arange(w.n_experts) // (w.n_experts // w.n_ranks)).all()


def test_tiny_x_is_bf16_normal():
    w = WL.get("tiny")
    x = WL.make_inputs(w)["x_bits"]
    assert x.shape == (256, 128) and x.dtype == np.uint16
    f = (x.astype(np.uint32) << 16).view(np.float32)
    assert abs(f.mean()) < 0.05 and abs(f.std() - 1) < 0.05


def test_pair_bias_workload(oracle_mod):
    """+3.0 on one of 64 seeded pairs for 40% of tokens (1638 of 4096)."""
    w = WL.get("deepseek_moe_16b")
    inp = WL.make_inputs(w, with_x=False)
    pl = inp["planted"]
    assert len(pl["tokens"]) == round(0.4 * 4096) == 1638
    assert len({tuple(p) for p in pl["pairs"].tolist()}) == 64
    idx, _ = oracle_mod.route_topk(inp["logits"], w.top_k)
    hit = 0
    for t, q in zip(pl["tokens"], pl["which"]):
        a, b = pl["pairs"][q]
        hit += (a in idx[t]) and (b in idx[t])
    # a +3.0 expert still falls below the 6th-largest of 62 N(0,1) logits ~7% of the time
    assert 0.8 < hit / len(pl["tokens"]) < 0.95


def test_zipf_workload_skews_load(oracle_mod):
    w = WL.get("qwen3_30b_a3b")
    inp = WL.make_inputs(w, with_x=False)
    idx, _ = oracle_mod.route_topk(inp["logits"], w.top_k)
    load = np.bincount(idx.ravel(), minlength=w.n_experts)
    rank = inp["planted"]["zipf_rank"]
    # the most popular ranks get many times the load of the least popular ones
    assert load[rank < 8].mean() > 4 * load[rank >= 120].mean()
    # monotone trend: Spearman correlation of load against Zipf rank is strongly negative
    r1 = np.argsort(np.argsort(load))
    r2 = np.argsort(np.argsort(rank))
    assert np.corrcoef(r1, r2)[0, 1] < -0.9


@pytest.mark.parametrize("name", ["zyphra_top2_ep8", "zyphra_top6_ep32"])
def test_zyphra_planted_pairs(oracle_mod, name):
    """Expert Coupling, within-layer correlation: 42% of tokens on 64 pairs; at
    top-2, 14 pairs at >= 50% confidence carrying 16% of tokens.  Correlated
    placement co-locates every planted pair."""
    w = WL.get(name)
    inp = WL.make_inputs(w, with_x=False)
    pl = inp["planted"]
    T = w.tokens
    assert len(pl["tokens"]) == round(0.16 * T) + round(0.26 * T)
    pairs = pl["pairs"]
    assert sorted(pairs.ravel().tolist()) == list(range(128))
    place = inp["placement_array"]
    assert (place[pairs[:, 0]] == place[pairs[:, 1]]).all()
    idx, _ = oracle_mod.route_topk(inp["logits"], w.top_k)
    W = oracle_mod.coselect(idx, w.n_experts)
    load = np.diag(W)
    conf = np.array([W[a, b] / min(load[a], load[b]) for a, b in pairs])
    on_pairs = sum(int(W[a, b]) for a, b in pairs)
    if w.top_k == 2:
        share = on_pairs / T
        assert 0.42 <= share <= 0.45        # planted 42% plus chance co-selections
        assert (conf[:14] >= 0.5).all() and (conf[14:] < 0.5).all()
        strong = sum(int(W[a, b]) for a, b in pairs[:14]) / T
        assert 0.155 <= strong <= 0.17
        # same-rank share and dedup share under correlated placement
        same = (place[idx[:, 0]] == place[idx[:, 1]]).mean()
        assert 0.45 <= same <= 0.53
    else:
        # at top-6 every planted token still selects its pair
        assert on_pairs / T >= 0.42


def test_dodoco_shaped_workloads_match_the_model_table():
    """Every 4096-token, EP16, contiguous workload takes (experts, top-k, hidden)
    from a row of the DODOCO "Models" table (fixture with its citation)."""
    import os
    golden = os.path.join(os.path.dirname(__file__), "golden", "dodoco_models.txt")
    with open(golden) as f:
        rows = {tuple(int(v) for v in l.split()[1:]) for l in f
                if l.strip() and not l.startswith("#")}
    shaped = [w for w in (WL.get(n) for n in WL.ORDER)
              if w.tokens == 4096 and w.n_ranks == 16]
    assert len(shaped) == 4
    for w in shaped:
        assert (w.n_experts, w.top_k, w.hidden_dim) in rows, w.name
        assert w.placement == "contiguous"


def test_layer_logits_cross_layer_correlation(oracle_mod):
    """The multi-layer generator gives the cross-layer statistic the Expert
    Coupling summary reports ("Key Theoretical Insight": most layer-l experts
    send >= 30% of their tokens to one layer-(l+1) expert, median share 48%),
    measured on the top-1 choices; reported, asserted only loosely."""
    w = WL.get("zyphra_top2_ep8")
    L = WL.make_layer_logits(w)
    assert len(L) == 3 and all(l.shape == (w.tokens, w.n_experts) for l in L)
    a = oracle_mod.route_topk(L[1][:8192], w.top_k)[0][:, 0]
    b = oracle_mod.route_topk(L[2][:8192], w.top_k)[0][:, 0]
    share = []
    for e in range(w.n_experts):
        m = a == e
        if m.any():
            share.append(np.bincount(b[m], minlength=w.n_experts).max() / m.sum())
    share = np.array(share)
    assert 0.35 <= np.median(share) <= 0.65
    assert (share >= 0.3).sum() >= 100
    again = WL.make_layer_logits(w)
    assert all((x == y).all() for x, y in zip(L, again))
