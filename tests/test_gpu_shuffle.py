"""GPU parity of the token-shuffle planner: fit tables bit for bit, prediction
scores bit for bit (fp64 in the oracle's order, one rounding), and the
assignment from those scores identical to the oracle's."""
import numpy as np
import pytest
import torch

from combine_top_router_select_amd import ops
from combine_top_router_select_amd import workloads as WL
from gpu_util import host, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.lib()
    yield
    torch.cuda.synchronize()


def _check(oracle_mod, prev, cur, nxt, E, R, place, min_obs):
    pair_o, single_o = oracle_mod.shuffle_fit(prev, cur, nxt, E, R, place)
    pair, single = ops.moe_shuffle_fit(to_dev(prev), to_dev(cur), to_dev(nxt), E, R,
                                       to_dev(place) if place is not None else None)
    torch.cuda.synchronize()
    assert (host(pair) == pair_o).all() and (host(single) == single_o).all()
    s_o = oracle_mod.shuffle_predict(prev, cur, pair_o, single_o, min_obs)
    s = host(ops.moe_shuffle_predict(to_dev(prev), to_dev(cur), pair, single, min_obs))
    assert (s.view(np.uint32) == s_o.view(np.uint32)).all()
    return s_o


@pytest.mark.parametrize("T,E,k,R,min_obs", [(200, 8, 2, 4, 1), (333, 16, 3, 8, 4),
                                             (1000, 64, 6, 16, 8), (64, 128, 16, 64, 2),
                                             (100, 4, 1, 2, 0), (257, 32, 4, 32, 1000),
                                             (50, 6, 2, 1, 1), (70, 12, 3, 3, 1)])
def test_shuffle_fit_predict_parity(oracle_mod, T, E, k, R, min_obs):
    say(f"[shuffle] T={T} E={E} k={k} R={R} min_obs={min_obs}")
    rng = np.random.default_rng(T * 3 + k)
    prev, cur, nxt = (np.array([rng.choice(E, k, replace=False) for _ in range(T)], np.int32)
                      for _ in range(3))
    place = WL.random_placement(E, R, seed=T) if R < E else None
    _check(oracle_mod, prev, cur, nxt, E, R, place, min_obs)


@pytest.mark.parametrize("name", ["zyphra_top2_ep8", "zyphra_top6_ep32"])
def test_shuffle_plan_workload(oracle_mod, name):
    """Fit on one batch of correlated three-layer routing, plan another batch:
    scores and owners equal the oracle's; locality beats the contiguous token
    ownership by a wide margin."""
    w = WL.get(name)
    E, k, R, T = w.n_experts, w.top_k, w.n_ranks, w.tokens
    cal = [oracle_mod.route_topk(l, k)[0] for l in WL.make_layer_logits(w, seed=1)]
    ev = [oracle_mod.route_topk(l, k)[0] for l in WL.make_layer_logits(w, seed=2)]
    pair, single = ops.moe_shuffle_fit(*(to_dev(x) for x in cal), E, R)
    s = ops.moe_shuffle_predict(to_dev(ev[0]), to_dev(ev[1]), pair, single, 8)
    owner = ops.moe_shuffle_assign(s).numpy()
    pair_o, single_o = oracle_mod.shuffle_fit(*cal, E, R)
    s_o = oracle_mod.shuffle_predict(ev[0], ev[1], pair_o, single_o, 8)
    assert (host(s).view(np.uint32) == s_o.view(np.uint32)).all()
    assert (owner == oracle_mod.shuffle_assign(s_o)).all()
    place = WL.contiguous_placement(E, R)
    served = place[ev[2]]                       # rank of each layer l+1 assignment
    base = (np.arange(T) * R // T)[:, None]     # contiguous sequence ownership
    loc_base = (served == base).mean()
    loc = (served == owner[:, None]).mean()
    say(f"  locality {loc_base:.3f} -> {loc:.3f}")
    assert loc > 2 * loc_base


def test_shuffle_predict_hand_cases(oracle_mod):
    """The hand-worked prediction fixture through the GPU: every score equals
    the worked value exactly."""
    from test_oracle_pins import load_shuffle_hand
    h, pair, single, groups = load_shuffle_hand()
    for prev, cur, want in groups:
        s = host(ops.moe_shuffle_predict(to_dev(prev), to_dev(cur), to_dev(pair),
                                         to_dev(single), h["min_obs"]))
        torch.cuda.synchronize()
        assert (s == want).all(), (prev.tolist(), cur.tolist(), s.tolist())
