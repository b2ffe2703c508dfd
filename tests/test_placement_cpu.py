"""The library's correlated-placement search (host code, no GPU) against the
oracle: identical placements, objectives and swap counts, bit for bit."""
import numpy as np
import pytest
import torch

from combine_top_router_select_amd import ops
from combine_top_router_select_amd import workloads as WL


@pytest.mark.parametrize("E,R,sym,init,max_swaps", [
    (8, 2, True, None, None), (16, 4, False, None, None), (64, 16, True, None, None),
    (64, 16, True, "random", None), (128, 32, True, None, None), (128, 8, False, "random", 7),
    (12, 3, True, None, 0), (512, 64, True, None, 3), (5, 1, True, None, None),
    (6, 6, True, None, None)])
def test_search_matches_oracle(oracle_mod, E, R, sym, init, max_swaps):
    rng = np.random.default_rng(E + R)
    W = rng.integers(0, 40, (E, E)).astype(np.int32)
    if sym:
        W = (W + W.T).astype(np.int32)
    initial = WL.random_placement(E, R, seed=E) if init == "random" else None
    p_o, obj_o, sw_o = oracle_mod.placement_search(W, R, initial=initial, max_swaps=max_swaps)
    p, obj, sw = ops.moe_placement_search(
        torch.from_numpy(W), R, None if initial is None else torch.from_numpy(initial),
        max_swaps=max_swaps)
    assert (p.numpy() == p_o).all()
    assert obj == obj_o and sw == sw_o


def test_search_on_workload_coselection(oracle_mod):
    """On the co-selection counts of the top-6 EP32 workload's first 4096
    tokens: same result as the oracle, and a higher objective than contiguous."""
    w = WL.get("zyphra_top6_ep32")
    inp = WL.make_inputs(w, with_x=False)
    idx, _ = oracle_mod.route_topk(inp["logits"][:w.coselect_tokens], w.top_k)
    W = oracle_mod.coselect(idx, w.n_experts)
    p_o, obj_o, sw_o = oracle_mod.placement_search(W, w.n_ranks)
    p, obj, sw = ops.moe_placement_search(torch.from_numpy(W), w.n_ranks)
    assert (p.numpy() == p_o).all() and obj == obj_o and sw == sw_o
    assert obj > oracle_mod.placement_objective(W, WL.contiguous_placement(w.n_experts,
                                                                           w.n_ranks))


def test_search_errors():
    from combine_top_router_select_amd._lib import MoeError
    W = torch.zeros((8, 8), dtype=torch.int32)
    with pytest.raises(MoeError):
        ops.moe_placement_search(W, 3)                       # 8 % 3 != 0
    with pytest.raises(MoeError):
        ops.moe_placement_search(W, 2, initial=torch.zeros(8, dtype=torch.int32))  # 8 on rank 0
    with pytest.raises(MoeError):
        ops.moe_placement_search(W, 2, initial=torch.full((8,), 5, dtype=torch.int32))
    with pytest.raises(MoeError):
        ops.moe_placement_search(W, 2, max_swaps=-1)
    with pytest.raises(MoeError):
        ops.moe_placement_search(torch.zeros((2048, 2048), dtype=torch.int32), 2)


# ------------------------------------------------------ shuffle assignment --

@pytest.mark.parametrize("T,R,ties", [(96, 4, False), (96, 4, True), (16384, 8, False),
                                      (4096, 32, True), (64, 64, False), (10, 1, False)])
def test_shuffle_assign_matches_oracle(oracle_mod, T, R, ties):
    rng = np.random.default_rng(T + R)
    s = rng.random((T, R)).astype(np.float32)
    if ties:   # many equal scores and equal confidences
        s = (rng.integers(0, 3, (T, R)) / 2).astype(np.float32)
        s[rng.random(T) < 0.1] = 0.0
    own_o = oracle_mod.shuffle_assign(s)
    own = ops.moe_shuffle_assign(torch.from_numpy(s))
    assert (own.numpy() == own_o).all()
    assert (np.bincount(own_o, minlength=R) == T // R).all()


def test_shuffle_assign_errors():
    from combine_top_router_select_amd._lib import MoeError
    with pytest.raises(MoeError):
        ops.moe_shuffle_assign(torch.zeros((10, 3)))          # 10 % 3 != 0
    with pytest.raises(MoeError):
        ops.moe_shuffle_assign(torch.zeros((130, 65)))        # R > 64
    assert ops.moe_shuffle_assign(torch.zeros((0, 4))).numel() == 0


def test_shuffle_assign_table_allocation_failure_is_an_error_code():
    """A token count whose host tables cannot be allocated returns
    MOE_EUNSUPPORTED instead of letting a C++ exception cross the C ABI (the
    tables are allocated before the scores are read, so a placeholder scores
    address is never dereferenced)."""
    import ctypes
    from combine_top_router_select_amd import _lib
    L = _lib.lib()
    owner = np.zeros(4, dtype=np.int32)
    scores = np.zeros(4, dtype=np.float32)
    rc = L.moe_shuffle_assign(scores.ctypes.data_as(ctypes.c_void_p), 1 << 62, 1,
                              owner.ctypes.data_as(ctypes.c_void_p))
    assert rc == 2   # MOE_EUNSUPPORTED
    assert (owner == 0).all()
