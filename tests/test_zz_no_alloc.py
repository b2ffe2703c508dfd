"""The dispatch entry point that allocates nothing (moe_dispatch_permute_noalloc)
against the workspace path it stands for: moe_send_counts (plain) followed by
moe_dispatch_permute.  Every output must be identical, bit for bit, on two
calls in a row (the second with a smaller input, so a stale plan left in the
shared scratch would show), with contiguous and explicit placements."""
import ctypes

import numpy as np
import pytest
import torch

from combine_top_router_select_amd import ops
from combine_top_router_select_amd import workloads as WL
from gpu_util import bf16_dev, bf16_host, host, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.lib()
    yield
    torch.cuda.synchronize()


KEYS = ("expert_counts", "rank_counts", "rank_offsets", "expert_offsets", "row_token",
        "row_expert", "slot_row")


def _case(T, H, E, k, R, seed, placement):
    inp = WL.make_custom_inputs(T, H, E, seed=seed)
    x = bf16_dev(inp["x_bits"])
    idx, gate = ops.moe_route_topk(to_dev(inp["logits"]), k)
    place = to_dev(placement) if placement is not None else None
    return x, idx, gate, place


def _compare(a, c, d, N):
    """a: the no-allocation call's outputs; c, d: the workspace path's."""
    ref = dict(c)
    ref.update(d)
    for key in KEYS:
        assert (host(a[key]) == host(ref[key])).all(), key
    assert (host(a["row_weight"]).view(np.uint32) == host(ref["row_weight"]).view(np.uint32)).all()
    assert (bf16_host(a["send"][:N]) == bf16_host(ref["send"][:N])).all()


def test_noalloc_matches_workspace_path_twice():
    """Call 1: the 4096-token, hidden-2048, 64-expert, top-6, 16-rank batch
    (contiguous placement).  Call 2, right after on the same stream: a smaller,
    ragged batch (777 tokens, 32 experts, top-4, 8 ranks) under an explicit
    random placement.  Both against moe_send_counts + moe_dispatch_permute."""
    cases = [(4096, 2048, 64, 6, 16, 0, None),
             (777, 512, 32, 4, 8, 1, WL.random_placement(32, 8, seed=3))]
    outs = []
    for T, H, E, k, R, seed, pl in cases:
        say(f"[noalloc] T={T} H={H} E={E} k={k} R={R} placement={'random' if pl is not None else 'contiguous'}")
        x, idx, gate, place = _case(T, H, E, k, R, seed, pl)
        a = ops.moe_dispatch_permute_noalloc(x, idx, gate, E, R, place)
        outs.append((a, x, idx, gate, place, E, R, T * k))
    torch.cuda.synchronize()
    for a, x, idx, gate, place, E, R, N in outs:
        c = ops.moe_send_counts(idx, E, R, place, dedup=False)
        d = ops.moe_dispatch_permute(x, idx, gate, E, R, c["ws"])
        torch.cuda.synchronize()
        _compare(a, c, d, N)


def test_noalloc_second_call_smaller_then_larger_again():
    """Three calls in a row on one stream with shrinking then growing plans;
    each call's outputs are compared right after it (the scratch keeps the
    previous call's plan)."""
    for T, H, E, k, R, seed in ((3000, 256, 128, 8, 16, 5), (65, 64, 8, 2, 4, 6),
                                (5000, 128, 64, 6, 16, 7)):
        say(f"[noalloc seq] T={T} H={H} E={E} k={k} R={R}")
        x, idx, gate, place = _case(T, H, E, k, R, seed, None)
        a = ops.moe_dispatch_permute_noalloc(x, idx, gate, E, R, place)
        torch.cuda.synchronize()
        c = ops.moe_send_counts(idx, E, R, place, dedup=False)
        d = ops.moe_dispatch_permute(x, idx, gate, E, R, c["ws"])
        torch.cuda.synchronize()
        _compare(a, c, d, T * k)


def test_noalloc_limits_and_zero_tokens():
    """A plan larger than the scratch is refused before any launch
    (MOE_EUNSUPPORTED, outputs untouched); zero tokens write zero counts."""
    L = ops.lib()
    E, k, R = 64, 8, 16
    T = 300000                                   # about 10 MB of plan
    need = L.moe_workspace_bytes(T, E, k, R, 0)
    assert need > (8 << 20)
    dv = torch.device("cuda:0")
    ec = torch.full((E,), 7, dtype=torch.int32, device=dv)
    rc = torch.full((R,), 7, dtype=torch.int32, device=dv)
    ro = torch.full((R + 1,), 7, dtype=torch.int32, device=dv)
    fake = ctypes.c_void_p(ec.data_ptr())       # never dereferenced: the call fails first
    st = torch.cuda.current_stream().cuda_stream
    rcode = L.moe_dispatch_permute_noalloc(fake, fake, fake, T, 64, E, k, R, None, 2,
                                           ec.data_ptr(), rc.data_ptr(), ro.data_ptr(), None,
                                           fake, fake, fake, fake, fake, st)
    torch.cuda.synchronize()
    assert rcode == 2                            # MOE_EUNSUPPORTED
    assert (host(ec) == 7).all() and (host(ro) == 7).all()
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=dv)
    idx = torch.empty((0, k), dtype=torch.int32, device=dv)
    gate = torch.empty((0, k), dtype=torch.float32, device=dv)
    a = ops.moe_dispatch_permute_noalloc(x, idx, gate, E, R)
    torch.cuda.synchronize()
    assert (host(a["rank_offsets"]) == 0).all() and (host(a["expert_counts"]) == 0).all()
