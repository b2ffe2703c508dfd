"""The C ABI from a plain C program (tests/abi_demo.c, built by the package
build with gcc as C11): one step through moe_route_plan, moe_dispatch_permute
and moe_combine on hipMalloc'd buffers, with its own checks (offsets scan the
counts, every row is its token's x, identity combine returns x), then three
batches through the pipelined loop (moe_combine_route routing the next batch,
moe_dispatch_routed) over two buffer sets, each against the one-call step."""
import os
import subprocess

import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu

DEMO = os.path.join(os.path.dirname(os.path.abspath(__file__)), "abi_demo")


def test_plain_c_user_of_the_abi():
    assert os.path.exists(DEMO), f"{DEMO} is missing: run __graft_entry__.build()"
    say("[abi_demo] plain C program over the C ABI")
    r = subprocess.run([DEMO], capture_output=True, text=True, timeout=120)
    say("  " + r.stdout.strip())
    assert r.returncode == 0 and "abi_demo ok" in r.stdout, r.stdout + r.stderr
