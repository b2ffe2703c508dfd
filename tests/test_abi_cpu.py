"""The C-ABI library loads without a GPU, exports what include/moe_route.h
declares, and rejects invalid arguments on the host with the documented codes.

Only argument checks that return before any launch are exercised here (no
compute call is made without a GPU).  Fake non-null pointers are never
dereferenced because every case below fails a host check first.
"""
import ctypes
import os
import re

import pytest

from combine_top_router_select_amd import _lib as L
from combine_top_router_select_amd.build import LIB

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_route.h")
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced in these tests

EINVAL, EUNSUP, EWS = L.MOE_EINVAL, L.MOE_EUNSUPPORTED, L.MOE_EWORKSPACE


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is not built: run python -m combine_top_router_select_amd.build")
    return L.lib()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(L.SYMBOLS)
    raw = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(raw, n), n


def test_status_strings(lib):
    for code in range(5):
        s = L.status_string(code)
        assert s and isinstance(s, str)
    assert "unknown" in L.status_string(99)


def test_workspace_bytes(lib):
    f = lib.moe_workspace_bytes
    # 4096 tokens, 64 experts, top-6, 16 ranks; 256-byte sections.
    # plain: one int32 base per 16-tile group (4 groups) per expert, one count
    # byte per tile (64) and expert, one 4-byte slot code per (token, slot)
    n = f(4096, 64, 6, 16, 0)
    assert n >= 4 * 64 * 4 + 64 * 64 + 4096 * 6 * 4 and n % 256 == 0
    # dedup: bases only for the 16 rank columns, counts for experts and ranks
    nd = f(4096, 64, 6, 16, 1)
    assert nd >= 4 * 16 * 4 + 64 * 80 + 4096 * 6 * 4 and nd % 256 == 0
    assert nd > n                                  # the rank count columns
    assert f(0, 64, 6, 16, 0) > 0
    assert f(10, 64, 6, 5, 0) == 0                 # E % R != 0
    assert f(10, 64, 65, 16, 0) == 0               # k > E
    assert f(10, 2048, 6, 16, 0) == 0              # E > 1024
    assert f(-1, 64, 6, 16, 0) == 0


def test_route_errors(lib):
    f = lib.moe_route_topk
    assert f(None, 10, 8, 2, FAKE, FAKE, None) == EINVAL
    assert f(FAKE, -1, 8, 2, FAKE, FAKE, None) == EINVAL
    assert f(FAKE, 10, 8, 0, FAKE, FAKE, None) == EINVAL
    assert f(FAKE, 10, 8, 9, FAKE, FAKE, None) == EINVAL
    assert f(FAKE, 10, 0, 1, FAKE, FAKE, None) == EINVAL
    assert f(FAKE, 10, 64, 17, FAKE, FAKE, None) == EUNSUP
    assert f(FAKE, 10, 2000, 2, FAKE, FAKE, None) == EUNSUP
    assert f(FAKE, 2 ** 30, 64, 6, FAKE, FAKE, None) == EUNSUP   # T*k >= 2^31
    assert f(None, 0, 8, 2, None, None, None) == L.MOE_OK      # empty: nothing launched


def test_send_counts_errors(lib):
    f = lib.moe_send_counts
    ws = lib.moe_workspace_bytes(100, 8, 2, 4, 0)
    ok = (FAKE, 100, 8, 2, 4, None, 0, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None)

    def call(**kw):
        a = list(ok)
        names = ["idx", "T", "E", "k", "R", "place", "dedup", "ec", "rc", "ro", "eo", "ws",
                 "wsb", "stream"]
        for key, v in kw.items():
            a[names.index(key)] = v
        return f(*a)

    assert call(R=3) == EINVAL
    assert call(R=0) == EINVAL
    assert call(E=128, R=128) == EUNSUP
    assert call(idx=None) == EINVAL
    assert call(ec=None) == EINVAL
    assert call(ws=None) == EINVAL
    assert call(wsb=ws - 1) == EWS
    wsd = lib.moe_workspace_bytes(6400, 8, 2, 4, 1)
    assert call(T=6400, dedup=1, wsb=wsd - 1) == EWS


def test_route_plan_errors(lib):
    f = lib.moe_route_plan
    ws = lib.moe_workspace_bytes(100, 8, 2, 4, 0)
    names = ["logits", "T", "E", "k", "gating", "R", "place", "dedup", "idx", "gate", "ec", "rc",
             "ro", "eo", "ncs", "W", "ws", "wsb", "stream"]
    ok = (FAKE, 100, 8, 2, 0, 4, None, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None, FAKE, ws,
          None)

    def call(**kw):
        a = list(ok)
        for key, v in kw.items():
            a[names.index(key)] = v
        return f(*a)

    assert call(gating=2) == EINVAL
    assert call(gating=-1) == EINVAL
    assert call(ncs=-1, W=FAKE) == EINVAL
    assert call(ncs=101, W=FAKE) == EINVAL                # more than tokens
    assert call(ncs=10, W=None) == EINVAL
    assert call(logits=None) == EINVAL
    assert call(idx=None) == EINVAL
    assert call(gate=None) == EINVAL
    assert call(ec=None) == EINVAL
    assert call(ws=None) == EINVAL
    assert call(R=3) == EINVAL
    assert call(k=9) == EINVAL
    assert call(k=17, E=64) == EUNSUP
    assert call(E=128, R=128) == EUNSUP
    assert call(wsb=ws - 1) == EWS
    wsd = lib.moe_workspace_bytes(6400, 8, 2, 4, 1)
    assert call(T=6400, dedup=1, wsb=wsd - 1) == EWS


def test_route_dispatch_errors(lib):
    f = lib.moe_route_dispatch
    ws = lib.moe_workspace_bytes(100, 8, 2, 4, 0)
    names = ["logits", "x", "T", "H", "E", "k", "gating", "R", "place", "dedup", "bpe", "idx",
             "gate", "ec", "rc", "ro", "eo", "send", "rt", "rx", "rg", "rw", "sr", "nr", "ncs", "W",
             "ws", "wsb", "stream"]
    ok = [FAKE, FAKE, 100, 128, 8, 2, 0, 4, None, 0, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
          FAKE, FAKE, None, FAKE, FAKE, None, 0, None, FAKE, ws, None]

    def call(**kw):
        a = list(ok)
        for key, v in kw.items():
            a[names.index(key)] = v
        return f(*a)

    assert call(gating=2) == EINVAL
    assert call(ncs=101, W=FAKE) == EINVAL                # more co-selection tokens than tokens
    assert call(ncs=-1, W=FAKE) == EINVAL
    for name in ("logits", "x", "idx", "gate", "ec", "rc", "ro", "send", "rt", "rx", "rw", "sr",
                 "ws"):
        assert call(**{name: None}) == EINVAL, name
    assert call(bpe=3) == EUNSUP
    assert call(H=4) == EUNSUP                            # 8-byte rows
    assert call(R=3) == EINVAL
    assert call(k=9) == EINVAL
    assert call(k=17, E=64) == EUNSUP
    assert call(wsb=ws - 1) == EWS
    wsd = lib.moe_workspace_bytes(100, 8, 2, 4, 1)
    assert call(dedup=1, wsb=wsd, rg=FAKE) == EINVAL      # dedup needs n_rows
    assert call(dedup=1, wsb=wsd, nr=FAKE) == EINVAL      # and row_gates
    assert call(dedup=1, wsb=wsd - 1, rg=FAKE, nr=FAKE) == EWS


def test_combine_route_errors(lib):
    f = lib.moe_combine_route
    ws = lib.moe_workspace_bytes(100, 8, 2, 4, 0)
    names = ["rows", "w", "sr", "T", "H", "k", "bpe", "out", "logits", "Tn", "E", "kn", "gating",
             "R", "place", "dedup", "idx", "gate", "ws", "wsb", "stream"]
    ok = [FAKE, None, FAKE, 50, 128, 2, 2, FAKE, FAKE, 100, 8, 2, 0, 4, None, 0, FAKE, FAKE, FAKE,
          ws, None]

    def call(**kw):
        a = list(ok)
        for key, v in kw.items():
            a[names.index(key)] = v
        return f(*a)

    assert call(gating=2) == EINVAL
    for name in ("rows", "sr", "out", "logits", "idx", "gate", "ws"):
        assert call(**{name: None}) == EINVAL, name
    assert call(bpe=4) == EUNSUP                           # the combine takes bf16 or fp8 rows
    assert call(H=4) == EUNSUP                             # 8-byte rows
    assert call(k=17) == EUNSUP
    assert call(T=-1) == EINVAL
    assert call(Tn=-1) == EINVAL
    assert call(R=3) == EINVAL
    assert call(kn=9) == EINVAL
    assert call(wsb=ws - 1) == EWS
    # no combine (tokens 0) needs no rows; no routed tokens need no logits or
    # ids (and nothing is launched)
    assert call(T=0, rows=None, sr=None, out=None, Tn=0, logits=None, idx=None, gate=None,
                wsb=lib.moe_workspace_bytes(0, 8, 2, 4, 0)) == 0


def test_dispatch_routed_errors(lib):
    f = lib.moe_dispatch_routed
    ws = lib.moe_workspace_bytes(100, 8, 2, 4, 0)
    names = ["x", "idx", "gate", "T", "H", "E", "k", "R", "place", "dedup", "bpe", "ec", "rc",
             "ro", "eo", "send", "rt", "rx", "rg", "rw", "sr", "nr", "ncs", "W", "ws", "wsb",
             "stream"]
    ok = [FAKE, FAKE, FAKE, 100, 128, 8, 2, 4, None, 0, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
          FAKE, None, FAKE, FAKE, None, 0, None, FAKE, ws, None]

    def call(**kw):
        a = list(ok)
        for key, v in kw.items():
            a[names.index(key)] = v
        return f(*a)

    assert call(ncs=101, W=FAKE) == EINVAL
    for name in ("x", "idx", "gate", "ec", "rc", "ro", "send", "rt", "rx", "rw", "sr", "ws"):
        assert call(**{name: None}) == EINVAL, name
    assert call(bpe=3) == EUNSUP
    assert call(H=4) == EUNSUP
    assert call(R=3) == EINVAL
    assert call(k=9) == EINVAL
    assert call(wsb=ws - 1) == EWS
    wsd = lib.moe_workspace_bytes(100, 8, 2, 4, 1)
    assert call(dedup=1, wsb=wsd, rg=FAKE) == EINVAL       # dedup needs n_rows
    assert call(dedup=1, wsb=wsd, nr=FAKE) == EINVAL       # and row_gates


def test_dispatch_errors(lib):
    f = lib.moe_dispatch_permute
    ws = lib.moe_workspace_bytes(100, 8, 2, 4, 0)
    base = [FAKE, FAKE, FAKE, 100, 128, 8, 2, 4, 2, FAKE, ws, FAKE, FAKE, FAKE, FAKE, FAKE,
            0, None, None]
    names = ["x", "idx", "gate", "T", "H", "E", "k", "R", "bpe", "ws", "wsb", "send", "rt", "re",
             "rw", "sr", "ncs", "W", "stream"]

    def call(**kw):
        a = list(base)
        for key, v in kw.items():
            a[names.index(key)] = v
        return f(*a)

    assert call(bpe=3) == EUNSUP
    assert call(bpe=0) == EINVAL
    assert call(H=4) == EUNSUP                     # 8 bytes per row: not a multiple of 16
    assert call(H=0) == EINVAL
    assert call(wsb=ws - 1) == EWS
    assert call(send=None) == EINVAL
    assert call(x=None) == EINVAL
    assert call(ws=None) == EINVAL
    assert call(W=FAKE, ncs=101) == EINVAL         # more co-selection tokens than tokens
    assert call(W=FAKE, ncs=-1) == EINVAL
    g = lib.moe_dispatch_permute_dedup
    wsd = lib.moe_workspace_bytes(6400, 8, 2, 4, 1)
    args = [FAKE, FAKE, FAKE, 6400, 128, 8, 2, 4, 2, FAKE, wsd, FAKE, FAKE, FAKE, FAKE, FAKE,
            FAKE, None, 0, None, None]
    assert g(*args) == EINVAL                      # n_rows is NULL
    args[17] = FAKE
    args[18], args[19] = 6401, FAKE                # more co-selection tokens than tokens
    assert g(*args) == EINVAL
    args[18], args[19] = 0, None
    args[10] = wsd - 1                             # one byte short
    assert g(*args) == EWS


def test_combine_and_coselect_errors(lib):
    c = lib.moe_combine
    assert c(FAKE, None, FAKE, 10, 128, 2, 4, FAKE, None) == EUNSUP   # bf16 or fp8 rows only
    assert c(FAKE, None, FAKE, 10, 128, 2, 3, FAKE, None) == EUNSUP
    assert c(FAKE, None, FAKE, 10, 8, 2, 1, FAKE, None) == EUNSUP     # 8-byte fp8 rows
    assert c(FAKE, None, FAKE, 10, 4, 2, 2, FAKE, None) == EUNSUP     # 8-byte rows
    assert c(None, None, FAKE, 10, 128, 2, 2, FAKE, None) == EINVAL
    assert c(FAKE, None, FAKE, 10, 128, 17, 2, FAKE, None) == EUNSUP
    assert c(FAKE, None, FAKE, -5, 128, 2, 2, FAKE, None) == EINVAL
    s = lib.moe_coselect_counts
    assert s(None, 10, 8, 2, FAKE, None) == EINVAL
    assert s(FAKE, 10, 8, 9, FAKE, None) == EINVAL                  # k > E
    assert s(FAKE, 10, 8, 2, None, None) == EINVAL
    assert s(FAKE, -1, 8, 2, FAKE, None) == EINVAL
    assert s(FAKE, 10, 2048, 2, FAKE, None) == EUNSUP               # E > 1024
    assert s(None, 0, 8, 2, None, None) == 0                        # no tokens: no-op


def test_receive_side_errors(lib):
    # the plain plan without the tile expert bitmaps (2 tiles x 8 experts x 8 bytes, aligned)
    assert lib.moe_expand_workspace_bytes(100, 8, 2, 4) == \
        lib.moe_workspace_bytes(100, 8, 2, 4, 0) - 256
    assert lib.moe_expand_workspace_bytes(100, 8, 9, 4) == 0
    ws = lib.moe_expand_workspace_bytes(100, 8, 2, 4)
    f = lib.moe_expand_counts
    base = [FAKE, FAKE, 100, 8, 2, 4, None, FAKE, FAKE, FAKE, None, FAKE, ws, None]
    names = ["rx", "n", "C", "E", "k", "R", "place", "ec", "rc", "ro", "eo", "ws", "wsb", "st"]

    def call(fn, base, names, **kw):
        a = list(base)
        for key, v in kw.items():
            a[names.index(key)] = v
        return fn(*a)

    assert call(f, base, names, n=None) == EINVAL      # the device row count is required
    assert call(f, base, names, rx=None) == EINVAL
    assert call(f, base, names, C=-1) == EINVAL
    assert call(f, base, names, R=3) == EINVAL         # E % R != 0
    assert call(f, base, names, k=17, E=32) == EUNSUP
    assert call(f, base, names, wsb=ws - 1) == EWS
    g = lib.moe_expand_permute
    gb = [FAKE, FAKE, FAKE, 100, 128, 8, 2, 4, 2, FAKE, ws, FAKE, 200, FAKE, FAKE, FAKE, FAKE,
          None]
    gn = ["rows", "rg", "n", "C", "H", "E", "k", "R", "bpe", "ws", "wsb", "ex", "excap", "er",
          "ee", "eg", "rs", "st"]
    assert call(g, gb, gn, n=None) == EINVAL
    assert call(g, gb, gn, excap=-1) == EINVAL
    assert call(g, gb, gn, excap=1 << 40) == EUNSUP
    assert call(g, gb, gn, bpe=3) == EUNSUP
    assert call(g, gb, gn, H=4) == EUNSUP
    assert call(g, gb, gn, wsb=ws - 1) == EWS
    assert call(g, gb, gn, rs=None) == EINVAL
    assert call(g, gb, gn, ex=None) == EINVAL
    assert call(g, gb, gn, C=0, wsb=lib.moe_expand_workspace_bytes(0, 8, 2, 4)) == 0  # no-op
    r = lib.moe_expand_reduce
    rb = [FAKE, None, FAKE, FAKE, 100, 128, 2, 2, FAKE, None]
    rn = ["y", "w", "rs", "n", "C", "H", "k", "bpe", "out", "st"]
    assert call(r, rb, rn, n=None) == EINVAL
    assert call(r, rb, rn, bpe=4) == EUNSUP
    assert call(r, rb, rn, k=17) == EUNSUP
    assert call(r, rb, rn, H=4) == EUNSUP
    assert call(r, rb, rn, out=None) == EINVAL
    assert call(r, rb, rn, C=-2) == EINVAL
    assert call(r, rb, rn, C=0) == 0                    # no-op


def test_noalloc_errors(lib):
    """The entry point that allocates nothing refuses, on the host, plans
    larger than its scratch and the argument errors of the calls it stands for
    (no HIP call is made in any of these cases)."""
    f = lib.moe_dispatch_permute_noalloc
    base = [FAKE, FAKE, FAKE, 4096, 2048, 64, 6, 16, None, 2, FAKE, FAKE, FAKE, None, FAKE, FAKE,
            FAKE, FAKE, FAKE, None]
    names = ["x", "idx", "gate", "T", "H", "E", "k", "R", "place", "bpe", "ec", "rc", "ro", "eo",
             "send", "rt", "re", "rw", "sr", "st"]

    def call(**kw):
        a = list(base)
        for key, v in kw.items():
            a[names.index(key)] = v
        return f(*a)

    big = 300000                                  # plan of about 10 MB > 8 MiB of scratch
    assert lib.moe_workspace_bytes(big, 64, 6, 16, 0) > (8 << 20)
    assert lib.moe_workspace_bytes(200000, 64, 6, 16, 0) <= (8 << 20)
    assert call(T=big) == EUNSUP
    assert call(T=-1) == EINVAL
    assert call(R=3) == EINVAL
    assert call(k=17, E=64) == EUNSUP
    assert call(bpe=3) == EUNSUP
    assert call(H=4) == EUNSUP
    assert call(ec=None) == EINVAL
    assert call(send=None) == EINVAL
    assert call(x=None) == EINVAL


def test_ceiling_library_exports_and_checks():
    """The benchmark's reference-kernel library loads without a GPU, exports
    its entry points and rejects bad sizes before any launch."""
    from combine_top_router_select_amd.build import CEILING_LIB
    if not os.path.exists(CEILING_LIB):
        pytest.fail(f"{CEILING_LIB} is not built")
    raw = ctypes.CDLL(CEILING_LIB)
    for n in ("hbm_read", "hbm_write", "hbm_copy", "hbm_scatter", "hbm_scatter_distinct",
              "hbm_gather_sum", "hbm_device_info"):
        assert hasattr(raw, n), n
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    raw.hbm_copy.argtypes = [P, P, i64, P]
    raw.hbm_scatter.argtypes = [P, P, i64, i32, i32, P, P]
    raw.hbm_scatter_distinct.argtypes = [P, P, i64, i32, i32, P, P]
    raw.hbm_gather_sum.argtypes = [P, P, i64, i32, i32, P, P]
    assert raw.hbm_copy(FAKE, FAKE, 24, None) == 2       # not a multiple of 16
    assert raw.hbm_copy(None, FAKE, 32, None) == 2
    for f in (raw.hbm_scatter, raw.hbm_scatter_distinct):
        assert f(FAKE, FAKE, 10, 24, 2, FAKE, None) == 2
        assert f(FAKE, FAKE, 10, 32, 0, FAKE, None) == 2
        assert f(FAKE, FAKE, 10, 32, 65, FAKE, None) == 2
        assert f(FAKE, FAKE, 0, 32, 2, FAKE, None) == 2
    g = raw.hbm_gather_sum
    assert g(FAKE, FAKE, 10, 24, 2, FAKE, None) == 2      # row bytes not a multiple of 16
    assert g(FAKE, FAKE, 10, 32, 17, FAKE, None) == 2     # k past 16
    assert g(FAKE, FAKE, 10, 32, 0, FAKE, None) == 2
    assert g(FAKE, FAKE, 0, 32, 2, FAKE, None) == 2
    assert g(None, FAKE, 10, 32, 2, FAKE, None) == 2


def test_product_path_does_not_touch_oracle():
    """The package sources never import, load or name the oracle."""
    pkg = os.path.join(ROOT, "combine_top_router_select_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                txt = open(os.path.join(dirpath, fn)).read()
                for pat in (r"^\s*(from|import)\s+oracle", r"liboracle", r"oracle\.c\b",
                            r"oracle_[a-z_]+\("):
                    assert not re.search(pat, txt, flags=re.M), (fn, pat)


def test_binding_rejects_host_tensors():
    """Every tensor the binding is handed must be on a GPU: host tensors are
    refused before the library is called."""
    import pytest
    import torch
    from combine_top_router_select_amd import ops
    t32 = torch.zeros((8, 2), dtype=torch.int32)
    f32 = torch.zeros((8, 2), dtype=torch.float32)
    logits = torch.zeros((8, 4), dtype=torch.float32)
    x = torch.zeros((8, 8), dtype=torch.bfloat16)
    calls = [
        lambda: ops.moe_route_topk(logits, 2),
        lambda: ops.moe_send_counts(t32, 4, 2),
        lambda: ops.moe_route_plan(logits, 2, 2),
        lambda: ops.moe_route_dispatch(logits, x, 2, 2),
        lambda: ops.moe_combine_route(None, None, None, logits, 2, 2),
        lambda: ops.moe_dispatch_permute(x, t32, f32, 4, 2, torch.zeros(16, dtype=torch.uint8)),
        lambda: ops.moe_combine(x, None, t32),
        lambda: ops.moe_coselect_counts(t32, 4),
        lambda: ops.moe_shuffle_predict(t32, t32, torch.zeros((4, 4, 2), dtype=torch.int32),
                                        torch.zeros((4, 2), dtype=torch.int32), 8),
    ]
    for i, call in enumerate(calls):
        with pytest.raises(ValueError, match="GPU device"):
            call()
