"""The benchmark's reference kernels (libmoe_hbm_ceiling.so) move the data they
are timed on: a copy is bit-identical, a scatter puts every row at its given
positions, a write covers the whole range.  Not part of the method; checked so
that the ceilings bench.py reports are real data movement."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_util import host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench
    return bench.ceiling_lib()


def test_copy_and_write(L):
    n = (3 << 20) + 4096 + 48            # a ragged last chunk
    st = torch.cuda.current_stream().cuda_stream
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda:0")
    dst = torch.zeros(n + 4096, dtype=torch.uint8, device="cuda:0")
    assert L.hbm_copy(src.data_ptr(), dst.data_ptr(), n, st) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst[:n], src) and bool((dst[n:] == 0).all())
    buf = torch.zeros(n + 4096, dtype=torch.uint8, device="cuda:0")
    assert L.hbm_write(buf.data_ptr(), n, st) == 0
    torch.cuda.synchronize()
    words = host(buf[:n].view(torch.int32)).reshape(-1, 4)
    lanes = np.arange(words.shape[0]) % 64
    assert (words[:, 1] == lanes).all()       # every 16-byte vector written
    assert bool((buf[n:] == 0).all())
    sink = torch.zeros(256, dtype=torch.int32, device="cuda:0")
    assert L.hbm_read(src.data_ptr(), n, sink.data_ptr(), st) == 0
    assert L.hbm_copy(src.data_ptr(), dst.data_ptr(), 8, st) == 2   # not a multiple of 16
    torch.cuda.synchronize()


@pytest.mark.parametrize("T,row_bytes,k", [(100, 4096, 6), (37, 8192, 2), (64, 272, 8)])
def test_scatter(L, T, row_bytes, k):
    say(f"[ceiling scatter] T={T} row_bytes={row_bytes} k={k}")
    rng = np.random.default_rng(T)
    pos = rng.permutation(T * k).astype(np.int32).reshape(T, k)
    x = torch.randint(0, 256, (T, row_bytes), dtype=torch.uint8, device="cuda:0")
    dst = torch.zeros((T * k, row_bytes), dtype=torch.uint8, device="cuda:0")
    p = torch.from_numpy(pos).to("cuda:0")
    st = torch.cuda.current_stream().cuda_stream
    assert L.hbm_scatter(x.data_ptr(), p.data_ptr(), T, row_bytes, k, dst.data_ptr(), st) == 0
    torch.cuda.synchronize()
    xh, dh = host(x), host(dst)
    for t in range(T):
        for j in range(k):
            assert (dh[pos[t, j]] == xh[t]).all()


@pytest.mark.parametrize("T,row_bytes,k", [(100, 4096, 6), (37, 8192, 8), (64, 272, 16)])
def test_scatter_distinct(L, T, row_bytes, k):
    """Positions that repeat within a token (slots sharing a row, as in the
    deduplicating dispatch): each distinct position gets the row, and no other
    row is written."""
    say(f"[ceiling scatter distinct] T={T} row_bytes={row_bytes} k={k}")
    rng = np.random.default_rng(T + k)
    n_distinct = rng.integers(1, k + 1, size=T)
    starts = np.concatenate([[0], np.cumsum(n_distinct)[:-1]])
    pos = np.empty((T, k), np.int32)
    for t in range(T):   # each slot takes one of the token's rows, every row at least once
        rows_t = starts[t] + np.arange(n_distinct[t])
        pos[t] = rng.permutation(np.concatenate([rows_t, rng.choice(rows_t, k - n_distinct[t])]))
    D = int(n_distinct.sum())
    x = torch.randint(0, 256, (T, row_bytes), dtype=torch.uint8, device="cuda:0")
    dst = torch.zeros((T * k, row_bytes), dtype=torch.uint8, device="cuda:0")
    p = torch.from_numpy(pos).to("cuda:0")
    st = torch.cuda.current_stream().cuda_stream
    assert L.hbm_scatter_distinct(x.data_ptr(), p.data_ptr(), T, row_bytes, k, dst.data_ptr(),
                                  st) == 0
    torch.cuda.synchronize()
    xh, dh = host(x), host(dst)
    for t in range(T):
        for r in starts[t] + np.arange(n_distinct[t]):
            assert (dh[r] == xh[t]).all()
    assert (dh[D:] == 0).all()


@pytest.mark.parametrize("T,row_bytes,k", [(100, 4096, 6), (37, 8192, 2), (64, 272, 8),
                                             (9, 5376, 16), (50, 2048, 3)])
def test_gather_sum(L, T, row_bytes, k):
    """Each token's output row is the fp32 sum, in slot order, of its distinct
    rows (positions repeat in half the tokens), truncated to bf16."""
    say(f"[ceiling gather_sum] T={T} row_bytes={row_bytes} k={k}")
    rng = np.random.default_rng(T * k)
    N = T * k
    pos = rng.integers(0, N, size=(T, k)).astype(np.int32)
    pos[::2, -1] = pos[::2, 0]                   # a repeated position
    H = row_bytes // 2
    vals = rng.standard_normal((N, H)).astype(np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)   # bf16 by truncation
    rows = torch.from_numpy(bits.view(np.int16)).to("cuda:0")
    out = torch.zeros((T, H), dtype=torch.int16, device="cuda:0")
    p = torch.from_numpy(pos).to("cuda:0")
    st = torch.cuda.current_stream().cuda_stream
    assert L.hbm_gather_sum(rows.data_ptr(), p.data_ptr(), T, row_bytes, k, out.data_ptr(),
                            st) == 0
    torch.cuda.synchronize()
    f = (bits.astype(np.uint32) << 16).view(np.float32)
    ref = np.empty((T, H), np.uint16)
    for t in range(T):
        acc = np.zeros(H, np.float32)
        seen = []
        for j in range(k):
            if pos[t, j] not in seen:
                seen.append(pos[t, j])
                acc = (acc + f[pos[t, j]]).astype(np.float32)
        ref[t] = (acc.view(np.uint32) >> 16).astype(np.uint16)
    assert (host(out).view(np.uint16) == ref).all()


def test_device_info(L):
    cu, mclk, bus, clk = (ctypes.c_int(0) for _ in range(4))
    arch = ctypes.create_string_buffer(64)
    assert L.hbm_device_info(ctypes.byref(cu), ctypes.byref(mclk), ctypes.byref(bus),
                             ctypes.byref(clk), arch, 64) == 0
    say(f"device: {arch.value.decode()} {cu.value} CUs, memory clock {mclk.value} kHz, "
        f"bus {bus.value} bits, clock {clk.value} kHz")
    assert arch.value.decode().startswith("gfx") and cu.value > 0
