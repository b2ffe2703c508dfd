"""Benchmark of the per-GPU MoE dispatch/combine hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--dedup]
                    [--receive] [--fp8] [--search] [--shuffle] [--streams {0,1,2,3,4}]
                    [--separate] [--plan-call] [--one-call] [--graph] [--overlap]
                    [--coselect-in {dispatch,route}] [--step-events]
                    [--no-cpu-baseline] [--no-reference] [--cpu-seconds S]
                    [--footprint-gib G] [--calib-copy]

A step is one pass of the whole path over one batch of the workload's seeded
synthetic input, with inputs resident in HBM: top-k routing, send counts,
offsets and the co-selection counts of the routed tokens (one combined call;
--separate uses their three entry points) -> dispatch permute -> combine
(identity experts: the combine reads the send buffer).  With --receive (dedup)
the receive side runs between dispatch and combine.  The workload defaults to
4096 tokens, hidden 2048 bf16, 64 experts, top-6, 16 logical ranks, contiguous
placement (DeepSeek-MoE-16B-shaped), plain (one row per token-expert) dispatch.

Without --steps the timed region holds as many steps as fill about 2 s
(between 200 and 100000), from the time of 50 untimed steps after the
warm-up; the JSON line's `warmup` counts those.

Steps are independent batches.  By default, when a batch's activations are
at most 64 MiB, consecutive steps alternate between two streams with no waits
between them (the way a server overlaps two micro-batches), so one batch's
latency-bound kernels can run beside the other batch's copies; each step's own
kernels stay in order on its stream.  Larger batches run on one stream
(measured: two vary by several percent from run to run there and are slower
on the receive side).  Each buffer set is only ever used on one stream.  The same K steps are then timed on the other setting
and reported as `other_streams`; --streams n fixes the setting.  --overlap instead forks only the co-selection
counts onto a second stream inside each step.

By default a step is moe_dispatch_routed (the plan's counts, offsets and scan,
the rows, and the co-selection counts of the workload's first tokens: one
launch, the dispatch workgroups scanning small plans themselves) and then
moe_combine_route, whose launch also routes the batch of the next step on the
same stream (routing, tile counts, slot codes: its workgroups run beside the
combine's copies); each batch is routed once, one step ahead.  --one-call takes
moe_route_dispatch (the routing and the dispatch of this batch) and then
moe_combine; --plan-call takes moe_route_plan and then the dispatch call;
--separate takes moe_route_topk, moe_send_counts and the dispatch call.  The
co-selection counts go with the dispatch launch, from the plan's expert
bitmaps; --coselect-in route takes them in the routing call instead (implies
--plan-call; with --separate, the stand-alone co-selection kernel at the end
of the step).

The timed steps call the C ABI directly with arguments marshalled once per
buffer set (the Python binding's per-call checks would otherwise cost about
10 us of host time per call and make short steps host-bound); the first
warm-up step goes through the binding.

To keep the last-level (Infinity) cache from serving the data, steps rotate
over enough independent buffer sets to exceed it several times over, so each
step's inputs and outputs were last touched many hundreds of MB earlier.

Prints one JSON line.  `roofline` reports the dominant kernel's algorithmic HBM
bytes per launch divided by its mean launch duration, measured with HIP events
on the stream the kernels run on around a run of back-to-back launches of that
kernel alone (queued behind a short GPU sleep so that host launch overhead
stays out); `traffic` is the HBM bytes per launch that rocprofv3's FETCH_SIZE
and WRITE_SIZE counters measured for that kernel (profiles/hbm_traffic_*.md,
scaled by a plain-copy calibration), or null when there is no such record for
the workload or the kernel's sources changed since.  `copy_reference` times a
plain device copy of the same bytes the same way; `hbm_ceiling` times
hand-written reference kernels (pure read, pure write, copy, and the plain
dispatch's own scatter without its plan and metadata) at the dispatch's sizes,
the practical ceilings its rate is compared with.  `device` names the GPU
(architecture, compute units, clocks).  `cpu_baseline` times the CPU oracle on
the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
PKG = os.path.join(ROOT, "combine_top_router_select_amd")
# The files that hold each entry point's kernel code (besides COMMON_SOURCES):
# a committed counter record counts only while their SHA-256 is unchanged.
_DISPATCH_SRC = ("csrc/dispatch.hip", "csrc/plan_order.hpp", "csrc/coselect_bm.hpp")
_COMBINE_SRC = ("csrc/combine.hip", "csrc/combine_rows.hpp")
KERNEL_SOURCES = {"moe_dispatch_permute": _DISPATCH_SRC,
                  "moe_dispatch_permute_dedup": _DISPATCH_SRC,
                  "moe_combine": _COMBINE_SRC,
                  "moe_expand_permute": _DISPATCH_SRC,
                  "moe_expand_reduce": _COMBINE_SRC,
                  "moe_route_dispatch": _DISPATCH_SRC,
                  "moe_dispatch_routed": _DISPATCH_SRC,
                  "moe_combine_route": ("csrc/combine_route.hip", "csrc/combine_rows.hpp",
                                        "csrc/route_tile.hpp")}
COMMON_SOURCES = ("csrc/common.hpp", "build.py")
METRIC = "dispatch+combine tokens/s and achieved HBM GB/s (% of MI355X peak)"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None,
                   help="timed steps (default: about 2 s of them, at least 200 and at most "
                        "100000, from the step time of 50 untimed steps after the warm-up)")
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="deepseek_moe_16b")
    p.add_argument("--dedup", action="store_true")
    p.add_argument("--fp8", action="store_true",
                   help="rows in fp8 E4M3 (activations quantised on the host): dispatch moves one "
                        "byte per element, combine decodes to bf16")
    p.add_argument("--receive", action="store_true",
                   help="dedup mode: also run the receive side (per-expert expansion, identity "
                        "experts, reduction) and combine the reduced rows with weight 1")
    p.add_argument("--search", action="store_true",
                   help="also fit a correlated placement to the co-selection counts of the "
                        "workload's first tokens and report the dedup rows it gives")
    p.add_argument("--shuffle", action="store_true",
                   help="also fit the token-shuffle planner on one batch of correlated "
                        "three-layer routing and plan another, reporting times and locality")
    p.add_argument("--streams", type=int, default=0, choices=(0, 1, 2, 3, 4),
                   help="n > 1: alternate the rotated buffer sets, i.e. consecutive "
                        "independent batches, between n streams so that one batch's "
                        "latency-bound kernels overlap another's copies (no cross-stream "
                        "waits); 1: every step on one stream; 0 (default): 2 when a batch's "
                        "activations are at most 64 MiB, else 1.  The other setting (1, or 2 "
                        "after 1) is timed too and reported as other_streams")
    p.add_argument("--separate", action="store_true",
                   help="route and count with moe_route_topk + moe_send_counts instead of the "
                        "fused moe_route_plan (one kernel more)")
    p.add_argument("--plan-call", action="store_true",
                   help="moe_route_plan then the dispatch call instead of moe_route_dispatch")
    p.add_argument("--one-call", action="store_true",
                   help="moe_route_dispatch then moe_combine instead of moe_dispatch_routed "
                        "then moe_combine_route (which routes the stream's next batch)")
    p.add_argument("--graph", action="store_true", help="replay the step as a HIP graph")
    p.add_argument("--overlap", action="store_true",
                   help="run the co-selection counts on a second stream")
    p.add_argument("--coselect-in", choices=("dispatch", "route"), default="dispatch",
                   help="the call that takes the co-selection counts (without --overlap)")
    p.add_argument("--step-events", action="store_true",
                   help="also record HIP events around the dispatch and combine launches of every "
                        "timed step (their in-step durations)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-reference", action="store_true",
                   help="skip the copy_reference and hbm_ceiling legs (short profiler runs)")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--footprint-gib", type=float, default=2.0,
                   help="total size of the rotated buffer sets")
    p.add_argument("--calib-copy", action="store_true",
                   help="only run a plain 1 GiB device copy (counter calibration)")
    return p.parse_args()


def calib_copy():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    b = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e)
    print(json.dumps({"calib_copy_bytes_read": n, "calib_copy_bytes_written": n,
                      "ms": ms, "GBps_rw": 2 * n / ms / 1e6}), flush=True)


def copy_reference(torch, nbytes, launches=100):
    """Device-to-device copies moving `nbytes` per launch (half read, half
    written), timed like the kernels: back-to-back launches over rotated
    buffers (about 1.5 GB, beyond the 256 MB Infinity Cache) queued behind a GPU
    sleep, bracketed by HIP events on the current stream."""
    half = max(1, nbytes // 2)
    pairs = max(2, int(np.ceil(1.5e9 / (2 * half))))
    bufs = [(torch.empty(half, dtype=torch.uint8, device="cuda:0"),
             torch.empty(half, dtype=torch.uint8, device="cuda:0")) for _ in range(pairs)]
    for a, b in bufs:
        a.fill_(1)
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(20_000_000)
    e0.record()
    for i in range(launches):
        a, b = bufs[i % pairs]
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / launches
    del bufs
    return {"bytes_per_copy": 2 * half, "us": round(t * 1e6, 2),
            "GBps": round(2 * half / t / 1e9, 1)}


def time_launches(torch, calls):
    """Mean duration of one launch over a run of back-to-back launches (each a
    (function, args) pair returning 0 on success), queued behind a GPU sleep
    and bracketed by HIP events on the current stream."""
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(20_000_000)
    e0.record()
    for fn, args in calls:
        rc = fn(*args)
        if rc != 0:
            raise RuntimeError(f"{getattr(fn, '__name__', fn)} returned {rc}")
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / len(calls)


def ceiling_lib():
    import ctypes
    from combine_top_router_select_amd.build import CEILING_LIB
    L = ctypes.CDLL(CEILING_LIB)
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.hbm_read.argtypes = [P, i64, P, P]
    L.hbm_write.argtypes = [P, i64, P]
    L.hbm_copy.argtypes = [P, P, i64, P]
    L.hbm_scatter.argtypes = [P, P, i64, i32, i32, P, P]
    L.hbm_scatter_distinct.argtypes = [P, P, i64, i32, i32, P, P]
    L.hbm_gather_sum.argtypes = [P, P, i64, i32, i32, P, P]
    L.hbm_device_info.argtypes = [P, P, P, P, ctypes.c_char_p, i32]
    for f in ("hbm_read", "hbm_write", "hbm_copy", "hbm_scatter", "hbm_scatter_distinct",
              "hbm_gather_sum", "hbm_device_info"):
        getattr(L, f).restype = i32
    return L


def device_info(torch):
    """The GPU the run used: name, architecture, compute units, clocks."""
    import ctypes
    info = {"name": torch.cuda.get_device_name(0)}
    try:
        L = ceiling_lib()
        cu, mclk, bus, clk = (ctypes.c_int(0) for _ in range(4))
        arch = ctypes.create_string_buffer(64)
        if L.hbm_device_info(ctypes.byref(cu), ctypes.byref(mclk), ctypes.byref(bus),
                             ctypes.byref(clk), arch, 64) == 0:
            info.update(arch=arch.value.decode(), compute_units=cu.value,
                        mem_clock_MHz=round(mclk.value / 1e3), mem_bus_width_bits=bus.value,
                        clock_MHz=round(clk.value / 1e3))
    except OSError:
        info["arch"] = getattr(torch.cuda.get_device_properties(0), "gcnArchName", None)
    return info


def hbm_ceiling(torch, sets, T, H, k, bpe, n_rows, dedup, launches=100):
    """Practical HBM ceilings at the dispatch's sizes: hand-written reference
    kernels (csrc/hbm_ceiling.hip) in the dispatch kernel's access pattern
    (one wave per 4 KiB chunk, 16-byte accesses, nontemporal loads) without its
    plan lookups and metadata, timed like the path's kernels (back-to-back
    launches over rotated buffers, about 1.5 GB, so nothing is served from the
    256 MB Infinity Cache):
      read     a pure read of the dispatch's algorithmic bytes;
      write    a pure write of them;
      copy     half of them read and written elsewhere;
      scatter  the dispatch's own data movement (each x row to its k send
               rows, or with dedup to its distinct ones, positions from the
               step's own slot_row), on the bench's buffer sets;
      gather_sum  the combine's own data movement (each token's distinct
               send rows summed into its output row, same positions), on the
               bench's buffer sets (bf16 rows only; null for fp8)."""
    L = ceiling_lib()
    st = torch.cuda.current_stream().cuda_stream
    read_b, write_b = T * H * bpe, n_rows * H * bpe
    total = (read_b + write_b) // 16 * 16
    half = total // 2 // 16 * 16
    nbuf = max(2, int(np.ceil(1.5e9 / total)))
    bufs = [torch.empty(total, dtype=torch.uint8, device="cuda:0") for _ in range(nbuf)]
    for b in bufs:
        b.fill_(1)
    sink = torch.zeros(256, dtype=torch.int32, device="cuda:0")
    res = {}
    t = time_launches(torch, [(L.hbm_read, (bufs[i % nbuf].data_ptr(), total, sink.data_ptr(),
                                            st)) for i in range(launches)])
    res["read"] = {"bytes": total, "us": round(t * 1e6, 2), "GBps": round(total / t / 1e9, 1)}
    t = time_launches(torch, [(L.hbm_write, (bufs[i % nbuf].data_ptr(), total, st))
                              for i in range(launches)])
    res["write"] = {"bytes": total, "us": round(t * 1e6, 2), "GBps": round(total / t / 1e9, 1)}
    t = time_launches(torch, [(L.hbm_copy, (bufs[i % nbuf].data_ptr(),
                                            bufs[i % nbuf].data_ptr() + half, half, st))
                              for i in range(launches)])
    res["copy"] = {"bytes": 2 * half, "us": round(t * 1e6, 2),
                   "GBps": round(2 * half / t / 1e9, 1)}
    del bufs
    fn = L.hbm_scatter_distinct if dedup else L.hbm_scatter
    calls = [(fn, (b.x.data_ptr(), b.disp["slot_row"].data_ptr(), T, H * bpe, k,
                   b.disp["send"].data_ptr(), st))
             for b in (sets[i % len(sets)] for i in range(launches))]
    t = time_launches(torch, calls)
    res["scatter"] = {"bytes": read_b + write_b, "us": round(t * 1e6, 2),
                      "GBps": round((read_b + write_b) / t / 1e9, 1)}
    res["gather_sum"] = None
    if bpe == 2:
        calls = [(L.hbm_gather_sum, (b.disp["send"].data_ptr(), b.disp["slot_row"].data_ptr(), T,
                                     H * bpe, k, b.out.data_ptr(), st))
                 for b in (sets[i % len(sets)] for i in range(launches))]
        t = time_launches(torch, calls)
        gb = write_b + read_b   # the dispatch's rows read, one output row per token written
        res["gather_sum"] = {"bytes": gb, "us": round(t * 1e6, 2), "GBps": round(gb / t / 1e9, 1)}
    return res


class BufferSet:
    """Device buffers for one step (inputs resident, outputs preallocated)."""

    def __init__(self, torch, ops, inp, w, dedup, dev, receive=False, fp8=False):
        T, H, E, k, R = w.tokens, w.hidden_dim, w.n_experts, w.top_k, w.n_ranks
        N = T * k
        rdt = torch.float8_e4m3fn if fp8 else torch.bfloat16  # row type of x, send, expanded
        self.logits = torch.from_numpy(inp["logits"]).to(dev)
        if fp8:
            self.x = torch.from_numpy(inp["x_fp8"]).view(torch.float8_e4m3fn).to(dev)
        else:
            self.x = torch.from_numpy(inp["x_bits"].view(np.int16)).view(torch.bfloat16).to(dev)
        self.place = (torch.from_numpy(inp["placement"]).to(dev)
                      if inp["placement"] is not None else None)
        i32, f32 = torch.int32, torch.float32
        self.idx = torch.empty((T, k), dtype=i32, device=dev)
        self.gate = torch.empty((T, k), dtype=f32, device=dev)
        self.ws = ops.workspace(T, E, k, R, dedup, dev)
        self.cnt = {"expert_counts": torch.empty(E, dtype=i32, device=dev),
                    "rank_counts": torch.empty(R, dtype=i32, device=dev),
                    "rank_offsets": torch.empty(R + 1, dtype=i32, device=dev)}
        if not dedup:
            self.cnt["expert_offsets"] = torch.empty(E, dtype=i32, device=dev)
        self.disp = {"send": torch.empty((N, H), dtype=rdt, device=dev),
                     "row_token": torch.empty(N, dtype=i32, device=dev),
                     "row_weight": torch.empty(N, dtype=f32, device=dev),
                     "slot_row": torch.empty((T, k), dtype=i32, device=dev)}
        if dedup:
            self.disp.update(row_experts=torch.empty((N, k), dtype=i32, device=dev),
                             row_gates=torch.empty((N, k), dtype=f32, device=dev),
                             n_rows=torch.empty(1, dtype=i32, device=dev))
        else:
            self.disp["row_expert"] = torch.empty(N, dtype=i32, device=dev)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        self.W = torch.zeros((E, E), dtype=i32, device=dev)
        if receive:  # the received rows are this set's dedup send buffer (capacity N)
            self.ews = ops.expand_workspace(N, E, k, R, dev)
            self.ecnt = {"expert_counts": torch.empty(E, dtype=i32, device=dev),
                         "rank_counts": torch.empty(R, dtype=i32, device=dev),
                         "rank_offsets": torch.empty(R + 1, dtype=i32, device=dev),
                         "expert_offsets": torch.empty(E, dtype=i32, device=dev)}
            self.exp = {"expanded": torch.empty((N, H), dtype=rdt, device=dev),
                        "exp_row": torch.empty(N, dtype=i32, device=dev),
                        "exp_expert": torch.empty(N, dtype=i32, device=dev),
                        "exp_gate": torch.empty(N, dtype=f32, device=dev),
                        "row_slot": torch.empty((N, k), dtype=i32, device=dev)}
            self.red = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
        self.ev_routed = torch.cuda.Event()
        self.ev_coselected = torch.cuda.Event()

    def nbytes(self):
        tot = 0
        for v in vars(self).values():
            if hasattr(v, "element_size"):
                tot += v.numel() * v.element_size()
            elif isinstance(v, dict):
                tot += sum(t.numel() * t.element_size() for t in v.values())
        return tot


def routed_of(b, w, dedup):
    """Buffer set b's routed batch as moe_dispatch_routed takes it."""
    return {"topk_idx": b.idx, "topk_gate": b.gate, "ws": b.ws, "n_experts": w.n_experts,
            "n_ranks": w.n_ranks, "placement": b.place, "dedup": dedup}


def gpu_step(torch, ops, b, w, dedup, side=None, receive=False, fused=True, cs_in="dispatch",
             one_call=False, nb=None):
    """One pass of the hot path.  one_call: moe_route_dispatch (with the
    co-selection counts), then the rest.  nb (pipelined): set b was routed by
    the previous step; moe_dispatch_routed, the rest, and a combine that also
    routes buffer set nb (moe_combine_route).  Otherwise the co-selection counts go
    with the dispatch (cs_in "dispatch") or the routing ("route") call, or with
    a side stream they run there, after the routing and concurrently with the
    rest.  With `receive` (dedup mode), the dedup rows are expanded per expert,
    passed through identity experts, reduced back to one row per received row,
    and those rows are combined with weight 1."""
    E, k, R = w.n_experts, w.top_k, w.n_ranks
    main = torch.cuda.current_stream()
    cs_route = side is None and cs_in == "route"
    cs_disp = side is None and cs_in == "dispatch"
    nxt = None
    if nb is not None:
        d = ops.moe_dispatch_routed(b.x, routed_of(b, w, dedup), out={**b.cnt, **b.disp},
                                    coselect=b.W, coselect_tokens=w.coselect_tokens)[1]
        nxt = {"topk_idx": nb.idx, "topk_gate": nb.gate, "ws": nb.ws}
    elif one_call:
        d = ops.moe_route_dispatch(b.logits, b.x, k, R, b.place, dedup,
                                   out={"topk_idx": b.idx, "topk_gate": b.gate, **b.cnt,
                                        **b.disp},
                                   ws=b.ws, coselect=b.W, coselect_tokens=w.coselect_tokens)[3]
    elif fused:
        c = ops.moe_route_plan(b.logits, k, R, b.place, dedup, topk_idx=b.idx, topk_gate=b.gate,
                               ws=b.ws, out=b.cnt, coselect=b.W if cs_route else None,
                               coselect_tokens=w.coselect_tokens)[2]
    else:
        ops.moe_route_topk(b.logits, k, b.idx, b.gate)
    if side is not None:
        b.ev_routed.record(main)
        side.wait_event(b.ev_routed)
        ops.moe_coselect_counts(b.idx, E, tokens=w.coselect_tokens, coselect=b.W,
                                stream=side)
        b.ev_coselected.record(side)
    if not fused and not one_call:
        c = ops.moe_send_counts(b.idx, E, R, b.place, dedup, ws=b.ws, out=b.cnt)
    if not one_call and nb is None:
        f = ops.moe_dispatch_permute_dedup if dedup else ops.moe_dispatch_permute
        d = f(b.x, b.idx, b.gate, E, R, c["ws"], out=b.disp, coselect=b.W if cs_disp else None,
              coselect_tokens=w.coselect_tokens)
    if receive:
        ops.moe_expand_counts(d["row_experts"], d["n_rows"], E, R, b.place, ws=b.ews, out=b.ecnt)
        ex = ops.moe_expand_permute(d["send"], d["row_gates"], d["n_rows"], E, R, b.ews,
                                    out=b.exp)
        red = ops.moe_expand_reduce(ex["expanded"], ex["exp_gate"], ex["row_slot"], d["n_rows"],
                                    out=b.red)
        rows, weight = red, None
    else:
        rows, weight = d["send"], d["row_weight"]
    if nb is not None:
        ops.moe_combine_route(rows, weight, d["slot_row"], nb.logits, k, R, nb.place, dedup,
                              out=b.out, next_out=nxt)
    else:
        ops.moe_combine(rows, weight, d["slot_row"], out=b.out)
    if side is not None:
        main.wait_event(b.ev_coselected)
    elif cs_route and not fused and not one_call:
        ops.moe_coselect_counts(b.idx, E, tokens=w.coselect_tokens, coselect=b.W)


def prepare_sets(torch, ops, sets, w, dedup, receive):
    """One whole step (the one-call path) on every buffer set before anything
    is timed: the per-kernel runs and the reference kernels read any set's
    plan, positions and rows, also those of sets that no timed step reaches in
    a short run, whose buffers would otherwise be uninitialised."""
    for b in sets:
        gpu_step(torch, ops, b, w, dedup, None, receive, True, "dispatch", True)
    torch.cuda.synchronize()


def algorithmic_bytes(T, H, E, k, bpe, n_rows, dedup, n_exp=None):
    """Bytes the method must move (each input read once, each output written
    once) for one step of T tokens, hidden H, E experts, top-k, rows of bpe
    bytes per element, n_rows rows sent (T*k, or D for dedup) and, on the
    receive side, n_exp expanded rows (None: no receive side).
      dispatch  read x once, write each sent row once
      combine   the send-side combine: read each sent row once, write out once
                (bf16)
      metadata  per sent row its token, expert(s), gate(s) and weight; per
                token-slot its row
      route     logits in, ids and gates out
      expand    read each received row once, write each expanded copy
      reduce    read each expert output once, write one bf16 row per received
                row
      job       everything a step moves; with a receive side the step's combine
                reads the reduced bf16 rows instead of the sent rows"""
    row_bytes = H * bpe
    out_bytes = H * 2
    res = {"dispatch": row_bytes * (T + n_rows),
           "combine": row_bytes * n_rows + out_bytes * T,
           "metadata": n_rows * (12 if not dedup else 8 + 8 * k) + T * k * 4,
           "route": T * E * 4 + T * k * 8}
    if n_exp is None:
        res["job"] = res["dispatch"] + res["combine"] + res["metadata"] + res["route"]
        return res
    res["expand"] = row_bytes * (n_rows + n_exp)
    res["reduce"] = row_bytes * n_exp + out_bytes * n_rows
    step_combine = out_bytes * n_rows + out_bytes * T
    res["job"] = (res["dispatch"] + step_combine + res["metadata"] + res["route"] +
                  res["expand"] + res["reduce"])
    return res


def sources_digest(kernel, pkg=PKG):
    """First 16 hex digits of the SHA-256 of the files that hold `kernel`'s
    code (KERNEL_SOURCES, then COMMON_SOURCES)."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel] + COMMON_SOURCES:
        with open(os.path.join(pkg, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic(kernel, workload, mode, dtype="bf16"):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summaries (FETCH_SIZE and WRITE_SIZE, each scaled by its plain-copy
    calibration), or None when there is none for this workload, dispatch mode
    and row type (a line without dtype= is bf16) or the kernel's sources have
    changed since the counters were taken."""
    import glob
    digest = sources_digest(kernel)
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "hbm_traffic_*.md"))):
        with open(path) as fh:
            for line in fh:
                if not line.startswith("traffic "):
                    continue
                kv = dict(t.split("=", 1) for t in line.split()[1:])
                if (kv.get("kernel"), kv.get("workload"), kv.get("dispatch"),
                        kv.get("dtype", "bf16"), kv.get("sources_sha256")) == \
                        (kernel, workload, mode, dtype, digest):
                    return int(kv["bytes"])
    return None


def raw_step_calls(torch, ops, b, w, dedup, receive, bpe, side=None, fused=True, stream=None,
                   cs_in="dispatch", one_call=False, nb=None):
    """The C-ABI calls of one step on buffer set b, with every argument
    marshalled once: the timed loop then costs a few microseconds of host time
    per step instead of the Python binding's checks.  one_call: routing, plan,
    rows and co-selection counts through moe_route_dispatch.  nb (pipelined): the
    set that this step's combine launch routes for the next step.  With a side stream
    the co-selection counts run there, forked after the routing and joined at
    the end of the step (event record and wait entries return 0)."""
    L = ops.lib()
    T, H, E, k, R = w.tokens, w.hidden_dim, w.n_experts, w.top_k, w.n_ranks
    N = T * k
    st = (stream or torch.cuda.current_stream()).cuda_stream
    p = lambda t: None if t is None else t.data_ptr()
    c, d = b.cnt, b.disp
    cargs = (int(dedup), p(c["expert_counts"]), p(c["rank_counts"]), p(c["rank_offsets"]),
             p(c.get("expert_offsets")))
    wsargs = (p(b.ws), b.ws.numel(), st)
    ncs = w.coselect_tokens if side is None and cs_in == "route" else 0
    dcs = w.coselect_tokens if side is None and cs_in == "dispatch" else 0
    if nb is not None:
        rx = d["row_experts"] if dedup else d["row_expert"]
        calls = [(L.moe_dispatch_routed, (
            p(b.x), p(b.idx), p(b.gate), T, H, E, k, R, p(b.place), int(dedup), bpe, *cargs[1:],
            p(d["send"]), p(d["row_token"]), p(rx), p(d.get("row_gates")), p(d["row_weight"]),
            p(d["slot_row"]), p(d.get("n_rows")), w.coselect_tokens, p(b.W), *wsargs))]
    elif one_call:
        rx = d["row_experts"] if dedup else d["row_expert"]
        calls = [(L.moe_route_dispatch, (
            p(b.logits), p(b.x), T, H, E, k, 0, R, p(b.place), int(dedup), bpe, p(b.idx),
            p(b.gate), *cargs[1:], p(d["send"]), p(d["row_token"]), p(rx), p(d.get("row_gates")),
            p(d["row_weight"]), p(d["slot_row"]), p(d.get("n_rows")), w.coselect_tokens,
            p(b.W), *wsargs))]
    elif fused:
        calls = [(L.moe_route_plan, (p(b.logits), T, E, k, 0, R, p(b.place), *cargs[:1],
                                     p(b.idx), p(b.gate), *cargs[1:], ncs,
                                     p(b.W) if ncs else None, *wsargs))]
    else:
        calls = [(L.moe_route_topk, (p(b.logits), T, E, k, p(b.idx), p(b.gate), st))]
    if side is not None:
        main = torch.cuda.current_stream()

        def fork():
            b.ev_routed.record(main)
            side.wait_event(b.ev_routed)
            return L.moe_coselect_counts(p(b.idx), w.coselect_tokens, E, k, p(b.W),
                                         side.cuda_stream) or b.ev_coselected.record(side) or 0

        def join():
            main.wait_event(b.ev_coselected)
            return 0
        calls.append((fork, ()))
    if not fused and not one_call and nb is None:
        calls.append((L.moe_send_counts, (p(b.idx), T, E, k, R, p(b.place), *cargs, *wsargs)))
    if one_call or nb is not None:
        pass
    elif dedup:
        calls.append((L.moe_dispatch_permute_dedup, (
            p(b.x), p(b.idx), p(b.gate), T, H, E, k, R, bpe, p(b.ws), b.ws.numel(),
            p(d["send"]), p(d["row_token"]), p(d["row_experts"]), p(d["row_gates"]),
            p(d["row_weight"]), p(d["slot_row"]), p(d["n_rows"]), dcs,
            p(b.W) if dcs else None, st)))
    else:
        calls.append((L.moe_dispatch_permute, (
            p(b.x), p(b.idx), p(b.gate), T, H, E, k, R, bpe, p(b.ws), b.ws.numel(),
            p(d["send"]), p(d["row_token"]), p(d["row_expert"]), p(d["row_weight"]),
            p(d["slot_row"]), dcs, p(b.W) if dcs else None, st)))
    if receive:
        ec, x = b.ecnt, b.exp
        calls += [
            (L.moe_expand_counts, (p(d["row_experts"]), p(d["n_rows"]), N, E, k, R, p(b.place),
                                   p(ec["expert_counts"]), p(ec["rank_counts"]),
                                   p(ec["rank_offsets"]), p(ec["expert_offsets"]), p(b.ews),
                                   b.ews.numel(), st)),
            (L.moe_expand_permute, (p(d["send"]), p(d["row_gates"]),
                                    p(d["n_rows"]), N, H, E, k, R, bpe, p(b.ews), b.ews.numel(),
                                    p(x["expanded"]), N, p(x["exp_row"]), p(x["exp_expert"]),
                                    p(x["exp_gate"]), p(x["row_slot"]), st)),
            (L.moe_expand_reduce, (p(x["expanded"]), p(x["exp_gate"]), p(x["row_slot"]),
                                   p(d["n_rows"]), N, H, k, bpe, p(b.red), st))]
        comb = (p(b.red), None, p(d["slot_row"]), T, H, k, 2, p(b.out))
    else:
        comb = (p(d["send"]), p(d["row_weight"]), p(d["slot_row"]), T, H, k, bpe, p(b.out))
    if nb is not None:
        calls.append((L.moe_combine_route, (*comb, p(nb.logits), T, E, k, 0, R, p(nb.place),
                                            int(dedup), p(nb.idx), p(nb.gate), p(nb.ws),
                                            nb.ws.numel(), st)))
    else:
        calls.append((L.moe_combine, (*comb, st)))
    if side is not None:
        calls.append((join, ()))
    elif not fused and not one_call and ncs:
        calls.append((L.moe_coselect_counts, (p(b.idx), w.coselect_tokens, E, k, p(b.W), st)))
    return calls


def placement_leg(torch, ops, b, w):
    """Correlated placement from this workload's co-selection counts (first
    coselect_tokens tokens, counted on the GPU), then the dedup rows of all
    tokens under the contiguous, the workload's own and the searched placement
    (counted on the GPU).  Not part of the timed step."""
    E, k, R, T = w.n_experts, w.top_k, w.n_ranks, w.tokens
    dev = b.idx.device
    W = torch.zeros((E, E), dtype=torch.int32, device=dev)
    ops.moe_coselect_counts(b.idx, E, tokens=w.coselect_tokens, coselect=W)
    torch.cuda.synchronize()
    Wh = W.cpu()
    t0 = time.perf_counter()
    place, obj, swaps = ops.moe_placement_search(Wh, R)
    search_ms = (time.perf_counter() - t0) * 1e3
    contiguous = (torch.arange(E, dtype=torch.int32) // (E // R))
    cands = {"contiguous": contiguous, "searched": place}
    if b.place is not None:
        cands["workload"] = b.place.cpu()
    rows, objective = {}, {}
    for name, pl in cands.items():
        c = ops.moe_send_counts(b.idx, E, R, pl.to(dev), dedup=True)
        rows[name] = int(c["rank_offsets"][R].item())
        objective[name] = ops.moe_placement_search(Wh, R, initial=pl, max_swaps=0)[1]
    return {"fit_tokens": w.coselect_tokens, "search_ms": round(search_ms, 2), "swaps": swaps,
            "objective": objective, "dedup_rows": rows,
            "rows_removed_pct": {n: round(100.0 * (1 - r / (T * k)), 2) for n, r in rows.items()}}


def shuffle_leg(torch, ops, WL, w):
    """Token-shuffle planner: fit on a calibration batch of three consecutive
    layers (l-1, l, l+1) under the contiguous expert placement, plan an
    evaluation batch, and report the share of layer l+1 token-expert
    assignments served on the token's own rank: contiguous token ownership vs
    the planned owners.  Not part of the timed step; GPU times are HIP events
    around single launches queued behind a GPU sleep (no host time inside)."""
    E, k, R, T = w.n_experts, w.top_k, w.n_ranks, w.tokens
    dev = torch.device("cuda:0")

    def routes(seed):
        return [ops.moe_route_topk(torch.from_numpy(l).to(dev), k)[0]
                for l in WL.make_layer_logits(w, seed=seed)]

    cal, ev = routes(1), routes(2)
    pair = torch.zeros((E, E, R), dtype=torch.int32, device=dev)
    single = torch.zeros((E, R), dtype=torch.int32, device=dev)
    pl = torch.from_numpy(WL.contiguous_placement(E, R)).to(dev)
    ops.moe_shuffle_predict(ev[0], ev[1],                      # untimed first launches
                            *ops.moe_shuffle_fit(cal[0], cal[1], cal[2], E, R, pl), 8)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    torch.cuda.synchronize()
    torch.cuda._sleep(5_000_000)   # the launches queue up behind it
    e[0].record()
    ops.moe_shuffle_fit(cal[0], cal[1], cal[2], E, R, pl, pair, single)
    e[1].record()
    torch.cuda.synchronize()
    torch.cuda._sleep(5_000_000)
    e[2].record()
    scores = ops.moe_shuffle_predict(ev[0], ev[1], pair, single, 8)
    e[3].record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    owner = ops.moe_shuffle_assign(scores)
    assign_ms = (time.perf_counter() - t0) * 1e3
    served = pl.cpu()[ev[2].cpu().long()]                     # rank of each l+1 assignment
    base = (torch.arange(T) * R // T)[:, None]
    return {"fit_us": round(e[0].elapsed_time(e[1]) * 1e3, 2),
            "predict_us": round(e[2].elapsed_time(e[3]) * 1e3, 2),
            "assign_ms": round(assign_ms, 2),
            "locality_contiguous": round(float((served == base).float().mean()), 4),
            "locality_planned": round(float((served == owner[:, None]).float().mean()), 4)}


def cpu_baseline(inp, w, dedup, seconds, receive=False, fp8=False):
    """The CPU oracle as it stands (single host thread), on whole steps of the
    same workload, repeated until `seconds` have elapsed."""
    from oracle import oracle as O
    O.lib()
    steps = 0
    t0 = time.perf_counter()
    while True:
        idx, gate = O.route_topk(inp["logits"], w.top_k)
        f = O.dispatch_dedup if dedup else O.dispatch
        x = inp["x_fp8"] if fp8 else inp["x_bits"]
        comb = O.combine_fp8 if fp8 else O.combine
        d = f(x, idx, gate, w.n_experts, w.n_ranks, inp["placement"])
        if receive:
            ex = O.expand_dedup(d["send"], d["row_experts"], d["row_gates"], d["n_rows"],
                                w.n_experts, w.n_ranks, inp["placement"])
            red = comb(ex["expanded"], ex["exp_gate"], ex["row_slot"][:d["n_rows"]])
            O.combine(red, None, d["slot_row"])
        else:
            comb(d["send"], d["row_weight"], d["slot_row"])
        O.coselect(idx, w.n_experts, tokens=w.coselect_tokens)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": steps * w.tokens / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} whole steps of the same workload ({w.tokens} tokens each), "
                      f"{el:.1f} s on one host thread"}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {a.gpus}): destination ranks are "
              "logical partitions of one GPU's buffers; there is no multi-GPU path to time.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if a.calib_copy:
        calib_copy()
        return
    from combine_top_router_select_amd import ops
    from combine_top_router_select_amd import workloads as WL
    ops.lib()
    w = WL.get(a.workload)
    dedup = bool(a.dedup)
    receive = bool(a.receive)
    fused = not a.separate
    # routing, plan, rows and co-selection counts in one call (the default)
    # the default: each step's combine launch routes the stream's next batch;
    # --one-call: routing and dispatch of this batch in one call
    # (graph replay takes the one-call step)
    direct = fused and not a.plan_call and not a.overlap and a.coselect_in == "dispatch"
    pipelined = direct and not a.one_call and not a.graph
    one_call = direct and (bool(a.one_call) or bool(a.graph))
    if receive and not dedup:
        print("--receive needs --dedup (the receive side expands deduplicated rows)",
              file=sys.stderr)
        sys.exit(2)
    if dedup and "dedup" not in w.dispatch:
        print(f"warning: {w.name} is not normally run with dedup dispatch", file=sys.stderr)
    dev = torch.device("cuda:0")
    inp = WL.make_inputs(w)
    fp8 = bool(a.fp8)
    bpe = 1 if fp8 else 2
    if fp8:  # synthetic fp8 activations: the bf16 ones rounded to E4M3 on the host
        xb = torch.from_numpy(inp["x_bits"].view(np.int16)).view(torch.bfloat16)
        inp["x_fp8"] = xb.float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    T, H, E, k, R = w.tokens, w.hidden_dim, w.n_experts, w.top_k, w.n_ranks

    # streams: the timed setting and the other one timed after it (None: none);
    # two by default, one for receive-side steps of batches over 64 MiB
    many = not a.overlap and not a.step_events and not a.graph
    want = a.streams if a.streams else (2 if T * H * bpe <= 64 * 2 ** 20 else 1)
    n_streams = want if many else 1
    other_ns = (1 if n_streams > 1 else 2) if many else None

    first = BufferSet(torch, ops, inp, w, dedup, dev, receive, fp8)
    per_set = first.nbytes()
    nsets = max(2, int(np.ceil(a.footprint_gib * 2 ** 30 / per_set)))
    # each buffer set always on the same stream (steps i and i + nsets use one
    # set): a multiple of both stream counts, and two sets per stream at least
    m = int(np.lcm(n_streams, other_ns or 1))
    nsets = max(nsets, 2 * m)
    nsets = (nsets + m - 1) // m * m
    sets = [first] + [BufferSet(torch, ops, inp, w, dedup, dev, receive, fp8)
                      for _ in range(nsets - 1)]
    prepare_sets(torch, ops, sets, w, dedup, receive)

    side = torch.cuda.Stream() if a.overlap else None
    graphs = None
    if a.graph:
        graphs = []
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for b in sets:       # warm the code paths once outside capture
                gpu_step(torch, ops, b, w, dedup, side, receive, fused, a.coselect_in,
                         one_call)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for b in sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                gpu_step(torch, ops, b, w, dedup, side, receive, fused, a.coselect_in,
                         one_call)
            graphs.append(g)
        torch.cuda.synchronize()

    raw = raw_other = None
    if graphs is None:
        streams = [torch.cuda.current_stream()] + [torch.cuda.Stream() for _ in range(3)]

        # pipelined: step i's combine launch routes the set of step i + ns, the
        # next step on the same stream
        def raw_sets(ns):
            return [raw_step_calls(torch, ops, b, w, dedup, receive, bpe, side, fused,
                                   streams[i % ns], a.coselect_in, one_call,
                                   sets[(i + ns) % nsets] if pipelined else None)
                    for i, b in enumerate(sets)]
        raw = raw_sets(n_streams)
        if other_ns is not None:
            raw_other = raw_sets(other_ns)

    timed_kernels = ("moe_route_dispatch", "moe_dispatch_permute", "moe_dispatch_permute_dedup",
                     "moe_combine", "moe_dispatch_routed", "moe_combine_route",
                     "moe_expand_permute", "moe_expand_reduce")
    step_ev = {}   # (step, entry point) -> (start event, end event)
    if a.steps is None and a.step_events:
        a.steps = 200   # one event pair per launch: a fixed count
    ev_pool = ([torch.cuda.Event(enable_timing=True) for _ in range(8 * a.steps + 8)]
               if a.step_events else [])

    def step(i, events=False):
        if graphs is not None:
            graphs[i % nsets].replay()
        elif raw is not None:
            for fn, args in raw[i % nsets]:
                name = getattr(fn, "__name__", "")
                ev = None
                if events and name in timed_kernels:
                    ev = step_ev[(i, name)] = (ev_pool.pop(), ev_pool.pop())
                    ev[0].record()
                rc = fn(*args)
                if ev is not None:
                    ev[1].record()
                if rc != 0:
                    raise ops.MoeError(rc, name)
        else:
            gpu_step(torch, ops, sets[i % nsets], w, dedup, side, receive, fused, a.coselect_in,
                     one_call, sets[(i + n_streams) % nsets] if pipelined else None)

    if pipelined:   # every set holds a routed batch before its first dispatch
        for b in sets:
            ops.moe_combine_route(None, None, None, b.logits, k, R, b.place, dedup,
                                  next_out={"topk_idx": b.idx, "topk_gate": b.gate, "ws": b.ws})
        torch.cuda.synchronize()
    for i in range(a.warmup):
        if i == 0 and graphs is None:   # once through the Python binding, with its checks
            gpu_step(torch, ops, sets[0], w, dedup, side, receive, fused, a.coselect_in,
                     one_call, sets[n_streams % nsets] if pipelined else None)
        else:
            step(i)
    torch.cuda.synchronize()
    # without --steps: as many steps as fill about 2 s, from the time of 50
    # untimed ones (counted with the warm-up); a long timed region leaves out
    # the start and the end of the launch queue
    pilot = 0
    if a.steps is None:
        pilot = 50
        p0 = time.perf_counter()
        for i in range(pilot):
            step(a.warmup + i)
        torch.cuda.synchronize()
        t_est = (time.perf_counter() - p0) / pilot
        a.steps = int(min(100000, max(200, round(2.0 / t_est))))
    a.warmup += pilot
    # timed region: exactly K steps, synchronised on both sides
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(a.warmup + i, a.step_events)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    other = None
    if raw_other is not None:   # the same K steps with the other stream setting
        raw, raw_main = raw_other, raw
        for i in range(a.warmup):
            step(i)
        torch.cuda.synchronize()
        u0 = time.perf_counter()
        for i in range(a.steps):
            step(a.warmup + i)
        torch.cuda.synchronize()
        other = {"streams": other_ns,
                 "ms_per_step": (time.perf_counter() - u0) / a.steps * 1e3}
        raw = raw_main
    in_step = {}
    for (i, name), (e0, e1) in step_ev.items():
        in_step.setdefault(name, []).append(e0.elapsed_time(e1) * 1e-3)
    in_step = {n: round(float(np.mean(v)) * 1e6, 2) for n, v in in_step.items()}

    # Per-kernel mean durations with HIP events on the stream the kernels run
    # on: each event pair brackets a run of back-to-back launches of that one
    # kernel over the rotated buffer sets (each set holds the plan and the send
    # buffer of its last step), so neither event overhead nor other kernels
    # enter the figure.
    K2 = min(a.steps, 100)
    order = [sets[(a.warmup + a.steps + i) % nsets] for i in range(K2)]
    L, st = ops.lib(), torch.cuda.current_stream().cuda_stream
    disp_calls, comb_calls = [], []
    dcs = w.coselect_tokens if side is None and a.coselect_in == "dispatch" else 0
    for b in order:
        d = b.disp
        wp = b.W.data_ptr() if dcs else None
        if dedup:
            disp_calls.append((L.moe_dispatch_permute_dedup, (
                b.x.data_ptr(), b.idx.data_ptr(), b.gate.data_ptr(), T, H, E, k, R, bpe,
                b.ws.data_ptr(), b.ws.numel(), d["send"].data_ptr(), d["row_token"].data_ptr(),
                d["row_experts"].data_ptr(), d["row_gates"].data_ptr(),
                d["row_weight"].data_ptr(), d["slot_row"].data_ptr(), d["n_rows"].data_ptr(),
                dcs, wp, st)))
        else:
            disp_calls.append((L.moe_dispatch_permute, (
                b.x.data_ptr(), b.idx.data_ptr(), b.gate.data_ptr(), T, H, E, k, R, bpe,
                b.ws.data_ptr(), b.ws.numel(), d["send"].data_ptr(), d["row_token"].data_ptr(),
                d["row_expert"].data_ptr(), d["row_weight"].data_ptr(),
                d["slot_row"].data_ptr(), dcs, wp, st)))
        comb_calls.append((L.moe_combine, (
            d["send"].data_ptr(), d["row_weight"].data_ptr(), d["slot_row"].data_ptr(), T, H, k,
            bpe, b.out.data_ptr(), st)))
    exp_calls, red_calls = [], []
    if receive:
        N = T * k
        for b in order:
            d, x = b.disp, b.exp
            exp_calls.append((L.moe_expand_permute, (
                d["send"].data_ptr(), d["row_gates"].data_ptr(),
                d["n_rows"].data_ptr(), N, H, E, k, R, bpe, b.ews.data_ptr(), b.ews.numel(),
                x["expanded"].data_ptr(), N, x["exp_row"].data_ptr(), x["exp_expert"].data_ptr(),
                x["exp_gate"].data_ptr(), x["row_slot"].data_ptr(), st)))
            red_calls.append((L.moe_expand_reduce, (
                x["expanded"].data_ptr(), x["exp_gate"].data_ptr(), x["row_slot"].data_ptr(),
                d["n_rows"].data_ptr(), N, H, k, bpe, b.red.data_ptr(), st)))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
    runs = [(disp_calls, ev[0], ev[1]), (comb_calls, ev[2], ev[3])]
    if receive:
        runs += [(exp_calls, ev[4], ev[5]), (red_calls, ev[6], ev[7])]
    for calls, e0, e1 in runs:
        torch.cuda.synchronize()
        torch.cuda._sleep(20_000_000)  # the GPU waits while the launches queue up
        e0.record()
        for fn, args in calls:
            rc = fn(*args)
            if rc != 0:
                raise ops.MoeError(rc, fn.__name__)
        e1.record()
    torch.cuda.synchronize()
    t_disp = ev[0].elapsed_time(ev[1]) * 1e-3 / K2
    t_comb = ev[2].elapsed_time(ev[3]) * 1e-3 / K2
    t_exp = ev[4].elapsed_time(ev[5]) * 1e-3 / K2 if receive else None
    t_red = ev[6].elapsed_time(ev[7]) * 1e-3 / K2 if receive else None

    # rows actually written (N, or D for dedup)
    b = sets[0]
    n_rows = int(b.cnt["rank_offsets"][R].item())
    n_exp = int(b.ecnt["rank_offsets"][R].item()) if receive else None
    ab = algorithmic_bytes(T, H, E, k, bpe, n_rows, dedup, n_exp)
    disp_bytes, comb_bytes = ab["dispatch"], ab["combine"]
    meta_bytes = ab["metadata"]
    dom = ("moe_dispatch_permute" + ("_dedup" if dedup else ""), t_disp, disp_bytes)
    if t_comb > t_disp:
        dom = ("moe_combine", t_comb, comb_bytes)
    achieved = dom[2] / dom[1] / 1e9
    dc_gbps = (disp_bytes + comb_bytes) / (t_disp + t_comb) / 1e9
    recv = None
    job_bytes = ab["job"]
    mode, dt = ("dedup" if dedup else "nondedup"), ("fp8" if fp8 else "bf16")
    if receive:
        exp_bytes, red_bytes = ab["expand"], ab["reduce"]
        recv = {"expanded_rows": n_exp,
                "expand_us": round(t_exp * 1e6, 2), "reduce_us": round(t_red * 1e6, 2),
                "expand_GBps": round(exp_bytes / t_exp / 1e9, 1),
                "reduce_GBps": round(red_bytes / t_red / 1e9, 1),
                "algorithmic_bytes": {"expand": exp_bytes, "reduce": red_bytes},
                "traffic": {"expand": counter_traffic("moe_expand_permute", w.name, mode, dt),
                            "reduce": counter_traffic("moe_expand_reduce", w.name, mode, dt)}}

    res = {
        "metric": METRIC,
        "value": T * a.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": elapsed / a.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": T, "hidden_dim": H, "n_experts": E,
                   "top_k": k, "n_ranks": R, "placement": w.placement,
                   "dispatch": "dedup" if dedup else "nondedup", "receive_side": receive,
                   "routing": ("pipelined" if pipelined else "one_call" if one_call
                               else ("fused" if fused else "separate")),
                   "bytes_per_element": bpe, "graph": bool(a.graph),
                   "coselect": "side_stream" if a.overlap else a.coselect_in + "_call",
                   "streams": n_streams,
                   "buffer_sets": nsets, "footprint_MiB": round(nsets * per_set / 2 ** 20)},
        "roofline": {"bound": "hbm", "kernel": dom[0], "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": counter_traffic(dom[0], w.name, mode, dt),
                     "algorithmic_bytes": dom[2]},
        "dispatch_us": round(t_disp * 1e6, 2),
        "in_step_event_us": in_step or None,
        "other_streams": other,
        "combine_us": round(t_comb * 1e6, 2),
        "dispatch_combine_tokens_per_s": T / (t_disp + t_comb),
        "dispatch_combine_GBps": round(dc_gbps, 1),
        # whole job: every algorithmic byte of a step (logits, ids, rows, metadata,
        # and with --receive the receive side) over the measured step time
        "job_GBps": round(job_bytes / (elapsed / a.steps) / 1e9, 1),
        "job_hbm_frac": round(job_bytes / (elapsed / a.steps) / 1e9 / HBM_PEAK_GBPS, 4),
        "dispatch_combine_hbm_frac": round(dc_gbps / HBM_PEAK_GBPS, 4),
        "rows": n_rows,
        "rows_removed_by_dedup_pct": round(100.0 * (1 - n_rows / (T * k)), 2) if dedup else 0.0,
        # rows that stay on source rank 0 (the diagonal of the send matrix)
        "self_rank_share": round(int(b.cnt["rank_counts"][0].item()) / n_rows, 4),
        "algorithmic_bytes": {"dispatch": disp_bytes, "combine": comb_bytes,
                              "metadata": meta_bytes},
        "copy_reference": None if a.no_reference else copy_reference(torch, dom[2]),
        "device": device_info(torch),
        "hip_version": getattr(torch.version, "hip", None),
        "host_cores_available": len(os.sched_getaffinity(0)),
    }
    if not a.no_reference:
        ceil = hbm_ceiling(torch, sets, T, H, k, bpe, n_rows, dedup)
        # the dispatch's achieved rate as a fraction of each reference rate
        disp_gbps = disp_bytes / t_disp / 1e9
        ceil["dispatch_frac_of"] = {name: round(disp_gbps / v["GBps"], 4)
                                    for name, v in ceil.items()
                                    if v is not None and name != "gather_sum"}
        if ceil["gather_sum"] is not None:   # the combine against its own data movement
            ceil["combine_frac_of_gather_sum"] = round(
                comb_bytes / t_comb / 1e9 / ceil["gather_sum"]["GBps"], 4)
        res["hbm_ceiling"] = ceil
    if recv is not None:
        res["receive"] = recv
    if a.search:
        res["placement_search"] = placement_leg(torch, ops, sets[0], w)
    if a.shuffle:
        res["token_shuffle"] = shuffle_leg(torch, ops, WL, w)
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, w, dedup, a.cpu_seconds, receive, fp8)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
