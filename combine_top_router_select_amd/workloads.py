"""Seeded synthetic workloads for per-GPU MoE dispatch/combine.

This module only draws inputs: router logits, bf16 activations and an
expert->rank placement table.  It contains none of the method's arithmetic
(no top-k, no counting, no packing, no combining), so both the HIP path and
the CPU oracle can be fed from it without sharing any of the computation.

Shapes and statistics follow the pages, not their data (which is not
available here):

* DeepSeek-MoE-16B and Qwen3-30B-A3B rows of the DODOCO model table (E, top-k,
  hidden size); 4096 routed tokens per rank, expert parallelism 16 and
  contiguous placement from its "Setup" section.
* Two further rows of the DODOCO model table as plain shapes: 256 experts,
  top-8, hidden 2048, and 128 experts, top-6, hidden 2688 (the hybrid
  Mamba-2 + attention row), with the same 4096 tokens, EP16 and contiguous
  placement.
* Zyphra's expert-coupling summary, "Model Configuration" (d_model 4096, 128
  experts, top-2/top-6, sequence length 8192), "Hardware"/"Measured A2A share"
  (EP8, EP32) and "Within-layer correlation" (42% of tokens on 64 pairs, 14
  pairs at >= 50% confidence carrying 16%).

Randomness: numpy PCG64 streams from ``SeedSequence(seed).spawn(6)`` in the
fixed order x, logits, pairs, planted tokens, placement, Zipf permutation.
Activations are N(0,1) fp32 rounded to bf16 (round to nearest even, done by
torch's CPU conversion) and stored as uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "make_inputs", "make_custom_inputs",
           "bf16_bits_from_f32", "contiguous_placement", "make_layer_logits", "random_placement"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    tokens: int
    hidden_dim: int
    n_experts: int
    top_k: int
    n_ranks: int
    placement: str          # "contiguous" | "correlated"
    recipe: str             # "plain" | "pair_bias" | "zipf" | "zyphra"
    dispatch: tuple         # dispatch modes this workload is run with
    coselect_tokens: int    # tokens accumulated into the co-selection counts (0 = none)
    bytes_per_element: int = 2
    seed: int = 0


# The five seeded workloads (names are what they are, with their sizes).
WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 256, 128, 8, 2, 4, "contiguous", "plain",
                     ("nondedup",), 256),
    "deepseek_moe_16b": Workload("deepseek_moe_16b", 4096, 2048, 64, 6, 16,
                                 "contiguous", "pair_bias", ("nondedup", "dedup"), 4096),
    "qwen3_30b_a3b": Workload("qwen3_30b_a3b", 4096, 2048, 128, 8, 16, "contiguous",
                              "zipf", ("nondedup", "dedup"), 4096),
    "e256_top8_h2048": Workload("e256_top8_h2048", 4096, 2048, 256, 8, 16, "contiguous",
                                "zipf", ("nondedup", "dedup"), 4096),
    "e128_top6_h2688": Workload("e128_top6_h2688", 4096, 2688, 128, 6, 16, "contiguous",
                                "plain", ("nondedup", "dedup"), 4096),
    "zyphra_top2_ep8": Workload("zyphra_top2_ep8", 16384, 4096, 128, 2, 8, "correlated",
                                "zyphra", ("dedup",), 4096),
    "zyphra_top6_ep32": Workload("zyphra_top6_ep32", 16384, 4096, 128, 6, 32, "correlated",
                                 "zyphra", ("dedup",), 4096),
}

ORDER: List[str] = list(WORKLOADS)


def get(name: str) -> Workload:
    return WORKLOADS[name]


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even) bit patterns, via torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def contiguous_placement(n_experts: int, n_ranks: int) -> np.ndarray:
    """Rank r holds experts r*E/R .. (r+1)*E/R-1 (DODOCO "Setup")."""
    m = n_experts // n_ranks
    return (np.arange(n_experts, dtype=np.int32) // m).astype(np.int32)


def _pair_from_index(i: int, n: int):
    """i-th unordered pair (a<b) of range(n) in lexicographic order."""
    a = 0
    while i >= n - 1 - a:
        i -= n - 1 - a
        a += 1
    return a, a + 1 + i


def make_inputs(w: Workload, seed: Optional[int] = None, with_x: bool = True) -> dict:
    """Draw the inputs of workload ``w``.

    Returns a dict with
      x_bits     uint16 [T][H]  bf16 activations (absent if with_x is False)
      logits     float32 [T][E]
      placement  int32 [E] or None (None = contiguous, the library default)
      placement_array int32 [E] (always materialised)
      planted    dict describing planted pairs (for generator statistics)
    """
    seed = w.seed if seed is None else seed
    ss = np.random.SeedSequence(seed)
    s_x, s_logits, s_pairs, s_planted, s_place, s_zipf = ss.spawn(6)
    T, H, E, k, R = w.tokens, w.hidden_dim, w.n_experts, w.top_k, w.n_ranks
    out: dict = {}
    if with_x:
        gx = np.random.Generator(np.random.PCG64(s_x))
        out["x_bits"] = bf16_bits_from_f32(gx.standard_normal((T, H), dtype=np.float32))
    gl = np.random.Generator(np.random.PCG64(s_logits))
    logits = gl.standard_normal((T, E), dtype=np.float32)
    planted = {}
    placement = None
    if w.recipe == "pair_bias":
        # +3.0 on both experts of one of 64 seeded distinct pairs, for 40% of tokens.
        gp = np.random.Generator(np.random.PCG64(s_pairs))
        npairs = E * (E - 1) // 2
        pidx = gp.choice(npairs, size=64, replace=False)
        pairs = np.array([_pair_from_index(int(i), E) for i in pidx], dtype=np.int32)
        gt = np.random.Generator(np.random.PCG64(s_planted))
        perm = gt.permutation(T)
        n_pl = int(round(0.4 * T))
        toks = np.sort(perm[:n_pl])
        which = gt.integers(0, 64, size=n_pl)
        logits[toks, pairs[which, 0]] += np.float32(3.0)
        logits[toks, pairs[which, 1]] += np.float32(3.0)
        planted = {"pairs": pairs, "tokens": toks, "which": which, "bias": 3.0}
    elif w.recipe == "zipf":
        # Expert popularity ~ Zipf(1.1) over a seeded permutation of the experts,
        # applied as a log-probability bias on the logits.
        gz = np.random.Generator(np.random.PCG64(s_zipf))
        pi = gz.permutation(E)
        bias = (-1.1 * np.log(pi.astype(np.float64) + 1.0)).astype(np.float32)
        logits += bias[None, :]
        planted = {"zipf_rank": pi, "bias": bias}
    elif w.recipe == "zyphra":
        # 64 planted pairs form a perfect matching of a permuted expert list;
        # 14 "strong" pairs take 16% of tokens, 50 "weak" pairs take 26% (42% in all).
        assert E == 128
        gp = np.random.Generator(np.random.PCG64(s_pairs))
        pi = gp.permutation(E)
        pairs = np.stack([pi[0::2], pi[1::2]], axis=1).astype(np.int32)  # [64][2]
        gt = np.random.Generator(np.random.PCG64(s_planted))
        perm = gt.permutation(T)
        n_strong = int(round(0.16 * T))
        n_weak = int(round(0.26 * T))
        strong_t = perm[:n_strong]
        weak_t = perm[n_strong:n_strong + n_weak]
        strong_w = gt.integers(0, 14, size=n_strong)
        weak_w = 14 + gt.integers(0, 50, size=n_weak)
        toks = np.concatenate([strong_t, weak_t])
        which = np.concatenate([strong_w, weak_w])
        logits[toks, pairs[which, 0]] += np.float32(6.0)
        logits[toks, pairs[which, 1]] += np.float32(6.0)
        planted = {"pairs": pairs, "tokens": toks, "which": which, "bias": 6.0,
                   "n_strong_pairs": 14}
        # Correlated placement: shuffle the pairs, give each rank whole pairs.
        gpl = np.random.Generator(np.random.PCG64(s_place))
        order = gpl.permutation(64)
        per_rank = (E // R) // 2
        placement = np.empty(E, dtype=np.int32)
        for slot, p in enumerate(order):
            r = slot // per_rank
            placement[pairs[p, 0]] = r
            placement[pairs[p, 1]] = r
    elif w.recipe != "plain":
        raise ValueError(w.recipe)
    if w.placement == "correlated":
        assert placement is not None
    out["logits"] = logits
    out["placement"] = placement
    out["placement_array"] = (placement if placement is not None
                              else contiguous_placement(E, R))
    out["planted"] = planted
    return out


def make_custom_inputs(tokens: int, hidden_dim: int, n_experts: int, seed: int = 0,
                       logit_values: Optional[np.ndarray] = None) -> dict:
    """Plain N(0,1) inputs of any shape (edge cases: ragged T, tiny T, ...).

    If ``logit_values`` is given, logits are drawn uniformly from that small
    set instead (dense ties, signed zeros)."""
    ss = np.random.SeedSequence(seed)
    s_x, s_logits = ss.spawn(2)
    gx = np.random.Generator(np.random.PCG64(s_x))
    gl = np.random.Generator(np.random.PCG64(s_logits))
    x = bf16_bits_from_f32(gx.standard_normal((tokens, hidden_dim), dtype=np.float32))
    if logit_values is None:
        logits = gl.standard_normal((tokens, n_experts), dtype=np.float32)
    else:
        vals = np.asarray(logit_values, dtype=np.float32)
        logits = vals[gl.integers(0, len(vals), size=(tokens, n_experts))]
    return {"x_bits": x, "logits": np.ascontiguousarray(logits, dtype=np.float32)}


def make_layer_logits(w: Workload, n_layers: int = 3, seed: int = 1,
                      path_share: float = 0.6, boost: float = 4.0) -> List[np.ndarray]:
    """Router logits of `n_layers` consecutive MoE layers with cross-layer
    correlation (Expert Coupling summary, "Key Theoretical Insight": the
    experts a token selects at one layer predict its experts at the next).

    E seeded expert paths are drawn, one expert per layer each, every expert on
    exactly one path at every layer (a permutation per layer); a `path_share` of
    the tokens each follows one path, uniformly chosen, and gets `boost` added
    to its path's expert at every layer.  The correlation comes from the shared
    latent path only: nothing here routes tokens.  The paths depend on the
    workload only; `seed` picks the batch (which tokens follow which path, and
    the noise), so a calibration batch and an evaluation batch share them."""
    # the paths are the model's (fixed by the workload's seed); the tokens and
    # the noise are the batch's (`seed`), so two batches share the structure
    s_paths = np.random.SeedSequence([w.seed, 0x9A7E])
    s_tok, *s_layers = np.random.SeedSequence([w.seed, seed]).spawn(1 + n_layers)
    T, E = w.tokens, w.n_experts
    gp = np.random.Generator(np.random.PCG64(s_paths))
    paths = np.stack([gp.permutation(E) for _ in range(n_layers)], axis=1)
    gt = np.random.Generator(np.random.PCG64(s_tok))
    follows = gt.random(T) < path_share
    which = gt.integers(0, E, size=T)
    out = []
    for layer in range(n_layers):
        g = np.random.Generator(np.random.PCG64(s_layers[layer]))
        lg = g.standard_normal((T, E), dtype=np.float32)
        toks = np.nonzero(follows)[0]
        lg[toks, paths[which[toks], layer]] += np.float32(boost)
        out.append(lg)
    return out


def random_placement(n_experts: int, n_ranks: int, seed: int) -> np.ndarray:
    """A seeded placement holding exactly E/R experts per rank."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    m = n_experts // n_ranks
    perm = g.permutation(n_experts)
    place = np.empty(n_experts, dtype=np.int32)
    place[perm] = np.arange(n_experts) // m
    return place

