"""Configuration search for the adapter down-projection (the SGMV operator).

"Efficient multi-tenant LoRA serving via SGMV-specific operator autotuning" (abstract) organises
the construction space of the SGMV operator as a graph and selects tiling, caching and
virtual-thread scheduling configurations with a hardware-aware Markov-style stochastic search,
used as a practical heuristic rather than a guarantee of optimality.  Here, for the gfx950
down-projection (``lora_shrink_configured``):

* nodes -- configurations ``(TG, JP, U, M, ORD)``:
    TG  in {0, 1, 2, 4}  tiling: token tiles of 16 per inner step on bf16 MFMA; 0 is the
                         wave-reduction kernel (BGMV: fp32 lane products, shuffle and LDS sums)
    JP  in {1, 2, 4}     tiling: rank tiles of 16 per workgroup item
    U   in {1, 2}        caching: 64-wide k-steps held per register prefetch buffer
    M   in {1, 2, 4}     scheduling: inner steps per item (TBLK = 16 TG M tokens of a segment);
                         for TG = 0 the positions of a segment per item (TBLK = M)
    ORD in {0, 1}        scheduling: items in workgroup-id order, or a contiguous run per XCD
* edges -- two configurations differing in one parameter by one step of its ordered domain;
* hardware awareness -- a node is kept only if its compiled instance spills no registers to
  scratch memory and needs no more LDS than a workgroup may have (the instance's resources
  are read from the runtime), and, for the shape, if an item's token block is no longer
  than a useful multiple of the batch;
* search -- a Metropolis walk: from the current node propose a uniformly chosen neighbour,
  accept it with probability min(1, exp(-(c' - c) / (tau c))) on the measured cost c; the best
  node seen is the result.  Costs are cached, so a revisit costs nothing.

Every MFMA configuration computes the same sums in the same order (the four waves of a
workgroup split K the same way whatever the tile shape), so t is bitwise the same for all of
them; the wave-reduction kernel sums in another order (t within fp32 rounding).
"""

from __future__ import annotations

import math
import random
from dataclasses import dataclass, field

DOMAINS = {"TG": (0, 1, 2, 4), "JP": (1, 2, 4), "U": (1, 2), "M": (1, 2, 4), "ORD": (0, 1)}
KEYS = ("TG", "JP", "U", "M", "ORD")
LDS_LIMIT = 64 * 1024


def space():
    """Every node of the configuration graph (before pruning)."""
    nodes = [()]
    for k in KEYS:
        nodes = [n + (v,) for n in nodes for v in DOMAINS[k]]
    return nodes


def neighbours(node):
    """Nodes that differ from ``node`` in one parameter by one step of its domain."""
    out = []
    for i, k in enumerate(KEYS):
        dom = DOMAINS[k]
        j = dom.index(node[i])
        for jj in (j - 1, j + 1):
            if 0 <= jj < len(dom):
                out.append(node[:i] + (dom[jj],) + node[i + 1:])
    return out


def to_config(node):
    """The int32[5] configuration of lora_shrink_configured for a node."""
    tg, jp, u, m, order = node
    return (tg, jp, u, m if tg == 0 else 16 * tg * m, order)


def feasible(node, info, T: int):
    """Hardware and shape constraints: a compiled instance (``info(tg, jp, u, m)`` is None
    otherwise) with no spill and LDS within a workgroup's share, and an item no longer than
    twice the batch (longer items only idle)."""
    tg, jp, u, m, _ = node
    r = info(tg, jp, u, m)
    if r is None or r["spill"] > 0 or r["lds"] > LDS_LIMIT:
        return False
    return m <= max(1, 2 * T) if tg == 0 else 16 * tg * m <= max(16, 2 * T)


def default_node(T: int):
    """The library's own choice for the standalone launch (the tile plan)."""
    if T <= 128:
        m = max(1, -(-T // 16))
        return (1, 4, 1, 4 if m > 2 else (2 if m > 1 else 1), 0)
    return (4, 2, 1, 1, 0)


@dataclass
class SearchResult:
    best: tuple
    best_cost: float
    start: tuple
    start_cost: float
    trace: list = field(default_factory=list)      # (step, proposed, cost, accepted)
    evaluated: dict = field(default_factory=dict)  # node -> cost


def metropolis(start, cost, nbrs, steps: int, tau: float = 0.05, seed: int = 0, allowed=None) -> SearchResult:
    """Markov-style stochastic search over a graph of configurations.

    ``cost(node)`` is measured once per node (cached); ``nbrs(node)`` lists the neighbours;
    ``allowed(node)`` prunes infeasible ones.  Acceptance: min(1, exp(-(c' - c) / (tau c))).
    """
    rng = random.Random(seed)
    cache = {}

    def c(n):
        if n not in cache:
            cache[n] = float(cost(n))
        return cache[n]

    cur = start
    cur_c = c(cur)
    res = SearchResult(best=cur, best_cost=cur_c, start=start, start_cost=cur_c)
    for step in range(steps):
        cand = [n for n in nbrs(cur) if allowed is None or allowed(n)]
        if not cand:
            break
        prop = cand[rng.randrange(len(cand))]
        pc = c(prop)
        accept = pc <= cur_c or rng.random() < math.exp(-(pc - cur_c) / (tau * cur_c))
        res.trace.append((step, prop, pc, accept))
        if accept:
            cur, cur_c = prop, pc
        if pc < res.best_cost:
            res.best, res.best_cost = prop, pc
    res.evaluated = dict(cache)
    return res


def tune_shrink(x, seg, ad, steps: int = 40, reps: int = 20, tau: float = 0.05, seed: int = 0) -> SearchResult:
    """Search the down-projection's configurations for these inputs on the current GPU.
    The cost of a node is the median over three batches of ``reps`` back-to-back launches,
    timed with HIP events on the launch stream (microseconds per launch)."""
    import torch
    from . import ops

    T = x.shape[0]
    t = torch.empty((T, ad.r_max), dtype=torch.float32, device=x.device)
    infos = {}

    def info(tg, jp, u, m):
        key = (tg, jp, u, m if tg == 0 else 0)
        if key not in infos:
            try:
                infos[key] = ops.shrink_config_info(tg, jp, u, nt=m)
            except Exception:  # not compiled
                infos[key] = None
        return infos[key]

    stream = torch.cuda.current_stream()

    def cost(node):
        cfg = to_config(node)
        ops.shrink_configured(x, seg, ad, cfg, t=t)   # warm
        times = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                ops.shrink_configured(x, seg, ad, cfg, t=t)
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3 / reps)
        return sorted(times)[1]

    start = default_node(T)
    return metropolis(start, cost, neighbours, steps, tau=tau, seed=seed,
                      allowed=lambda n: feasible(n, info, T))
