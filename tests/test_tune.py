"""The configuration search of the down-projection (precision_gemm_amd.tune) on synthetic costs:
the graph, its neighbourhoods, and the Metropolis walk (no GPU)."""

import math
from collections import deque

from precision_gemm_amd import tune


def test_space_and_neighbours():
    nodes = tune.space()
    assert len(nodes) == 4 * 3 * 2 * 3 * 2 and len(set(nodes)) == len(nodes)
    for n in nodes:
        nb = tune.neighbours(n)
        assert n not in nb and len(set(nb)) == len(nb)
        for m in nb:
            assert n in tune.neighbours(m)                        # symmetric
            assert sum(a != b for a, b in zip(n, m)) == 1          # one parameter changes
        cfg = tune.to_config(n)
        if n[0] == 0:
            assert cfg[3] == n[3] and cfg[0] == 0          # wave reductions: positions per item
        else:
            assert cfg[3] % 16 == 0 and cfg[3] == 16 * n[0] * n[3]
    # connected: every node is reachable from the default of any batch size
    for T in (1, 16, 64, 128, 4096):
        start = tune.default_node(T)
        assert start in nodes
        seen, q = {start}, deque([start])
        while q:
            for m in tune.neighbours(q.popleft()):
                if m not in seen:
                    seen.add(m)
                    q.append(m)
        assert len(seen) == len(nodes)


def test_feasibility_prunes_spills_lds_and_long_items():
    def info(tg, jp, u, m):
        if tg == 0 and u == 2 and m != 1:
            return None                                              # not compiled
        return {"regs": 128, "spill": 16 if (tg, jp, u) == (4, 4, 2) else 0, "lds": 4 * max(tg, 1) * jp * 256 * 4}
    assert not tune.feasible((4, 4, 2, 1, 0), info, 4096)            # spills
    assert tune.feasible((4, 4, 1, 1, 0), info, 4096)                # 64 KB of LDS: fits
    assert not tune.feasible((4, 2, 1, 4, 0), info, 16)              # 256-token items for 16 tokens
    assert tune.feasible((1, 1, 2, 1, 0), info, 16)
    assert not tune.feasible((1, 1, 1, 1, 0), lambda *a: None, 16)   # not compiled
    assert tune.feasible((0, 4, 1, 4, 0), info, 16) and not tune.feasible((0, 4, 2, 4, 0), info, 16)
    assert not tune.feasible((0, 1, 1, 4, 1), info, 1)               # 4 positions per item for 1 token


def test_metropolis_finds_the_minimum_and_is_reproducible():
    target = (2, 4, 1, 2, 1)

    def cost(n):  # a bowl around the target in index space, with a plateau to cross
        d = sum(abs(tune.DOMAINS[k].index(a) - tune.DOMAINS[k].index(b)) for k, a, b in zip(tune.KEYS, n, target))
        return 10.0 + d * d + (3.0 if n[4] != target[4] else 0.0)

    r1 = tune.metropolis(tune.default_node(4096), cost, tune.neighbours, steps=300, tau=0.2, seed=3)
    r2 = tune.metropolis(tune.default_node(4096), cost, tune.neighbours, steps=300, tau=0.2, seed=3)
    assert r1.best == target and r1.best_cost == 10.0
    assert r1.trace == r2.trace and r1.best == r2.best
    assert r1.best_cost <= r1.start_cost
    assert all(cost(n) == c for n, c in r1.evaluated.items())


def test_metropolis_acceptance_rule():
    # two nodes: from a (cost 1) the only move is to b (cost 1 + d); it is accepted with
    # probability exp(-d / (tau * 1)), and never at tau -> 0
    nb = {"a": ["b"], "b": ["a"]}
    costs = {"a": 1.0, "b": 1.2}
    r = tune.metropolis("a", costs.get, nb.get, steps=1, tau=1e-9, seed=0)
    assert r.trace[0][3] is False and r.best == "a"
    acc = 0
    for seed in range(2000):
        acc += tune.metropolis("a", costs.get, nb.get, steps=1, tau=0.5, seed=seed).trace[0][3]
    p = math.exp(-0.2 / 0.5)
    assert abs(acc / 2000 - p) < 0.04
    r = tune.metropolis("b", costs.get, nb.get, steps=1, tau=1e-9, seed=0)
    assert r.trace[0][3] is True and r.best == "a"           # downhill is always taken
