"""Pins of the scheduler model (CPU only): the task graph of every workload shape runs
to completion in static ticket order and through the dynamic ready queue, under
random interleavings and worker counts; every task runs once and after its waits;
the counters end exactly at their targets; a dropped signal is detected."""

import random

import numpy as np
import pytest

from oracle import moe as om
from oracle import sched_model as sm


def _graph_from_routing(T, H, F, k, E, layers_idx, plan):
    counts, tors = [], []
    for idx in layers_idx:
        c = om.expert_counts(idx, E)
        sa, _ = om.permutation(idx, E)
        off = om.exclusive_scan(c)
        counts.append(c)
        tors.append([list(sa[off[e]:off[e + 1]] // k) for e in range(E)])
    return sm.build_graph(T, H, F, k, counts, tors, plan)


def _random_idx(rng, T, E, k, skew=0.0):
    logits = rng.standard_normal((T, E)) - skew * np.log1p(np.arange(E))[None, :]
    return om.topk_experts(logits, k)


CASES = [
    # T, H, F, E, k, layers, plan
    (16, 128, 256, 4, 2, 1, sm.Plan(BT=16, BM=128, BN1=64, BN2=128, GPC=4)),
    (1, 4096, 14336, 8, 2, 1, sm.Plan(BT=16, BM=128, BN1=64, BN2=128, GPC=8)),
    (64, 4096, 14336, 8, 2, 1, sm.Plan(BT=16, BM=32, BN1=512, BN2=256, GPC=4)),
    (256, 2048, 768, 128, 8, 1, sm.Plan(BT=16, BM=64, BN1=128, BN2=256, GPC=6)),
    (300, 512, 384, 16, 6, 2, sm.Plan(BT=16, BM=64, BN1=64, BN2=128, GPC=6)),
    (33, 256, 192, 8, 3, 3, sm.Plan(BT=8, BM=16, BN1=32, BN2=64, GPC=2)),
    # few routing tiles: S scatters the permutation, no P tasks
    (1, 4096, 14336, 8, 2, 2, sm.Plan(BT=16, BM=128, BN1=128, BN2=256, GPC=7, PI=4)),
    (64, 4096, 14336, 8, 2, 1, sm.Plan(BT=16, BM=128, BN1=128, BN2=256, GPC=4, PI=4)),
    (33, 256, 192, 8, 3, 3, sm.Plan(BT=8, BM=16, BN1=32, BN2=64, GPC=2, PI=5)),
    # router slices: each routing tile's router in Q tasks, the last one finishing it
    (1, 4096, 14336, 8, 2, 2, sm.Plan(BT=16, BM=128, BN1=128, BN2=256, GPC=7, PI=4, Q=8)),
    (64, 4096, 14336, 8, 2, 1, sm.Plan(BT=16, BM=128, BN1=128, BN2=256, GPC=4, PI=4, Q=3)),
    (256, 2048, 768, 128, 8, 2, sm.Plan(BT=16, BM=64, BN1=128, BN2=256, GPC=6, PI=4, Q=8)),
]


@pytest.mark.parametrize("T,H,F,E,k,L,plan", CASES)
def test_static_and_dynamic_complete(T, H, F, E, k, L, plan):
    rng = np.random.default_rng(T + E)
    idx = [_random_idx(rng, T, E, k, skew=1.1 if E >= 64 else 0.0) for _ in range(L)]
    graph = _graph_from_routing(T, H, F, k, E, idx, plan)
    final = sm.expected_final_counters(graph)
    for workers in (1, 3, 17):
        for seed in range(3):
            ex, ctr = sm.simulate_static(graph, workers, random.Random(seed))
            assert sm.check_execution(ex, graph) == final
            assert ctr == final
            ex, ctr = sm.simulate_dynamic(graph, workers, random.Random(seed))
            assert sm.check_execution(ex, graph) == final
            assert ctr == final


@pytest.mark.parametrize("T,H,F,E,k,L,plan", CASES)
def test_static_xcd_queues_complete(T, H, F, E, k, L, plan):
    """The static order dealt in chunks to up to 8 queues (one per XCD), each worker
    drawing only from its own queue: every task runs once and every counter ends at
    its target, for worker counts that do and do not divide into the queues, with and
    without gate/up and down tasks drawing their worker's next ticket ahead."""
    rng = np.random.default_rng(T + 3 * E)
    idx = [_random_idx(rng, T, E, k, skew=1.1 if E >= 64 else 0.0) for _ in range(L)]
    graph = _graph_from_routing(T, H, F, k, E, idx, plan)
    final = sm.expected_final_counters(graph)
    for workers in (1, 2, 8, 17, 64):
        queues = min(8, workers)
        for seed in range(2):
            for prefetch in (False, True):
                ex, ctr = sm.simulate_static(graph, workers, random.Random(seed), queues=queues,
                                             chunk=workers // queues, prefetch=prefetch)
                assert sm.check_execution(ex, graph) == final
                assert ctr == final


def test_queue_tickets_partition_the_order():
    """Queue tickets cover every position of the order exactly once, in increasing
    order within each queue."""
    for queues, chunk in ((1, 1), (8, 32), (8, 2), (3, 5)):
        seen = []
        for q in range(queues):
            pos = [sm.queue_ticket(q, i, queues, chunk) for i in range(200)]
            assert pos == sorted(pos)
            seen += pos
        n = 200 * queues
        assert sorted(p for p in seen if p < n - queues * chunk) == list(range(n - queues * chunk))


def test_unserved_queue_deadlocks():
    """More queues than workers leaves a queue nobody draws from: the model reports the
    deadlock (the kernel therefore uses at most as many queues as workgroups)."""
    rng = np.random.default_rng(5)
    plan = sm.Plan(BT=8, BM=16, BN1=32, BN2=64, GPC=2)
    graph = _graph_from_routing(24, 128, 128, 2, 8, [_random_idx(rng, 24, 8, 2)], plan)
    with pytest.raises(RuntimeError, match="deadlocked"):
        sm.simulate_static(graph, 2, queues=3, chunk=1)


@pytest.mark.parametrize("T,H,F,E,k,L,plan", CASES)
def test_targets_equal_final_counts(T, H, F, E, k, L, plan):
    """Every wait target is exactly the value its counter reaches: the targets computed
    from the routing (counts, rows per routing tile) match what the producers signal."""
    rng = np.random.default_rng(T * 7 + E)
    idx = [_random_idx(rng, T, E, k) for _ in range(L)]
    graph = _graph_from_routing(T, H, F, k, E, idx, plan)
    final = sm.expected_final_counters(graph)
    for R, S, P, GU, D, Fin in graph:
        for t in R + [S] + P + GU + D + Fin:
            for ctr, tgt in t.waits:
                if t.kind == "R":
                    assert final[ctr] == tgt  # one F per routing tile
                else:
                    assert final[ctr] == tgt, (t.kind, t.key, ctr)
    # routing-tile targets: rows * k * n2 * nS sum to the total D row work
    n_rt, n1, n2, nS = sm.layer_shape(T, H, F, plan)
    total = sum(final[("comb", 0, tau)] for tau in range(n_rt))
    assert total == T * k * n2 * nS


def test_dropped_signal_detected():
    """A producer that never signals must not go unnoticed: static mode deadlocks with
    workers holding the starved tasks, dynamic mode starves."""
    rng = np.random.default_rng(1)
    plan = sm.Plan(BT=8, BM=16, BN1=32, BN2=64, GPC=2)
    idx = [_random_idx(rng, 24, 8, 2)]
    graph = _graph_from_routing(24, 128, 128, 2, 8, idx, plan)
    R, S, P, GU, D, Fin = graph[0]
    GU[5].signals = []  # planted mistake: one gate/up tile never signals
    with pytest.raises(RuntimeError, match="deadlocked"):
        sm.simulate_static(graph, 4)
    with pytest.raises(RuntimeError, match="starved"):
        sm.simulate_dynamic(graph, 4)


def test_static_ticket_order_is_topological():
    rng = np.random.default_rng(2)
    plan = sm.Plan(BT=16, BM=64, BN1=64, BN2=128, GPC=3)
    graph = _graph_from_routing(100, 256, 384, 2, 8, [_random_idx(rng, 100, 8, 2)] * 2, plan)
    # one worker executing the ticket order without ever waiting proves every task's
    # producers hold smaller tickets (deadlock freedom with co-resident workers)
    sm.check_execution(sm.replay_static(graph), graph)
    # S has no ticket: it runs inside the routing task that completes route[l]
    assert all(t.kind != "S" for t in sm.static_order(graph))


def test_inline_permutation_replaces_p_tasks():
    rng = np.random.default_rng(3)
    idx = [_random_idx(rng, 40, 8, 2)] * 2
    few = _graph_from_routing(40, 256, 384, 2, 8, idx, sm.Plan(BT=16, BM=64, BN1=64, BN2=128, GPC=3, PI=4))
    many = _graph_from_routing(40, 256, 384, 2, 8, idx, sm.Plan(BT=16, BM=64, BN1=64, BN2=128, GPC=3, PI=2))
    for R, S, P, GU, D, Fin in few:
        assert P == [] and (("perm", S.layer), len(R)) in S.signals
    for R, S, P, GU, D, Fin in many:
        assert len(P) == len(R)
    # both reach the same final counters, and both schedules complete
    assert sm.expected_final_counters(few) == sm.expected_final_counters(many)
    for g in (few, many):
        sm.check_execution(sm.simulate_static(g, 3, queues=2, chunk=2)[0], g)
        sm.check_execution(sm.simulate_dynamic(g, 3)[0], g)


def test_splitk_graph():
    P, K = sm.splitk_graph(64, 4096, 8, 64, 128)
    assert len(P) == 32 * 8 and len(K) == 32
    counters = {}
    for t in P:
        for c, a in t.signals:
            counters[c] = counters.get(c, 0) + a
    assert all(counters[t.waits[0][0]] == 8 for t in K)


def test_router_slices_finish_each_tile_once():
    """With Q slices per routing tile, the slice counter of every tile ends at Q, the
    route counter at the number of tiles (one finish per tile), and S runs after the
    last finish; a slice whose signal is dropped leaves its tile unfinished and the
    static schedule stuck."""
    plan = sm.Plan(BT=16, BM=64, BN1=64, BN2=128, GPC=3, PI=4, Q=4)
    rng = np.random.default_rng(5)
    graph = _graph_from_routing(40, 256, 384, 2, 8, [_random_idx(rng, 40, 8, 2)], plan)
    final = sm.expected_final_counters(graph)
    R, S, P, GU, D, Fin = graph[0]
    assert len(R) == 3 * 4 and all(final[("rq", 0, tau)] == 4 for tau in range(3))
    assert final[("route", 0)] == 3
    ex = sm.replay_static(graph)
    assert ex.index(S) > max(ex.index(t) for t in R)
    dropped = R[5]
    dropped.signals = []
    with pytest.raises(RuntimeError):
        sm.simulate_static(graph, 3, random.Random(0))
