"""CPU model of the event-tensor task graph (test infrastructure only).

What the pages fix: event tensors are counters that encode the dependencies between
tiled tasks (OpenAlex record of "Event Tensor: A Unified Abstraction for Compiling
Dynamic Megakernel", abstract); a task waits until its counter reaches a target, and
with MoE routing the target depends on how many producer tasks the routing creates,
so it is computed on the GPU before anyone waits (chapter "5 · Event Tensor et le
dynamisme", §5.5 Obstacle 1); with unpredictable task sizes the work is handed out
online through atomics (§5.5 Obstacle 3); static scheduling suits regular work and
dynamic scheduling irregular work such as MoE (podcast episode page "Prompt
Boundary-Aware Scheduling with Event Tensors for Dynamic Kernels", summary).

reading (tiling): per layer, with BT tokens per routing tile, BM rows per expert row
tile, BN1 ffn columns per gate/up tile, BN2 hidden columns per down tile and the
down projection split along ffn into chunks of GPC gate/up tiles:

  R(tau)          routing tile tau                      waits  done[l-1][tau] >= 1 (l > 0)
                                                        signals route[l] += 1
  S               counts, scans, per-tile row offsets   runs in the R task whose signal
                                                        brings route[l] to n_rt
                                                        signals scan[l] = 1 (and perm[l] = n_rt
                                                        when it scatters the permutation)
  P(tau)          permutation scatter of tile tau       waits  scan[l] >= 1
                                                        signals perm[l] += 1
  GU(e, m, n)     gate/up tile                          waits  perm[l] >= n_rt
                                                        signals gu[l][e,m][n // GPC] += 1
  D(e, m, n2, s)  down tile over ffn chunk s            waits  gu[l][e,m][s] >= tiles in chunk s
                                                        signals comb[l][tau] += rows of (e,m) in tau
  F(tau)          finalize the output rows of tau       waits  comb[l][tau] >= |tau| * k * n2 * nS
                                                        signals done[l][tau] += 1

reading (few routing tiles): with at most Plan.PI routing tiles S also scatters the
permutation and there are no P tasks (a hand-off less on a short critical path).

reading (router slices, Plan.Q > 1): the router of a routing tile is cut along H into Q
slice tasks R(tau*Q + q), each waiting like R(tau) and signalling rq[l][tau] += 1; the
slice whose signal completes rq[l][tau] (target Q) finishes the tile in the same worker
and signals route[l] += 1.  Like S, that finish is not a task of its own: it is the
task's `finish` field, (counter, target, counter it then signals).

S is not a ticket of its own: in both modes the R task whose signal completes
route[l] (the last arriver) runs it.  Static mode runs the other tasks in one fixed
ticket order (per layer: all R, all P, all GU, all D, all F) and each worker spins on
the dependencies of the task it drew.  Dynamic mode keeps a FIFO ready queue: the R
tasks of the first layer are queued at the start; the worker whose signal completes a
counter makes the dependents ready -- S queues every P task (or every GU task when it
scattered the permutation), the last P queues every GU task, a full gu chunk queues its
D tasks, a full comb tile queues its F, and F queues the next layer's R for the same
tokens.
"""

from dataclasses import dataclass, field
import random


def cdiv(a, b):
    return -(-a // b)


@dataclass(frozen=True)
class Plan:
    BT: int  # tokens per routing tile
    BM: int  # rows per expert row tile
    BN1: int  # ffn columns per gate/up tile
    BN2: int  # hidden columns per down tile
    GPC: int  # gate/up tiles per down chunk (ffn split of the down projection)
    PI: int = 0  # up to this many routing tiles S scatters the permutation (no P tasks)
    Q: int = 1  # router slices per routing tile


@dataclass
class Task:
    kind: str
    layer: int
    key: tuple
    waits: list = field(default_factory=list)  # [(counter, target)]
    signals: list = field(default_factory=list)  # [(counter, amount)]
    finish: tuple = None  # (counter, target, next): when the task's signal completes
    #                       counter, the same worker then signals next += 1


def layer_shape(T, H, F, plan):
    n_rt = cdiv(T, plan.BT)
    n1 = cdiv(F, plan.BN1)
    n2 = cdiv(H, plan.BN2)
    nS = cdiv(n1, plan.GPC)
    return n_rt, n1, n2, nS


def rows_per_routing_tile(T, plan):
    return [min(plan.BT, T - tau * plan.BT) for tau in range(cdiv(T, plan.BT))]


def build_layer(l, T, H, F, k, counts, plan, tokens_of_rows):
    """Tasks of layer ``l``.  ``tokens_of_rows[e]`` lists the token of every row of
    expert e in row order (the permutation), used to count rows per routing tile."""
    n_rt, n1, n2, nS = layer_shape(T, H, F, plan)
    tile_rows = rows_per_routing_tile(T, plan)
    R, GU, D, Fin = [], [], [], []
    Q = plan.Q
    for tau in range(n_rt):
        waits = [(("done", l - 1, tau), 1)] if l > 0 else []
        if Q == 1:
            R.append(Task("R", l, (tau,), waits, [(("route", l), 1)]))
        else:
            for q in range(Q):
                R.append(Task("R", l, (tau * Q + q,), list(waits), [(("rq", l, tau), 1)],
                              finish=(("rq", l, tau), Q, ("route", l))))
    if n_rt <= plan.PI:
        S = Task("S", l, (), [(("route", l), n_rt)], [(("scan", l), 1), (("perm", l), n_rt)])
        P = []
    else:
        S = Task("S", l, (), [(("route", l), n_rt)], [(("scan", l), 1)])
        P = [Task("P", l, (tau,), [(("scan", l), 1)], [(("perm", l), 1)]) for tau in range(n_rt)]
    for e, c in enumerate(counts):
        for m in range(cdiv(int(c), plan.BM)):
            for n in range(n1):
                GU.append(Task("GU", l, (e, m, n), [(("perm", l), n_rt)],
                               [(("gu", l, e, m, n // plan.GPC), 1)]))
    for e, c in enumerate(counts):
        for m in range(cdiv(int(c), plan.BM)):
            rows = tokens_of_rows[e][m * plan.BM:(m + 1) * plan.BM]
            per_tau = {}
            for t in rows:
                per_tau[t // plan.BT] = per_tau.get(t // plan.BT, 0) + 1
            sig = [(("comb", l, tau), cnt) for tau, cnt in sorted(per_tau.items())]
            for s in range(nS):
                need = min(plan.GPC, n1 - s * plan.GPC)
                for n2i in range(n2):
                    D.append(Task("D", l, (e, m, n2i, s), [(("gu", l, e, m, s), need)], sig))
    for tau in range(n_rt):
        target = tile_rows[tau] * k * n2 * nS
        Fin.append(Task("F", l, (tau,), [(("comb", l, tau), target)], [(("done", l, tau), 1)]))
    return R, S, P, GU, D, Fin


def build_graph(T, H, F, k, layer_counts, layer_tokens_of_rows, plan):
    """All layers, each as (R, S, P, GU, D, F) lists."""
    return [build_layer(l, T, H, F, k, c, plan, tr)
            for l, (c, tr) in enumerate(zip(layer_counts, layer_tokens_of_rows))]


def expected_final_counters(graph):
    """Every counter's value once all tasks have signalled (and every router slice
    counter has been completed once, moving its `next` counter by one)."""
    final = {}
    finishes = set()
    for R, S, P, GU, D, Fin in graph:
        for t in R + [S] + P + GU + D + Fin:
            for ctr, amt in t.signals:
                final[ctr] = final.get(ctr, 0) + amt
            if t.finish is not None:
                finishes.add((t.finish[0], t.finish[2]))
    for _, nxt in finishes:
        final[nxt] = final.get(nxt, 0) + 1
    return final


def static_order(graph):
    """The ticket order (S runs inside the last R of its layer and has no ticket)."""
    order = []
    for R, S, P, GU, D, Fin in graph:
        order += R + P + GU + D + Fin
    return order


def _scan_of(graph):
    """S of each layer by the route counter its last routing tile completes (its target
    is the number of routing tiles)."""
    return {("route", l): (g[1], g[1].waits[0][1]) for l, g in enumerate(graph)}


def _run_finish(task, before, counters):
    """A router slice whose signal completed its tile's slice counter finishes the tile
    in the same worker (its `next` counter moves by one)."""
    if task.finish is not None:
        ctr, target, nxt = task.finish
        if before.get(ctr, 0) < target <= counters.get(ctr, 0):
            counters[nxt] = counters.get(nxt, 0) + 1


def _run_inline_scan(task, before, counters, scans, executed):
    """After ``task`` (an R, or a router slice that finished its tile) signalled: if its
    layer's route counter is now complete, S runs right after it in the same worker.
    Returns S or None."""
    _run_finish(task, before, counters)
    ctrs = [c for c, _ in task.signals] + ([task.finish[2]] if task.finish else [])
    for ctr in ctrs:
        if ctr in scans:
            S, n_rt = scans[ctr]
            if before.get(ctr, 0) < n_rt <= counters.get(ctr, 0):
                assert _ready(S, counters)
                _signal(S, counters)
                executed.append(S)
                return S
    return None


def replay_static(graph):
    """One worker taking the tickets in order and never waiting (S inline after the R
    that completes its layer's route counter); raises if a ticket's task is not ready
    when its turn comes.  Returns the execution order."""
    scans = _scan_of(graph)
    counters, executed = {}, []
    for t in static_order(graph):
        if not _ready(t, counters):
            raise RuntimeError(f"ticket {t.kind}{t.key} of layer {t.layer} is not ready in order")
        before = dict(counters)
        _signal(t, counters)
        executed.append(t)
        _run_inline_scan(t, before, counters, scans, executed)
    return executed


def _ready(task, counters):
    return all(counters.get(c, 0) >= tgt for c, tgt in task.waits)


def _signal(task, counters):
    for c, amt in task.signals:
        counters[c] = counters.get(c, 0) + amt


def queue_ticket(q, i, queues, chunk):
    """Position in the static order of the i-th ticket of queue q when the order is cut
    into chunks of `chunk` consecutive tasks dealt round-robin to `queues` queues."""
    return ((i // chunk) * queues + q) * chunk + i % chunk


def simulate_static(graph, workers, rng=None, queues=1, chunk=1, prefetch=False):
    """Workers draw tickets and spin on the drawn task's waits.  With queues > 1 the
    order is dealt to the queues in chunks (queue_ticket) and worker w draws only from
    queue w mod queues, each queue in its own order.  With prefetch, a worker that runs
    a GU or D task draws its next ticket while running it (the kernel overlaps that
    atomic with the task) and takes that ticket afterwards.  Returns the execution
    order; raises RuntimeError on deadlock (no worker can move)."""
    rng = rng or random.Random(0)
    order = static_order(graph)
    scans = _scan_of(graph)
    counters, executed = {}, []
    next_local = [0] * queues
    holding = [None] * workers  # task drawn by each worker
    pending = [None] * workers  # ticket drawn ahead (prefetch), False: queue drained
    total = len(order) + len(graph)  # the tickets and one S per layer

    def draw(w):
        q = w % queues
        g = queue_ticket(q, next_local[q], queues, chunk)
        if g >= len(order):
            return False
        next_local[q] += 1
        return order[g]

    while len(executed) < total:
        # every idle worker draws its queue's next ticket (an atomic increment), or takes
        # the one it drew ahead; a ticket past the end of the order means the queue is
        # drained
        for w in range(workers):
            if holding[w] is None:
                t = pending[w] if pending[w] is not None else draw(w)
                pending[w] = None
                if t is not False:
                    holding[w] = t
        movable = [w for w in range(workers)
                   if holding[w] is not None and _ready(holding[w], counters)]
        if not movable:
            stuck = [holding[w] for w in range(workers) if holding[w] is not None]
            raise RuntimeError(f"static schedule deadlocked holding {[(t.kind, t.key) for t in stuck]}")
        w = rng.choice(movable)
        t = holding[w]
        if prefetch and t.kind in ("GU", "D"):
            pending[w] = draw(w)
        before = dict(counters)
        _signal(t, counters)
        executed.append(t)
        _run_inline_scan(t, before, counters, scans, executed)
        holding[w] = None
    return executed, counters


def simulate_dynamic(graph, workers, rng=None):
    """FIFO ready queue filled by last arrivers.  Returns (execution order, counters);
    raises RuntimeError if work remains but nothing is queued or running."""
    rng = rng or random.Random(0)
    counters, executed = {}, []
    layers = len(graph)
    queue = list(graph[0][0])  # R tasks of the first layer
    running = []
    # lookups of the dependents that a completed counter releases
    p_by_layer = [g[2] for g in graph]
    gu_by_layer = [g[3] for g in graph]
    d_by_chunk = []
    f_by_tau = []
    r_by_tau = []
    for R, S, P, GU, D, Fin in graph:
        dd = {}
        for t in D:
            e, m, _, s = t.key
            dd.setdefault((e, m, s), []).append(t)
        d_by_chunk.append(dd)
        f_by_tau.append({t.key[0]: t for t in Fin})
        rt = {}
        for t in R:  # the routing tasks (slices) of each tile
            tau = t.finish[0][2] if t.finish else t.key[0]
            rt.setdefault(tau, []).append(t)
        r_by_tau.append(rt)
    total = sum(len(R) + len(P) + len(GU) + len(D) + len(Fin) + 1 for R, S, P, GU, D, Fin in graph)
    while len(executed) < total:
        while queue and len(running) < workers:
            running.append(queue.pop(0))
        if not running:
            raise RuntimeError("dynamic schedule starved: no task queued or running")
        t = running.pop(rng.randrange(len(running)))
        if not _ready(t, counters):
            raise RuntimeError(f"task {t.kind}{t.key} was queued before it was ready")
        before = dict(counters)
        _signal(t, counters)
        _run_finish(t, before, counters)
        executed.append(t)
        l = t.layer
        R, S, P, GU, D, Fin = graph[l]
        n_rt = S.waits[0][1]
        ctrs = [c for c, _ in t.signals] + ([t.finish[2]] if t.finish else [])
        for ctr in ctrs:
            old, new = before.get(ctr, 0), counters.get(ctr, 0)
            kind = ctr[0]
            if kind == "route" and new == n_rt and old < new:
                # the last routing tile runs S inline; S queues the P tasks, or the GU
                # tasks when it scattered the permutation itself
                assert _ready(S, counters)
                _signal(S, counters)
                executed.append(S)
                queue.extend(p_by_layer[l] if p_by_layer[l] else gu_by_layer[l])
            elif kind == "perm" and P and new == len(P) and old < new:
                queue.extend(gu_by_layer[l])
            elif kind == "gu":
                _, _, e, m, s = ctr
                deps = d_by_chunk[l].get((e, m, s), [])
                if deps and old < deps[0].waits[0][1] <= new:
                    queue.extend(deps)
            elif kind == "comb":
                ft = f_by_tau[l][ctr[2]]
                if old < ft.waits[0][1] <= new:
                    queue.append(ft)
            elif kind == "done" and l + 1 < layers:
                queue.extend(r_by_tau[l + 1][ctr[2]])
    return executed, counters


def check_execution(executed, graph):
    """Each task ran once and only after its waits were met (replays the order)."""
    counters = {}
    seen = set()
    for t in executed:
        ident = (t.kind, t.layer, t.key)
        if ident in seen:
            raise AssertionError(f"{ident} ran twice")
        seen.add(ident)
        if not _ready(t, counters):
            raise AssertionError(f"{ident} ran before its dependencies")
        before = dict(counters)
        _signal(t, counters)
        _run_finish(t, before, counters)
    n = sum(len(R) + 1 + len(P) + len(GU) + len(D) + len(Fin) for R, S, P, GU, D, Fin in graph)
    if len(seen) != n:
        raise AssertionError(f"{len(seen)} of {n} tasks ran")
    return counters


# ------------------------------------------------------------------ split-K graph


def splitk_graph(M, N, split_k, BM, BN):
    """P(tile, s) partial tasks signal ev[tile]; the reduction of a tile waits for
    ev[tile] >= split_k (podcast episode summary: the split-K summation example)."""
    tiles = [(i, j) for i in range(cdiv(M, BM)) for j in range(cdiv(N, BN))]
    P = [Task("P", 0, (tile, s), [], [(("ev", tile), 1)]) for s in range(split_k) for tile in tiles]
    K = [Task("K", 0, (tile,), [(("ev", tile), split_k)], [(("out", tile), 1)]) for tile in tiles]
    return P, K
