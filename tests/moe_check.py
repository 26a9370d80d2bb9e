"""Parity rules between the HIP MoE path and the oracle (used by the GPU tests).

Every layer is checked on the same input on both sides: layer 0 on x, layer l > 0 on
the GPU's own output of layer l-1 (bfloat16 or float32 values, which the oracle takes
exactly).  Rules, per layer, for every token:
  * routing: the GPU's expert list of a token equals the oracle's, slot by slot, unless
    the oracle's gap l_(k) - l_(k+1) is below TIE = 1e-5 (then any valid top-k set
    within TIE of the boundary is accepted, and slots may swap between logits closer
    than TIE); the number of such near-tie tokens is reported;
  * gates: within 1e-5 absolute of the oracle's for the same expert;
  * counts and sorted_assign: always the stable grouping of the GPU's own topk_idx, and
    bit-exact to the oracle's whenever every token's expert set agrees with the oracle;
  * outputs: max |gpu - ref| <= tol * max |ref| with tol 2e-2 for bfloat16 and 1e-4 for
    float32, where ref follows the GPU's expert choice for tokens that took another
    valid set (the oracle computes every valid alternative itself).
One end-to-end check follows for a chain of layers: the oracle runs the whole chain from
x on its own (each layer fed its own rounded output) and the GPU's last output must
match it within the same output tolerance, on every token whose expert sets agree in
every layer.  A token whose sets differ there must sit within CHAIN_TIE of a tie in the
first layer where they differ: from layer 1 on, the two chains' inputs differ by
rounding flips of the previous output (one flip of a 2**-8-relative step moves a logit
by about |w| * |x| * 2**-8 ~ 1e-4), so near-ties there may resolve either way.
"""

import numpy as np

from oracle import moe as om

# routing tiles up to which the library's scan task scatters the permutation itself
# (no P tasks; PERM_INLINE_RT in csrc/moe.hip)
PERM_INLINE_RT = 4

TIE = 1e-5
GATE_TOL = 1e-5
CHAIN_TIE = 2e-3
OUT_TOL = {"bf16": 2e-2, "f32": 1e-4}


def check_grouping(idx, counts, sorted_assign, E):
    """counts / sorted_assign are the stable per-expert grouping of idx."""
    flat = np.asarray(idx).reshape(-1)
    n = flat.size
    assert np.array_equal(counts, np.bincount(flat, minlength=E)), "counts != histogram of topk_idx"
    assert np.array_equal(np.sort(sorted_assign), np.arange(n)), "sorted_assign is not a permutation"
    off = np.concatenate([[0], np.cumsum(counts)])
    for e in range(E):
        seg = sorted_assign[off[e]:off[e + 1]]
        assert np.all(flat[seg] == e), f"expert {e} segment holds other experts"
        assert np.all(np.diff(seg) > 0), f"expert {e} segment is not token-ascending"


def _check_layer(l, h_in, layer, k, eps, act, gidx, gw, gcounts, gsa, gout, stats):
    """One layer on the GPU's own input h_in (see the module docstring).  Returns the
    boolean mask of tokens that took another valid expert set."""
    T = h_in.shape[0]
    E = layer["w_router"].shape[0]
    r, out_ref = om.moe_layer(h_in, layer, k, eps, act)
    gap = om.topk_gap(r.logits, k)
    stats["near_tie"][l] = int(np.sum(gap < TIE))
    other = np.zeros(T, dtype=bool)
    for t in np.nonzero(~np.all(gidx == r.idx, axis=1))[0]:
        gs, os_ = [int(e) for e in gidx[t]], [int(e) for e in r.idx[t]]
        if set(gs) != set(os_):
            valid = om.valid_topk_sets(r.logits[t], k, TIE)
            assert frozenset(gs) in valid, (
                f"layer {l} token {t}: experts {gs} vs oracle {os_}, gap {gap[t]:.3g}")
            other[t] = True
            out_ref[t] = om.token_output_for_set(h_in[t], layer, set(gs), eps, act)
        else:  # same set, slots swapped: only between near-equal logits
            lg = r.logits[t]
            for j in range(k):
                assert abs(lg[gs[j]] - lg[os_[j]]) < TIE, f"layer {l} token {t}: slot order {gs} vs {os_}"
    stats["other_set"][l] = int(other.sum())
    # gates of the tokens that took the oracle's set, per expert
    dense = np.zeros((T, E))
    np.put_along_axis(dense, r.idx, r.gates, axis=1)
    keep = ~other
    diff = np.abs(np.take_along_axis(dense, gidx, axis=1) - gw)[keep]
    worst = float(diff.max()) if diff.size else 0.0
    stats["max_gate_err"][l] = worst
    assert worst <= GATE_TOL, f"layer {l}: gate error {worst:.3g} > {GATE_TOL}"
    ref_max = float(np.max(np.abs(out_ref)))
    err = float(np.max(np.abs(gout - out_ref)))
    stats["max_err"][l], stats["max_ref"][l] = err, ref_max
    assert err <= OUT_TOL[act] * ref_max, f"layer {l}: max err {err:.4g} > {OUT_TOL[act]} * {ref_max:.4g}"
    # grouping: always valid for the GPU's own routing; exact while no set differs
    check_grouping(gidx, gcounts, gsa, E)
    if not other.any():
        assert np.array_equal(gcounts, r.counts), f"layer {l}: counts differ"
        assert np.array_equal(gsa, r.sorted_assign), f"layer {l}: sorted_assign differs"
    return other


def compare(x, layers, k, eps, act, gpu):
    """Compare one GPU run with the oracle (rules in the module docstring).

    x: [T][H] float array (exact input values); layers: list of float weight dicts;
    gpu: dict of numpy arrays idx [L][T][k], w [L][T][k], counts [L][E], sa [L][T*k],
    outs [L][T][H] (output of every layer, the last being the call's output).
    Returns a stats dict.
    """
    L = len(layers)
    x = np.asarray(x, np.float64)
    stats = {"near_tie": [0] * L, "other_set": [0] * L, "max_err": [0.0] * L, "max_ref": [0.0] * L,
             "max_gate_err": [0.0] * L}
    for l, layer in enumerate(layers):
        h_in = x if l == 0 else np.asarray(gpu["outs"][l - 1], np.float64)
        _check_layer(l, h_in, layer, k, eps, act, np.asarray(gpu["idx"][l]), np.asarray(gpu["w"][l]),
                     np.asarray(gpu["counts"][l]), np.asarray(gpu["sa"][l]),
                     np.asarray(gpu["outs"][l], np.float64), stats)
    if L > 1:
        stats.update(compare_chain(x, layers, k, eps, act, gpu))
    return stats


def compare_chain(x, layers, k, eps, act, gpu):
    """End-to-end check of a chain of layers against the oracle's own chain from x."""
    routings, outs = om.moe_forward(x, layers, k, eps, act)
    T = x.shape[0]
    agree = np.ones(T, dtype=bool)
    for l, r in enumerate(routings):
        gidx = np.asarray(gpu["idx"][l])
        same = np.sort(gidx, axis=1) == np.sort(r.idx, axis=1)
        first_diff = agree & ~np.all(same, axis=1)
        if first_diff.any():
            gap = om.topk_gap(r.logits[first_diff], k)
            lim = TIE if l == 0 else CHAIN_TIE
            assert np.all(gap < lim), (
                f"chain layer {l}: tokens {np.nonzero(first_diff)[0][:8]} took other experts with "
                f"gaps {gap[:8]} >= {lim}")
        agree &= ~first_diff
    ref = outs[-1][agree]
    ref_max = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(np.asarray(gpu["outs"][-1], np.float64)[agree] - ref))) if ref.size else 0.0
    assert err <= OUT_TOL[act] * ref_max, f"chain: max err {err:.4g} > {OUT_TOL[act]} * {ref_max:.4g}"
    return {"chain_max_err": err, "chain_max_ref": ref_max, "chain_excluded": int(T - agree.sum())}


def check_event_tensor(read_i32, layout, T, H, F, k, E, gpu, layers):
    """Final state of every counter of the event tensor (call made with the counters
    kept) against the scheduler model, given the GPU's own routing and down split.

    read_i32(byte_offset, count) -> int array from the workspace; layout(l) -> the
    etc_moe_workspace_layout words of layer l."""
    from oracle import sched_model as sm

    for l in range(layers):
        lay = layout(l)
        max_rt, n1, n_rt_cap, BT, BM, BN1, BN2 = lay[6:13]
        pw = [int(v) for v in read_i32(lay[5], 8)]
        RT, ngu, nd, nf, nS, gpc, Q = pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[7]
        counts = gpu["counts"][l]
        sa = gpu["sa"][l]
        off = np.concatenate([[0], np.cumsum(counts)])
        tors = [list(sa[off[e]:off[e + 1]] // k) for e in range(E)]
        plan = sm.Plan(BT=BT, BM=BM, BN1=BN1, BN2=BN2, GPC=gpc, PI=PERM_INLINE_RT, Q=Q)
        final = sm.expected_final_counters(sm.build_graph(T, H, F, k, [counts], [tors], plan))
        n_rt, n1m, n2, nSm = sm.layer_shape(T, H, F, plan)
        assert (n1m, nSm) == (n1, nS) and RT == sum(-(-int(c) // BM) for c in counts)
        assert ngu == RT * n1 and nd == RT * n2 * nS and nf == n_rt
        assert int(read_i32(lay[0], 1)[0]) == final[("route", 0)]
        assert int(read_i32(lay[1], 1)[0]) == 1
        assert int(read_i32(lay[15], 1)[0]) == final[("perm", 0)] == n_rt
        ev_gu = np.asarray(read_i32(lay[2], max_rt * n1)).reshape(max_rt, n1)
        rt = 0
        for e in range(E):
            for m in range(-(-int(counts[e]) // BM)):
                for s in range(nS):
                    assert ev_gu[rt, s] == final[("gu", 0, e, m, s)], (l, e, m, s)
                rt += 1
        assert not ev_gu[rt:].any() and not ev_gu[:, nS:].any()
        comb = np.asarray(read_i32(lay[3], n_rt_cap))
        done = np.asarray(read_i32(lay[4], n_rt_cap))
        for tau in range(n_rt):
            assert comb[tau] == final[("comb", 0, tau)], (l, tau)
            assert done[tau] == 1
        assert not comb[n_rt:].any() and not done[n_rt:].any()
        # router slices: every tile's slice counter ends at Q (untouched with one slice)
        rq = np.asarray(read_i32(lay[16], n_rt_cap))
        assert 1 <= Q <= 8
        for tau in range(n_rt):
            assert rq[tau] == (final[("rq", 0, tau)] if Q > 1 else 0), (l, tau, rq[tau], Q)
        assert not rq[n_rt:].any()


TRACE_KIND = {"R": 1, "S": 2, "GU": 3, "D": 4, "F": 5, "P": 6}


def check_trace_causality(records, T, H, F, k, E, gpu, layout, read_i32, layers,
                          slack_ticks=200):
    """The event tensor's dependencies, read off a trace of one call (ETC_FLAG_TRACE):
    every task of the scheduler model (built from the GPU's own routing and down split)
    has exactly one record, and no task began its body before every task whose signals
    it waits for had signalled.

    A record holds the task's claim start, the ticks spent claiming and waiting and the
    ticks running, on the device's 100 MHz clock.  A producer's signal falls between
    the start of its body and its end stamp, which is taken right after the signal, so
    a consumer's body must start no earlier than the producer's end minus slack_ticks.
    S runs inside the routing task whose signal completed ev_route; that task's record
    ends after S, so S is only required to start after every routing task started."""
    from oracle import sched_model as sm
    from moe_layer_scheduling_amd import trace

    d = trace.decode(records)
    t_run = d["start"] + d["wait"]
    t_end = t_run + d["run"]
    index = {}
    for i in range(len(d["kind"])):
        key = (int(d["kind"][i]), int(d["layer"][i]), int(d["a"][i]), int(d["b"][i]),
               int(d["c"][i]), int(d["d"][i]))
        assert key not in index, f"task recorded twice: {key}"
        index[key] = i

    def rec(task):
        f = list(task.key) + [0] * (4 - len(task.key))
        return index[(TRACE_KIND[task.kind], task.layer, *f)]

    tasks = []
    for l in range(layers):
        lay = layout(l)
        _, _, _, BT, BM, BN1, BN2 = lay[6:13]
        pw = [int(v) for v in read_i32(lay[5], 8)]
        gpc, Q = pw[5], pw[7]
        counts = gpu["counts"][l]
        sa = gpu["sa"][l]
        off = np.concatenate([[0], np.cumsum(counts)])
        tors = [list(sa[off[e]:off[e + 1]] // k) for e in range(E)]
        plan = sm.Plan(BT=BT, BM=BM, BN1=BN1, BN2=BN2, GPC=gpc, PI=PERM_INLINE_RT, Q=Q)
        R, S, P, GU, D, Fin = sm.build_layer(l, T, H, F, k, counts, plan, tors)
        tasks += R + [S] + P + GU + D + Fin
    assert len(tasks) == len(index), (len(tasks), len(index))
    producers = {}
    for t in tasks:
        for ctr, _ in t.signals:
            producers.setdefault(ctr, []).append(t)
        if t.finish is not None:  # a router slice may be the one that moves `next`
            producers.setdefault(t.finish[2], []).append(t)
    checked = 0
    for t in tasks:
        i = rec(t)
        for ctr, _ in t.waits:
            for p in {id(x): x for x in producers[ctr]}.values():
                j = rec(p)
                if t.kind == "S":
                    assert t_run[i] >= t_run[j], ("S before a routing task", t.layer, p.key)
                else:
                    assert t_run[i] >= t_end[j] - slack_ticks, (
                        f"{t.kind}{t.key} (layer {t.layer}) began {int(t_end[j] - t_run[i])} ticks "
                        f"before {p.kind}{p.key} signalled {ctr}")
                checked += 1
    return checked


def check_data_dependencies(records, T, H, k, E, gpu, layout, read_i32, layers, atomic=True,
                            slack_ticks=200):
    """The trace of one call against the data each task reads, derived from the routing
    the GPU produced and the tiling alone (not from the counters or the scheduler
    model): a task's body begins no earlier than the end of every task that writes what
    it reads, less slack_ticks.  With a counter target set too low in both the kernel
    and the model, the event-tensor checks would still pass; this one would not.

    Reads and writes, per layer:
      R (every slice of tile tau) writes xq rows of tau's tokens and, with the atomic
        combine, clears their accumulator rows; layer l+1's R of tau reads F(l, tau)'s rows.
      P(tau), or S when there are no P tasks, writes tau's entries of the permutation.
      GU(e, m, n) reads the xq rows and permutation entries of row tile (e, m).
      D(e, m, n2, s) reads the h rows of (e, m) that GU(e, m, n) wrote for n in chunk s,
        and adds into the accumulator rows of its tokens.
      F(tau) reads the accumulator rows of tau's tokens: every D whose row tile holds one.
    Returns the number of (consumer, producer) pairs checked."""
    from moe_layer_scheduling_amd import trace

    d = trace.decode(records)
    t_run = d["start"] + d["wait"]
    t_end = t_run + d["run"]
    index = {}
    for i in range(len(d["kind"])):
        index[(int(d["kind"][i]), int(d["layer"][i]), int(d["a"][i]), int(d["b"][i]),
               int(d["c"][i]), int(d["d"][i]))] = i
    K_R, K_S, K_GU, K_D, K_F, K_P = (TRACE_KIND[n] for n in ("R", "S", "GU", "D", "F", "P"))
    checked = 0

    def after(consumer, producers, what):
        nonlocal checked
        i = index[consumer]
        for pk in producers:
            j = index[pk]
            assert t_run[i] >= t_end[j] - slack_ticks, (
                f"task {consumer} began {int(t_end[j] - t_run[i])} ticks before {pk} "
                f"finished ({what})")
            checked += 1

    for l in range(layers):
        lay = layout(l)
        _, n1, _, BT, BM, BN1, BN2 = (int(v) for v in lay[6:13])
        pw = [int(v) for v in read_i32(lay[5], 8)]
        nS, gpc, Q = pw[4], pw[5], pw[7]
        n2 = -(-H // BN2)
        n_rt = -(-T // BT)
        counts = np.asarray(gpu["counts"][l])
        sa = np.asarray(gpu["sa"][l])
        off = np.concatenate([[0], np.cumsum(counts)]).astype(int)
        perm_by_p = n_rt > PERM_INLINE_RT
        d_of_tau = [[] for _ in range(n_rt)]
        for e in range(E):
            for m in range(-(-int(counts[e]) // BM)):
                rows = sa[off[e] + m * BM:min(off[e] + (m + 1) * BM, off[e + 1])]
                taus = sorted({int(t) // BT for t in rows // k})
                routing = [(K_R, l, tau * Q + q, 0, 0, 0) for tau in taus for q in range(Q)]
                perm = ([(K_P, l, tau, 0, 0, 0) for tau in taus] if perm_by_p
                        else [(K_S, l, 0, 0, 0, 0)])
                for n in range(n1):
                    after((K_GU, l, e, m, n, 0), routing + perm, "xq rows and permutation")
                for n2i in range(n2):
                    for s_ in range(nS):
                        gus = [(K_GU, l, e, m, n, 0) for n in range(s_ * gpc, min((s_ + 1) * gpc, n1))]
                        after((K_D, l, e, m, n2i, s_), gus + (routing if atomic else []),
                              "h rows of its chunk, cleared accumulator rows")
                        for tau in taus:
                            d_of_tau[tau].append((K_D, l, e, m, n2i, s_))
        for tau in range(n_rt):
            after((K_F, l, tau, 0, 0, 0), d_of_tau[tau], "accumulator rows of its tokens")
            if l + 1 < layers:
                Qn = int(read_i32(layout(l + 1)[5], 8)[7])
                for q in range(Qn):
                    after((K_R, l + 1, tau * Qn + q, 0, 0, 0), [(K_F, l, tau, 0, 0, 0)], "layer input rows")
    return checked


def check_identical_experts(x, layers, eps, out):
    """Every expert holds the same weights: whatever the routing, each token's output is
    the single FFN of its normalised input (the gates sum to 1), rounded to bfloat16.
    Returns (max error, max |reference|)."""
    from oracle.numerics import round_bf16

    lay = layers[0]
    xn = om.rmsnorm(x, lay["gamma"], eps)
    ffn = om.expert_ffn(round_bf16(xn), lay["w_gate"][0], lay["w_up"][0], lay["w_down"][0], "bf16")
    ref = round_bf16(ffn)
    err = float(np.max(np.abs(out - ref)))
    ref_max = float(np.max(np.abs(ref)))
    assert err <= OUT_TOL["bf16"] * ref_max, (err, ref_max)
    return err, ref_max


DEGENERATE = {
    # one expert, top-1: every gate is 1
    "one_expert": dict(name="one", tokens=(40,), hidden=256, experts=1, top_k=1, ffn=128, layers=2),
    # top-k = E: every expert for every token, the gates are the full softmax
    "all_experts": dict(name="all", tokens=(40,), hidden=256, experts=4, top_k=4, ffn=128, layers=1),
    # every expert with the same weights: the output does not depend on the routing
    "identical_experts": dict(name="same", tokens=(40,), hidden=256, experts=8, top_k=2, ffn=128,
                              layers=1),
}


def degenerate_case(which):
    """(config, layers, x) of a degenerate case of the method (see DEGENERATE)."""
    from moe_layer_scheduling_amd import synth

    cfg = synth.MoEConfig(**DEGENERATE[which])
    layers = synth.make_layers(cfg)
    if which == "identical_experts":
        for lay in layers:
            for key in ("w_gate", "w_up", "w_down"):
                lay[key][:] = lay[key][0:1]
    return cfg, layers, synth.make_x(cfg, 40)


def check_degenerate(which, cfg, x, layers, gpu):
    from moe_layer_scheduling_amd import synth

    st = compare(synth.as_numpy(x), synth.layers_as_numpy(layers), cfg.top_k, cfg.eps, cfg.dtype, gpu)
    if which == "one_expert":
        assert np.all(gpu["w"] == 1.0) and np.all(gpu["idx"] == 0)
    if which == "all_experts":
        for l in range(cfg.layers):
            assert np.array_equal(np.sort(gpu["idx"][l], axis=1), np.tile(np.arange(cfg.experts), (x.shape[0], 1)))
    if which == "identical_experts":
        check_identical_experts(synth.as_numpy(x), synth.layers_as_numpy(layers), cfg.eps, gpu["outs"][0])
    return st
