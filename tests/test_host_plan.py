"""The host plan of a trajectory (engine.make_plan / engine.schedule) against the oracle's
schedule and recent-segment edges.  CPU only: the plan is host arithmetic.

The GPU parity tests take slow/fast decisions and recent edges from the oracle and assert
that the engine's plan agrees; these tests cover the plan itself over many flag patterns,
budgets and window sizes, including the sliding edge and the selected-row counts."""
import numpy as np
import pytest

from oracle import sfi_oracle as O
from sparse_kv_attention_decode_amd.engine import make_plan, schedule

rng = np.random.default_rng(77)


def _oracle_tables(flags, context, budget, n_sink, n_recent, top_k, sliding):
    """mode [B, S], recent edge [S, B] and K_eff [S, B] from the oracle's readings: the edge
    in force at a step is the one of the last slow step (recent_start_at), or with a sliding
    window the newest W positions (recent_start_sliding); K_eff is the size of the last slow
    step's selection, min(K, |C|)."""
    mode = O.schedule(flags, budget)
    B, S = flags.shape
    edge = np.zeros((S, B), np.int64)
    keff = np.zeros((S, B), np.int64)
    for b in range(B):
        e = k = 0
        for s in range(S):
            N = context + s
            if mode[b, s]:
                e = O.recent_start_at(N, n_sink, n_recent)
                lo, hi = O.candidates(N, n_sink, n_recent)
                k = min(top_k, hi - lo)
            elif sliding:
                e = O.recent_start_sliding(N, n_sink, n_recent)
            edge[s, b] = e
            keff[s, b] = k
    return mode, edge, keff


@pytest.mark.parametrize("budget", [0, 1, 4, 32])
@pytest.mark.parametrize("sliding", [False, True])
@pytest.mark.parametrize("context,n_sink,n_recent,top_k", [
    (1024, 4, 64, 128),      # the tiny workload's shape
    (40, 4, 64, 16),         # no candidates: N - W <= n_sink
    (300, 0, 0, 1000),       # no sink, no recent window, K > |C|
    (8192, 4, 256, 1024),
])
def test_plan_matches_oracle_schedule_and_edges(budget, sliding, context, n_sink, n_recent,
                                                top_k):
    B, S = 3, 120
    flags = (rng.random((B, S)) < 0.08).astype(np.uint8)
    plan = make_plan(flags, context, budget, n_sink, n_recent, top_k, sliding=sliding)
    mode, edge, keff = _oracle_tables(flags, context, budget, n_sink, n_recent, top_k, sliding)
    np.testing.assert_array_equal(plan.mode, mode)
    np.testing.assert_array_equal(schedule(flags, budget), mode)
    np.testing.assert_array_equal(plan.seq_len, (context + np.arange(S))[:, None].repeat(B, 1))
    fast = mode.T == 0
    # the edge is what a fast step reads; at slow steps the plan holds the new edge too
    np.testing.assert_array_equal(plan.recent_start[fast], edge[fast])
    np.testing.assert_array_equal(plan.recent_start[mode.T == 1], edge[mode.T == 1])
    np.testing.assert_array_equal(plan.keff, keff)
    for s in range(S):
        np.testing.assert_array_equal(plan.slow_ids[s], np.nonzero(mode[:, s])[0])
        np.testing.assert_array_equal(plan.fast_ids[s], np.nonzero(mode[:, s] == 0)[0])
    # max_recent bounds every fast step's recent segment and is reached (at least 1: it
    # sizes the split of the recent segment)
    seg = plan.seq_len - plan.recent_start
    assert plan.max_recent == max([1] + [int(x) for x in seg[fast]])


def test_plan_of_the_seeded_workloads_matches_the_oracle():
    """The flags the generator draws for every workload give the oracle's schedule."""
    from workload import get, WORKLOADS
    from workload.gen import gen_flags
    for name in WORKLOADS:
        w = get(name)
        flags = gen_flags(w).numpy()
        plan = make_plan(flags, w.context, w.refresh_budget, w.n_sink, w.n_recent, w.top_k,
                         sliding=w.sliding_recent)
        mode, edge, _ = _oracle_tables(flags, w.context, w.refresh_budget, w.n_sink,
                                       w.n_recent, w.top_k, w.sliding_recent)
        np.testing.assert_array_equal(plan.mode, mode, err_msg=name)
        np.testing.assert_array_equal(plan.recent_start, edge, err_msg=name)


def test_incremental_pack_slot_model():
    """The slot arithmetic of the incremental pack (tests' model of the documented order,
    which the GPU test compares slot by slot with the device) over seeded random selection
    sequences: the buffer always holds exactly sink + selection, kept rows never move, freed
    slots are refilled first in slot order, and nothing lies past the new length."""
    import sys, os
    sys.path.insert(0, os.path.dirname(__file__))
    from sfi_testlib import model_pack_update
    r = np.random.default_rng(9)
    n_sink, K, lo, hi = 4, 60, 4, 400
    cap = (n_sink + K + 15) // 16 * 16
    for trial in range(40):
        ppos, plen = [-1] * cap, 0
        sel = np.sort(r.choice(np.arange(lo, hi), int(r.integers(10, K)), replace=False))
        for step in range(12):
            prev, prev_len = list(ppos), plen
            ppos, plen = model_pack_update(ppos, plen, sel, n_sink)
            assert plen == n_sink + len(sel)
            assert ppos[:n_sink] == list(range(n_sink))
            assert sorted(ppos[n_sink:plen]) == sorted(sel.tolist())
            assert all(x == -1 for x in ppos[plen:])
            rebuilt = prev_len == 0 or len(sel) < prev_len - n_sink
            if rebuilt:
                assert ppos[n_sink:plen] == sel.tolist()
            else:
                for s in range(n_sink, prev_len):           # kept rows keep their slot
                    if prev[s] in set(sel.tolist()):
                        assert ppos[s] == prev[s]
                moved_in = [s for s in range(n_sink, plen) if ppos[s] != prev[s]]
                freed = [s for s in range(n_sink, prev_len) if prev[s] not in set(sel.tolist())]
                assert moved_in[:len(freed)] == freed        # freed slots are filled first
            # next selection: keep most, swap a few, grow by 0-3 or shrink now and then
            keep = r.choice(sel, int(len(sel) * r.uniform(0.7, 1.0)), replace=False)
            pool = np.setdiff1d(np.arange(lo, hi), keep)
            n_new = min(K, len(sel) + int(r.integers(-8, 4))) - len(keep)
            sel = np.sort(np.concatenate([keep, r.choice(pool, max(0, n_new), replace=False)]))
