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
