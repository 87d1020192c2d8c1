"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: worked examples
derived by hand (tests/golden), closed forms, library routines on special cases,
brute force on tiny inputs and invariants.  CPU only.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import sfi_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(20260312)


def _rand_qkv(Hq=4, Hkv=2, n=37, D=8, scale=1.0, seed=0):
    r = np.random.default_rng(seed)
    q = r.standard_normal((Hq, D)) * scale
    K = r.standard_normal((Hkv, n, D)) * scale
    V = r.standard_normal((Hkv, n, D))
    return q, K, V


# ---------------------------------------------------------------------------- attention
def test_attention_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "fusion_and_softmax.json")))["attention"]
    q = np.array([[1.0, 0.0]])
    K = np.array([[[0.0, 0.0], [math.sqrt(2) * math.log(3), 0.0]]])
    V = np.array([g["v"]])
    o, z, lse, p = O.attention(q, K, V)
    np.testing.assert_allclose(p[0], g["p"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(o[0], g["o"], rtol=0, atol=1e-14)
    assert abs(lse[0] - math.log(4)) < 1e-15


def test_softmax_sums_to_one_and_lse():
    q, K, V = _rand_qkv(scale=3.0)
    o, z, lse, p = O.attention(q, K, V)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-14)
    assert (p >= 0).all()
    # lse is the log of the partition function of z, evaluated directly
    np.testing.assert_allclose(lse, [math.log(sum(math.exp(x) for x in row)) for row in z],
                               rtol=1e-13)


def test_attention_matches_torch_sdpa_fp64():
    Hq, Hkv, n, D = 8, 2, 53, 16
    q, K, V = _rand_qkv(Hq, Hkv, n, D, scale=2.0, seed=3)
    o, _, _, _ = O.attention(q, K, V)
    G = Hq // Hkv
    tq = torch.from_numpy(q)[None, :, None, :]                   # [1, Hq, 1, D]
    tk = torch.from_numpy(K).repeat_interleave(G, dim=0)[None]   # [1, Hq, n, D]
    tv = torch.from_numpy(V).repeat_interleave(G, dim=0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[0, :, 0].numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)


def test_attention_explicit_loops_tiny():
    q, K, V = _rand_qkv(2, 1, 5, 3, seed=5)
    o, z, lse, p = O.attention(q, K, V)
    for h in range(2):
        zz = [sum(q[h][d] * K[0][j][d] for d in range(3)) / math.sqrt(3) for j in range(5)]
        ee = [math.exp(x) for x in zz]
        tot = sum(ee)
        for d in range(3):
            ref = sum(ee[j] / tot * V[0][j][d] for j in range(5))
            assert abs(o[h][d] - ref) < 1e-13
        np.testing.assert_allclose(z[h], zz, rtol=1e-13)


def test_attention_key_permutation_invariance():
    q, K, V = _rand_qkv(seed=7)
    perm = rng.permutation(K.shape[1])
    o1, z1, l1, _ = O.attention(q, K, V)
    o2, z2, l2, _ = O.attention(q, K[:, perm], V[:, perm])
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)
    np.testing.assert_allclose(z1[:, perm], z2, atol=1e-13)


def test_lse_merge_of_splits_equals_unsplit():
    q, K, V = _rand_qkv(n=61, seed=9, scale=2.5)
    o, _, lse, _ = O.attention(q, K, V)
    cuts = [0, 7, 30, 31, 61]
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        oo, _, ll, _ = O.attention(q, K[:, a:b], V[:, a:b])
        parts.append((oo, ll))
    om, lm = O.merge_segments(parts)
    np.testing.assert_allclose(om, o, atol=1e-13)
    np.testing.assert_allclose(lm, lse, atol=1e-13)


# ------------------------------------------------------------------------------ schedule
def _schedule_by_segments(flags, budget):
    """Independent construction: slow steps are step 0, the flagged steps, and then every
    (budget+1)-th step inside each gap between consecutive such anchors."""
    B, S = flags.shape
    out = np.zeros((B, S), np.uint8)
    for b in range(B):
        anchors = sorted({0} | {s for s in range(S) if flags[b, s]})
        anchors.append(S)
        for a0, a1 in zip(anchors[:-1], anchors[1:]):
            for s in range(a0, a1, budget + 1):
                out[b, s] = 1
    return out


@pytest.mark.parametrize("budget", [0, 1, 3, 8, 32])
def test_schedule_against_direct_construction(budget):
    flags = (rng.random((5, 300)) < 0.07).astype(np.uint8)
    m = O.schedule(flags, budget)
    np.testing.assert_array_equal(m, _schedule_by_segments(flags, budget))
    for b in range(5):
        run = 0
        for s in range(300):
            run = 0 if m[b, s] else run + 1
            assert run <= budget
        assert m[b, 0] == 1
        assert all(m[b, s] == 1 for s in range(300) if flags[b, s])


def test_schedule_budget_zero_is_all_slow():
    assert O.schedule(np.zeros((2, 9), np.uint8), 0).all()


def test_boundary_flags_worked_example():
    tok = np.array([[5, 1001, 7, 1005], [1003, 1003, 0, 999999]])
    np.testing.assert_array_equal(O.boundary_flags(tok, (1001, 1002, 1003, 1004, 1005)),
                                  [[0, 1, 0, 1], [1, 1, 0, 0]])
    assert not O.boundary_flags(tok, ()).any()


def test_step_control_worked_example():
    """Two rows, six steps, budget 2, 10 stored positions, n_sink 1, W 4, worked by hand.
    Row 0 decodes a boundary token at step 3, row 1 at step 1; row 1's budget runs out at
    step 4.  N_s = 11 + s; a slow step at N sets the edge max(1, N - 4)."""
    B = 1001
    tok = np.array([[7, 8, 9, B, 10, 11],
                    [7, B, 9, 10, 11, 12]])
    st = O.step_control(tok, (B,), budget=2, n_stored=10, n_sink=1, n_recent=4)
    np.testing.assert_array_equal(st["mode"].T, [[1, 0, 0, 1, 0, 0], [1, 1, 0, 0, 1, 0]])
    np.testing.assert_array_equal(st["seq_len"][:, 0], [11, 12, 13, 14, 15, 16])
    np.testing.assert_array_equal(st["recent_start"].T, [[7, 7, 7, 10, 10, 10],
                                                         [7, 8, 8, 8, 11, 11]])
    np.testing.assert_array_equal(st["slow_ids"], [[0, 1], [1, -1], [-1, -1], [0, -1],
                                                   [1, -1], [-1, -1]])
    np.testing.assert_array_equal(st["fast_ids"], [[-1, -1], [0, -1], [0, 1], [1, -1],
                                                   [0, -1], [0, 1]])
    np.testing.assert_array_equal(st["counts"], [[2, 0], [1, 1], [0, 2], [1, 1], [1, 1],
                                                 [0, 2]])
    # a purely sliding window follows every step: max(1, N - 4)
    sl = O.step_control(tok, (B,), budget=2, n_stored=10, n_sink=1, n_recent=4, sliding=True)
    np.testing.assert_array_equal(sl["recent_start"].T, [[7, 8, 9, 10, 11, 12]] * 2)
    np.testing.assert_array_equal(sl["mode"], st["mode"])
    # budget 0: every step is slow; no boundary and a long budget: only the first step
    assert O.step_control(tok, (B,), 0, 10, 1, 4)["mode"].all()
    m = O.step_control(tok, (), 100, 10, 1, 4)["mode"]
    assert m[0].all() and not m[1:].any()


def test_sliding_fast_step_attends_to_sink_selection_and_newest_window():
    """With a purely sliding window a fast step attends to exactly the sink, the slow step's
    selection and the newest W positions: a softmax over that set written out by hand."""
    r = np.random.default_rng(21)
    Hq, Hkv, D, ctx, S = 4, 2, 8, 60, 7
    n_sink, W, K = 2, 6, 5
    q = r.standard_normal((S, Hq, D))
    Kc = r.standard_normal((Hkv, ctx + S, D))
    Vc = r.standard_normal((Hkv, ctx + S, D))
    flags = np.zeros(S, np.uint8)
    recs = O.run_sequence(q, Kc, Vc, flags, ctx, n_sink, W, K, 1, 0.5, 0.5, 0.3, budget=100,
                          sliding=True)
    sel = recs[0].selection.sel
    G = Hq // Hkv
    for rec in recs[1:]:
        N = rec.N
        assert rec.recent_start == N - W
        for h in range(Hq):
            g = h // G
            keep = sorted(set(range(n_sink)) | set(int(j) for j in sel[g] if j >= 0)
                          | set(range(N - W, N)))
            z = np.array([q[rec.step, h] @ Kc[g, j] / math.sqrt(D) for j in keep])
            p = np.exp(z - z.max())
            p /= p.sum()
            o = sum(p[i] * Vc[g, j] for i, j in enumerate(keep))
            np.testing.assert_allclose(rec.o[h], o, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------------------ Selector
def test_evidence_is_distribution():
    q, K, V = _rand_qkv(Hq=8, Hkv=2, n=40, seed=11)
    _, _, _, p = O.attention(q, K, V)
    f = O.evidence(p, 2)
    np.testing.assert_allclose(f.sum(axis=1), 1.0, atol=1e-14)
    assert (f >= 0).all()
    # one query head per KV head: f is that head's distribution
    np.testing.assert_allclose(O.evidence(p, 8), p, atol=0)


def test_evidence_grouping_worked_example():
    """Two KV heads of two query heads each: each KV head's f is the mean of its own query
    heads' rows (h div G), evaluated by hand in the golden file.  An interleaved grouping
    (h mod Hkv) gives different values there, so it fails this pin."""
    g = json.load(open(os.path.join(GOLDEN, "evidence_grouping.json")))
    p = np.array(g["p"])
    f = O.evidence(p, g["num_kv_heads"])
    np.testing.assert_allclose(f, g["f"], rtol=0, atol=1e-15)
    assert np.abs(f - np.array(g["f_interleaved_wrong"])).max() > 0.1
    # the same grouping when the evidence is pooled over a window of two slots
    P = np.stack([p, p[g["window_slot1_head_order"]]])
    fw = O.window_evidence(P, g["num_kv_heads"])
    np.testing.assert_allclose(fw, g["f_window2"], rtol=0, atol=1e-15)


def test_window_evidence_worked_example():
    """Two slots, two query heads of one KV head, three positions, summed by hand:
    f = (0.5+0.2+1+0, 0.25+0.3+0+0, 0.25+0.5+0+1) / 4."""
    P = np.array([[[0.5, 0.25, 0.25], [0.2, 0.3, 0.5]],
                  [[1.0, 0.0, 0.0], [0.0, 0.0, 1.0]]])
    np.testing.assert_allclose(O.window_evidence(P, 1), [[0.425, 0.1375, 0.4375]], atol=1e-15)


def test_window_evidence_reduces_to_single_query_evidence():
    q, K, V = _rand_qkv(Hq=8, Hkv=2, n=40, seed=12)
    _, _, _, p = O.attention(q, K, V)
    # a window of one slot, and a window whose slots all hold the same query
    np.testing.assert_allclose(O.window_evidence(p[None], 2), O.evidence(p, 2), atol=1e-16)
    np.testing.assert_allclose(O.window_evidence(np.stack([p] * 3), 2), O.evidence(p, 2),
                               atol=1e-16)


def test_window_evidence_is_the_mean_of_per_slot_evidence():
    """Linearity: pooling over the window equals averaging each slot's own evidence; the
    result is a distribution and does not depend on the order of the slots."""
    r = np.random.default_rng(13)
    Q = r.standard_normal((4, 8, 8))
    _, K, V = _rand_qkv(Hq=8, Hkv=2, n=33, seed=13)
    P = np.stack([O.attention(Q[k], K, V)[3] for k in range(4)])
    f = O.window_evidence(P, 2)
    np.testing.assert_allclose(f, np.mean([O.evidence(P[k], 2) for k in range(4)], axis=0),
                               atol=1e-15)
    np.testing.assert_allclose(f.sum(axis=1), 1.0, atol=1e-14)
    np.testing.assert_allclose(O.window_evidence(P[[2, 0, 3, 1]], 2), f, atol=1e-15)


def test_window_queries_slots():
    q = np.arange(5 * 2 * 3, dtype=float).reshape(5, 2, 3)
    Wq = O.window_queries(q, 3, 3)
    for k, step in enumerate((3, 2, 1)):
        np.testing.assert_array_equal(Wq[k], q[step])
    # at the first steps the missing slots repeat the first query
    np.testing.assert_array_equal(O.window_queries(q, 0, 3), np.stack([q[0]] * 3))
    np.testing.assert_array_equal(O.window_queries(q, 1, 3), np.stack([q[1], q[0], q[0]]))


def test_window_selector_keeps_what_each_slot_attends_to():
    """Slot 0 attends to position 10, slot 1 to position 30 (one KV head, no prior, no
    refinement).  With K = 2 the current query alone keeps 10 and its next-largest
    position; the window keeps 10 and 30."""
    N = 48
    P = np.full((2, 1, N), 0.1 / (N - 1))
    P[0, 0, 10] = 0.9
    P[1, 0, 30] = 0.9
    P[0, 0, 20] = P[0, 0, 20] + 1e-3
    P[0, 0] /= P[0, 0].sum()
    norms = np.ones((1, N))
    kw = dict(N=N, num_kv_heads=1, n_sink=2, n_recent=4, top_k=2, R=0, alpha_soft=0.0,
              alpha_cross=0.0, lam=0.0)
    np.testing.assert_array_equal(O.select(P[0], norms, **kw).sel, [[10, 20]])
    np.testing.assert_array_equal(O.select_window(P, norms, **kw).sel, [[10, 30]])
    # identical slots: the window changes nothing
    same = np.stack([P[0]] * 2)
    np.testing.assert_array_equal(O.select_window(same, norms, **kw).sel,
                                  O.select(P[0], norms, **kw).sel)


def test_refine_greedy_worked_example():
    """One head, R = 1, α_soft = 0.5, scores 0.1 0.5 0.4 0.45 0.05, by hand.  Greedy: take
    1 (0.5), halving 0 and 2 to 0.05 and 0.2; take 3 (0.45), halving 2 to 0.1 and 4 to
    0.025; then 2, 0, 4.  The one-pass reading halves only the initially dominated 0, 2, 4:
    position 2 ends at 0.2 instead of 0.1."""
    s = np.array([[0.1, 0.5, 0.4, 0.45, 0.05]])
    np.testing.assert_allclose(O.refine_greedy(s, 0, 5, 1, 0.5, 0.0),
                               [[0.05, 0.5, 0.1, 0.45, 0.025]], rtol=1e-15)
    np.testing.assert_allclose(np.exp(O.refine(s, 0, 5, 1, 0.5, 0.0).ellp),
                               [[0.05, 0.5, 0.2, 0.45, 0.025]], rtol=1e-15)


def _greedy_quadratic(cur, R, a):
    """The greedy taken one argmax at a time over a plain list (no heap)."""
    val = list(cur)
    n = len(val)
    taken = [False] * n
    final = [0.0] * n
    for _ in range(n):
        best = None
        for c in range(n):
            if not taken[c] and (best is None or val[c] > val[best]):
                best = c
        taken[best] = True
        final[best] = val[best]
        for d in range(max(0, best - R), min(n, best + R + 1)):
            if not taken[d]:
                val[d] *= 1.0 - a
    return final


def test_refine_greedy_matches_quadratic_simulation_and_reductions():
    r = np.random.default_rng(31)
    for trial in range(20):
        Hkv, n, R = 3, 40, int(r.integers(0, 5))
        a_s, a_c = float(r.choice([0.0, 0.3, 0.5, 1.0])), float(r.choice([0.0, 0.5, 1.0]))
        s = r.random((Hkv, n + 6))
        if trial % 4 == 0:
            s = np.round(s * 4) / 4 + 0.01           # many exact ties
        lo, hi = 2, n + 2
        got = O.refine_greedy(s, lo, hi, R, a_s, a_c)
        own = np.argmax(s[:, lo:hi], axis=0)
        for g in range(Hkv):
            cur = s[g, lo:hi] * np.where(own != g, 1.0 - a_c, 1.0)
            np.testing.assert_allclose(got[g], _greedy_quadratic(cur, R, a_s), rtol=0, atol=0)
        # no penalty or no neighbours: only exclusivity is left, as in the one-pass reading
        base = np.exp(O.refine(s, lo, hi, R, 0.0, a_c).ellp)
        np.testing.assert_allclose(O.refine_greedy(s, lo, hi, R, 0.0, a_c), base, rtol=1e-15)
        np.testing.assert_allclose(O.refine_greedy(s, lo, hi, 0, a_s, a_c),
                                   np.exp(O.refine(s, lo, hi, 0, a_s, a_c).ellp), rtol=1e-15)


def test_refine_greedy_hard_nms_at_alpha_one():
    """α_soft = 1 is hard NMS: the kept positions are at least R + 1 apart, the first is the
    global maximum, and every dropped position has a kept neighbour within R."""
    r = np.random.default_rng(32)
    s = r.random((1, 200))
    R = 3
    fin = O.refine_greedy(s, 0, 200, R, 1.0, 0.0)[0]
    kept = np.nonzero(fin > 0)[0]
    assert np.all(np.diff(kept) > R)
    assert int(np.argmax(s[0])) in kept
    for j in np.nonzero(fin == 0)[0]:
        assert np.any(np.abs(kept - j) <= R)


def test_key_norms_library():
    K = rng.standard_normal((3, 20, 16))
    np.testing.assert_allclose(O.key_norms(K), np.sqrt((K ** 2).sum(-1)), rtol=1e-14)


def test_prior_worked_example():
    """The prior's form as read (key-norm floor, distance from the newest position counted
    N-1-j, the +1 terms, the normalisation over [0, N)) against hand-derived values (golden)."""
    g = json.load(open(os.path.join(GOLDEN, "prior_worked_example.json")))
    np.testing.assert_allclose(O.prior(np.array(g["norms"])), np.array(g["r"]), rtol=1e-14,
                               atol=0)


def test_prior_invariants():
    norms = np.exp(rng.standard_normal((3, 50)))
    r = O.prior(norms)
    np.testing.assert_allclose(r.sum(axis=1), 1.0, atol=1e-14)
    assert (r > 0).all()
    # equal norms: depends on position only and grows with distance from the newest
    re = O.prior(np.full((2, 50), 1.7))
    np.testing.assert_allclose(re[0], re[1], atol=0)
    assert (np.diff(re[0]) < 0).all()
    # a larger key norm lowers that position's prior (key-norm suppression)
    n2 = norms.copy()
    n2[1, 20] *= 4.0
    r2 = O.prior(n2)
    assert r2[1, 20] < r[1, 20]
    # common rescaling of every norm does not change the distribution
    np.testing.assert_allclose(O.prior(norms * 3.0), r, rtol=1e-13)
    # the 1e-6 floor keeps zero-norm keys finite
    z = norms.copy()
    z[0, 3] = 0.0
    assert np.isfinite(O.prior(z)).all()


def test_fusion_worked_example_and_endpoints():
    g = json.load(open(os.path.join(GOLDEN, "fusion_and_softmax.json")))["fusion"]
    s = O.fuse(np.array(g["f"]), np.array(g["r"]), g["lambda"])
    np.testing.assert_allclose(s, g["s"], atol=1e-16)
    f = rng.dirichlet(np.ones(30), size=2)
    r = rng.dirichlet(np.ones(30), size=2)
    np.testing.assert_array_equal(O.fuse(f, r, 0.0), f)
    np.testing.assert_array_equal(O.fuse(f, r, 1.0), r)
    np.testing.assert_allclose(O.fuse(f, r, 0.3).sum(axis=1), 1.0, atol=1e-14)


def test_adaptive_lambda_worked_examples():
    """The clipped adaptive fusion weight min(λclip, H(f)/ln N) on hand-evaluated entropies
    (golden), the point-mass and uniform limits, and λclip = 0 (evidence only)."""
    g = json.load(open(os.path.join(GOLDEN, "adaptive_lambda.json")))
    f4 = np.array(g["f4"])
    np.testing.assert_allclose(O.adaptive_lambda(f4, 0.8), g["lam_clip08"], atol=1e-15)
    np.testing.assert_allclose(O.adaptive_lambda(f4, 0.3), g["lam_clip03"], atol=1e-15)
    np.testing.assert_allclose(O.adaptive_lambda(np.array(g["f8"]), 1.0), g["lam8_clip1"],
                               atol=1e-15)
    np.testing.assert_array_equal(O.adaptive_lambda(np.array([[0.0, 1.0, 0.0]]), 0.9), [0.0])
    np.testing.assert_array_equal(O.adaptive_lambda(np.array([[1.0]]), 0.9), [0.0])
    np.testing.assert_array_equal(O.adaptive_lambda(f4, 0.0), [0.0, 0.0])
    s = O.fuse_per_head(f4[:1], np.full((1, 4), 0.25), [0.5])
    np.testing.assert_allclose(s[0], g["fused_f0_uniform_half"], atol=1e-15)


def test_adaptive_lambda_grows_with_flatness_and_keeps_a_distribution():
    N = 50
    point = np.zeros(N)
    point[7] = 1.0
    lams = [O.adaptive_lambda(((1 - t) * point + t / N)[None, :], 1.0)[0]
            for t in np.linspace(0, 1, 11)]
    assert lams[0] == 0.0 and abs(lams[-1] - 1.0) < 1e-12
    assert all(b > a for a, b in zip(lams, lams[1:]))
    q, K, V = _rand_qkv(Hq=8, Hkv=2, n=N, seed=21, scale=2.0)
    _, _, _, p = O.attention(q, K, V)
    f = O.evidence(p, 2)
    r = O.prior(O.key_norms(K))
    lam = O.adaptive_lambda(f, 0.3)
    assert ((lam >= 0) & (lam <= 0.3)).all()
    s = O.fuse_per_head(f, r, lam)
    np.testing.assert_allclose(s.sum(axis=1), 1.0, atol=1e-14)
    # the Selector with the adaptive weight equals the fixed-weight Selector at those weights
    # for one head (per-head weights only differ across heads)
    sel = O.select_from_evidence(f, O.key_norms(K), N, 4, 8, 10, 2, 0.5, 0.5, 0.7, 0.3)
    np.testing.assert_allclose(sel.s, s, atol=1e-15)


def _kl_objective(s, f, r, lam):
    s = np.clip(s, 1e-300, None)
    return (1 - lam) * np.sum(f * np.log(f / s)) + lam * np.sum(r * np.log(r / s))


@pytest.mark.parametrize("lam", [0.1, 0.3, 0.7])
def test_fusion_is_kl_minimiser(lam):
    from scipy.optimize import minimize
    for n in (3, 7, 12):
        f = rng.dirichlet(np.ones(n))
        r = rng.dirichlet(np.ones(n))
        s_star = O.fuse(f, r, lam)
        res = minimize(lambda x: _kl_objective(x, f, r, lam), np.full(n, 1.0 / n),
                       method="SLSQP", bounds=[(1e-12, 1)] * n,
                       constraints=[{"type": "eq", "fun": lambda x: x.sum() - 1}],
                       options={"ftol": 1e-15, "maxiter": 1000})
        np.testing.assert_allclose(res.x, s_star, atol=1e-6)
        base = _kl_objective(s_star, f, r, lam)
        for _ in range(200):
            d = rng.standard_normal(n)
            d -= d.mean()
            d *= 1e-3 * s_star.min() / np.abs(d).max()
            assert _kl_objective(s_star + d, f, r, lam) >= base - 1e-15


def test_refine_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "selector_worked_example.json")))
    s = np.array(g["scores"], float)
    lo, hi = O.candidates(g["N"], g["n_sink"], g["n_recent"])
    assert (lo, hi) == (2, 10)
    ref = O.refine(s, lo, hi, g["R"], g["alpha_soft"], g["alpha_cross"])
    np.testing.assert_array_equal(ref.dom.astype(int), g["dom"])
    owner = np.where(~ref.exc[0], 0, 1)
    np.testing.assert_array_equal(owner, g["owner"])
    np.testing.assert_allclose(np.exp(ref.ellp), np.array(g["refined"], float), rtol=1e-14)
    for K, key in ((3, "top3"), (2, "top2")):
        sel = O.select_from_scores(s, g["N"], g["n_sink"], g["n_recent"], K, g["R"],
                                   g["alpha_soft"], g["alpha_cross"])
        np.testing.assert_array_equal(sel, g[key])


def test_refine_identity_at_zero_alpha():
    s = rng.dirichlet(np.ones(80), size=3)
    ref = O.refine(s, 4, 70, 4, 0.0, 0.0)
    np.testing.assert_array_equal(ref.ellp, np.log(s[:, 4:70]))


def test_refine_soft_one_keeps_only_local_maxima():
    from scipy.ndimage import maximum_filter1d
    for R in (1, 3, 8):
        s = rng.dirichlet(np.ones(120), size=3)
        lo, hi = 5, 100
        ref = O.refine(s, lo, hi, R, 1.0, 0.0)
        ell = np.log(s[:, lo:hi])
        mx = maximum_filter1d(ell, size=2 * R + 1, axis=1, mode="constant", cval=-np.inf)
        np.testing.assert_array_equal(np.isfinite(ref.ellp), ell >= mx)


def test_refine_cross_one_keeps_only_owned():
    s = rng.dirichlet(np.ones(90), size=4)
    lo, hi = 3, 80
    ref = O.refine(s, lo, hi, 2, 0.0, 1.0)
    owner = np.argmax(s[:, lo:hi], axis=0)
    for g in range(4):
        np.testing.assert_array_equal(np.isfinite(ref.ellp[g]), owner == g)
    # each head owns >= K candidates here, so the selections are pairwise disjoint
    counts = np.bincount(owner, minlength=4)
    K = int(counts.min())
    sel = O.topk(ref.ellp, lo, K)
    sets = [set(row.tolist()) for row in sel]
    for a, b in itertools.combinations(range(4), 2):
        assert not (sets[a] & sets[b])


def test_refine_single_head_has_no_exclusivity():
    s = rng.dirichlet(np.ones(30), size=1)
    ref = O.refine(s, 0, 30, 2, 0.0, 0.9)
    assert not ref.exc.any()


def _brute_topk(vals, K):
    n = len(vals)
    best = None
    for sub in itertools.combinations(range(n), K):
        key = (sum(vals[i] for i in sub), tuple(-i for i in sub))
        if best is None or key > best[0]:
            best = (key, sub)
    return list(best[1])


def test_topk_brute_force_with_ties():
    for trial in range(60):
        n = int(rng.integers(1, 11))
        K = int(rng.integers(1, n + 1))
        # small integers force many exact ties
        vals = rng.integers(-3, 4, size=n).astype(float)
        sel = O.topk(vals[None, :], 10, K)[0]
        assert list(sel - 10) == _brute_topk(list(vals), K)


def test_topk_padding_and_order():
    ellp = np.log(rng.dirichlet(np.ones(6), size=2))
    sel = O.topk(ellp, 4, 9)
    assert (sel[:, 6:] == -1).all()
    assert (np.diff(sel[:, :6], axis=1) > 0).all()
    assert set(sel[0, :6]) == set(range(4, 10))
    sel0 = O.topk(np.zeros((2, 0)), 4, 3)
    assert (sel0 == -1).all()


def test_topk_with_neg_inf_scores():
    v = np.array([[-np.inf, 0.0, -np.inf, -1.0, -np.inf]])
    np.testing.assert_array_equal(O.topk(v, 0, 3)[0], [0, 1, 3])


# ---------------------------------------------------------------------------------- pack
def test_pack_rows_are_stored_rows():
    K = rng.standard_normal((2, 50, 8)).astype(np.float32)
    V = rng.standard_normal((2, 50, 8)).astype(np.float32)
    sel = np.array([[7, 9, 30, -1], [5, 6, 40, 41]])
    pos, pk, pv = O.pack(K, V, sel, 3)
    assert list(pos[0]) == [0, 1, 2, 7, 9, 30]
    assert list(pos[1]) == [0, 1, 2, 5, 6, 40, 41]
    for g in range(2):
        for i, j in enumerate(pos[g]):
            assert pk[g][i].tobytes() == K[g, j].tobytes()
            assert pv[g][i].tobytes() == V[g, j].tobytes()


# ---------------------------------------------------------------------------- fast step
def test_fast_two_segments_equal_single_pass():
    q, K, V = _rand_qkv(Hq=6, Hkv=3, n=70, D=8, seed=13, scale=2.0)
    packed = [np.array([0, 1, 5, 9, 20]), np.array([0, 1, 2, 3]), np.array([0, 1, 44])]
    a = O.fast_attention(q, K, V, packed, 50, 70)
    b = O.fast_attention_single_pass(q, K, V, packed, 50, 70)
    np.testing.assert_allclose(a[0], b[0], atol=1e-13)
    np.testing.assert_allclose(a[1], b[1], atol=1e-13)


def test_fast_equals_dense_when_k_covers_candidates():
    """With K >= |C| every fast step equals dense attention: sink, selected memory and
    recent segment then cover the whole history."""
    Hq, Hkv, D, ctx, S = 4, 2, 8, 60, 25
    r = np.random.default_rng(17)
    K = r.standard_normal((Hkv, ctx + S, D)) * 2
    V = r.standard_normal((Hkv, ctx + S, D))
    q = r.standard_normal((S, Hq, D)) * 2
    flags = (r.random(S) < 0.2).astype(np.uint8)
    recs = O.run_sequence(q, K, V, flags, ctx, 3, 8, 10_000, 2, 0.5, 0.5, 0.3, 5)
    assert any(rc.mode == 0 for rc in recs) and sum(rc.mode for rc in recs) > 1
    for rc in recs:
        o, _, lse, _ = O.attention(q[rc.step], K[:, :rc.N], V[:, :rc.N])
        np.testing.assert_allclose(rc.o, o, atol=1e-12)
        np.testing.assert_allclose(rc.lse, lse, atol=1e-12)


def test_fast_memory_partitions_history():
    """Sink, candidates and the frozen-edge recent window cover [0, N) exactly once."""
    for N0, W, ns in ((100, 10, 4), (10, 20, 4), (5, 1, 4), (64, 60, 4)):
        lo, hi = O.candidates(N0, ns, W)
        rs = O.recent_start_at(N0, ns, W)
        assert hi == rs
        for c in range(0, 6):
            N = N0 + c
            cover = list(range(0, ns)) + list(range(lo, hi)) + list(range(rs, N))
            assert sorted(cover) == list(range(N)) or N0 < ns


def test_packed_positions_brute_force():
    """The compact buffer's positions are the sink tokens, then the selection in the order
    sfi_select writes it (ascending), with the -1 padding dropped; pack gathers exactly those
    rows."""
    r = np.random.default_rng(23)
    for n_sink, K, N in ((4, 6, 40), (0, 5, 12), (3, 1, 9), (2, 7, 7)):
        keff = int(r.integers(0, K + 1))
        chosen = np.sort(r.choice(np.arange(n_sink, N), min(keff, N - n_sink), replace=False))
        sel = np.full(K, -1)
        sel[:len(chosen)] = chosen
        want = []
        for p in range(n_sink):
            want.append(p)
        for p in chosen:
            want.append(int(p))
        assert O.packed_positions(sel, n_sink).tolist() == want
        Kt = r.standard_normal((1, N, 3))
        Vt = r.standard_normal((1, N, 3))
        pos, pk, pv = O.pack(Kt, Vt, sel[None, :], n_sink)
        assert pos[0].tolist() == want
        for i, p in enumerate(want):
            assert (pk[0][i] == Kt[0, p]).all() and (pv[0][i] == Vt[0, p]).all()


def test_greedy_selection_without_soft_nms_is_the_one_pass_selection():
    """With alpha_soft = 0 neither reading of soft-NMS scales a score, so the greedy
    selection equals the one-pass one (exclusivity applies the same in both)."""
    r = np.random.default_rng(29)
    for Hkv, N, K, R, a_c in ((1, 50, 10, 2, 0.5), (3, 80, 17, 4, 0.3), (2, 30, 40, 1, 1.0)):
        s = r.random((Hkv, N))
        s[:, 7] = s[:, 8]  # an exact tie between neighbours
        np.testing.assert_array_equal(
            O.select_greedy_from_scores(s, N, 3, 5, K, R, 0.0, a_c),
            O.select_from_scores(s, N, 3, 5, K, R, 0.0, a_c))


def test_sliding_recent_segment():
    """The sliding reading keeps exactly the newest min(W, N - n_sink) positions (never a
    sink position), and at a slow step it starts where the frozen reading does."""
    for N, ns, W in ((100, 4, 10), (12, 4, 10), (4, 4, 3), (50, 0, 50), (51, 0, 50)):
        rs = O.recent_start_sliding(N, ns, W)
        assert N - rs == min(W, max(N - ns, 0)) and rs >= ns
        assert rs == O.recent_start_at(N, ns, W)
