"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on one MI355X.

Inputs come from the seeded generator on the GPU; the oracle reads host fp64 copies of
the very same stored values.  Comparison rules are in sfi_testlib.
"""
import numpy as np
import pytest
import torch

from oracle import sfi_oracle as O
from workload import get
from workload.gen import make_layer
from sfi_testlib import (check_lse, check_logits, check_out, explain_selection_diff,
                         host64, model_pack_update, oracle_layer_arrays, oracle_schedule)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sparse_kv_attention_decode_amd import lib as L
    from sparse_kv_attention_decode_amd.engine import Engine


def _setup(w, dbg=False, two_streams=True, layer=0, incremental_pack=None):
    d = make_layer(w, layer, device="cuda")
    eng = Engine(w, d["flags"], two_streams=two_streams, dbg_scores=dbg,
                 incremental_pack=incremental_pack)
    lb = eng.add_layer(d["k_cache"], d["v_cache"], d["block_table"], d["q"])
    return d, eng, lb


def _slow(eng, lb, q, N, ids=None):
    B = eng.w.batch
    seq_len = torch.full((B,), N, dtype=torch.int32, device="cuda")
    ids = eng.all_ids_d if ids is None else ids
    L.sfi_slow_attn(eng.shape, q, lb.k_cache, lb.v_cache, lb.block_table, seq_len, ids,
                    ids.numel(), eng.max_len, lb.out, lb.logits, eng.stride, lb.lse,
                    eng.ws_slow)
    return seq_len


SMALL = ["tiny_fp32_1k", "qwen3_0p6b_8k"]


def _lc(w):
    """The oracle's lambda_clip argument for a workload (None: the fixed weight lam)."""
    return w.lambda_clip if w.lambda_clip >= 0 else None


def _bits(t: torch.Tensor) -> torch.Tensor:
    """Bit pattern of a bf16 / fp32 tensor, for byte-exact comparisons."""
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.parametrize("name", SMALL)
def test_key_norms(name):
    w = get(name)
    d, eng, lb = _setup(w)
    torch.cuda.synchronize()
    for b in range(w.batch):
        ref = O.key_norms(host64(d["K"][b]))
        got = host64(lb.key_norm[b, :, :w.total_len])
        np.testing.assert_allclose(got, ref, rtol=1e-6)


@pytest.mark.parametrize("name", SMALL)
def test_slow_attention(name):
    w = get(name)
    d, eng, lb = _setup(w)
    for s in (0, 1, 7, w.steps - 1):
        N = w.seq_len(s)
        _slow(eng, lb, d["q"][s], N)
        torch.cuda.synchronize()
        for b in range(w.batch):
            q, K, V = oracle_layer_arrays(d, b)
            o, z, lse, p = O.attention(q[s], K[:, :N], V[:, :N])
            check_out(host64(lb.out[b]), o)
            check_lse(host64(lb.lse[b]), lse, p, q[s], K[:, :N])
            check_logits(host64(lb.logits[b, :, :N]), z, q[s], K[:, :N], w.head_dim)


@pytest.mark.parametrize("name", SMALL)
def test_full_kv_mode_without_logits(name):
    """logits == NULL: same output, nothing written to the logits buffer."""
    w = get(name)
    d, eng, lb = _setup(w)
    N = w.seq_len(3)
    lb.logits.fill_(7.0)
    seq_len = torch.full((w.batch,), N, dtype=torch.int32, device="cuda")
    L.sfi_slow_attn(eng.shape, d["q"][3], lb.k_cache, lb.v_cache, lb.block_table, seq_len,
                    eng.all_ids_d, w.batch, eng.max_len, lb.out, None, 0, lb.lse, eng.ws_slow)
    torch.cuda.synchronize()
    assert bool((lb.logits == 7.0).all())
    q, K, V = oracle_layer_arrays(d, 0)
    o, _, lse, p = O.attention(q[3], K[:, :N], V[:, :N])
    check_out(host64(lb.out[0]), o)
    check_lse(host64(lb.lse[0]), lse, p, q[3], K[:, :N])


def _select_and_check(w, d, eng, lb, s):
    """Slow step s on the device + Selector; checks exact Top-K on the device scores and
    the end-to-end near-tie rule against the oracle's own selection."""
    N = w.seq_len(s)
    seq_len = _slow(eng, lb, d["q"][s], N)
    L.sfi_select(eng.shape, eng.params, lb.logits, eng.stride, lb.lse, lb.key_norm, eng.stride,
                 seq_len, eng.all_ids_d, w.batch, eng.max_len, lb.sel_idx, eng.dbg_buf,
                 eng.ws_sel)
    torch.cuda.synchronize()
    stats = []
    for b in range(w.batch):
        sel_gpu = lb.sel_idx[b].cpu().numpy()
        s_gpu = host64(eng.dbg_buf[b, :, :N])
        # exact Top-K on the device's own fused scores
        ref_sel = O.select_from_scores(s_gpu, N, w.n_sink, w.n_recent, w.top_k, w.nms_radius,
                                       w.alpha_soft, w.alpha_cross)
        np.testing.assert_array_equal(sel_gpu, ref_sel)
        # fused scores against the oracle pipeline
        q, K, V = oracle_layer_arrays(d, b)
        _, _, _, p = O.attention(q[s], K[:, :N], V[:, :N])
        sel = O.select(p, O.key_norms(K[:, :N]), N, w.num_kv_heads, w.n_sink, w.n_recent,
                       w.top_k, w.nms_radius, w.alpha_soft, w.alpha_cross, w.lam, _lc(w))
        np.testing.assert_allclose(s_gpu, sel.s, rtol=1e-3, atol=1e-12)
        stats.append(explain_selection_diff(sel_gpu, sel, N))
    return stats


@pytest.mark.parametrize("name", SMALL)
def test_select(name):
    w = get(name)
    d, eng, lb = _setup(w, dbg=True)
    for s in (0, 9):
        stats = _select_and_check(w, d, eng, lb, s)
        print(name, "step", s, "(diff, kth-ties, decision-ties) per row:", stats)


@pytest.mark.parametrize("name", SMALL)
@pytest.mark.parametrize("clip", [0.3, 0.9])
def test_select_adaptive_lambda(name, clip):
    """The clipped adaptive fusion weight (lambda_clip): fused scores against the oracle,
    exact Top-K on the device's own scores, the near-tie rule end to end."""
    w = get(name).replace(lambda_clip=clip, name=f"{name}_clip{clip}")
    d, eng, lb = _setup(w, dbg=True)
    for s in (0, 9):
        stats = _select_and_check(w, d, eng, lb, s)
        print(name, "clip", clip, "step", s, "(diff, kth, decision, score) per row:", stats)


@pytest.mark.parametrize("name", SMALL)
@pytest.mark.parametrize("clip", [None, 0.3])
def test_select_greedy_soft_nms(name, clip):
    """Greedy soft-NMS on the device (nms_greedy = 1): the selection equals the oracle's
    greedy reading (refine_greedy, then Top-K) run on the device's own fused scores, and
    the fused scores match the oracle's; also with the adaptive fusion weight."""
    w = get(name).replace(nms_greedy=True, lambda_clip=-1.0 if clip is None else clip,
                          name=f"{name}_greedy")
    d, eng, lb = _setup(w, dbg=True)
    for s in (0, 9):
        N = w.seq_len(s)
        seq_len = _slow(eng, lb, d["q"][s], N)
        L.sfi_select(eng.shape, eng.params, lb.logits, eng.stride, lb.lse, lb.key_norm,
                     eng.stride, seq_len, eng.all_ids_d, w.batch, eng.max_len, lb.sel_idx,
                     eng.dbg_buf, eng.ws_sel)
        torch.cuda.synchronize()
        for b in range(w.batch):
            sel_gpu = lb.sel_idx[b].cpu().numpy()
            s_gpu = host64(eng.dbg_buf[b, :, :N])
            ref = O.select_greedy_from_scores(s_gpu, N, w.n_sink, w.n_recent, w.top_k,
                                              w.nms_radius, w.alpha_soft, w.alpha_cross)
            np.testing.assert_array_equal(sel_gpu, ref)
            q, K, V = oracle_layer_arrays(d, b)
            _, _, _, p = O.attention(q[s], K[:, :N], V[:, :N])
            sel = O.select(p, O.key_norms(K[:, :N]), N, w.num_kv_heads, w.n_sink, w.n_recent,
                           w.top_k, w.nms_radius, w.alpha_soft, w.alpha_cross, w.lam, _lc(w))
            np.testing.assert_allclose(s_gpu, sel.s, rtol=1e-3, atol=1e-12)
            one_pass = O.select_from_scores(s_gpu, N, w.n_sink, w.n_recent, w.top_k,
                                            w.nms_radius, w.alpha_soft, w.alpha_cross)
            jac = [len(set(a) & set(c)) / max(1, len(set(a) | set(c)))
                   for a, c in zip(sel_gpu, one_pass)]
            print(name, "step", s, "row", b, "greedy vs one-pass Jaccard per head:",
                  np.round(jac, 3).tolist())


@pytest.mark.parametrize("name", SMALL)
def test_pack_bit_exact(name):
    w = get(name)
    d, eng, lb = _setup(w, dbg=True)
    _select_and_check(w, d, eng, lb, 0)
    L.sfi_pack(eng.shape, eng.params, lb.k_cache, lb.v_cache, lb.block_table, lb.sel_idx,
               eng.all_ids_d, w.batch, lb.packed_k, lb.packed_v, lb.packed_pos, lb.packed_len,
               eng.packed_cap)
    torch.cuda.synchronize()
    for b in range(w.batch):
        sel = lb.sel_idx[b].cpu().numpy()
        pk = lb.packed_k[b].cpu()
        pv = lb.packed_v[b].cpu()
        ppos = lb.packed_pos[b].cpu().numpy()
        plen = lb.packed_len[b].cpu().numpy()
        Kb, Vb = d["K"][b].cpu(), d["V"][b].cpu()
        for g in range(w.num_kv_heads):
            pos = O.packed_positions(sel[g], w.n_sink)
            n = len(pos)
            assert plen[g] == n
            np.testing.assert_array_equal(ppos[g, :n], pos)
            assert (ppos[g, n:] == -1).all()
            assert (np.diff(pos[w.n_sink:]) > 0).all()
            idx = torch.from_numpy(pos)
            assert torch.equal(_bits(pk[g, :n]), _bits(Kb[g, idx]))
            assert torch.equal(_bits(pv[g, :n]), _bits(Vb[g, idx]))
            assert bool((_bits(pk[g, n:]) == 0).all()) and bool((_bits(pv[g, n:]) == 0).all())


# Four rows, an odd context and a 600-position recent window: the fast calls split that
# window into eight half-size paged splits with a ragged last one (the split plan gives paged
# splits half the tiles of packed ones).
RAGGED_RECENT = dict(batch=4, context=6000, n_recent=600, top_k=1500, steps=40, refresh_budget=8,
                     name="ragged_recent_b4")


@pytest.mark.parametrize("name,win,sliding,inc,over", [(n, 1, False, None, None) for n in SMALL] +
                         [("tiny_fp32_1k", 3, False, None, None),
                          ("qwen3_0p6b_8k", 4, False, None, None),
                          ("qwen3_0p6b_8k", 1, True, None, None),
                          ("tiny_fp32_1k", 1, False, True, None),
                          ("qwen3_0p6b_8k", 1, False, True, None),
                          pytest.param("qwen3_0p6b_8k", 1, False, True, RAGGED_RECENT,
                                       id="ragged_recent_b4"),
                          pytest.param("qwen3_0p6b_8k", 1, False, None,
                                       dict(lambda_clip=0.3, name="lambda_clip_8k"),
                                       id="lambda_clip"),
                          pytest.param("qwen3_0p6b_8k", 1, False, True,
                                       dict(batch=48, context=1536, num_q_heads=8,
                                            num_kv_heads=4, top_k=256, n_recent=128, steps=10,
                                            name="batch48"),
                                       id="batch48_incremental")])
def test_trajectory_lockstep(name, win, sliding, inc, over):
    """Every step of the seeded trajectory through the two-stream engine.  Slow steps:
    dense output and the selection (near-tie rule); the oracle then continues with the
    device's selection (teacher forcing) so the two cannot drift.  Fast steps: the
    two-segment output against the oracle's fast step on the same memory.  win > 1 pools
    the Selector's evidence over that many decode queries; sliding moves the recent
    segment to the newest W positions at every step; inc forces the incremental pack (a
    one-layer engine packs in full by default); over replaces workload fields."""
    w = get(name).replace(evidence_window=win, sliding_recent=sliding, **(over or {}))
    d, eng, lb = _setup(w, incremental_pack=inc)
    B = w.batch
    omode = oracle_schedule(w, d["flags"], eng.plan)
    host = [oracle_layer_arrays(d, b) for b in range(B)]
    norms = [O.key_norms(K) for _, K, _ in host]
    packed = [None] * B
    rstart = [0] * B
    worst = 0.0
    n_slow = n_fast = 0
    for s in range(w.steps):
        eng.step(s)
        torch.cuda.synchronize()
        N = w.seq_len(s)
        out = host64(lb.out)
        mode = omode[:, s]
        for b in range(B):
            q, K, V = host[b]
            if mode[b]:
                n_slow += 1
                o, z, lse, p = O.attention(q[s], K[:, :N], V[:, :N])
                worst = max(worst, check_out(out[b], o, f"slow s={s} b={b}"))
                if win == 1:
                    sel = O.select(p, norms[b][:, :N], N, w.num_kv_heads, w.n_sink,
                                   w.n_recent, w.top_k, w.nms_radius, w.alpha_soft,
                                   w.alpha_cross, w.lam, _lc(w))
                else:
                    Qw = O.window_queries(q, s, win)
                    P = np.stack([p] + [O.attention(Qw[k], K[:, :N], V[:, :N])[3]
                                        for k in range(1, win)])
                    sel = O.select_window(P, norms[b][:, :N], N, w.num_kv_heads, w.n_sink,
                                          w.n_recent, w.top_k, w.nms_radius, w.alpha_soft,
                                          w.alpha_cross, w.lam, _lc(w))
                sel_gpu = lb.sel_idx[b].cpu().numpy()
                explain_selection_diff(sel_gpu, sel, N)
                packed[b] = [O.packed_positions(sel_gpu[g], w.n_sink)
                             for g in range(w.num_kv_heads)]
                rstart[b] = O.recent_start_at(N, w.n_sink, w.n_recent)
            else:
                n_fast += 1
                if sliding:
                    rstart[b] = O.recent_start_sliding(N, w.n_sink, w.n_recent)
                o, lse = O.fast_attention(q[s], K, V, packed[b], rstart[b], N)
                worst = max(worst, check_out(out[b], o, f"fast s={s} b={b}"))
    assert eng.device_status() == 0
    print(f"{name} window {win} sliding {sliding}: {n_slow} slow / {n_fast} fast steps, "
          f"worst row rel err {worst:.2e}")


@pytest.mark.parametrize("name,win", [("tiny_fp32_1k", 3), ("qwen3_0p6b_8k", 4),
                                      ("qwen3_0p6b_8k", 8)])
def test_slow_attention_and_select_window(name, win):
    """sfi_slow_attn_window + sfi_select_window against the oracle's window readings: the
    logits and lse of every slot, the output of slot 0, the pooled fused scores and the
    selection.  Steps 0 and 1 have slots filled by the first query."""
    w = get(name).replace(evidence_window=win)
    d, eng, lb = _setup(w, dbg=True)
    Hq, Hkv, G, B = w.num_q_heads, w.num_kv_heads, w.group, w.batch
    out1 = torch.zeros_like(lb.out)
    lse1 = torch.zeros(B, Hq, dtype=torch.float32, device="cuda")
    for s in (0, 1, 5, w.steps - 1):
        N = w.seq_len(s)
        seq_len = torch.full((B,), N, dtype=torch.int32, device="cuda")
        L.sfi_slow_attn_window(eng.shape, win, lb.q_win[s], lb.k_cache, lb.v_cache,
                               lb.block_table, seq_len, eng.all_ids_d, B, eng.max_len, lb.out,
                               lb.logits, eng.stride, lb.lse, eng.ws_slow)
        L.sfi_select_window(eng.shape, eng.params, win, lb.logits, eng.stride, lb.lse,
                            lb.key_norm, eng.stride, seq_len, eng.all_ids_d, B, eng.max_len,
                            lb.sel_idx, eng.dbg_buf, eng.ws_sel)
        # the step's own output does not depend on the window
        L.sfi_slow_attn(eng.shape, d["q"][s], lb.k_cache, lb.v_cache, lb.block_table, seq_len,
                        eng.all_ids_d, B, eng.max_len, out1, None, 0, lse1, eng.ws_slow)
        torch.cuda.synchronize()
        assert bool((_bits(out1) == _bits(lb.out)).all())
        for b in range(B):
            q, K, V = oracle_layer_arrays(d, b)
            Qw = O.window_queries(q, s, win)
            z_gpu = host64(lb.logits[b, :, :N]).reshape(Hkv, win, G, N)
            lse_gpu = host64(lb.lse[b]).reshape(Hkv, win, G)
            P = []
            for k in range(win):
                o, z, lse, p = O.attention(Qw[k], K[:, :N], V[:, :N])
                P.append(p)
                if k == 0:
                    check_out(host64(lb.out[b]), o, f"s={s} b={b}")
                check_lse(lse_gpu[:, k].reshape(Hq), lse, p, Qw[k], K[:, :N])
                check_logits(z_gpu[:, k].reshape(Hq, N), z, Qw[k], K[:, :N], w.head_dim)
            sel = O.select_window(np.stack(P), O.key_norms(K[:, :N]), N, Hkv, w.n_sink,
                                  w.n_recent, w.top_k, w.nms_radius, w.alpha_soft,
                                  w.alpha_cross, w.lam, _lc(w))
            s_gpu = host64(eng.dbg_buf[b, :, :N])
            np.testing.assert_allclose(s_gpu, sel.s, rtol=1e-3, atol=1e-12)
            sel_gpu = lb.sel_idx[b].cpu().numpy()
            np.testing.assert_array_equal(
                sel_gpu, O.select_from_scores(s_gpu, N, w.n_sink, w.n_recent, w.top_k,
                                              w.nms_radius, w.alpha_soft, w.alpha_cross))
            print(name, win, "step", s, "row", b, explain_selection_diff(sel_gpu, sel, N))


def _stack_outputs(w, ds, **engine_kw):
    """Issue every step of a layer stack with no host synchronisation between steps (the
    host runs ahead of the GPU) and copy each layer's output on the attention stream after
    every step.  Returns the outputs [S, layers, B, Hq, D], the final Selector and pack
    state of every layer and the engine."""
    eng = Engine(w, ds[0]["flags"], **engine_kw)
    lbs = [eng.add_layer(d["k_cache"], d["v_cache"], d["block_table"], d["q"]) for d in ds]
    outs = torch.empty((w.steps, w.layers) + tuple(lbs[0].out.shape), device="cuda")
    eng.stream1.wait_stream(torch.cuda.current_stream())
    for s in range(w.steps):
        eng.step(s)
        with torch.cuda.stream(eng.stream1):
            for li, lb in enumerate(lbs):
                outs[s, li].copy_(lb.out)
    eng.join()
    torch.cuda.synchronize()
    state = [(lb.sel_idx.clone(), lb.packed_pos.clone(), lb.packed_len.clone(),
              lb.packed_k.clone(), lb.packed_v.clone()) for lb in lbs]
    return outs, state, eng


def test_two_streams_bit_identical_to_one_stream():
    """Race check of the overlap on a three-layer stack issued with no host synchronisation
    between steps: with two Selector streams layer i's Selector and pack run while stream 1
    runs the attention of layer i + 1 and of the next steps.  Every step's output of every
    layer, and the final selections and packed buffers, must be bit-identical to the same
    work serialised on one stream."""
    w = get("qwen3_0p6b_8k").replace(steps=70, layers=3, name="overlap_3l")
    ds = [make_layer(w, layer, device="cuda") for layer in range(w.layers)]
    o2, st2, eng2 = _stack_outputs(w, ds)
    assert len(eng2.sel_streams) == 2 and eng2.sel_streams[0] is not eng2.stream1
    o1, st1, eng1 = _stack_outputs(w, ds, two_streams=False)
    assert eng1.sel_streams[0] is eng1.stream1
    mode = oracle_schedule(w, ds[0]["flags"], eng1.plan)
    assert int(mode[0].sum()) >= 3  # several slow steps, each with its Selector overlap
    for s in range(w.steps):
        assert torch.equal(o1[s], o2[s]), s
    for a, b in zip(st1, st2):
        for x, y in zip(a, b):
            assert torch.equal(_bits(x) if x.is_floating_point() else x,
                               _bits(y) if y.is_floating_point() else y)


def test_paced_issue_bit_identical_to_unpaced():
    """Pacing and the Selector lookahead change only when the host queues work.  A three-layer
    stack issued with no host synchronisation between steps (so the host runs ahead of the
    GPU) gives bit-identical outputs at every step of every layer, and the same packed
    buffers at the end, paced with the lookahead as unpaced."""
    w = get("qwen3_0p6b_8k").replace(steps=70, layers=3, name="paced_3l")
    ds = [make_layer(w, layer, device="cuda") for layer in range(w.layers)]
    runs = []
    for paced in (False, True):
        eng = Engine(w, ds[0]["flags"], paced=paced, sel_lookahead=2 if paced else 0)
        lbs = [eng.add_layer(d["k_cache"], d["v_cache"], d["block_table"], d["q"])
               for d in ds]
        outs = torch.empty((w.steps, w.layers) + tuple(lbs[0].out.shape), device="cuda")
        eng.stream1.wait_stream(torch.cuda.current_stream())
        for s in range(w.steps):
            eng.step(s)
            with torch.cuda.stream(eng.stream1):
                for li, lb in enumerate(lbs):
                    outs[s, li].copy_(lb.out)
        eng.join()
        torch.cuda.synchronize()
        assert eng.paced == paced and (eng.sel_lookahead or 0) == (2 if paced else 0)
        runs.append((outs, [(lb.packed_k.clone(), lb.packed_pos.clone()) for lb in lbs],
                     eng.plan.mode.copy()))
    (o0, p0, mode), (o1, p1, _) = runs
    assert int(mode[0].sum()) >= 3  # several slow steps, each with its Selector overlap
    for s in range(w.steps):
        assert torch.equal(o0[s], o1[s]), s
    for (k0, q0), (k1, q1) in zip(p0, p1):
        assert torch.equal(q0, q1)
        assert torch.equal(_bits(k0), _bits(k1))


@pytest.mark.parametrize("batch", [1, 3])
def test_fast_step_graph_bit_identical_to_eager(batch):
    """Fast steps replayed from the captured two-layer graph, with eager slow steps,
    Selector and pack work and host synchronisations between the replays, give
    bit-identical outputs to the same trajectory issued call by call.  With three rows,
    steps that mix slow and fast rows take the call-by-call path and all-fast steps the
    graph."""
    w = get("qwen3_0p6b_8k").replace(steps=48, batch=batch, context=4096,
                                     name=f"graph_b{batch}")
    runs = []
    for graphs in (False, True):
        ds = [make_layer(w, layer, device="cuda") for layer in (0, 1)]
        eng = Engine(w, ds[0]["flags"])
        lbs = [eng.add_layer(d["k_cache"], d["v_cache"], d["block_table"], d["q"])
               for d in ds]
        if graphs:
            eng.enable_graphs(min_layers=1)
            assert eng.graphs
        res = []
        for s in range(w.steps):
            eng.step(s)
            eng.join()
            torch.cuda.synchronize()
            res.append(torch.stack([lb.out.clone() for lb in lbs]))
        runs.append((res, eng.plan.mode.copy()))
    (eager, mode), (graph, _) = runs
    all_fast = (mode == 0).all(axis=0)
    assert int(all_fast.sum()) >= 10  # many replays, interleaved with slow steps
    assert int((~all_fast).sum()) >= 2
    for s, (a, b) in enumerate(zip(eager, graph)):
        assert torch.equal(a, b), s


def test_fast_equals_dense_when_k_covers_candidates():
    """Invariant on the device: with K >= |C| every fast step equals the dense
    step (same positions, so equal up to fp32 rounding)."""
    w = get("qwen3_0p6b_8k").replace(steps=40, top_k=9000, context=2048)
    d, eng, lb = _setup(w)
    for s in range(w.steps):
        eng.step(s)
        torch.cuda.synchronize()
        fast_out = lb.out.clone()
        _slow(eng, lb, d["q"][s], w.seq_len(s))
        torch.cuda.synchronize()
        err = (fast_out - lb.out).abs().amax(dim=-1) / lb.out.abs().amax(dim=-1)
        assert float(err.max()) <= 2e-3, (s, float(err.max()))


# ------------------------------------------------------------------------- edge cases
EDGE = {
    "empty_candidates": dict(context=40, n_recent=64, steps=6),            # N - W <= n_sink
    "k_exceeds_candidates": dict(context=300, top_k=1000, steps=6),        # -1 padding
    "no_sink": dict(n_sink=0, steps=6),
    "no_recent_window": dict(n_recent=0, steps=6),
    "ragged_tail": dict(context=1000 + 13, steps=5),                       # partial pages
    "single_kv_head": dict(num_q_heads=8, num_kv_heads=1, steps=5),
    "group_16": dict(num_q_heads=32, num_kv_heads=2, steps=5),
    "head_dim_64_bf16": dict(head_dim=64, steps=5),
    "f32_head_dim_128": dict(dtype="f32", head_dim=128, steps=5),
    "alpha_one": dict(alpha_soft=1.0, alpha_cross=1.0, steps=5),
    "alpha_zero": dict(alpha_soft=0.0, alpha_cross=0.0, steps=5),
    "budget_zero": dict(refresh_budget=0, steps=5),
}


@pytest.mark.parametrize("case", sorted(EDGE))
def test_edge_cases(case):
    base = get("qwen3_0p6b_8k").replace(context=1024, top_k=128, n_recent=64, steps=8,
                                        name="edge_" + case)
    w = base.replace(**EDGE[case])
    d, eng, lb = _setup(w, dbg=True)
    _select_and_check(w, d, eng, lb, 0)
    # run the trajectory through the engine and compare every step
    d, eng, lb = _setup(w)
    omode = oracle_schedule(w, d["flags"], eng.plan)
    q, K, V = oracle_layer_arrays(d, 0)
    norms = O.key_norms(K)
    packed, rstart = None, 0
    for s in range(w.steps):
        eng.step(s)
        torch.cuda.synchronize()
        N = w.seq_len(s)
        if omode[0, s]:
            o, z, lse, p = O.attention(q[s], K[:, :N], V[:, :N])
            sel = O.select(p, norms[:, :N], N, w.num_kv_heads, w.n_sink, w.n_recent, w.top_k,
                           w.nms_radius, w.alpha_soft, w.alpha_cross, w.lam, _lc(w))
            sel_gpu = lb.sel_idx[0].cpu().numpy()
            explain_selection_diff(sel_gpu, sel, N)
            packed = [O.packed_positions(sel_gpu[g], w.n_sink) for g in range(w.num_kv_heads)]
            rstart = O.recent_start_at(N, w.n_sink, w.n_recent)
        else:
            o, _ = O.fast_attention(q[s], K, V, packed, rstart, N)
        check_out(host64(lb.out[0]), o, f"{case} s={s}")
    assert eng.device_status() == 0


def test_ragged_batch_lengths():
    """Rows of one call with different KV lengths (partial last pages, one row much
    shorter than the call's max_seq_len)."""
    w = get("qwen3_0p6b_8k").replace(batch=3, context=2000, steps=4, name="ragged_batch")
    d, eng, lb = _setup(w, dbg=True)
    lens = [2003, 517, 1290]
    seq_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
    ids = torch.tensor([2, 0, 1], dtype=torch.int32, device="cuda")
    q = d["q"][0]
    L.sfi_slow_attn(eng.shape, q, lb.k_cache, lb.v_cache, lb.block_table, seq_len, ids, 3,
                    eng.max_len, lb.out, lb.logits, eng.stride, lb.lse, eng.ws_slow)
    L.sfi_select(eng.shape, eng.params, lb.logits, eng.stride, lb.lse, lb.key_norm, eng.stride,
                 seq_len, ids, 3, eng.max_len, lb.sel_idx, eng.dbg_buf, eng.ws_sel)
    torch.cuda.synchronize()
    for b in range(3):
        N = lens[b]
        qh, K, V = oracle_layer_arrays(d, b)
        o, z, lse, p = O.attention(qh[0], K[:, :N], V[:, :N])
        check_out(host64(lb.out[b]), o, f"row {b}")
        check_lse(host64(lb.lse[b]), lse, p, qh[0], K[:, :N])
        s_gpu = host64(eng.dbg_buf[b, :, :N])
        ref_sel = O.select_from_scores(s_gpu, N, w.n_sink, w.n_recent, w.top_k, w.nms_radius,
                                       w.alpha_soft, w.alpha_cross)
        np.testing.assert_array_equal(lb.sel_idx[b].cpu().numpy(), ref_sel)


def test_fast_and_pack_on_a_row_subset():
    """Pack and fast attention serve only the rows listed in seq_ids (here rows 2 and 0 of
    three, in that order, with their own lengths and recent starts); the other row's
    outputs are left untouched."""
    w = get("qwen3_0p6b_8k").replace(batch=3, context=2000, steps=4, name="row_subset")
    d, eng, lb = _setup(w)
    N0 = w.seq_len(0)
    lens0 = torch.full((3,), N0, dtype=torch.int32, device="cuda")
    L.sfi_slow_attn(eng.shape, d["q"][0], lb.k_cache, lb.v_cache, lb.block_table, lens0,
                    eng.all_ids_d, 3, eng.max_len, lb.out, lb.logits, eng.stride, lb.lse,
                    eng.ws_slow)
    L.sfi_select(eng.shape, eng.params, lb.logits, eng.stride, lb.lse, lb.key_norm, eng.stride,
                 lens0, eng.all_ids_d, 3, eng.max_len, lb.sel_idx, None, eng.ws_sel)
    ids = torch.tensor([2, 0], dtype=torch.int32, device="cuda")
    lb.packed_len.fill_(-5)
    lb.packed_pos.fill_(-5)
    L.sfi_pack(eng.shape, eng.params, lb.k_cache, lb.v_cache, lb.block_table, lb.sel_idx, ids,
               2, lb.packed_k, lb.packed_v, lb.packed_pos, lb.packed_len, eng.packed_cap)
    torch.cuda.synchronize()
    assert bool((lb.packed_len[1] == -5).all()) and bool((lb.packed_pos[1] == -5).all())
    # fast step of rows 2 and 0 at their own lengths
    lens = torch.tensor([N0 + 3, N0, N0 + 2], dtype=torch.int32, device="cuda")
    rs = O.recent_start_at(N0, w.n_sink, w.n_recent)
    rstart = torch.full((3,), rs, dtype=torch.int32, device="cuda")
    lb.out.fill_(123.0)
    L.sfi_fast_attn(eng.shape, d["q"][1], lb.packed_k, lb.packed_v, lb.packed_len,
                    eng.packed_cap, lb.k_cache, lb.v_cache, lb.block_table, rstart, lens, ids, 2,
                    eng.max_recent, lb.out, None, eng.ws_fast)
    torch.cuda.synchronize()
    assert bool((lb.out[1] == 123.0).all())
    out = host64(lb.out)
    for b in (2, 0):
        sel = lb.sel_idx[b].cpu().numpy()
        pos = [O.packed_positions(sel[g], w.n_sink) for g in range(w.num_kv_heads)]
        for g in range(w.num_kv_heads):
            assert int(lb.packed_len[b, g]) == len(pos[g])
        q, K, V = oracle_layer_arrays(d, b)
        o, _ = O.fast_attention(q[1], K, V, pos, rs, int(lens[b]))
        check_out(out[b], o, f"fast row {b}")


# ------------------------------------------------------------ full-size sampled checks
FULL = ["qwen3_4b_32k_b4", "qwen3_4b_128k_36l", "g16_64k_b8"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    """At the full sizes and in the engine's launch configuration: step 0 (slow) of
    layer 0 for the first and last row -- dense output, lse, exact Top-K on the device
    scores, the near-tie rule end to end and the bit-exact pack -- then the first fast
    step against the oracle's fast step on the device's memory."""
    w = get(name)
    d, eng, lb = _setup(w, dbg=True)
    eng.step(0)
    eng.join()
    torch.cuda.synchronize()
    rows = sorted({0, w.batch - 1})
    N = w.seq_len(0)
    # one extra Selector call with the debug scores on (same inputs, same kernels)
    seq_len = torch.full((w.batch,), N, dtype=torch.int32, device="cuda")
    sel_before = lb.sel_idx.clone()
    L.sfi_select(eng.shape, eng.params, lb.logits, eng.stride, lb.lse, lb.key_norm, eng.stride,
                 seq_len, eng.all_ids_d, w.batch, eng.max_len, lb.sel_idx, eng.dbg_buf,
                 eng.ws_sel)
    torch.cuda.synchronize()
    assert torch.equal(sel_before, lb.sel_idx)
    out0 = host64(lb.out)
    for b in rows:
        q, K, V = oracle_layer_arrays(d, b)
        o, z, lse, p = O.attention(q[0], K[:, :N], V[:, :N])
        check_out(out0[b], o, f"{name} slow b={b}")
        check_lse(host64(lb.lse[b]), lse, p, q[0], K[:, :N])
        s_gpu = host64(eng.dbg_buf[b, :, :N])
        sel_gpu = lb.sel_idx[b].cpu().numpy()
        np.testing.assert_array_equal(
            sel_gpu, O.select_from_scores(s_gpu, N, w.n_sink, w.n_recent, w.top_k,
                                          w.nms_radius, w.alpha_soft, w.alpha_cross))
        sel = O.select(p, O.key_norms(K[:, :N]), N, w.num_kv_heads, w.n_sink, w.n_recent,
                       w.top_k, w.nms_radius, w.alpha_soft, w.alpha_cross, w.lam, _lc(w))
        print(name, "row", b, "selection diff (n, kth, decision):",
              explain_selection_diff(sel_gpu, sel, N))
        pos = [O.packed_positions(sel_gpu[g], w.n_sink) for g in range(w.num_kv_heads)]
        for g in range(w.num_kv_heads):
            n = len(pos[g])
            assert int(lb.packed_len[b, g]) == n
            idx = torch.from_numpy(pos[g]).cuda()
            assert torch.equal(_bits(lb.packed_k[b, g, :n]), _bits(d["K"][b, g, idx]))
            assert torch.equal(_bits(lb.packed_v[b, g, :n]), _bits(d["V"][b, g, idx]))
    # first fast step of those rows (if the schedule makes it fast)
    omode = oracle_schedule(w, d["flags"], eng.plan)
    eng.step(1)
    torch.cuda.synchronize()
    out1 = host64(lb.out)
    for b in rows:
        if omode[b, 1]:
            continue
        q, K, V = oracle_layer_arrays(d, b)
        sel_gpu = lb.sel_idx[b].cpu().numpy()
        pos = [O.packed_positions(sel_gpu[g], w.n_sink) for g in range(w.num_kv_heads)]
        o, _ = O.fast_attention(q[1], K, V, pos, O.recent_start_at(N, w.n_sink, w.n_recent),
                                w.seq_len(1))
        check_out(out1[b], o, f"{name} fast b={b}")
    assert eng.device_status() == 0


# ------------------------------------------------------------- Top-K selection paths
def _select_direct(shape, params, logits, lse, key_norm, N, stride):
    B = shape.batch
    seq_lens = torch.full((B,), N, dtype=torch.int32, device="cuda")
    ids = torch.arange(B, dtype=torch.int32, device="cuda")
    sel = torch.full((B, shape.num_kv_heads, params.top_k), -7, dtype=torch.int32, device="cuda")
    dbg = torch.zeros(B, shape.num_kv_heads, stride, dtype=torch.float32, device="cuda")
    ws = L.workspace(L.sfi_select_ws(shape, params, B, N), "cuda")
    L.sfi_select(shape, params, logits, stride, lse, key_norm, stride, seq_lens, ids, B, N, sel,
                 dbg, ws)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), host64(dbg)


def test_topk_concentrated_scores_need_several_passes():
    """Prior-only scores (lambda = 1) with equal key norms vary by a few percent over 128K
    positions, so the bin of the K-th key holds far more keys than the LDS candidate list
    takes and the selection needs further passes over global memory."""
    import math
    Hq, Hkv, D, N, K = 8, 2, 128, 131072 + 100, 19456
    stride = (N + 63) // 64 * 64
    shape = L.make_shape(1, Hq, Hkv, D, (N + 15) // 16, "bf16")
    params = L.make_params(4, 1024, K, 4, 1.0, 0.5, 0.5)
    logits = torch.zeros(1, Hq, stride, device="cuda")
    lse = torch.full((1, Hq), math.log(N), device="cuda")
    key_norm = torch.full((1, Hkv, stride), 2.0, device="cuda")
    sel, dbg = _select_direct(shape, params, logits, lse, key_norm, N, stride)
    ref = O.select_from_scores(dbg[0, :, :N], N, 4, 1024, K, 4, 0.5, 0.5)
    np.testing.assert_array_equal(sel[0], ref)


def test_topk_heavy_exact_ties():
    """alpha_soft = alpha_cross = 1 zeroes every dominated or non-owned score, so the K-th
    key is 0 and thousands of candidates tie with it: the lowest positions must win."""
    w = get("qwen3_0p6b_8k").replace(alpha_soft=1.0, alpha_cross=1.0, steps=4,
                                     name="heavy_ties_8k")
    d, eng, lb = _setup(w, dbg=True)
    _select_and_check(w, d, eng, lb, 0)


@pytest.mark.parametrize("levels", [16, 4])
def test_topk_ties_across_slices(levels):
    """Score levels 22% apart (each its own 11-bit bin), interleaved over 70000 positions
    (18 slices of 4096 candidates); the K-th key sits inside a level, so only part of its
    exactly tied positions is taken, lowest positions first.  With 16 levels (about 4400
    positions each) the level fits the candidate list; with 4 (about 17500 each) it does
    not and the one-block path over global memory selects."""
    Hq, Hkv, D, N, K = 4, 2, 128, 70000, 30000
    stride = (N + 63) // 64 * 64
    shape = L.make_shape(1, Hq, Hkv, D, (N + 15) // 16, "bf16")
    params = L.make_params(4, 64, K, 4, 0.0, 0.0, 0.0)  # lambda = 0: s = f; no refinement
    j = torch.arange(stride, device="cuda")
    level = (j * 7919) % levels  # levels interleaved over positions, not in runs
    logits = (-0.2 * level.float()).expand(1, Hq, stride).contiguous()
    lse = torch.zeros(1, Hq, device="cuda")
    key_norm = torch.ones(1, Hkv, stride, device="cuda")
    sel, dbg = _select_direct(shape, params, logits, lse, key_norm, N, stride)
    s = dbg[0, :, :N]
    assert len(np.unique(s[0, 4:N - 64])) == levels
    ref = O.select_from_scores(s, N, 4, 64, K, 4, 0.0, 0.0)
    np.testing.assert_array_equal(sel[0], ref)


@pytest.mark.parametrize("N,batch", [(16384, 2), (16385, 2), (3000, 3)])
def test_topk_one_block_path_and_its_bound(N, batch):
    """Rows of at most 16384 positions (four slices) are ranked by one block per (row, head);
    longer ones by the four-kernel chain.  On both sides of the bound, with exact ties inside
    the K-th score's level and rows of different lengths, the selection equals the oracle's
    Top-K on the device's own scores."""
    Hq, Hkv, D, K = 4, 2, 128, N // 3
    stride = (N + 63) // 64 * 64
    shape = L.make_shape(batch, Hq, Hkv, D, (N + 15) // 16, "bf16")
    params = L.make_params(4, 64, K, 4, 0.0, 0.0, 0.0)  # lambda = 0: s = f; no refinement
    j = torch.arange(stride, device="cuda")
    level = (j * 7919) % 5  # five score levels interleaved over positions
    logits = (-0.2 * level.float()).expand(batch, Hq, stride).contiguous()
    lse = torch.zeros(batch, Hq, device="cuda")
    key_norm = torch.ones(batch, Hkv, stride, device="cuda")
    lens = [N - 97 * b for b in range(batch)]
    seq_lens = torch.tensor(lens, dtype=torch.int32, device="cuda")
    ids = torch.arange(batch, dtype=torch.int32, device="cuda")
    sel = torch.full((batch, Hkv, K), -7, dtype=torch.int32, device="cuda")
    dbg = torch.zeros(batch, Hkv, stride, dtype=torch.float32, device="cuda")
    ws = L.workspace(L.sfi_select_ws(shape, params, batch, N), "cuda")
    L.sfi_select(shape, params, logits, stride, lse, key_norm, stride, seq_lens, ids, batch, N,
                 sel, dbg, ws)
    torch.cuda.synchronize()
    sel = sel.cpu().numpy()
    for b in range(batch):
        n = lens[b]
        s = host64(dbg[b, :, :n])
        ref = O.select_from_scores(s, n, 4, 64, K, 4, 0.0, 0.0)
        np.testing.assert_array_equal(sel[b], ref)


def test_select_at_maximum_length():
    """The Selector at its longest KV length (2^22 positions: 1024 top-K slices of 4096
    candidates, 1024 prior-normaliser chunks), from seeded logits, lse and key norms: fused
    scores against the oracle pipeline, exact Top-K on the device's own scores, and the
    near-tie rule end to end."""
    Hq, Hkv, D, N, K = 2, 1, 128, 1 << 22, 65536
    n_sink, n_recent, R, lam, a_soft, a_cross = 4, 1024, 4, 0.3, 0.5, 0.5
    rng = np.random.default_rng(20261203)
    z = (3.0 * rng.standard_normal((Hq, N))).astype(np.float32)
    zmax = z.max(axis=1, keepdims=True).astype(np.float64)
    lse64 = zmax[:, 0] + np.log(np.exp(z.astype(np.float64) - zmax).sum(axis=1))
    lse32 = lse64.astype(np.float32)
    norms = rng.lognormal(0.0, 0.5, (Hkv, N)).astype(np.float32)
    stride = N
    shape = L.make_shape(1, Hq, Hkv, D, N // 16, "bf16")
    params = L.make_params(n_sink, n_recent, K, R, lam, a_soft, a_cross)
    logits = torch.from_numpy(z).reshape(1, Hq, N).cuda()
    lse = torch.from_numpy(lse32).reshape(1, Hq).cuda()
    key_norm = torch.from_numpy(norms).reshape(1, Hkv, N).cuda()
    sel, dbg = _select_direct(shape, params, logits, lse, key_norm, N, stride)
    s_gpu = dbg[0]
    ref_sel = O.select_from_scores(s_gpu, N, n_sink, n_recent, K, R, a_soft, a_cross)
    np.testing.assert_array_equal(sel[0], ref_sel)
    # the oracle pipeline on the same inputs (p from the logits and the stored lse)
    p = np.exp(z.astype(np.float64) - lse32.astype(np.float64)[:, None])
    oracle_sel = O.select(p, norms.astype(np.float64), N, Hkv, n_sink, n_recent, K, R, a_soft,
                          a_cross, lam, None)
    np.testing.assert_allclose(s_gpu, oracle_sel.s, rtol=1e-3, atol=1e-12)
    print("maximum length (diff, kth-ties, decision-ties, score-ties):",
          explain_selection_diff(sel[0], oracle_sel, N))


# ------------------------------------------------------------------ incremental pack
def _check_pack_state(w, lb, d, b, want_pos, N, ordered=False):
    """Rows [0, packed_len) hold exactly sink + want_pos, each the stored row of its slot's
    position; slot_map is the inverse of packed_pos and -1 elsewhere."""
    Hkv = w.num_kv_heads
    ppos = lb.packed_pos[b].cpu().numpy()
    plen = lb.packed_len[b].cpu().numpy()
    smap = lb.slot_map[b, :, :N].cpu().numpy()
    for g in range(Hkv):
        want = O.packed_positions(np.asarray(want_pos[g]), w.n_sink)
        n = len(want)
        assert plen[g] == n
        held = ppos[g, :n]
        if ordered:
            np.testing.assert_array_equal(held, want)
        assert sorted(held.tolist()) == sorted(want.tolist())
        assert (ppos[g, n:] == -1).all()
        idx = torch.from_numpy(held.astype(np.int64)).cuda()
        assert torch.equal(_bits(lb.packed_k[b, g, :n]), _bits(d["K"][b, g, idx]))
        assert torch.equal(_bits(lb.packed_v[b, g, :n]), _bits(d["V"][b, g, idx]))
        inv = np.full(N, -1)
        inv[held] = np.arange(n)
        np.testing.assert_array_equal(smap[g], inv)


def test_pack_update_keeps_held_rows_and_adds_new_ones():
    """A run of selections through sfi_pack_update: growing K_eff with 0-100% turnover, a
    shrink (rebuilt in sfi_pack's order), an emptied buffer, and a row the list skips.
    Before every call the workspace is filled with seeded integers in [-2, top_k + 2), so
    that leftover per-slot claims look valid: the result must not depend on them."""
    w = get("qwen3_0p6b_8k").replace(batch=2, top_k=300, name="pack_update")
    d, eng, lb = _setup(w)
    dev = "cuda"
    N = w.context
    lo, hi = O.candidates(N, w.n_sink, w.n_recent)
    rng = np.random.default_rng(5)
    ws = L.workspace(L.sfi_pack_update_ws(eng.shape, eng.params, w.batch), dev)
    scramble = torch.Generator(device=dev)
    scramble.manual_seed(11)
    ids = torch.tensor([0, 1], dtype=torch.int32, device=dev)
    cur = [[np.sort(rng.choice(np.arange(lo, hi), 200, replace=False)) for _ in range(8)]
           for _ in range(2)]
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    def apply(sets, ids, n):
        sel = torch.full((w.batch, w.num_kv_heads, w.top_k), -1, dtype=torch.int32)
        for b in range(w.batch):
            for g in range(w.num_kv_heads):
                sel[b, g, :len(sets[b][g])] = torch.from_numpy(sets[b][g].astype(np.int32))
        lb.sel_idx.copy_(sel.to(dev))
        ws.view(torch.int32).random_(-2, w.top_k + 2, generator=scramble)
        prev_pos = lb.packed_pos.cpu().numpy()
        prev_len = lb.packed_len.cpu().numpy()
        L.sfi_pack_update(eng.shape, eng.params, lb.k_cache, lb.v_cache, lb.block_table,
                          lb.sel_idx, ids, n, lb.packed_k, lb.packed_v, lb.packed_pos,
                          lb.packed_len, eng.packed_cap, lb.slot_map, eng.stride, ws,
                          status=status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        # the device's slot of every row equals the documented order, slot by slot
        got = lb.packed_pos.cpu().numpy()
        for b in [int(x) for x in ids.cpu().numpy() if x >= 0]:
            for g in range(w.num_kv_heads):
                want, wlen = model_pack_update(prev_pos[b, g], int(prev_len[b, g]),
                                               sets[b][g], w.n_sink)
                np.testing.assert_array_equal(got[b, g], want, err_msg=f"row {b} head {g}")
                assert int(lb.packed_len[b, g]) == wlen

    # first call: an empty buffer is built in the full pack's order
    apply(cur, ids, 2)
    for b in range(2):
        _check_pack_state(w, lb, d, b, cur[b], N, ordered=True)
    plan = [(0.0, 0), (0.05, 10), (0.5, 20), (1.0, 30), (0.2, 0)]
    plan += [(float(rng.choice([0.0, 0.01, 0.1, 0.3, 1.0])), int(rng.integers(0, 3)))
             for _ in range(15)]  # seeded random turnovers, growing by at most 2
    for turnover, grow in plan:
        new = []
        for b in range(2):
            rows = []
            for g in range(8):
                keep_n = int(round(len(cur[b][g]) * (1 - turnover)))
                keep = rng.choice(cur[b][g], keep_n, replace=False)
                pool = np.setdiff1d(np.arange(lo, hi), keep)
                add = rng.choice(pool, len(cur[b][g]) + grow - keep_n, replace=False)
                rows.append(np.sort(np.concatenate([keep, add])))
            new.append(rows)
        apply(new, ids, 2)
        cur = new
        for b in range(2):
            _check_pack_state(w, lb, d, b, cur[b], N)
    # row 1 only (row 0's slot skipped with -1): row 0 keeps its state
    before = lb.packed_pos[0].clone()
    new = [cur[0], [np.sort(np.concatenate([c[:-3], [hi - 1]])) if hi - 1 not in c else c
                    for c in cur[1]]]
    apply(new, torch.tensor([-1, 1], dtype=torch.int32, device=dev), 2)
    assert torch.equal(before, lb.packed_pos[0])
    _check_pack_state(w, lb, d, 1, new[1], N)
    cur = new
    # a smaller selection is rebuilt in order
    small = [[c[:50] for c in cur[b]] for b in range(2)]
    apply(small, ids, 2)
    for b in range(2):
        _check_pack_state(w, lb, d, b, small[b], N, ordered=True)
    # an emptied buffer (a new sequence) is rebuilt in order, with no stale map entries
    lb.packed_len.zero_()
    apply(cur, ids, 2)
    for b in range(2):
        _check_pack_state(w, lb, d, b, cur[b], N, ordered=True)


def test_pack_update_rebuilds_beside_a_busy_stream():
    """Rebuilds (emptied buffer) and growing updates of sfi_pack_update while another stream
    keeps the CUs busy, so that the workgroups of one (row, KV head) start at different times.
    The assign kernel publishes the new packed length from one workgroup; every other
    workgroup must still work from the old one (a workgroup that read the new length at a
    rebuild would place rows past the buffer).  Each round must leave exactly sink +
    selection in the buffer."""
    w = get("qwen3_0p6b_8k").replace(batch=2, top_k=4096, name="pack_update_busy")
    d, eng, lb = _setup(w, incremental_pack=True)
    dev = "cuda"
    N = w.context
    lo, hi = O.candidates(N, w.n_sink, w.n_recent)
    rng = np.random.default_rng(11)
    ws = L.workspace(L.sfi_pack_update_ws(eng.shape, eng.params, w.batch), dev)
    ids = torch.tensor([0, 1], dtype=torch.int32, device=dev)
    busy = torch.cuda.Stream()
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    busy.wait_stream(torch.cuda.current_stream())

    def apply(sets):
        sel = torch.full((w.batch, w.num_kv_heads, w.top_k), -1, dtype=torch.int32)
        for b in range(w.batch):
            for g in range(w.num_kv_heads):
                sel[b, g, :len(sets[b][g])] = torch.from_numpy(sets[b][g].astype(np.int32))
        with torch.cuda.stream(side):
            lb.sel_idx.copy_(sel.to(dev))
            L.sfi_pack_update(eng.shape, eng.params, lb.k_cache, lb.v_cache, lb.block_table,
                              lb.sel_idx, ids, 2, lb.packed_k, lb.packed_v, lb.packed_pos,
                              lb.packed_len, eng.packed_cap, lb.slot_map, eng.stride, ws,
                              stream=side, status=status)

    for rnd in range(6):
        n0 = int(rng.integers(3000, 3900))
        cur = [[np.sort(rng.choice(np.arange(lo, hi), n0, replace=False)) for _ in range(8)]
               for _ in range(2)]
        with torch.cuda.stream(busy):
            for _ in range(4):
                dst.copy_(src)
        with torch.cuda.stream(side):
            lb.packed_len.zero_()
        apply(cur)
        torch.cuda.synchronize()
        for b in range(2):
            _check_pack_state(w, lb, d, b, cur[b], N, ordered=True)
        grow = int(rng.integers(1, 4096 - n0))
        new = []
        for b in range(2):
            rows = []
            for g in range(8):
                keep = rng.choice(cur[b][g], int(0.9 * len(cur[b][g])), replace=False)
                pool = np.setdiff1d(np.arange(lo, hi), keep)
                add = rng.choice(pool, len(cur[b][g]) + grow - len(keep), replace=False)
                rows.append(np.sort(np.concatenate([keep, add])))
            new.append(rows)
        with torch.cuda.stream(busy):
            for _ in range(4):
                dst.copy_(src)
        apply(new)
        torch.cuda.synchronize()
        for b in range(2):
            _check_pack_state(w, lb, d, b, new[b], N)
    assert int(status.item()) == 0


def test_pack_update_full_size():
    """The incremental pack at the benchmark's full size (131072-token context, K = 19456, one
    layer): a rebuild at the first slow step, then updates at later slow steps of the seeded
    schedule, each leaving exactly sink + selection in the buffer, byte for byte."""
    w = get("qwen3_4b_128k_36l").replace(layers=1)
    d, eng, lb = _setup(w, incremental_pack=True)
    slow = [s for s in range(w.steps) if oracle_schedule(w, d["flags"], eng.plan)[0, s]][:3]
    for s in range(slow[-1] + 1):
        eng.step(s)
        if s in slow:
            eng.join()
            torch.cuda.synchronize()
            N = w.seq_len(s)
            sel = lb.sel_idx[0].cpu().numpy()
            want = [sel[g][sel[g] >= 0] for g in range(w.num_kv_heads)]
            _check_pack_state(w, lb, d, 0, want, N, ordered=(s == slow[0]))
    assert eng.device_status() == 0
    print("slow steps checked:", slow)


def test_full_stack_in_bench_configuration():
    """The benchmark's own launch configuration: all 36 layers of the 128K workload, fast steps
    replayed from graphs, the incremental pack, two Selector streams.  The schedule and the
    recent edge come from the oracle (the engine's plan must agree).  At a slow step, for
    layers 0, 17 and 35: the dense output, the selection against the oracle's Selector (the
    near-tie rule) and the packed buffer, which must hold exactly the sink rows and that
    selection, byte for byte.  At the last fast step before the next slow step (a graph
    replay): the fast output against the oracle's fast step on that memory."""
    w = get("qwen3_4b_128k_36l")
    sample = (0, 17, 35)
    data, eng, flags = {}, None, None
    for li in range(w.layers):
        d = make_layer(w, li, device="cuda", keep_logical=li in sample)
        if eng is None:
            eng = Engine(w, d["flags"])
            flags = d["flags"]
        eng.add_layer(d["k_cache"], d["v_cache"], d["block_table"], d["q"])
        if li in sample:
            data[li] = {k: d[k] for k in ("q", "K", "V")}
        del d
    eng.enable_graphs()
    assert eng.graph is not None and eng.incremental_pack and len(eng.sel_streams) == 2
    omode = oracle_schedule(w, flags, eng.plan)
    slow = [s for s in range(w.steps) if omode[0, s]]
    i = next(i for i in range(1, len(slow) - 1) if slow[i + 1] - slow[i] >= 3)
    s_slow, s_fast = slow[i], slow[i + 1] - 1
    host = {li: (host64(data[li]["q"][:, 0]), host64(data[li]["K"][0]), host64(data[li]["V"][0]))
            for li in sample}
    packed = {}
    rstart = O.recent_start_at(w.seq_len(s_slow), w.n_sink, w.n_recent)
    for s in range(s_fast + 1):
        eng.step(s)
        if s not in (s_slow, s_fast):
            continue
        eng.join()
        torch.cuda.synchronize()
        N = w.seq_len(s)
        for li in sample:
            lb = eng.layers[li]
            q, K, V = host[li]
            if s == s_slow:
                o, _, _, p = O.attention(q[s], K[:, :N], V[:, :N])
                check_out(host64(lb.out[0]), o, f"layer {li} step {s}")
                sel = O.select(p, O.key_norms(K[:, :N]), N, w.num_kv_heads, w.n_sink,
                               w.n_recent, w.top_k, w.nms_radius, w.alpha_soft, w.alpha_cross,
                               w.lam, _lc(w))
                sel_gpu = lb.sel_idx[0].cpu().numpy()
                print(f"layer {li} step {s} selection diff (n, kth, decision, score):",
                      explain_selection_diff(sel_gpu, sel, N))
                packed[li] = [O.packed_positions(sel_gpu[g], w.n_sink)
                              for g in range(w.num_kv_heads)]
                plen = lb.packed_len[0].cpu().numpy()
                ppos = lb.packed_pos[0].cpu().numpy()
                for g in range(w.num_kv_heads):
                    n = len(packed[li][g])
                    assert plen[g] == n, (li, g)
                    held = ppos[g, :n]
                    assert sorted(held.tolist()) == packed[li][g].tolist(), (li, g)
                    idx = torch.from_numpy(held.astype(np.int64)).cuda()
                    assert torch.equal(_bits(lb.packed_k[0, g, :n]), _bits(data[li]["K"][0, g, idx]))
                    assert torch.equal(_bits(lb.packed_v[0, g, :n]), _bits(data[li]["V"][0, g, idx]))
            else:
                o, _ = O.fast_attention(q[s], K, V, packed[li], rstart, N)
                check_out(host64(lb.out[0]), o, f"layer {li} step {s}")
    assert eng.device_status() == 0
    print(f"checked slow step {s_slow} and graph-replayed fast step {s_fast}")


def test_device_status_flags_broken_contracts():
    """Lengths, packed lengths and recent edges that break a call's contract are clamped by
    the kernels (no access leaves the buffers) and reported in the status word; consistent
    arguments leave it at 0."""
    w = get("qwen3_0p6b_8k").replace(batch=2, context=2000, steps=4, name="status_word")
    d, eng, lb = _setup(w)
    eng.step(0)
    eng.join()
    torch.cuda.synchronize()
    assert eng.device_status() == 0
    N = w.seq_len(1)
    rs = O.recent_start_at(w.seq_len(0), w.n_sink, w.n_recent)
    ids = eng.all_ids_d

    def fast(lens, rstart, plen):
        st = torch.zeros(1, dtype=torch.int32, device="cuda")
        L.sfi_fast_attn(eng.shape, d["q"][1], lb.packed_k, lb.packed_v, plen, eng.packed_cap,
                        lb.k_cache, lb.v_cache, lb.block_table, rstart, lens, ids, w.batch,
                        eng.max_recent, lb.out, None, eng.ws_fast, status=st)
        torch.cuda.synchronize()
        return int(st.item())

    full = lambda v: torch.full((w.batch,), v, dtype=torch.int32, device="cuda")  # noqa: E731
    assert fast(full(N), full(rs), lb.packed_len) == 0
    # a recent segment longer than max_recent (the edge moved back), an edge past N
    assert fast(full(N), full(rs - eng.max_recent - 40), lb.packed_len) == L.SFI_DEV_RECENT
    assert fast(full(N), full(N + 5), lb.packed_len) == L.SFI_DEV_RECENT
    # packed_len beyond the buffer, negative
    big = torch.full_like(lb.packed_len, eng.packed_cap + 16)
    assert fast(full(N), full(rs), big) == L.SFI_DEV_PACKED_LEN
    assert fast(full(N), full(rs), torch.full_like(lb.packed_len, -3)) == L.SFI_DEV_PACKED_LEN
    # a row longer than the page table
    assert fast(full(w.pages_per_seq * 16 + 7), full(rs), lb.packed_len) & L.SFI_DEV_SEQ_LEN
    # slow call: a row longer than max_seq_len
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    L.sfi_slow_attn(eng.shape, d["q"][0], lb.k_cache, lb.v_cache, lb.block_table,
                    full(eng.max_len + 3), ids, w.batch, eng.max_len, lb.out, lb.logits,
                    eng.stride, lb.lse, eng.ws_slow, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == L.SFI_DEV_SEQ_LEN
