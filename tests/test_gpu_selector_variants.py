"""Selector variants on one MI355X: the greedy Soft-NMS reading against the one-pass reading
the kernels implement, on the device's own fused scores.

The greedy reading has no kernel (each take depends on the takes before it along a run of
neighbours), so it runs in the oracle on the scores the device computed; both selections are
then judged by the dense attention mass their fast memory keeps at the following fast steps.
"""
import numpy as np
import pytest
import torch

from oracle import sfi_oracle as O
from workload import get
from workload.gen import make_layer

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sparse_kv_attention_decode_amd import lib as L
    from sparse_kv_attention_decode_amd.coverage import coverage_of, memory_mask
    from sparse_kv_attention_decode_amd.engine import Engine


def _packed(sel: np.ndarray, n_sink: int, dev):
    rows = [O.packed_positions(sel[g], n_sink) for g in range(sel.shape[0])]
    cap = max(len(r) for r in rows)
    pos = torch.full((len(rows), cap), -1, dtype=torch.int32)
    for g, r in enumerate(rows):
        pos[g, :len(r)] = torch.from_numpy(r.astype(np.int32))
    return pos.to(dev), torch.tensor([len(r) for r in rows], dtype=torch.int32, device=dev)


@pytest.mark.parametrize("name,top_k", [("qwen3_0p6b_8k", 1024), ("qwen3_0p6b_8k", 64)])
def test_greedy_soft_nms_against_one_pass(name, top_k):
    """Prints, per slow step, the overlap of the two selections and the dense attention mass
    each fast memory keeps; checks that both selections are valid Top-K sets and that the
    device's selection is the one-pass reading of its own scores."""
    w = get(name).replace(top_k=top_k)
    dev = "cuda"
    d = make_layer(w, 0, device=dev)
    eng = Engine(w, d["flags"], dbg_scores=True)
    lb = eng.add_layer(d["k_cache"], d["v_cache"], d["block_table"], d["q"])
    mode = O.schedule(d["flags"].cpu().numpy(), w.refresh_budget)[0]
    slow_steps = [s for s in range(w.steps) if mode[s]][:5]
    z = torch.empty(1, w.num_q_heads, eng.stride, device=dev)
    lse = torch.empty(1, w.num_q_heads, device=dev)
    out = torch.empty(1, w.num_q_heads, w.head_dim, device=dev)
    rows = []
    for s0 in slow_steps:
        N0 = w.seq_len(s0)
        lens = torch.full((1,), N0, dtype=torch.int32, device=dev)
        L.sfi_slow_attn(eng.shape, d["q"][s0], lb.k_cache, lb.v_cache, lb.block_table, lens,
                        eng.all_ids_d, 1, eng.max_len, lb.out, lb.logits, eng.stride, lb.lse,
                        eng.ws_slow)
        L.sfi_select(eng.shape, eng.params, lb.logits, eng.stride, lb.lse, lb.key_norm,
                     eng.stride, lens, eng.all_ids_d, 1, eng.max_len, lb.sel_idx, eng.dbg_buf,
                     eng.ws_sel)
        torch.cuda.synchronize()
        s_dev = eng.dbg_buf[0, :, :N0].double().cpu().numpy()
        args = (N0, w.n_sink, w.n_recent, w.top_k, w.nms_radius, w.alpha_soft, w.alpha_cross)
        one = O.select_from_scores(s_dev, *args)
        np.testing.assert_array_equal(lb.sel_idx[0].cpu().numpy(), one)
        greedy = O.select_greedy_from_scores(s_dev, *args)
        lo, hi = O.candidates(N0, w.n_sink, w.n_recent)
        keff = min(w.top_k, hi - lo)
        for g in range(w.num_kv_heads):
            v = greedy[g][:keff]
            assert np.all(np.diff(v) > 0) and v[0] >= lo and v[-1] < hi
            assert np.all(greedy[g][keff:] == -1)
        jac = np.mean([len(set(one[g][:keff]) & set(greedy[g][:keff])) /
                       len(set(one[g][:keff]) | set(greedy[g][:keff]))
                       for g in range(w.num_kv_heads)])
        # dense mass each memory keeps at the fast steps up to the next slow step
        rs = O.recent_start_at(N0, w.n_sink, w.n_recent)
        mem = {k: _packed(v, w.n_sink, dev) for k, v in (("one", one), ("greedy", greedy))}
        cov = {"one": [], "greedy": []}
        s = s0 + 1
        while s < w.steps and not mode[s] and s - s0 <= 8:
            N = w.seq_len(s)
            lens = torch.full((1,), N, dtype=torch.int32, device=dev)
            L.sfi_slow_attn(eng.shape, d["q"][s], lb.k_cache, lb.v_cache, lb.block_table,
                            lens, eng.all_ids_d, 1, eng.max_len, out, z, eng.stride, lse,
                            eng.ws_slow)
            torch.cuda.synchronize()
            for k, (pp, pl) in mem.items():
                c = coverage_of(z[0, :, :N], lse[0], memory_mask(N, w.n_sink, pp, pl, rs))
                assert bool(((c > 0) & (c <= 1 + 1e-4)).all())  # fp32 logits and lse
                cov[k].append(float(c.mean()))
            s += 1
        rows.append((s0, jac, np.mean(cov["one"]) if cov["one"] else np.nan,
                     np.mean(cov["greedy"]) if cov["greedy"] else np.nan, len(cov["one"])))
    print(f"\n{name} K {top_k}: slow step | Jaccard(one-pass, greedy) | dense mass kept: "
          "one-pass / greedy | fast steps")
    for r in rows:
        print(f"  {r[0]:4d} | {r[1]:.3f} | {r[2]:.4f} / {r[3]:.4f} | {r[4]}")
    assert rows
