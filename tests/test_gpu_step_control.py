"""On-device step control and KV append (sfi_step_control, sfi_kv_append) on one MI355X.

The decisions are integer work and must match the oracle exactly; the appended rows and key
norms must be the very bits the generator stored and sfi_key_norms computes; and a trajectory
driven on the device must give bit-identical results to the same trajectory scheduled by the
host, call by call and replayed from per-step graphs.
"""
import numpy as np
import pytest
import torch

from oracle import sfi_oracle as O
from workload import get
from workload.gen import BOUNDARY_TOKENS, gen_tokens, make_layer

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sparse_kv_attention_decode_amd import lib as L
    from sparse_kv_attention_decode_amd.engine import Engine, recent_bound


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.parametrize("batch,steps,budget,sliding", [(1, 40, 3, False), (5, 64, 4, False),
                                                       (600, 12, 2, False), (5, 64, 4, True)])
def test_step_control_matches_oracle(batch, steps, budget, sliding):
    """Every output of every step, bit-exact, against the oracle's step control.  600 rows
    span three chunks of the control kernel's workgroup."""
    rng = np.random.default_rng(batch * 1000 + steps)
    n_stored, n_sink, n_recent = 500, 4, 64
    tokens = rng.integers(0, 2000, size=(batch, steps)).astype(np.int32)
    tokens[rng.random((batch, steps)) < 0.15] = 1003
    shape = L.make_shape(batch, 8, 2, 128, 64, "bf16")
    params = L.make_params(n_sink, n_recent, 128, 4, 0.3, 0.5, 0.5)
    dev = "cuda"
    tok_d = torch.from_numpy(tokens.T.copy()).to(dev)            # [S, B]
    bnd = torch.tensor(BOUNDARY_TOKENS, dtype=torch.int32, device=dev)
    state = torch.stack([torch.full((batch,), n_stored, dtype=torch.int32),
                         torch.full((batch,), -1, dtype=torch.int32),
                         torch.zeros(batch, dtype=torch.int32)]).to(dev)
    # alternate two buffers as the engine does; every other step runs in place
    other = torch.empty_like(state)
    slow = torch.empty(batch, dtype=torch.int32, device=dev)
    fast = torch.empty(batch, dtype=torch.int32, device=dev)
    cnt = torch.empty(2, dtype=torch.int32, device=dev)
    ref = O.step_control(tokens, BOUNDARY_TOKENS, budget, n_stored, n_sink, n_recent,
                         sliding=sliding)
    for s in range(steps):
        out = state if s % 3 == 0 else other
        L.sfi_step_control(shape, params, budget, tok_d[s], bnd, len(BOUNDARY_TOKENS), state,
                           out, slow, fast, cnt, sliding_recent=sliding)
        torch.cuda.synchronize()
        state, other = out, (other if out is state else state)
        np.testing.assert_array_equal(state[0].cpu().numpy(), ref["seq_len"][s], f"step {s}")
        np.testing.assert_array_equal(state[2].cpu().numpy(), ref["recent_start"][s],
                                      f"step {s}")
        np.testing.assert_array_equal(slow.cpu().numpy(), ref["slow_ids"][s], f"step {s}")
        np.testing.assert_array_equal(fast.cpu().numpy(), ref["fast_ids"][s], f"step {s}")
        np.testing.assert_array_equal(cnt.cpu().numpy(), ref["counts"][s], f"step {s}")


def _engines(w, layers, graphs=False, inc=None):
    """A host-scheduled and a device-controlled engine over the same generated layers."""
    data = [make_layer(w, li, device="cuda") for li in range(layers)]
    tokens = gen_tokens(w, data[0]["flags"])
    # the host engine passes whole -1-padded lists too, so both launch the same splits
    host = Engine(w, data[0]["flags"], max_recent=recent_bound(w), full_lists=True,
                  incremental_pack=inc)
    devc = Engine(w, data[0]["flags"], device_control=True, tokens=tokens,
                  boundary_tokens=BOUNDARY_TOKENS, incremental_pack=inc)
    for d in data:
        host.add_layer(d["k_cache"], d["v_cache"], d["block_table"], d["q"])
        devc.add_layer(d["k_cache"].clone(), d["v_cache"].clone(), d["block_table"], d["q"])
    if graphs:
        devc.enable_device_graphs()
    return data, host, devc


@pytest.mark.parametrize("name,batch,layers,graphs,sliding,inc",
                         [("tiny_fp32_1k", 1, 1, False, False, None),
                          ("qwen3_0p6b_8k", 3, 1, False, False, None),
                          ("qwen3_0p6b_8k", 3, 2, True, False, None),
                          ("qwen3_0p6b_8k", 3, 1, False, True, None),
                          ("qwen3_0p6b_8k", 3, 1, False, False, True)])
def test_device_trajectory_bit_identical_to_host(name, batch, layers, graphs, sliding, inc):
    """The whole trajectory decided on the device (tokens -> modes, K/V appended step by
    step) against the host schedule: outputs after every step, then the selections, the
    packed buffers, the re-filled caches and the key norms, all bit for bit."""
    w = get(name).replace(batch=batch, name=f"{name}_b{batch}", sliding_recent=sliding)
    data, host, devc = _engines(w, layers, graphs, inc)
    for s in range(w.steps):
        host.step(s)
        devc.step(s)
        host.join()
        devc.join()
        torch.cuda.synchronize()
        for li in range(layers):
            assert bool((_bits(host.layers[li].out) == _bits(devc.layers[li].out)).all()), \
                f"step {s} layer {li} mode {host.mode(s)}"
    for li in range(layers):
        hl, dl = host.layers[li], devc.layers[li]
        assert torch.equal(hl.sel_idx, dl.sel_idx)
        assert torch.equal(hl.packed_pos, dl.packed_pos)
        assert torch.equal(hl.packed_len, dl.packed_len)
        assert bool((_bits(hl.packed_k) == _bits(dl.packed_k)).all())
        # every appended row is back in the cache, and its norm is the stored statistic
        n_used = w.context + w.steps - 1
        assert bool((_bits(hl.k_cache) == _bits(dl.k_cache)).all())
        assert bool((_bits(hl.v_cache) == _bits(dl.v_cache)).all())
        assert bool((_bits(hl.key_norm[:, :, :n_used]) == _bits(dl.key_norm[:, :, :n_used]))
                    .all())
    # the device's own state at the end
    ref = O.step_control(gen_tokens(w, data[0]["flags"]).numpy().T, BOUNDARY_TOKENS,
                         w.refresh_budget, w.context - 1, w.n_sink, w.n_recent,
                         sliding=sliding)
    st = devc.device_state(w.steps - 1)
    np.testing.assert_array_equal(st[0].cpu().numpy(), ref["seq_len"][-1])
    np.testing.assert_array_equal(st[2].cpu().numpy(), ref["recent_start"][-1])


def test_device_trajectory_restarts():
    """Running the trajectory twice (step 0 resets the state) gives the same results."""
    w = get("qwen3_0p6b_8k").replace(steps=48, name="qwen3_0p6b_8k_s48")
    data, host, devc = _engines(w, 1, inc=True)
    outs = []
    for rep in range(2):
        for s in range(w.steps):
            devc.step(s)
        devc.join()
        torch.cuda.synchronize()
        outs.append(devc.layers[0].out.clone())
    assert bool((_bits(outs[0]) == _bits(outs[1])).all())


@pytest.mark.parametrize("name,win", [("qwen3_0p6b_8k", 1), ("qwen3_0p6b_8k", 4),
                                      ("tiny_fp32_1k", 2)])
def test_decode_attn_matches_separate_calls(name, win):
    """sfi_decode_attn (fast and slow rows in one launch pair) against sfi_fast_attn plus
    sfi_slow_attn_window with the same lists: output, logits and lse bit for bit."""
    B = 3
    w = get(name).replace(batch=B, name=f"{name}_b{B}", evidence_window=win)
    d = make_layer(w, 0, device="cuda")
    eng = Engine(w, d["flags"])
    lb = eng.add_layer(d["k_cache"], d["v_cache"], d["block_table"], d["q"])
    dev = "cuda"
    all_ids = eng.all_ids_d
    # a slow step of every row fills the packed buffers
    s0 = 5
    N0 = w.seq_len(s0)
    lens0 = torch.full((B,), N0, dtype=torch.int32, device=dev)
    L.sfi_slow_attn_window(eng.shape, win, lb.q_win[s0] if win > 1 else d["q"][s0], lb.k_cache,
                           lb.v_cache, lb.block_table, lens0, all_ids, B, eng.max_len, lb.out,
                           lb.logits, eng.stride, lb.lse, eng.ws_slow)
    L.sfi_select_window(eng.shape, eng.params, win, lb.logits, eng.stride, lb.lse, lb.key_norm,
                        eng.stride, lens0, all_ids, B, eng.max_len, lb.sel_idx, None,
                        eng.ws_sel)
    L.sfi_pack(eng.shape, eng.params, lb.k_cache, lb.v_cache, lb.block_table, lb.sel_idx,
               all_ids, B, lb.packed_k, lb.packed_v, lb.packed_pos, lb.packed_len,
               eng.packed_cap)
    # three steps later rows 0 and 2 are fast, row 1 is slow
    s1 = s0 + 3
    N1 = w.seq_len(s1)
    lens1 = torch.full((B,), N1, dtype=torch.int32, device=dev)
    rstart = torch.full((B,), O.recent_start_at(N0, w.n_sink, w.n_recent), dtype=torch.int32,
                        device=dev)
    fast_ids = torch.tensor([0, 2, -1], dtype=torch.int32, device=dev)
    slow_ids = torch.tensor([1, -1, -1], dtype=torch.int32, device=dev)
    max_recent = recent_bound(w)
    q = d["q"][s1]
    qw = lb.q_win[s1] if win > 1 else q
    Hq = w.num_q_heads

    def buffers():
        return (torch.full((B, Hq, w.head_dim), 7.0, device=dev),
                torch.full((B, Hq * win, eng.stride), 7.0, device=dev),
                torch.full((B, Hq * win), 7.0, device=dev))

    out_a, z_a, lse_a = buffers()
    ws = L.workspace(L.sfi_decode_attn_ws(eng.shape, win, B, eng.packed_cap, max_recent,
                                          eng.max_len), dev)
    L.sfi_decode_attn(eng.shape, win, q, qw, lb.packed_k, lb.packed_v, lb.packed_len,
                      eng.packed_cap, lb.k_cache, lb.v_cache, lb.block_table, rstart, lens1,
                      fast_ids, slow_ids, B, max_recent, eng.max_len, out_a, z_a, eng.stride,
                      lse_a, ws)
    out_b, z_b, lse_b = buffers()
    ws_f = L.workspace(L.sfi_fast_attn_ws(eng.shape, B, eng.packed_cap, max_recent), dev)
    L.sfi_fast_attn(eng.shape, q, lb.packed_k, lb.packed_v, lb.packed_len, eng.packed_cap,
                    lb.k_cache, lb.v_cache, lb.block_table, rstart, lens1, fast_ids, B,
                    max_recent, out_b, None, ws_f)
    L.sfi_slow_attn_window(eng.shape, win, qw, lb.k_cache, lb.v_cache, lb.block_table, lens1,
                           slow_ids, B, eng.max_len, out_b, z_b, eng.stride, lse_b, eng.ws_slow)
    torch.cuda.synchronize()
    assert bool((_bits(out_a) == _bits(out_b)).all())
    assert bool((_bits(z_a) == _bits(z_b)).all())
    assert bool((_bits(lse_a) == _bits(lse_b)).all())
    # rows of neither list are untouched; the slow row's logits and lse were written
    assert bool((z_a[0] == 7.0).all()) and bool((lse_a[2] == 7.0).all())
    assert not bool((z_a[1, :, :N1] == 7.0).any())
