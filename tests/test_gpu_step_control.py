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


@pytest.mark.parametrize("batch,steps,budget", [(1, 40, 3), (5, 64, 4), (600, 12, 2)])
def test_step_control_matches_oracle(batch, steps, budget):
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
    seq = torch.full((batch,), n_stored, dtype=torch.int32, device=dev)
    since = torch.full((batch,), -1, dtype=torch.int32, device=dev)
    rs = torch.zeros(batch, dtype=torch.int32, device=dev)
    slow = torch.empty(batch, dtype=torch.int32, device=dev)
    fast = torch.empty(batch, dtype=torch.int32, device=dev)
    cnt = torch.empty(2, dtype=torch.int32, device=dev)
    ref = O.step_control(tokens, BOUNDARY_TOKENS, budget, n_stored, n_sink, n_recent)
    for s in range(steps):
        L.sfi_step_control(shape, params, budget, tok_d[s], bnd, len(BOUNDARY_TOKENS), seq,
                           since, rs, slow, fast, cnt)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(seq.cpu().numpy(), ref["seq_len"][s], f"step {s}")
        np.testing.assert_array_equal(rs.cpu().numpy(), ref["recent_start"][s], f"step {s}")
        np.testing.assert_array_equal(slow.cpu().numpy(), ref["slow_ids"][s], f"step {s}")
        np.testing.assert_array_equal(fast.cpu().numpy(), ref["fast_ids"][s], f"step {s}")
        np.testing.assert_array_equal(cnt.cpu().numpy(), ref["counts"][s], f"step {s}")


def _engines(w, layers, graphs=False):
    """A host-scheduled and a device-controlled engine over the same generated layers."""
    data = [make_layer(w, li, device="cuda") for li in range(layers)]
    tokens = gen_tokens(w, data[0]["flags"])
    # the host engine passes whole -1-padded lists too, so both launch the same splits
    host = Engine(w, data[0]["flags"], max_recent=recent_bound(w), full_lists=True)
    devc = Engine(w, data[0]["flags"], device_control=True, tokens=tokens,
                  boundary_tokens=BOUNDARY_TOKENS)
    for d in data:
        host.add_layer(d["k_cache"], d["v_cache"], d["block_table"], d["q"])
        devc.add_layer(d["k_cache"].clone(), d["v_cache"].clone(), d["block_table"], d["q"])
    if graphs:
        devc.enable_device_graphs()
    return data, host, devc


@pytest.mark.parametrize("name,batch,layers,graphs",
                         [("tiny_fp32_1k", 1, 1, False), ("qwen3_0p6b_8k", 3, 1, False),
                          ("qwen3_0p6b_8k", 3, 2, True)])
def test_device_trajectory_bit_identical_to_host(name, batch, layers, graphs):
    """The whole trajectory decided on the device (tokens -> modes, K/V appended step by
    step) against the host schedule: outputs after every step, then the selections, the
    packed buffers, the re-filled caches and the key norms, all bit for bit."""
    w = get(name).replace(batch=batch, name=f"{name}_b{batch}")
    data, host, devc = _engines(w, layers, graphs)
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
                         w.refresh_budget, w.context - 1, w.n_sink, w.n_recent)
    np.testing.assert_array_equal(devc.state[0].cpu().numpy(), ref["seq_len"][-1])
    np.testing.assert_array_equal(devc.state[2].cpu().numpy(), ref["recent_start"][-1])


def test_device_trajectory_restarts():
    """Running the trajectory twice (step 0 resets the state) gives the same results."""
    w = get("qwen3_0p6b_8k").replace(steps=48, name="qwen3_0p6b_8k_s48")
    data, host, devc = _engines(w, 1)
    outs = []
    for rep in range(2):
        for s in range(w.steps):
            devc.step(s)
        devc.join()
        torch.cuda.synchronize()
        outs.append(devc.layers[0].out.clone())
    assert bool((_bits(outs[0]) == _bits(outs[1])).all())
