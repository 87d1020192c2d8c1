"""The allocation-free fast call (sfi_fast_attn_noalloc) against sfi_fast_attn, through the C
ABI on the GPU: two calls in a row, the second on a smaller input, each bit-identical to the
workspace call on the same inputs and within the parity bar of the fp64 oracle."""
import numpy as np
import pytest
import torch

from oracle import sfi_oracle as O
from workload import get
from workload.gen import make_layer
from sfi_testlib import check_out, host64, oracle_layer_arrays, oracle_schedule

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sparse_kv_attention_decode_amd import lib as L
    from sparse_kv_attention_decode_amd.engine import Engine


def test_noalloc_fast_attn_matches_workspace_call():
    w = get("qwen3_0p6b_8k").replace(batch=2, context=4096, steps=4, name="noalloc_b2")
    d = make_layer(w, 0, device="cuda")
    eng = Engine(w, d["flags"])
    lb = eng.add_layer(d["k_cache"], d["v_cache"], d["block_table"], d["q"])
    assert oracle_schedule(w, d["flags"], eng.plan)[:, 0].all()
    eng.step(0)  # slow step: dense attention, Selector, pack of both rows
    eng.join()
    torch.cuda.synchronize()
    N0 = w.seq_len(0)
    rs = O.recent_start_at(N0, w.n_sink, w.n_recent)
    q = d["q"][1]

    def both(ids, lens, plen):
        """The fast call on the listed rows through both entry points."""
        n = ids.numel()
        rstart = torch.full((w.batch,), rs, dtype=torch.int32, device="cuda")
        out_ws = torch.full_like(lb.out, 77.0)
        out_na = torch.full_like(lb.out, 77.0)
        ws = L.workspace(L.sfi_fast_attn_ws(eng.shape, n, eng.packed_cap, eng.max_recent),
                         "cuda")
        L.sfi_fast_attn(eng.shape, q, lb.packed_k, lb.packed_v, plen, eng.packed_cap,
                        lb.k_cache, lb.v_cache, lb.block_table, rstart, lens, ids, n,
                        eng.max_recent, out_ws, None, ws)
        L.sfi_fast_attn_noalloc(eng.shape, q, lb.packed_k, lb.packed_v, plen, eng.packed_cap,
                                lb.k_cache, lb.v_cache, lb.block_table, rstart, lens, ids, n,
                                eng.max_recent, out_na, None)
        torch.cuda.synchronize()
        assert torch.equal(out_ws.view(torch.int32), out_na.view(torch.int32))
        return out_na

    # first call: both rows at the next step's length, the whole packed memory
    ids = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    lens = torch.full((w.batch,), w.seq_len(1), dtype=torch.int32, device="cuda")
    out = host64(both(ids, lens, lb.packed_len))
    # second call, smaller: one row, a shorter history and half of its packed rows
    ids2 = torch.tensor([1], dtype=torch.int32, device="cuda")
    lens2 = torch.full((w.batch,), N0 + 0, dtype=torch.int32, device="cuda")
    plen2 = (lb.packed_len // 2).contiguous()
    out2 = both(ids2, lens2, plen2)
    assert bool((out2[0] == 77.0).all())  # row 0 is not listed: untouched
    out2 = host64(out2)

    ppos = lb.packed_pos.cpu().numpy()
    for b, o_dev, N, pl in [(0, out, w.seq_len(1), lb.packed_len), (1, out, w.seq_len(1),
                                                                     lb.packed_len),
                            (1, out2, N0, plen2)]:
        qh, K, V = oracle_layer_arrays(d, b)
        n = pl[b].cpu().numpy()
        packed = [np.sort(ppos[b, g, :n[g]]) for g in range(w.num_kv_heads)]
        o, _ = O.fast_attention(qh[1], K, V, packed, rs, N)
        check_out(o_dev[b], o, f"row {b} N {N}")
