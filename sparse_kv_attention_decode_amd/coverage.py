"""Fast-memory quality on synthetic inputs: how much of the dense attention the fast memory
keeps.

A fast step attends to the sink, the selected rows of the last slow step and the recent
segment instead of the whole history (es "2. Metodología", zh "2.1 慢快推理框架").  At every fast step
of a one-layer trajectory this tool also runs the dense attention of the same query and
reports, per (row, query head):
  * coverage   the dense softmax mass on the positions of the fast memory, sum_{j in M} p_j;
  * rel_err    |o_fast - o_dense| / |o_dense| of the attention output.
Coverage 1 means the fast step is exact.  Settings vary the knobs the pages name (the prior
weight lambda, soft-NMS and exclusivity strength, K, the recent window's behaviour, the
evidence window), which makes this a model-free proxy for the pages' ablation next to the
topic recall of recall.py.

    python -m sparse_kv_attention_decode_amd.coverage --workload qwen3_4b_32k_b4
"""
from __future__ import annotations

import argparse
import os
import sys
from typing import Dict, List, Optional

import numpy as np
import torch

if __package__ in (None, ""):
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from sparse_kv_attention_decode_amd import lib as L  # noqa: E402
from sparse_kv_attention_decode_amd.engine import Engine  # noqa: E402


def memory_mask(N: int, n_sink: int, packed_pos: torch.Tensor, packed_len: torch.Tensor,
                recent_start: int) -> torch.Tensor:
    """Positions of one row's fast memory, bool [Hkv, N]: the sink, the packed rows of each
    KV head (packed_pos [Hkv, cap], the first packed_len [Hkv] valid) and [recent_start, N)."""
    Hkv, cap = packed_pos.shape
    m = torch.zeros(Hkv, N, dtype=torch.bool, device=packed_pos.device)
    m[:, :min(n_sink, N)] = True
    valid = torch.arange(cap, device=packed_pos.device)[None, :] < packed_len[:, None]
    g_idx = torch.arange(Hkv, device=packed_pos.device)[:, None].expand(Hkv, cap)
    m[g_idx[valid], packed_pos[valid].long()] = True
    m[:, recent_start:N] = True
    return m


def coverage_of(z: torch.Tensor, lse: torch.Tensor, mask: torch.Tensor) -> torch.Tensor:
    """Dense softmax mass on the masked positions per query head: z [Hq, N] logits, lse [Hq],
    mask [Hkv, N] (query head h reads KV head h // G)."""
    Hq = z.shape[0]
    G = Hq // mask.shape[0]
    p = torch.exp(z.double() - lse.double()[:, None])
    return (p * mask.repeat_interleave(G, dim=0)).sum(dim=1)


def default_settings(w) -> List[Dict]:
    base = dict(label="workload setting")
    return [base,
            dict(label="sliding recent window", sliding_recent=True),
            dict(label="strict exclusivity (alpha_cross = 1)", alpha_cross=1.0),
            dict(label="no exclusivity (alpha_cross = 0)", alpha_cross=0.0),
            dict(label="no soft-NMS (alpha_soft = 0)", alpha_soft=0.0),
            dict(label="evidence only (lambda = 0)", lam=0.0),
            dict(label="evidence window 4", evidence_window=4),
            dict(label="K x 0.5", top_k=max(1, w.top_k // 2)),
            dict(label="K x 2", top_k=w.top_k * 2)]


def run(w, settings: Optional[List[Dict]] = None, layer: int = 0, device: str = "cuda",
        max_fast_steps: Optional[int] = None) -> List[Dict]:
    from workload.gen import make_layer
    settings = default_settings(w) if settings is None else settings
    d = make_layer(w, layer, device=device, keep_logical=False)
    results = []
    for st in settings:
        over = {k: v for k, v in st.items() if k != "label"}
        wv = w.replace(**over)
        if wv.evidence_window * wv.group > 16:
            continue
        eng = Engine(wv, d["flags"], device=device)
        lb = eng.add_layer(d["k_cache"], d["v_cache"], d["block_table"], d["q"])
        B, Hq = wv.batch, wv.num_q_heads
        z_d = torch.empty(B, Hq, eng.stride, dtype=torch.float32, device=device)
        lse_d = torch.empty(B, Hq, dtype=torch.float32, device=device)
        out_d = torch.empty(B, Hq, wv.head_dim, dtype=torch.float32, device=device)
        cov, err = [], []
        n_fast = 0
        for s in range(wv.steps):
            eng.step(s)
            eng.join()
            fast_rows = eng.plan.fast_ids[s]
            if len(fast_rows) == 0:
                continue
            if max_fast_steps is not None and n_fast >= max_fast_steps:
                break
            n_fast += 1
            N = wv.seq_len(s)
            lens = torch.full((B,), N, dtype=torch.int32, device=device)
            with torch.cuda.stream(eng.stream1):
                L.sfi_slow_attn(eng.shape, d["q"][s], lb.k_cache, lb.v_cache, lb.block_table,
                                lens, eng.all_ids_d, B, eng.max_len, out_d, z_d, eng.stride,
                                lse_d, eng.ws_slow, stream=eng.stream1)
            torch.cuda.synchronize()
            for b in fast_rows:
                b = int(b)
                m = memory_mask(N, wv.n_sink, lb.packed_pos[b], lb.packed_len[b],
                                int(eng.plan.recent_start[s, b]))
                cov.append(coverage_of(z_d[b, :, :N], lse_d[b], m).cpu().numpy())
                num = (lb.out[b].double() - out_d[b].double()).norm(dim=1)
                err.append((num / out_d[b].double().norm(dim=1)).cpu().numpy())
        cov_a = np.concatenate(cov) if cov else np.array([np.nan])
        err_a = np.concatenate(err) if err else np.array([np.nan])
        results.append(dict(st, coverage=float(cov_a.mean()), coverage_min=float(cov_a.min()),
                            rel_err=float(err_a.mean()), rel_err_max=float(err_a.max()),
                            fast_steps=n_fast, samples=int(cov_a.size)))
        del eng, lb
        torch.cuda.empty_cache()
    return results


def main() -> None:
    from workload import get
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--workload", default="qwen3_4b_32k_b4")
    ap.add_argument("--max-fast-steps", type=int, default=None,
                    help="stop after this many fast steps per setting")
    ap.add_argument("--layer", type=int, default=0)
    ap.add_argument("--k-scale", type=float, default=1.0,
                    help="scale the workload's K first (a small K makes the settings differ)")
    a = ap.parse_args()
    w = get(a.workload)
    if w.layers > 1:
        w = w.replace(layers=1)
    if a.k_scale != 1.0:
        w = w.replace(top_k=max(1, int(round(w.top_k * a.k_scale))))
    res = run(w, layer=a.layer, max_fast_steps=a.max_fast_steps)
    print(f"| setting ({a.workload}, layer {a.layer}, K {w.top_k}) | dense mass on the fast "
          f"memory (mean / min) "
          f"| fast vs dense output rel. error (mean / max) | fast steps |")
    print("|---|---|---|---|")
    for r in res:
        print(f"| {r['label']} | {r['coverage']:.4f} / {r['coverage_min']:.4f} | "
              f"{r['rel_err']:.4f} / {r['rel_err_max']:.4f} | {r['fast_steps']} |")


if __name__ == "__main__":
    main()
