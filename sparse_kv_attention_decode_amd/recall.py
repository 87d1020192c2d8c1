"""Selector quality on synthetic inputs: recall of the generator's topic positions.

The seeded generator builds every span's queries from the keys at a few topic positions per
query head (plus noise), so those positions are the support a good selection keeps while the
span lasts (the within-span stability the pages build on: nl "Kernobservatie", zh
"1 问题背景").  At every span start this runs the slow attention and the Selector on the
device and measures, for each setting of (K, lambda, alpha_soft, alpha_cross), the fraction
of the span's topic positions -- those of the G query heads of each KV head that lie among the
candidates [n_sink, N - W) -- that the KV head's selection contains.  It is a model-free proxy
for the pages' ablation of the prior fusion and the score refinement (zh "4. 实验结果").

A setting may also pool the evidence over a window of decode queries.  Then every setting is
measured at the step window_max - 1 after the span start (spans shorter than that are
skipped), so that all windows lie inside the span and all settings see the same steps.

    python -m sparse_kv_attention_decode_amd.recall --workload qwen3_4b_32k_b4
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


def topic_recall(sel: np.ndarray, topics: np.ndarray, G: int, lo: int, hi: int) -> np.ndarray:
    """Per KV head g: |topics of query heads g*G .. g*G+G-1 within [lo, hi) ∩ sel[g]| divided
    by the number of those topics (NaN when there are none).  sel [Hkv, K] (-1 padded),
    topics [Hq, t]."""
    Hkv = sel.shape[0]
    out = np.full(Hkv, np.nan)
    for g in range(Hkv):
        want = np.unique(topics[g * G:(g + 1) * G].reshape(-1))
        want = want[(want >= lo) & (want < hi)]
        if len(want):
            out[g] = np.isin(want, sel[g][sel[g] >= 0]).mean()
    return out


def default_settings(w) -> List[Dict]:
    K = w.top_k
    base = dict(top_k=K, lam=w.lam, alpha_soft=w.alpha_soft, alpha_cross=w.alpha_cross)
    out = [dict(base, label="workload setting")]
    out.append(dict(base, lam=0.0, alpha_soft=0.0, alpha_cross=0.0, label="evidence only"))
    out.append(dict(base, alpha_soft=0.0, alpha_cross=0.0, label="fusion, no refinement"))
    out.append(dict(base, lam=1.0, label="prior only (+ refinement)"))
    out.append(dict(base, alpha_soft=0.0, label="no soft-NMS"))
    out.append(dict(base, alpha_cross=0.0, label="no exclusivity"))
    out.append(dict(base, alpha_soft=0.9, alpha_cross=0.9, label="strong refinement (0.9)"))
    for f in (0.25, 0.5, 2.0):
        out.append(dict(base, top_k=max(1, int(K * f)), label=f"K x {f}"))
    return out


def run(w, settings: Optional[List[Dict]] = None, layer: int = 0, device: str = "cuda"):
    from workload.gen import make_layer
    from sparse_kv_attention_decode_amd.engine import window_query_table
    settings = default_settings(w) if settings is None else settings
    wmax = max(st.get("window", 1) for st in settings)
    d = make_layer(w, layer, device=device, keep_logical=False)
    # sized for the widest window: logits, lse and the slow workspace
    eng = Engine(w, d["flags"], device=device, window=wmax)
    lb = eng.add_layer(d["k_cache"], d["v_cache"], d["block_table"], d["q"])
    B, G = w.batch, w.group
    q_tables = {1: d["q"]}
    by_step: Dict[int, list] = {}
    for b, s0, s1, pos in d["topics"]:
        s = s0 + wmax - 1
        if s < s1:
            by_step.setdefault(s, []).append((b, pos.numpy()))
    results = []
    for st in settings:
        win = st.get("window", 1)
        if win not in q_tables:
            q_tables[win] = window_query_table(d["q"], w.num_kv_heads, win)
        params = L.make_params(w.n_sink, w.n_recent, st["top_k"], w.nms_radius, st["lam"],
                               st["alpha_soft"], st["alpha_cross"])
        sel_buf = torch.full((B, w.num_kv_heads, st["top_k"]), -1, dtype=torch.int32,
                             device=device)
        ws = L.workspace(L.sfi_select_window_ws(eng.shape, params, win, B, eng.max_len), device)
        rec, rnd = [], []
        for s, rows in sorted(by_step.items()):
            N = w.seq_len(s)
            lens = torch.full((B,), N, dtype=torch.int32, device=device)
            L.sfi_slow_attn_window(eng.shape, win, q_tables[win][s], lb.k_cache, lb.v_cache,
                                   lb.block_table, lens, eng.all_ids_d, B, eng.max_len, lb.out,
                                   lb.logits, eng.stride, lb.lse, eng.ws_slow)
            L.sfi_select_window(eng.shape, params, win, lb.logits, eng.stride, lb.lse,
                                lb.key_norm, eng.stride, lens, eng.all_ids_d, B, eng.max_len,
                                sel_buf, None, ws)
            torch.cuda.synchronize()
            sel = sel_buf.cpu().numpy()
            lo, hi = w.n_sink, max(w.n_sink, N - w.n_recent)
            for b, pos in rows:
                r = topic_recall(sel[b], pos, G, lo, hi)
                rec.extend(r[~np.isnan(r)].tolist())
                rnd.append(min(1.0, st["top_k"] / max(1, hi - lo)))
        results.append(dict(st, window=win, recall=float(np.mean(rec)),
                            recall_min=float(np.min(rec)), random=float(np.mean(rnd)),
                            samples=len(rec)))
    return results


def main() -> None:
    from workload import get
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--workload", default="qwen3_4b_32k_b4")
    ap.add_argument("--n-topics", type=int, default=None,
                    help="override the topic positions per query head and span")
    ap.add_argument("--sigma", type=float, default=None,
                    help="override the log-normal key-scale sigma")
    ap.add_argument("--query-noise", type=float, default=None,
                    help="override the std of the per-step query noise")
    ap.add_argument("--windows", default=None,
                    help="comma-separated evidence windows: run the workload setting with "
                         "each instead of the default table")
    a = ap.parse_args()
    w = get(a.workload)
    over = {}
    if a.n_topics is not None:
        over["n_topics"] = a.n_topics
    if a.sigma is not None:
        over["key_scale_sigma"] = a.sigma
    if a.query_noise is not None:
        over["query_noise"] = a.query_noise
    name = a.workload
    if over:
        name += " " + ", ".join(f"{k}={v}" for k, v in over.items())
        w = w.replace(name=w.name + "_recall_" + "_".join(f"{k}{v}" for k, v in over.items()),
                      **over)
    settings = None
    if a.windows:
        base = default_settings(w)[0]
        settings = [dict(base, window=int(x), label=f"window {int(x)}")
                    for x in a.windows.split(",")]
    res = run(w, settings)
    print(f"| setting ({name}) | K | lambda | alpha_soft | alpha_cross | window | topic recall "
          f"(mean / min over spans x KV heads) | K/|C| (random) |")
    print("|---|---|---|---|---|---|---|---|")
    for r in res:
        print(f"| {r['label']} | {r['top_k']} | {r['lam']} | {r['alpha_soft']} | "
              f"{r['alpha_cross']} | {r['window']} | {r['recall']:.3f} / "
              f"{r['recall_min']:.3f} (n={r['samples']}) | {r['random']:.3f} |")


if __name__ == "__main__":
    main()
