"""Shared helpers of the GPU parity tests: device inputs from the seeded generator, host
fp64 copies for the oracle, and the comparison rules.

Parity rules (fp32 device arithmetic on bf16/fp32 stored K/V against the fp64 oracle):
  * attention output: per (row, query head) max|o_gpu - o_ref| / max|o_ref| <= 2e-3;
  * lse: |lse_gpu - lse_ref| <= max(1e-4, 1e-5 * sum_j p_j |q|·|k_j| / sqrt(D)), the
    larger of a flat 1e-4 and the logit bound below propagated through the softmax
    (check_lse);
  * logits: |z_gpu - z_ref| <= 1e-5 * |q|·|k| / sqrt(D)  (relative to the Cauchy-Schwarz
    scale of the dot product, which a cancelling sum cannot undercut);
  * key norms: relative 1e-6;
  * Top-K on the device's own fused scores: identical index lists;
  * Top-K end to end: the device set may differ from the oracle's only at positions whose
    oracle refined log-score ln s' is within relative 1e-5 of the K-th one, or where a
    refinement decision (soft-NMS dominance, head ownership) is within relative 1e-5 of
    ln s in the oracle.  The allowance is taken on the log-score, where the refinement
    and the Top-K compare; with |ln s'| around 7-12 it admits score differences of about
    1e-4 relative, the size of the fp32 logit error (1e-5 of the Cauchy-Schwarz scale)
    after the softmax.  How many of the differences also lie within relative 1e-5 of the
    K-th score s' itself is counted and reported;
  * pack: bit-exact.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import sfi_oracle as O

O_TOL = 2e-3
LSE_TOL = 1e-4
Z_TOL = 1e-5
TIE_TOL = 1e-5


def host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def check_out(o_gpu: np.ndarray, o_ref: np.ndarray, what: str = "o"):
    """o arrays [..., D]; per-row relative max error."""
    o_gpu = np.asarray(o_gpu, np.float64).reshape(-1, o_ref.shape[-1])
    o_ref = np.asarray(o_ref, np.float64).reshape(-1, o_ref.shape[-1])
    den = np.maximum(np.abs(o_ref).max(axis=1), 1e-30)
    err = np.abs(o_gpu - o_ref).max(axis=1) / den
    assert err.max() <= O_TOL, f"{what}: max row rel err {err.max():.3e} (row {err.argmax()})"
    return float(err.max())


def check_lse(l_gpu, l_ref, p=None, q=None, K=None, what="lse"):
    """|dlse| <= max(LSE_TOL, Z_TOL * sum_j p_j |q||k_j| / sqrt(D)).

    lse is a smooth maximum of the logits (d lse / d z_j = p_j), so its error is at most the
    p-weighted logit error; with the logit bound of check_logits that is the second term.
    p [Hq, N], q [Hq, D], K [Hkv, N, D] of the oracle give the bound per head."""
    d = np.abs(np.asarray(l_gpu, np.float64) - np.asarray(l_ref, np.float64))
    tol = np.full(d.shape, LSE_TOL)
    if p is not None:
        Hq, D = q.shape
        G = Hq // K.shape[0]
        kn = np.linalg.norm(K, axis=2)
        qn = np.linalg.norm(q, axis=1)
        for h in range(Hq):
            tol[h] = max(LSE_TOL, Z_TOL * qn[h] * float(p[h] @ kn[h // G]) / np.sqrt(D))
    assert (d <= tol).all(), f"{what}: |dlse| {d.max():.3e} vs tol {tol[d.argmax()]:.3e}"
    return float(d.max())


def check_logits(z_gpu, z_ref, q, K, D):
    """z [Hq, N] for one row; q [Hq, D]; K [Hkv, N, D]."""
    Hq = q.shape[0]
    G = Hq // K.shape[0]
    qn = np.linalg.norm(q, axis=1)
    kn = np.linalg.norm(K, axis=2)
    worst = 0.0
    for h in range(Hq):
        scale = qn[h] * kn[h // G] / np.sqrt(D)
        err = np.abs(z_gpu[h] - z_ref[h]) / np.maximum(scale, 1e-30)
        worst = max(worst, float(err.max()))
    assert worst <= Z_TOL, f"logits: max scaled err {worst:.3e}"
    return worst


def explain_selection_diff(sel_gpu: np.ndarray, selection: "O.Selection", N: int):
    """Check that every difference between the device and oracle index sets is a near-tie
    (the end-to-end rule in the module docstring).  Returns (n_diff, n_kth_ties,
    n_decision_ties, n_score_ties): the K-th ties are counted on ln s', and n_score_ties
    counts those of them that are also within relative 1e-5 of the K-th score s'."""
    ref = selection.refined
    lo = selection.lo
    n_diff = n_kth = n_dec = n_score = 0
    for g in range(sel_gpu.shape[0]):
        a = set(int(x) for x in sel_gpu[g] if x >= 0)
        b = set(int(x) for x in selection.sel[g] if x >= 0)
        if len(a) != len(b):
            raise AssertionError(f"head {g}: |sel| {len(a)} vs {len(b)}")
        diff = a ^ b
        if not diff:
            continue
        keff = len(b)
        vals = ref.ellp[g]
        order = np.lexsort((np.arange(len(vals)), -vals))
        kth = vals[order[keff - 1]] if keff else 0.0
        for j in diff:
            c = j - lo
            v = vals[c]
            n_diff += 1
            if np.isfinite(kth) and abs(v - kth) <= TIE_TOL * max(abs(kth), 1e-30):
                n_kth += 1
                if abs(np.expm1(v - kth)) <= TIE_TOL:
                    n_score += 1
            elif ref.dom_margin[g, c] <= TIE_TOL or ref.own_margin[c] <= TIE_TOL:
                n_dec += 1
            else:
                raise AssertionError(
                    f"head {g} position {j}: ell'={v:.9g} K-th={kth:.9g} not a near-tie "
                    f"(dom margin {ref.dom_margin[g, c]:.2e}, own margin {ref.own_margin[c]:.2e})")
    return n_diff, n_kth, n_dec, n_score


def oracle_schedule(w, flags, plan=None) -> np.ndarray:
    """Slow/fast mode [B, S] of a trajectory from the oracle's schedule of the seeded flags.
    When the engine's host plan is given, it must agree: the tests then follow the oracle's
    decisions, never the plan's."""
    flags = flags.cpu().numpy() if torch.is_tensor(flags) else np.asarray(flags)
    mode = O.schedule(flags, w.refresh_budget)
    if plan is not None:
        np.testing.assert_array_equal(plan.mode, mode, err_msg="host plan vs oracle schedule")
    return mode


def oracle_layer_arrays(d: dict, b: int):
    """fp64 host copies of row b: q [S, Hq, D], K/V [Hkv, total, D]."""
    return host64(d["q"][:, b]), host64(d["K"][b]), host64(d["V"][b])


def model_pack_update(ppos, plen, sel, n_sink):
    """Slot-by-slot state of one (row, KV head) of the packed buffer after sfi_pack_update,
    from the order the call documents: ppos [cap] positions per slot (-1 empty), plen the
    held length before the update, sel the new selection (ascending, valid entries only).

    An empty buffer (plen 0) or a selection smaller than what is held is rebuilt in the
    full pack's order: sink rows, then sel.  Otherwise every held row whose position stays
    selected keeps its slot; the slots of the others are freed, in ascending slot order; the
    newly selected positions, in ascending order, take the freed slots first and then the
    slots from the old end on.  Returns (ppos', plen')."""
    ppos = [int(x) for x in ppos]
    cap = len(ppos)
    sel = [int(x) for x in sel]
    keff = len(sel)
    if plen == 0 or keff < max(0, plen - n_sink):
        new = list(range(n_sink)) + sel
        return new + [-1] * (cap - len(new)), n_sink + keff
    held = {ppos[s]: s for s in range(n_sink, plen)}
    chosen = set(sel)
    free = [s for s in range(n_sink, plen) if ppos[s] not in chosen]
    added = [p for p in sel if p not in held]
    new = list(ppos)
    for j, p in enumerate(added):
        slot = free[j] if j < len(free) else plen + (j - len(free))
        new[slot] = p
    return new, n_sink + keff
