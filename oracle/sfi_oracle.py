"""Plain fp64 CPU oracle of the Slow-Fast Inference (SFI) decode path.

TEST INFRASTRUCTURE ONLY.  Only tests, the smoke check and the benchmark's CPU-baseline
leg may import this module.  The device path never calls it, and it shares no code with
the device path: it reads only NumPy arrays handed to it.

Sources (the pages are five summaries of one paper, "Slow-Fast Inference: Training-Free
Inference Acceleration via Within-Sentence Support Stability"; cited by language and
section):
  * fast / slow steps and the fast memory (sink + recent window + selected memory):
    es "2. Metodología", fr "2.A Le Paradigme Lente-Rapide", zh "2.1 慢快推理框架";
  * Selector (evidence f, prior r, fusion s = (1-λ)f + λr, soft-NMS, cross-head
    exclusivity, Top-K): zh "2.2 训练无感的 Selector", fr "2.B Le Sélecteur",
    nl "De Selector";
  * compact buffer of sink + selected tokens, recent tokens read from the paged cache:
    zh "2.3 系统级优化", nl "Systeemontwerp en Kernel-optimalisatie".

Where the pages leave a step open, the plainest reading is taken; each reading is named
in the docstring of the function that applies it.

Parity status of each function:
  attention, merge_segments, evidence, window_evidence, window_queries, fuse, topk, pack,
  packed_positions, fast_attention, fast_attention_single_pass, schedule, boundary_flags,
  step_control, candidates, recent_start_at, recent_start_sliding, run_sequence:
      pinned by tests (closed forms, library routines, brute force, partition and
      equivalence invariants).
  select, select_window, select_from_evidence, select_from_scores,
  select_greedy_from_scores: compositions of the pinned steps, each also checked end to
      end (worked examples, K covering the candidates, the greedy reading's reduction to
      the one-pass one without soft-NMS).
  key_norms: pinned (library norm).
  prior: pinned to its reading by a hand-derived example (the key-norm floor, the
      distance N-1-j, the +1 terms and the normalisation) and by invariants (normalisation,
      positivity, monotonicity).  The functional form itself is a reading the pages do not
      fix: the pin checks the oracle against the reading, not the reading against the pages.
  refine: pinned by a hand-derived worked example at α_soft = α_cross = 0.5 (dominance,
      ownership with a tie, the refined products, Top-K with a tie) and by special cases
      (identity at α=0, local maxima at α_soft=1, ownership at α_cross=1).
  refine_greedy (an alternative reading): pinned by a worked example, a plain
      quadratic simulation, its reductions (α_soft = 0 or R = 0) and hard NMS at α_soft = 1.
  adaptive_lambda, fuse_per_head (the clipped adaptive fusion weight, a reading): pinned by
      hand-worked entropies, the point-mass and uniform limits, λclip = 0 (evidence only)
      and the per-head fusion staying a distribution.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

F64 = np.float64


# ----------------------------------------------------------------------------- attention
def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray):
    """Dense GQA decode attention of one query token over rows K, V.

    Slow steps run dense attention over the whole accessible history (es "2. Metodología",
    zh "2.1 慢快推理框架").  q [Hq, D]; K, V [Hkv, n, D]; query head h reads KV head h // G.
    Logits z = q·k / sqrt(D) (no positional term: keys are taken as already rotated).
    Returns o [Hq, D], z [Hq, n], lse [Hq], p [Hq, n] (softmax probabilities).
    """
    q = np.asarray(q, F64)
    K = np.asarray(K, F64)
    V = np.asarray(V, F64)
    Hq, D = q.shape
    Hkv, n, _ = K.shape
    G = Hq // Hkv
    z = np.empty((Hq, n), F64)
    for h in range(Hq):
        z[h] = K[h // G] @ q[h] / math.sqrt(D)
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    o = np.empty((Hq, D), F64)
    for h in range(Hq):
        o[h] = p[h] @ V[h // G]
    lse = (m + np.log(l))[:, 0]
    return o, z, lse, p


def merge_segments(parts: List[Tuple[np.ndarray, np.ndarray]]):
    """Combine attention results over disjoint row sets by log-sum-exp weights.

    parts: list of (o [Hq, D], lse [Hq]), each normalised over its own rows.  The union's
    output is sum_s exp(lse_s - lse) o_s with lse = log sum_s exp(lse_s).
    """
    lses = np.stack([np.asarray(l, F64) for _, l in parts])          # [S, Hq]
    m = lses.max(axis=0)
    w = np.exp(lses - m)
    tot = w.sum(axis=0)
    o = sum(w[i][:, None] * np.asarray(parts[i][0], F64) for i in range(len(parts)))
    return o / tot[:, None], m + np.log(tot)


# ------------------------------------------------------------------------------ schedule
def schedule(flags: np.ndarray, budget: int) -> np.ndarray:
    """Slow/fast mode of every (sequence, step): 1 = SLOW, 0 = FAST.

    Slow steps fire near semantic boundaries or when the reuse budget is spent (es "Pasos
    Lentos", fr "2.A", zh "2.1 慢快推理框架").  Reading: step 0 is slow (nothing is selected
    yet); a step is slow when its boundary flag is set or when `budget` fast steps have run
    since the last slow step.
    """
    flags = np.asarray(flags)
    B, S = flags.shape
    mode = np.zeros((B, S), np.uint8)
    for b in range(B):
        run = 0
        for s in range(S):
            if s == 0 or flags[b, s] or run == budget:
                mode[b, s] = 1
                run = 0
            else:
                run += 1
    return mode


def boundary_flags(tokens: np.ndarray, boundary_tokens) -> np.ndarray:
    """flag = 1 where the decoded token is one of the semantic-boundary tokens (sentence
    punctuation, line or paragraph breaks: es "2. Metodología", zh "2.1 慢快推理框架")."""
    tokens = np.asarray(tokens)
    bset = set(int(t) for t in boundary_tokens)
    out = np.zeros(tokens.shape, np.uint8)
    for idx in np.ndindex(tokens.shape):
        out[idx] = 1 if int(tokens[idx]) in bset else 0
    return out


def step_control(tokens: np.ndarray, boundary_tokens, budget: int, n_stored: int,
                 n_sink: int, n_recent: int, sliding: bool = False) -> Dict[str, np.ndarray]:
    """The per-step state of a trajectory driven by decoded tokens, tokens [B, S].

    Before step 0 every row stores n_stored positions; step s decodes token [b, s], which
    joins the history, so N_s = n_stored + s + 1.  The mode is `schedule` of the tokens'
    boundary flags; a slow step freezes the recent segment's left edge (recent_start_at),
    or, with sliding, the edge follows every step (recent_start_sliding).
    Returns mode [S, B], seq_len [S, B], recent_start [S, B] (the edge in force at the
    step), slow / fast row lists [S, B] in ascending order padded with -1, and the counts
    [S, 2]."""
    mode = schedule(boundary_flags(tokens, boundary_tokens), budget).T
    S, B = mode.shape
    seq_len = np.zeros((S, B), np.int64)
    rstart = np.zeros((S, B), np.int64)
    slow_ids = np.full((S, B), -1, np.int64)
    fast_ids = np.full((S, B), -1, np.int64)
    counts = np.zeros((S, 2), np.int64)
    edge = np.zeros(B, np.int64)
    for s in range(S):
        for b in range(B):
            N = n_stored + s + 1
            seq_len[s, b] = N
            if sliding:
                edge[b] = recent_start_sliding(N, n_sink, n_recent)
            elif mode[s, b]:
                edge[b] = recent_start_at(N, n_sink, n_recent)
            rstart[s, b] = edge[b]
        sl = [b for b in range(B) if mode[s, b]]
        fa = [b for b in range(B) if not mode[s, b]]
        slow_ids[s, :len(sl)] = sl
        fast_ids[s, :len(fa)] = fa
        counts[s] = (len(sl), len(fa))
    return dict(mode=mode, seq_len=seq_len, recent_start=rstart, slow_ids=slow_ids,
                fast_ids=fast_ids, counts=counts)


# ------------------------------------------------------------------------------ Selector
def evidence(p: np.ndarray, num_kv_heads: int) -> np.ndarray:
    """Evidence distribution f per KV head.

    The Selector's evidence is the slow step's attention distribution (zh "2.2 训练无感的 Selector").  Reading: f of KV head g is the mean of the softmax probabilities of its G query
    heads, because selection and the compact buffer are per KV head; the mean keeps f a
    distribution.  p [Hq, N] -> f [Hkv, N].
    """
    p = np.asarray(p, F64)
    Hq, N = p.shape
    G = Hq // num_kv_heads
    return p.reshape(num_kv_heads, G, N).mean(axis=1)


def window_queries(q_steps: np.ndarray, s: int, window: int) -> np.ndarray:
    """The queries of the slow step's window at decode step s: slot k holds the query of
    step max(0, s - k), k < window.

    The pages call the Selector's evidence the attention observed in the slow step's window
    (es "2. Metodología", zh "2.2 训练无感的 Selector") without sizing the window.  Reading:
    the window is the current decode query and the window - 1 decode queries before it;
    before the first decode step there are none, so the first query fills the missing
    slots.  q_steps [S, Hq, D] -> [window, Hq, D]."""
    q_steps = np.asarray(q_steps, F64)
    return np.stack([q_steps[max(0, s - k)] for k in range(window)])


def window_evidence(P: np.ndarray, num_kv_heads: int) -> np.ndarray:
    """Evidence f per KV head pooled over a window of queries (es "Metodología / El
    Selector": the attention distribution observed in the slow step's window).  Reading:
    every query of the window and every query head of the group weighs the same, so f of
    KV head g is the mean over the window slots k and the G heads of g of the softmax
    probabilities; each of them attends to all N positions of the current history (no
    causal mask between the slots).  P [window, Hq, N] -> f [Hkv, N]."""
    P = np.asarray(P, F64)
    W, Hq, N = P.shape
    G = Hq // num_kv_heads
    f = np.zeros((num_kv_heads, N), F64)
    for g in range(num_kv_heads):
        f[g] = P[:, g * G:(g + 1) * G, :].sum(axis=(0, 1)) / (W * G)
    return f


def key_norms(K: np.ndarray) -> np.ndarray:
    """Cached key statistic: Euclidean norm of every stored key row.  K [Hkv, N, D]."""
    return np.linalg.norm(np.asarray(K, F64), axis=2)


def prior(norms: np.ndarray) -> np.ndarray:
    """Cache-aware structural prior r over positions [0, N) per KV head.

    The pages give the purpose of the two factors only (zh "2.2 训练无感的 Selector"): a key-norm
    factor that suppresses spuriously high logits of large-norm keys, and a position
    factor that discourages concentration on recent positions.  Reading:
      phi_key(g, j) = 1 / max(||k_{g,j}||, 1e-6)
      phi_pos(j)    = 1 + ln(1 + (N - 1 - j))       (grows with distance from the newest)
      r(g, j)       = phi_key * phi_pos / sum_{j'<N} phi_key * phi_pos
    norms [Hkv, N] -> r [Hkv, N].  The form is a reading; the implementation is pinned to it.
    """
    a = np.asarray(norms, F64)
    Hkv, N = a.shape
    phi_key = 1.0 / np.maximum(a, 1e-6)
    dist = (N - 1) - np.arange(N, dtype=F64)
    phi_pos = 1.0 + np.log1p(dist)
    w = phi_key * phi_pos[None, :]
    return w / w.sum(axis=1, keepdims=True)


def fuse(f: np.ndarray, r: np.ndarray, lam: float) -> np.ndarray:
    """Reverse-KL fusion in closed form, s = (1 - λ) f + λ r (nl "De Selector",
    zh "2.2 训练无感的 Selector").  The printed formula is the arithmetic mixture; it minimises
    (1-λ) KL(f||s) + λ KL(r||s) over the simplex."""
    return (1.0 - lam) * np.asarray(f, F64) + lam * np.asarray(r, F64)


def adaptive_lambda(f: np.ndarray, lambda_clip: float) -> np.ndarray:
    """Per-KV-head fusion weight of the clipped, adaptive reading of the prior fusion.

    The pages name the prior fusion's knob λclip in the Selector ablation (zh "4. 实验结果")
    and give no rule for it.  Reading: the weight of the prior follows how little the
    evidence says, measured by the normalised entropy of f, and is clipped at λclip:
      λ_g = min(λclip, H(f_g) / ln N),   H(f) = -sum_j f_j ln f_j  (0 ln 0 = 0),
    so a flat evidence (H = ln N) leans on the prior up to λclip and a point mass (H = 0)
    keeps the evidence alone.  With N = 1 there is nothing to weigh and λ_g = 0.
    f [Hkv, N] -> λ [Hkv]."""
    f = np.asarray(f, F64)
    Hkv, N = f.shape
    if N <= 1:
        return np.zeros(Hkv, F64)
    t = np.zeros_like(f)
    pos = f > 0
    t[pos] = f[pos] * np.log(f[pos])
    H = -t.sum(axis=1)
    return np.minimum(float(lambda_clip), H / math.log(N))


def fuse_per_head(f: np.ndarray, r: np.ndarray, lam: np.ndarray) -> np.ndarray:
    """The closed-form fusion with one weight per KV head: s_g = (1 - λ_g) f_g + λ_g r_g."""
    lam = np.asarray(lam, F64)[:, None]
    return (1.0 - lam) * np.asarray(f, F64) + lam * np.asarray(r, F64)


def candidates(N: int, n_sink: int, n_recent: int) -> Tuple[int, int]:
    """Candidate range C = [n_sink, N - W) of the selected memory (empty if N-W <= n_sink).
    Sink [0, n_sink) and the recent window are always in the fast memory
    (es "2. Metodología", zh "2.1 慢快推理框架"), so the Selector chooses among the rest."""
    lo = n_sink
    hi = max(lo, N - n_recent)
    return lo, hi


@dataclass
class Refined:
    ellp: np.ndarray        # refined log-scores over C, [Hkv, |C|]
    dom: np.ndarray         # soft-NMS decision, bool [Hkv, |C|]
    exc: np.ndarray         # cross-head exclusivity decision, bool [Hkv, |C|]
    dom_margin: np.ndarray  # relative gap of the deciding soft-NMS comparison
    own_margin: np.ndarray  # relative gap between the two best heads at each position


def refine(s: np.ndarray, lo: int, hi: int, R: int, alpha_soft: float,
           alpha_cross: float) -> Refined:
    """Log-score refinement before discretisation (zh "2.2 训练无感的 Selector", fr "2.B 2.").

    The pages name soft-NMS (penalise high-scoring neighbours in the same local region
    within a head) and cross-head exclusivity (discourage different heads from choosing
    the same position).  Reading, with ℓ = ln s on the candidates C = [lo, hi):
      dom(g, j) = some i in C with 0 < |i - j| <= R has ℓ(g, i) > ℓ(g, j)
      own(j)    = the smallest g that maximises ℓ(g, j);  exc(g, j) = g != own(j)
      ℓ'(g, j)  = ℓ + dom·ln(1 - α_soft) + exc·ln(1 - α_cross)
    Both decisions read the unrefined ℓ, so the order of the two refinements is
    immaterial.  ℓ' is evaluated as ln(s·(1-α_soft)^dom·(1-α_cross)^exc): the same real
    number, but two candidates whose penalised scores are equal stay exactly equal, so the
    lowest-position tie rule of topk sees them as ties.  ln 0 = -inf.
    """
    s = np.asarray(s, F64)
    Hkv = s.shape[0]
    sc = s[:, lo:hi]
    n = sc.shape[1]
    with np.errstate(divide="ignore"):
        ell = np.log(sc)
    dom = np.zeros((Hkv, n), bool)
    nbr_max = np.full((Hkv, n), -np.inf)
    for d in range(1, R + 1):
        if d >= n:
            break
        right = ell[:, d:]            # neighbour at j + d
        left = ell[:, :-d]            # neighbour at j - d
        nbr_max[:, :-d] = np.maximum(nbr_max[:, :-d], right)
        nbr_max[:, d:] = np.maximum(nbr_max[:, d:], left)
    dom = nbr_max > ell
    own = np.argmax(ell, axis=0) if n else np.zeros(0, int)   # first maximum = lowest g
    exc = np.arange(Hkv)[:, None] != own[None, :]
    if Hkv == 1:
        exc[:] = False
    w = np.where(dom, 1.0 - alpha_soft, 1.0) * np.where(exc, 1.0 - alpha_cross, 1.0)
    with np.errstate(divide="ignore"):
        ellp = np.log(sc * w)
    with np.errstate(invalid="ignore", divide="ignore"):
        dom_margin = np.abs(nbr_max - ell) / np.maximum(np.abs(ell), 1e-300)
        if Hkv > 1 and n:
            srt = np.sort(ell, axis=0)
            own_margin = np.abs(srt[-1] - srt[-2]) / np.maximum(np.abs(srt[-1]), 1e-300)
        else:
            own_margin = np.full(n, np.inf)
    return Refined(ellp, dom, exc, dom_margin, own_margin)


def refine_greedy(s: np.ndarray, lo: int, hi: int, R: int, alpha_soft: float,
                  alpha_cross: float) -> np.ndarray:
    """Classic greedy Soft-NMS as an alternative reading of the refinement's soft-NMS
    (zh "2.2 训练无感的 Selector": penalise high-scoring neighbours within a head).

    Exclusivity is that of `refine` (owner = the smallest g with the largest unrefined s;
    other heads' scores times 1 - α_cross).  Then, per head, the candidates are taken one
    at a time: the one with the largest current score (the lower position on ties) keeps
    that score for good, and every not yet taken candidate within ±R has its current score
    multiplied by 1 - α_soft.  A score is thus penalised once for every neighbour taken
    before it, where the one-pass reading penalises it once if any neighbour is larger to
    begin with.  Scores taken are non-increasing, so the first K taken are the Top-K.
    Returns the final scores [Hkv, |C|] (product form; take the log for `topk`)."""
    import heapq
    s = np.asarray(s, F64)
    Hkv = s.shape[0]
    sc = s[:, lo:hi]
    n = sc.shape[1]
    own = np.argmax(sc, axis=0) if n else np.zeros(0, int)
    exc = (np.arange(Hkv)[:, None] != own[None, :]) & (Hkv > 1)
    cur = sc * np.where(exc, 1.0 - alpha_cross, 1.0)
    final = np.zeros((Hkv, n), F64)
    for g in range(Hkv):
        val = cur[g].copy()
        taken = np.zeros(n, bool)
        heap = [(-val[c], c) for c in range(n)]
        heapq.heapify(heap)
        while heap:
            negv, c = heapq.heappop(heap)
            if taken[c] or -negv != val[c]:
                continue  # taken already, or an entry from before a penalty
            taken[c] = True
            final[g, c] = val[c]
            for d in range(max(0, c - R), min(n, c + R + 1)):
                if not taken[d]:
                    val[d] *= 1.0 - alpha_soft
                    heapq.heappush(heap, (-val[d], d))
    return final


def topk(ellp: np.ndarray, lo: int, K: int) -> np.ndarray:
    """Top-K discretisation (zh "2.2 训练无感的 Selector").

    Per KV head: the K_eff = min(K, |C|) candidates with the largest ℓ'; equal scores go
    to the lower position.  Output ascending positions, padded with -1 to K.
    ellp [Hkv, |C|] over positions lo + c -> sel int64 [Hkv, K].
    """
    ellp = np.asarray(ellp, F64)
    Hkv, n = ellp.shape
    keff = min(K, n)
    sel = np.full((Hkv, K), -1, np.int64)
    pos = np.arange(n)
    for g in range(Hkv):
        order = np.lexsort((pos, -ellp[g]))   # primary: ℓ' descending; then position
        chosen = np.sort(order[:keff]) + lo
        sel[g, :keff] = chosen
    return sel


@dataclass
class Selection:
    sel: np.ndarray          # [Hkv, K] ascending, -1 padded
    f: np.ndarray
    r: np.ndarray
    s: np.ndarray
    refined: Refined
    lo: int
    hi: int


def select(p: np.ndarray, norms: np.ndarray, N: int, num_kv_heads: int, n_sink: int,
           n_recent: int, top_k: int, R: int, alpha_soft: float, alpha_cross: float,
           lam: float, lambda_clip: Optional[float] = None) -> Selection:
    """The whole Selector of one slow step: evidence, prior, fusion, refinement, Top-K.
    p [Hq, N] slow-step softmax probabilities; norms [Hkv, N] cached key norms.  With
    lambda_clip (not None) the fusion weight is adaptive_lambda per KV head and lam is
    not used."""
    return select_from_evidence(evidence(p, num_kv_heads), norms, N, n_sink, n_recent, top_k,
                                R, alpha_soft, alpha_cross, lam, lambda_clip)


def select_window(P: np.ndarray, norms: np.ndarray, N: int, num_kv_heads: int, n_sink: int,
                  n_recent: int, top_k: int, R: int, alpha_soft: float, alpha_cross: float,
                  lam: float, lambda_clip: Optional[float] = None) -> Selection:
    """The Selector with evidence pooled over a window of queries, P [window, Hq, N]."""
    return select_from_evidence(window_evidence(P, num_kv_heads), norms, N, n_sink, n_recent,
                                top_k, R, alpha_soft, alpha_cross, lam, lambda_clip)


def select_from_evidence(f: np.ndarray, norms: np.ndarray, N: int, n_sink: int,
                         n_recent: int, top_k: int, R: int, alpha_soft: float,
                         alpha_cross: float, lam: float,
                         lambda_clip: Optional[float] = None) -> Selection:
    """Prior, fusion, refinement and Top-K on given evidence f [Hkv, N]."""
    r = prior(norms[:, :N])
    if lambda_clip is None:
        s = fuse(f, r, lam)
    else:
        s = fuse_per_head(f, r, adaptive_lambda(f, lambda_clip))
    lo, hi = candidates(N, n_sink, n_recent)
    ref = refine(s, lo, hi, R, alpha_soft, alpha_cross)
    sel = topk(ref.ellp, lo, top_k)
    return Selection(sel, f, r, s, ref, lo, hi)


def select_greedy_from_scores(s: np.ndarray, N: int, n_sink: int, n_recent: int, top_k: int,
                              R: int, alpha_soft: float, alpha_cross: float) -> np.ndarray:
    """Top-K after the greedy Soft-NMS reading (refine_greedy) of given fused scores."""
    lo, hi = candidates(N, n_sink, n_recent)
    final = refine_greedy(np.asarray(s, F64)[:, :N], lo, hi, R, alpha_soft, alpha_cross)
    with np.errstate(divide="ignore"):
        return topk(np.log(final), lo, top_k)


def select_from_scores(s: np.ndarray, N: int, n_sink: int, n_recent: int, top_k: int,
                       R: int, alpha_soft: float, alpha_cross: float) -> np.ndarray:
    """Refinement and Top-K applied to given fused scores s [Hkv, >=N]."""
    lo, hi = candidates(N, n_sink, n_recent)
    ref = refine(np.asarray(s, F64)[:, :N], lo, hi, R, alpha_soft, alpha_cross)
    return topk(ref.ellp, lo, top_k)


# ---------------------------------------------------------------------------------- pack
def packed_positions(sel_row: np.ndarray, n_sink: int) -> np.ndarray:
    """Positions of the compact buffer of one KV head: the sink tokens then the selected
    ones in ascending order (zh "2.3 系统级优化")."""
    sel_row = np.asarray(sel_row)
    return np.concatenate([np.arange(n_sink, dtype=np.int64), sel_row[sel_row >= 0]])


def pack(K: np.ndarray, V: np.ndarray, sel: np.ndarray, n_sink: int):
    """Gather sink + selected rows of every KV head into contiguous buffers.  The rows are
    the stored rows, unchanged.  Returns (list of positions, list of K rows, list of V
    rows), one entry per KV head."""
    pos, pk, pv = [], [], []
    for g in range(K.shape[0]):
        pp = packed_positions(sel[g], n_sink)
        pos.append(pp)
        pk.append(K[g][pp])
        pv.append(V[g][pp])
    return pos, pk, pv


# ---------------------------------------------------------------------------- fast step
def fast_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, packed_pos: List[np.ndarray],
                   recent_start: int, N: int):
    """Fast step: attention over the compact buffer (sink + selected) and the recent
    window [recent_start, N) read from the cache (zh "2.3 系统级优化"; nl "Memory-Coalesced
    Kernel").  Computed per segment and merged by log-sum-exp.  The compact buffer's
    positions all lie below recent_start.  Returns o [Hq, D], lse [Hq]."""
    Hq, D = q.shape
    Hkv = K.shape[0]
    G = Hq // Hkv
    o = np.empty((Hq, D), F64)
    lse = np.empty(Hq, F64)
    for g in range(Hkv):
        qg = q[g * G:(g + 1) * G]
        seg_a = attention(qg, K[g:g + 1, packed_pos[g]], V[g:g + 1, packed_pos[g]])
        rows_b = np.arange(recent_start, N)
        parts = [(seg_a[0], seg_a[2])]
        if len(rows_b):
            seg_b = attention(qg, K[g:g + 1, rows_b], V[g:g + 1, rows_b])
            parts.append((seg_b[0], seg_b[2]))
        og, lg = merge_segments(parts)
        o[g * G:(g + 1) * G] = og
        lse[g * G:(g + 1) * G] = lg
    return o, lse


def fast_attention_single_pass(q, K, V, packed_pos, recent_start, N):
    """The same fast step as one attention over the union of the two segments."""
    Hq, D = q.shape
    Hkv = K.shape[0]
    G = Hq // Hkv
    o = np.empty((Hq, D), F64)
    lse = np.empty(Hq, F64)
    for g in range(Hkv):
        J = np.concatenate([packed_pos[g], np.arange(recent_start, N)])
        og, _, lg, _ = attention(q[g * G:(g + 1) * G], K[g:g + 1, J], V[g:g + 1, J])
        o[g * G:(g + 1) * G] = og
        lse[g * G:(g + 1) * G] = lg
    return o, lse


def recent_start_at(N_slow: int, n_sink: int, n_recent: int) -> int:
    """Left edge of the recent segment after a slow step at KV length N_slow.

    Reading of "sliding window" for the fast steps after a slow step: the edge is frozen
    at max(n_sink, N_slow - W) and the window grows by one row per fast step, so every
    position is in exactly one of sink, candidates or recent until the next slow step."""
    return max(n_sink, N_slow - n_recent)


def recent_start_sliding(N: int, n_sink: int, n_recent: int) -> int:
    """Left edge of a purely sliding recent segment at KV length N: always the newest W
    positions (the literal reading of the sliding window, es "2. Metodología", nl
    "Methodologie").  After a slow step at N0 the positions [N0 - W, N - W) then belong to
    no segment of the fast memory until the next slow step."""
    return max(n_sink, N - n_recent)


# --------------------------------------------------------------------------- trajectory
@dataclass
class StepRecord:
    step: int
    mode: int                   # 1 slow, 0 fast
    N: int
    o: np.ndarray
    lse: np.ndarray
    selection: Optional[Selection] = None
    recent_start: int = 0


def run_sequence(q: np.ndarray, K: np.ndarray, V: np.ndarray, flags_row: np.ndarray,
                 context: int, n_sink: int, n_recent: int, top_k: int, R: int,
                 alpha_soft: float, alpha_cross: float, lam: float, budget: int,
                 steps: Optional[int] = None, sel_override: Optional[Dict[int, np.ndarray]] = None,
                 sliding: bool = False) -> List[StepRecord]:
    """Decode trajectory of one sequence in one layer.

    q [S, Hq, D]; K, V [Hkv, context + S, D] stored values; flags_row [S].
    At step s the KV length is N = context + s (the current token is already appended).
    sel_override maps a slow step to a selection to continue with (teacher forcing), so a
    comparison can follow another implementation's choice at near-ties.
    """
    S = q.shape[0] if steps is None else steps
    Hkv = K.shape[0]
    mode = schedule(np.asarray(flags_row)[None, :S], budget)[0]
    norms = key_norms(K)
    recs: List[StepRecord] = []
    packed = None
    rstart = n_sink
    for s in range(S):
        N = context + s
        if mode[s]:
            o, z, lse, p = attention(q[s], K[:, :N], V[:, :N])
            sel = select(p, norms[:, :N], N, Hkv, n_sink, n_recent, top_k, R, alpha_soft,
                         alpha_cross, lam)
            use = sel.sel if not sel_override or s not in sel_override else sel_override[s]
            packed = [packed_positions(use[g], n_sink) for g in range(Hkv)]
            rstart = recent_start_at(N, n_sink, n_recent)
            recs.append(StepRecord(s, 1, N, o, lse, sel, rstart))
        else:
            if sliding:
                rstart = recent_start_sliding(N, n_sink, n_recent)
            o, lse = fast_attention(q[s], K, V, packed, rstart, N)
            recs.append(StepRecord(s, 0, N, o, lse, None, rstart))
    return recs
