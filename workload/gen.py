"""Seeded synthetic inputs for the SFI decode path.

Everything here is input generation: random keys/values, boundary flags, span-drift
queries and the paged-cache packaging of K/V.  None of the method's arithmetic
(attention, Selector, pack) lives here, so the oracle and the device path can both take
their inputs from this module.

Recipe (one attention layer, one sequence b; per layer an independent stream):
  * key scale   a_j ~ LogNormal(0, sigma_k) per position, shared by the KV heads;
  * keys        K[g, j] = a_j * N(0, I_D), values V[g, j] = N(0, I_D), rounded to the
                storage dtype (bf16 round-to-nearest-even, or kept fp32);
  * flags       flag[b, s] ~ Bernoulli(p) per decode step, shared by all layers;
  * tokens      the id decoded at step s: one of five synthetic boundary ids (standing for
                '.', '?', '!', a line break and a paragraph break) where flag[b, s] is set,
                otherwise a uniform id from the rest of a 151936-entry vocabulary;
  * spans       a span starts at step 0 and at every flagged step.  At a span start s,
                each query head h draws n_topics positions uniformly without replacement
                from [n_sink, N_s - W) and its span base is the sum of the stored keys
                of its KV head at those positions;
  * queries     q[s, h] = base_h + query_noise * N(0, I_D), fp32.
  * paging      physical pages are a seeded random permutation, so paged reads scatter.

The attention support this produces is stable within a span and moves at flagged steps,
the behaviour the pages describe for sentences (nl "Kernobservatie", zh "1. 问题背景").

Random numbers come from torch's generators on the device where the tensors are made
(Philox on a GPU, Mersenne Twister on the CPU), so the same seed gives different values
on the two devices; tests always hand the very same tensors to both sides.
"""
from __future__ import annotations

import hashlib
from typing import Optional, Tuple

import torch

from .configs import Workload

ROOT_SEED = 1234
STREAM_KV, STREAM_FLAGS, STREAM_TOPICS, STREAM_NOISE, STREAM_PAGES, STREAM_TOKENS = range(6)

VOCAB = 151936
# Synthetic ids of the boundary tokens (a contiguous block, so other ids can skip it).
BOUNDARY_TOKENS = (1001, 1002, 1003, 1004, 1005)


def seed_for(w: Workload, stream: int, layer: int = 0) -> int:
    """Seed of one generator stream, derived from (root seed, workload, stream, layer)."""
    h = hashlib.sha256(f"{ROOT_SEED}/{w.name}/{stream}/{layer}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(w: Workload, stream: int, layer: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(w, stream, layer))
    return g


def storage_dtype(w: Workload) -> torch.dtype:
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def gen_layer_kv(w: Workload, layer: int, device="cpu") -> Tuple[torch.Tensor, torch.Tensor]:
    """Logical K, V of one layer: [B, Hkv, total_len, D] in the storage dtype."""
    g = _gen(w, STREAM_KV, layer, device)
    B, Hkv, N, D = w.batch, w.num_kv_heads, w.total_len, w.head_dim
    dt = storage_dtype(w)
    a = torch.exp(w.key_scale_sigma * torch.randn(B, 1, N, 1, generator=g, device=device))
    k = torch.randn(B, Hkv, N, D, generator=g, device=device)
    k.mul_(a)
    K = k.to(dt)
    del k
    v = torch.randn(B, Hkv, N, D, generator=g, device=device)
    V = v.to(dt)
    del v
    return K, V


def gen_flags(w: Workload, device="cpu") -> torch.Tensor:
    """Boundary flags [B, steps] uint8, shared by every layer."""
    g = _gen(w, STREAM_FLAGS, 0, device)
    u = torch.rand(w.batch, w.steps, generator=g, device=device)
    return (u < w.p_boundary).to(torch.uint8)


def gen_tokens(w: Workload, flags: torch.Tensor, device="cpu") -> torch.Tensor:
    """Token id decoded at every step, [steps, B] int32: a boundary id where the step's flag
    is set, any other id of the vocabulary otherwise."""
    g = _gen(w, STREAM_TOKENS, 0, "cpu")
    B, S = flags.shape
    nb = len(BOUNDARY_TOKENS)
    pick = torch.randint(0, nb, (S, B), generator=g)
    other = torch.randint(0, VOCAB - nb, (S, B), generator=g)
    other = other + (other >= BOUNDARY_TOKENS[0]).long() * nb
    bnd = torch.tensor(BOUNDARY_TOKENS)[pick]
    tok = torch.where(flags.cpu().t().bool(), bnd, other).to(torch.int32)
    return tok.to(device)


def span_starts(w: Workload, flags_row) -> list:
    """Steps at which a query span starts: step 0 and every flagged step."""
    fl = [int(x) for x in flags_row]
    return [s for s in range(w.steps) if s == 0 or fl[s]]


def gen_queries(w: Workload, layer: int, K: torch.Tensor, flags: torch.Tensor,
                device=None, topics: Optional[list] = None) -> torch.Tensor:
    """Span-drift queries of one layer: [steps, B, Hq, D] fp32.

    K is the layer's stored logical key tensor [B, Hkv, total_len, D].  When `topics` is
    a list, (b, s0, s1, positions [Hq, t]) is appended for every span: the topic positions
    whose keys make up the span's query base (the support a selection should recover).
    """
    device = K.device if device is None else device
    gt = _gen(w, STREAM_TOPICS, layer, device)
    gn = _gen(w, STREAM_NOISE, layer, device)
    B, Hq, D, G = w.batch, w.num_q_heads, w.head_dim, w.group
    S = w.steps
    q = torch.empty(S, B, Hq, D, dtype=torch.float32, device=device)
    flags_cpu = flags.cpu()
    kv_of_head = torch.arange(Hq, device=device) // G
    for b in range(B):
        starts = span_starts(w, flags_cpu[b])
        ends = starts[1:] + [S]
        for s0, s1 in zip(starts, ends):
            lo = w.n_sink
            hi = max(lo, w.seq_len(s0) - w.n_recent)
            n = hi - lo
            if n <= 0:
                base = torch.zeros(Hq, D, device=device)
            else:
                t = min(w.n_topics, n)
                u = torch.rand(Hq, n, generator=gt, device=device)
                pos = u.topk(t, dim=1).indices + lo                         # [Hq, t]
                rows = K[b][kv_of_head[:, None], pos].to(torch.float32)   # [Hq, t, D]
                base = rows.sum(dim=1)
                if topics is not None:
                    topics.append((b, s0, s1, pos.cpu()))
            noise = torch.randn(s1 - s0, Hq, D, generator=gn, device=device)
            q[s0:s1, b] = base[None] + w.query_noise * noise
    return q


def gen_block_table(w: Workload, layer: int, device="cpu") -> torch.Tensor:
    """Block table [B, pages_per_seq] int32: a seeded permutation of the physical pages."""
    g = _gen(w, STREAM_PAGES, layer, device)
    P = w.batch * w.pages_per_seq
    perm = torch.randperm(P, generator=g, device=device).to(torch.int32)
    return perm.view(w.batch, w.pages_per_seq).contiguous()


def paginate(w: Workload, X: torch.Tensor, block_table: torch.Tensor,
             num_pages: Optional[int] = None) -> torch.Tensor:
    """Place logical rows [B, Hkv, total_len, D] into a paged cache [pages, Hkv, 16, D].

    Logical position j of sequence b lives in physical page block_table[b, j // 16], slot
    j % 16.  Slots past total_len in the last page are zero.
    """
    B, Hkv, N, D = X.shape
    P16 = w.page_size
    npg = w.pages_per_seq
    num_pages = B * npg if num_pages is None else num_pages
    pad = npg * P16 - N
    if pad:
        X = torch.cat([X, X.new_zeros(B, Hkv, pad, D)], dim=2)
    tiles = X.view(B, Hkv, npg, P16, D).permute(0, 2, 1, 3, 4).reshape(B * npg, Hkv, P16, D)
    cache = X.new_zeros(num_pages, Hkv, P16, D)
    cache[block_table.reshape(-1).long()] = tiles
    return cache


def make_layer(w: Workload, layer: int, device="cpu", keep_logical: bool = True):
    """All inputs of one layer.  Returns a dict with K/V (logical, optional), the paged
    caches, the block table, the queries [steps, B, Hq, D] and the spans' topic positions
    (see gen_queries)."""
    K, V = gen_layer_kv(w, layer, device)
    flags = gen_flags(w, device)
    topics: list = []
    q = gen_queries(w, layer, K, flags, topics=topics)
    bt = gen_block_table(w, layer, device)
    kc = paginate(w, K, bt)
    vc = paginate(w, V, bt)
    out = dict(q=q, flags=flags, block_table=bt, k_cache=kc, v_cache=vc, topics=topics)
    if keep_logical:
        out["K"], out["V"] = K, V
    else:
        del K, V
    return out
