"""Host-side checks of the C ABI: the library loads, exports every function include/sfi.h
declares, and rejects bad arguments with the documented codes before launching anything.
No GPU is needed: every call here fails validation (or is a pure host query)."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

from sparse_kv_attention_decode_amd import lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sfi.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(sfi_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    lib = L.load()
    declared = _declared_functions()
    assert len(declared) >= 11
    assert sorted(L.EXPORTS) == declared
    for name in declared:
        assert hasattr(lib, name), name
    assert L.sfi_abi_version() == 8


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert L.status_str(code) and L.status_str(code) != "unknown status"
    assert L.status_str(42) == "unknown status"


def _shape(**kw):
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, max_pages_per_seq=64,
                dtype="bf16")
    base.update(kw)
    return L.make_shape(**base)


def _params(**kw):
    base = dict(n_sink=4, n_recent=64, top_k=128, nms_radius=4, lam=0.3, alpha_soft=0.5,
                alpha_cross=0.5)
    base.update(kw)
    return L.make_params(**base)


FAKE = 1 << 20          # a 16-byte aligned non-null address; never dereferenced
MIS = (1 << 20) + 4     # misaligned


def _slow(shape, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, ids=FAKE, n=1, maxlen=100, out=FAKE,
             logits=FAKE, stride=128, lse=FAKE, ws=FAKE, wsb=1 << 40)
    a.update(over)
    return L.load().sfi_slow_attn(ctypes.byref(shape), a["q"], a["k"], a["v"], a["bt"], a["sl"],
                                  a["ids"], a["n"], a["maxlen"], a["out"], a["logits"],
                                  a["stride"], a["lse"], None, a["ws"], a["wsb"], None)


def test_slow_attn_validation():
    s = _shape()
    assert _slow(s, q=None) == L.SFI_E_ARG
    assert _slow(s, lse=None) == L.SFI_E_ARG
    assert _slow(_shape(num_q_heads=7)) == L.SFI_E_ARG
    assert _slow(_shape(num_kv_heads=0)) == L.SFI_E_ARG
    assert _slow(_shape(head_dim=96)) == L.SFI_E_UNSUPPORTED
    assert _slow(_shape(num_q_heads=64, num_kv_heads=2)) == L.SFI_E_UNSUPPORTED   # G = 32
    assert _slow(_shape(dtype=7)) == L.SFI_E_UNSUPPORTED
    s16 = _shape()
    s16.page_size = 32
    assert _slow(s16) == L.SFI_E_UNSUPPORTED
    assert _slow(s, n=3) == L.SFI_E_ARG                    # more rows than the batch
    assert _slow(s, n=-1) == L.SFI_E_ARG
    assert _slow(s, maxlen=0) == L.SFI_E_ARG
    assert _slow(s, maxlen=64 * 16 + 1) == L.SFI_E_CAPACITY
    assert _slow(s, q=MIS) == L.SFI_E_ALIGN
    assert _slow(s, k=MIS) == L.SFI_E_ALIGN
    assert _slow(s, logits=MIS) == L.SFI_E_ALIGN
    assert _slow(s, stride=130) == L.SFI_E_ALIGN
    assert _slow(s, stride=96) == L.SFI_E_CAPACITY         # stride < max_seq_len
    assert _slow(s, ws=None) == L.SFI_E_WORKSPACE
    need = L.sfi_slow_attn_ws(s, 1, 100)
    assert need > 0
    assert _slow(s, wsb=need - 1) == L.SFI_E_WORKSPACE
    assert _slow(s, ws=FAKE + 16) == L.SFI_E_WORKSPACE     # not 256-byte aligned
    assert _slow(s, n=0, wsb=need) == L.SFI_OK             # no rows: nothing to launch


def test_workspace_queries_reject_bad_arguments():
    s, p = _shape(), _params()
    assert L.sfi_slow_attn_ws(_shape(head_dim=80), 1, 10) == 0
    assert L.sfi_slow_attn_ws(s, 1, 64 * 16 + 1) == 0
    assert L.sfi_select_ws(s, _params(top_k=0), 1, 10) == 0
    assert L.sfi_fast_attn_ws(s, 1, 17, 10) == 0
    assert L.sfi_fast_attn_ws(s, 1, 144, 10) > 0
    assert L.sfi_packed_cap(p) == 144
    assert L.sfi_packed_cap(_params(n_sink=0, top_k=16)) == 16
    assert L.sfi_packed_cap(_params(alpha_soft=1.5)) == 0


def _select(shape, params, **over):
    a = dict(logits=FAKE, lstride=128, lse=FAKE, norm=FAKE, nstride=128, sl=FAKE, ids=FAKE, n=1,
             maxlen=100, sel=FAKE, dbg=None, ws=FAKE, wsb=1 << 40)
    a.update(over)
    return L.load().sfi_select(ctypes.byref(shape), ctypes.byref(params), a["logits"],
                               a["lstride"], a["lse"], a["norm"], a["nstride"], a["sl"], a["ids"],
                               a["n"], a["maxlen"], a["sel"], a["dbg"], a["ws"], a["wsb"], None)


def test_select_validation():
    s, p = _shape(), _params()
    assert _select(s, p, logits=None) == L.SFI_E_ARG
    assert _select(s, _params(top_k=0)) == L.SFI_E_ARG
    assert _select(s, _params(nms_radius=-1)) == L.SFI_E_ARG
    assert _select(s, _params(lam=1.5)) == L.SFI_E_ARG
    assert _select(s, _params(lambda_clip=1.5)) == L.SFI_E_ARG
    assert _select(s, _params(lambda_clip=float("nan"))) == L.SFI_E_ARG
    assert _select(s, _params(lambda_clip=-1.0, lam=1.5)) == L.SFI_E_ARG
    bad = _params()
    bad.nms_greedy = 2
    assert _select(s, bad) == L.SFI_E_ARG
    # the greedy soft-NMS needs two more arrays per candidate in the workspace
    assert L.sfi_select_ws(s, _params(nms_greedy=True), 2, 1000) > \
        L.sfi_select_ws(s, _params(), 2, 1000)
    assert _select(s, _params(lam=float("nan"))) == L.SFI_E_ARG
    assert _select(s, _params(alpha_soft=-0.1)) == L.SFI_E_ARG
    assert _select(s, _params(alpha_cross=2.0)) == L.SFI_E_ARG
    assert _select(s, _params(n_sink=-1)) == L.SFI_E_ARG
    assert _select(s, p, lstride=64) == L.SFI_E_CAPACITY
    assert _select(s, p, nstride=130) == L.SFI_E_ALIGN
    assert _select(s, _params(nms_radius=5000)) == L.SFI_E_UNSUPPORTED
    assert _select(s, p, wsb=10) == L.SFI_E_WORKSPACE
    assert _select(s, p, n=0) == L.SFI_OK
    # the top-K takes at most 1024 slices of 4096 candidates
    big = _shape(max_pages_per_seq=(1 << 22) // 16 + 8)
    stride = (1 << 22) + 64
    assert L.sfi_select_ws(big, p, 1, 1 << 22) > 0
    assert L.sfi_select_ws(big, p, 1, (1 << 22) + 1) == 0
    assert _select(big, p, maxlen=(1 << 22) + 1, lstride=stride, nstride=stride) == \
        L.SFI_E_UNSUPPORTED


def test_window_calls_validate_and_size_like_the_widened_shape():
    """A window of w slots is the model's shape with Hq * w query heads (G * w <= 16)."""
    s, p = _shape(), _params()              # Hq 8, Hkv 2: G = 4
    lib = L.load()
    for n, maxlen in ((1, 100), (2, 1000)):
        assert L.sfi_slow_attn_window_ws(s, 1, n, maxlen) == L.sfi_slow_attn_ws(s, n, maxlen)
        assert L.sfi_select_window_ws(s, p, 1, n, maxlen) == L.sfi_select_ws(s, p, n, maxlen)
        wide = _shape(num_q_heads=32)
        assert L.sfi_slow_attn_window_ws(s, 4, n, maxlen) == L.sfi_slow_attn_ws(wide, n, maxlen)
        assert L.sfi_select_window_ws(s, p, 4, n, maxlen) == L.sfi_select_ws(wide, p, n, maxlen)
    assert L.sfi_slow_attn_window_ws(s, 0, 1, 100) == 0
    assert L.sfi_slow_attn_window_ws(s, 5, 1, 100) == 0      # G * w = 20 > 16
    assert L.sfi_select_window_ws(s, p, 5, 1, 100) == 0

    def slow_w(win, **over):
        a = dict(q=FAKE, n=1, ws=FAKE, wsb=1 << 40)
        a.update(over)
        return lib.sfi_slow_attn_window(ctypes.byref(s), win, a["q"], FAKE, FAKE, FAKE, FAKE,
                                        FAKE, a["n"], 100, FAKE, FAKE, 128, FAKE, None,
                                        a["ws"], a["wsb"], None)

    def select_w(win):
        return lib.sfi_select_window(ctypes.byref(s), ctypes.byref(p), win, FAKE, 128, FAKE, FAKE,
                                     128, FAKE, FAKE, 1, 100, FAKE, None, FAKE, 1 << 40, None)

    assert slow_w(0) == L.SFI_E_ARG
    assert slow_w(-3) == L.SFI_E_ARG
    assert slow_w(5) == L.SFI_E_UNSUPPORTED
    assert slow_w(2, q=None) == L.SFI_E_ARG
    assert slow_w(2, q=MIS) == L.SFI_E_ALIGN
    assert slow_w(2, ws=None) == L.SFI_E_WORKSPACE
    assert slow_w(2, wsb=L.sfi_slow_attn_window_ws(s, 2, 1, 100) - 1) == L.SFI_E_WORKSPACE
    assert slow_w(4, n=0) == L.SFI_OK                         # no rows: nothing to launch
    assert select_w(0) == L.SFI_E_ARG
    assert select_w(5) == L.SFI_E_UNSUPPORTED


def _pack(shape, params, **over):
    a = dict(k=FAKE, v=FAKE, bt=FAKE, sel=FAKE, ids=FAKE, n=1, pk=FAKE, pv=FAKE, pp=FAKE,
             pl=FAKE, cap=L.sfi_packed_cap(params))
    a.update(over)
    return L.load().sfi_pack(ctypes.byref(shape), ctypes.byref(params), a["k"], a["v"], a["bt"],
                             a["sel"], a["ids"], a["n"], a["pk"], a["pv"], a["pp"], a["pl"],
                             a["cap"], None)


def test_pack_validation():
    s, p = _shape(), _params()
    assert _pack(s, p, sel=None) == L.SFI_E_ARG
    assert _pack(s, p, cap=128) == L.SFI_E_CAPACITY
    assert _pack(s, p, pk=MIS) == L.SFI_E_ALIGN
    assert _pack(s, p, n=5) == L.SFI_E_ARG
    assert _pack(s, p, n=0) == L.SFI_OK


def _fast(shape, **over):
    a = dict(q=FAKE, pk=FAKE, pv=FAKE, pl=FAKE, cap=144, k=FAKE, v=FAKE, bt=FAKE, rs=FAKE,
             sl=FAKE, ids=FAKE, n=1, maxrec=100, out=FAKE, lse=None, ws=FAKE, wsb=1 << 40)
    a.update(over)
    return L.load().sfi_fast_attn(ctypes.byref(shape), a["q"], a["pk"], a["pv"], a["pl"],
                                  a["cap"], a["k"], a["v"], a["bt"], a["rs"], a["sl"], a["ids"],
                                  a["n"], a["maxrec"], a["out"], a["lse"], None, a["ws"],
                                  a["wsb"], None)


def test_fast_attn_validation():
    s = _shape()
    assert _fast(s, rs=None) == L.SFI_E_ARG
    assert _fast(s, cap=100) == L.SFI_E_CAPACITY
    assert _fast(s, cap=0) == L.SFI_E_CAPACITY
    assert _fast(s, maxrec=-1) == L.SFI_E_ARG
    assert _fast(s, maxrec=64 * 16 + 1) == L.SFI_E_CAPACITY
    assert _fast(s, pv=MIS) == L.SFI_E_ALIGN
    assert _fast(s, wsb=0) == L.SFI_E_WORKSPACE
    assert _fast(s, n=0) == L.SFI_OK


def _fast_noalloc(shape, **over):
    a = dict(q=FAKE, pk=FAKE, pv=FAKE, pl=FAKE, cap=144, k=FAKE, v=FAKE, bt=FAKE, rs=FAKE,
             sl=FAKE, ids=FAKE, n=1, maxrec=100, out=FAKE, lse=None)
    a.update(over)
    return L.load().sfi_fast_attn_noalloc(
        ctypes.byref(shape), a["q"], a["pk"], a["pv"], a["pl"], a["cap"], a["k"], a["v"],
        a["bt"], a["rs"], a["sl"], a["ids"], a["n"], a["maxrec"], a["out"], a["lse"], None,
        None)


def test_fast_attn_noalloc_validation():
    """The allocation-free fast call rejects what sfi_fast_attn rejects, and calls whose split
    partials exceed its fixed scratch array, before touching the device."""
    s = _shape()
    assert _fast_noalloc(s, rs=None) == L.SFI_E_ARG
    assert _fast_noalloc(s, cap=100) == L.SFI_E_CAPACITY
    assert _fast_noalloc(s, maxrec=-1) == L.SFI_E_ARG
    assert _fast_noalloc(s, pv=MIS) == L.SFI_E_ALIGN
    assert _fast_noalloc(s, n=3) == L.SFI_E_ARG            # more rows than the batch
    assert _fast_noalloc(s, n=0) == L.SFI_OK
    # 64 rows of 16 KV heads with G = 16: the partials outgrow the 8 MiB array
    big = _shape(batch=64, num_q_heads=256, num_kv_heads=16, max_pages_per_seq=8192)
    need = L.sfi_fast_attn_ws(big, 64, 65536, 4096)
    assert need > 8 << 20
    assert _fast_noalloc(big, n=64, cap=65536, maxrec=4096) == L.SFI_E_WORKSPACE


def test_key_norms_validation():
    s = _shape()
    lib = L.load()

    def call(**over):
        a = dict(k=FAKE, bt=FAKE, sl=FAKE, ids=FAKE, n=1, pb=0, pe=100, out=FAKE, stride=128)
        a.update(over)
        return lib.sfi_key_norms(ctypes.byref(s), a["k"], a["bt"], a["sl"], a["ids"], a["n"],
                                 a["pb"], a["pe"], a["out"], a["stride"], None)

    assert call(out=None) == L.SFI_E_ARG
    assert call(pb=10, pe=5) == L.SFI_E_ARG
    assert call(pe=64 * 16 + 1, stride=2048) == L.SFI_E_CAPACITY
    assert call(stride=64) == L.SFI_E_CAPACITY
    assert call(k=MIS) == L.SFI_E_ALIGN
    assert call(pb=7, pe=7) == L.SFI_OK


def test_binding_fails_loudly_without_library(tmp_path):
    import importlib
    mod = importlib.reload(L)
    try:
        mod._lib = None
        with pytest.raises(RuntimeError, match="missing"):
            mod.load(str(tmp_path / "nope.so"))
    finally:
        importlib.reload(L)


def test_topic_recall_counts_candidate_topics_only():
    """The recall measurement: topics of the G query heads of a KV head, restricted to the
    candidate range, found in that head's selection."""
    import numpy as np
    from sparse_kv_attention_decode_amd.recall import topic_recall
    sel = np.array([[5, 9, 12, -1], [3, 4, -1, -1]])
    topics = np.array([[5, 9, 2], [12, 30, 9],   # KV head 0 (query heads 0, 1)
                       [3, 7, 50], [4, 7, 8]])   # KV head 1 (query heads 2, 3)
    r = topic_recall(sel, topics, G=2, lo=4, hi=40)
    # head 0: candidates {5, 9, 12, 30} (2 is below lo), selected {5, 9, 12} -> 3/4
    # head 1: candidates {4, 7, 8} (3 below lo, 50 above hi), selected {4} -> 1/3
    assert np.allclose(r, [0.75, 1 / 3])
    assert np.isnan(topic_recall(sel[:1], np.array([[1, 2]]), G=1, lo=4, hi=40)[0])


def test_synthetic_tokens_follow_the_boundary_flags():
    """Boundary ids exactly at the flagged steps; other ids avoid the boundary block."""
    from oracle import sfi_oracle as O
    from workload import get
    from workload.gen import BOUNDARY_TOKENS, VOCAB, gen_flags, gen_tokens
    w = get("qwen3_4b_32k_b4")
    flags = gen_flags(w)
    tok = gen_tokens(w, flags)
    assert tok.shape == (w.steps, w.batch) and tok.dtype == torch.int32
    assert int(tok.min()) >= 0 and int(tok.max()) < VOCAB
    np.testing.assert_array_equal(O.boundary_flags(tok.numpy().T, BOUNDARY_TOKENS),
                                  flags.numpy())


def test_step_control_and_append_validation():
    s, p = _shape(), _params()
    lib = L.load()

    def ctrl(budget=4, tok=FAKE, bnd=FAKE, nb=5, sl=FAKE, outs=FAKE, shape=s, params=p,
             slide=0):
        return lib.sfi_step_control(ctypes.byref(shape), ctypes.byref(params), budget, slide,
                                    tok, bnd, nb, sl, FAKE, outs, FAKE, FAKE, None)

    assert ctrl(budget=-1) == L.SFI_E_ARG
    assert ctrl(slide=2) == L.SFI_E_ARG
    assert ctrl(nb=-1) == L.SFI_E_ARG
    assert ctrl(nb=1025) == L.SFI_E_UNSUPPORTED
    assert ctrl(tok=None) == L.SFI_E_ARG
    assert ctrl(bnd=None) == L.SFI_E_ARG          # a table is needed when nb > 0
    assert ctrl(sl=None) == L.SFI_E_ARG
    assert ctrl(outs=None) == L.SFI_E_ARG
    assert ctrl(shape=_shape(num_kv_heads=0)) == L.SFI_E_ARG
    assert ctrl(params=_params(top_k=0)) == L.SFI_E_ARG

    def app(kn=FAKE, kc=FAKE, n=1, norm=FAKE, stride=128, shape=s):
        return lib.sfi_kv_append(ctypes.byref(shape), kn, FAKE, kc, FAKE, FAKE, FAKE, FAKE, n,
                                 norm, stride, None)

    assert app(kn=None) == L.SFI_E_ARG
    assert app(kn=MIS) == L.SFI_E_ALIGN
    assert app(kc=MIS) == L.SFI_E_ALIGN
    assert app(n=3) == L.SFI_E_ARG                 # more rows than the batch
    assert app(norm=FAKE, stride=0) == L.SFI_E_ARG
    assert app(shape=_shape(head_dim=96)) == L.SFI_E_UNSUPPORTED
    assert app(n=0) == L.SFI_OK                    # nothing to launch


def test_coverage_helpers():
    """memory_mask marks sink, packed rows and the recent segment; coverage_of sums the
    softmax mass over them (uniform logits: |M| / N per head)."""
    from sparse_kv_attention_decode_amd.coverage import coverage_of, memory_mask
    N, n_sink = 20, 2
    pos = torch.tensor([[0, 1, 5, 9, -1], [0, 1, 7, -1, -1]], dtype=torch.int32)
    plen = torch.tensor([4, 3], dtype=torch.int32)
    m = memory_mask(N, n_sink, pos, plen, 16)
    want0 = {0, 1, 5, 9, 16, 17, 18, 19}
    want1 = {0, 1, 7, 16, 17, 18, 19}
    assert set(torch.nonzero(m[0]).flatten().tolist()) == want0
    assert set(torch.nonzero(m[1]).flatten().tolist()) == want1
    z = torch.zeros(4, N, dtype=torch.float64)     # G = 2
    lse = torch.full((4,), float(np.log(N)), dtype=torch.float64)
    c = coverage_of(z, lse, m)
    np.testing.assert_allclose(c.numpy(), [8 / N, 8 / N, 7 / N, 7 / N], rtol=1e-12)
