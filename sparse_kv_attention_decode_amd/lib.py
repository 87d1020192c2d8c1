"""ctypes binding of libsfi.so: the C ABI in include/sfi.h, one Python function per entry
point with the same name.  Argument marshalling only -- every step runs in the HIP
kernels.  Tensors are torch tensors on the GPU (torch provides device memory and
streams); pointers, sizes and the current stream are handed to the library as-is.

Loading fails loudly when libsfi.so has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsfi.so")

SFI_OK, SFI_E_ARG, SFI_E_UNSUPPORTED, SFI_E_ALIGN, SFI_E_WORKSPACE, SFI_E_CAPACITY, SFI_E_HIP = (
    0, -1, -2, -3, -4, -5, -6)
SFI_BF16, SFI_F32 = 0, 1
# device contract flags (enum sfi_device_status)
SFI_DEV_SEQ_LEN, SFI_DEV_PACKED_LEN, SFI_DEV_RECENT, SFI_DEV_PACK_SLOT = 1, 2, 4, 8

EXPORTS = ["sfi_abi_version", "sfi_status_str", "sfi_slow_attn_ws", "sfi_fast_attn_ws",
           "sfi_select_ws", "sfi_packed_cap", "sfi_key_norms", "sfi_slow_attn", "sfi_select",
           "sfi_pack", "sfi_fast_attn", "sfi_slow_attn_window_ws", "sfi_select_window_ws",
           "sfi_slow_attn_window", "sfi_select_window", "sfi_step_control", "sfi_kv_append",
           "sfi_decode_attn_ws", "sfi_decode_attn", "sfi_pack_update_ws", "sfi_pack_update",
           "sfi_fast_attn_noalloc"]


class SfiShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class SfiSelectParams(ctypes.Structure):
    _fields_ = [("n_sink", ctypes.c_int32), ("n_recent", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("nms_radius", ctypes.c_int32),
                ("lambda_", ctypes.c_float), ("alpha_soft", ctypes.c_float),
                ("alpha_cross", ctypes.c_float), ("lambda_clip", ctypes.c_float),
                ("nms_greedy", ctypes.c_int32)]


class SfiError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed with {code}: {msg}")
        self.code = code


_lib: Optional[ctypes.CDLL] = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_SHP = ctypes.POINTER(SfiShape)
_PRM = ctypes.POINTER(SfiSelectParams)

_SIGS = {
    "sfi_abi_version": (ctypes.c_int, []),
    "sfi_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "sfi_slow_attn_ws": (_SZ, [_SHP, _I32, _I32]),
    "sfi_fast_attn_ws": (_SZ, [_SHP, _I32, _I32, _I32]),
    "sfi_select_ws": (_SZ, [_SHP, _PRM, _I32, _I32]),
    "sfi_packed_cap": (_I32, [_PRM]),
    "sfi_key_norms": (ctypes.c_int, [_SHP, _P, _P, _P, _P, _I32, _I32, _I32, _P, _I64, _P]),
    "sfi_slow_attn": (ctypes.c_int, [_SHP, _P, _P, _P, _P, _P, _P, _I32, _I32, _P, _P, _I64, _P,
                                     _P, _P, _SZ, _P]),
    "sfi_select": (ctypes.c_int, [_SHP, _PRM, _P, _I64, _P, _P, _I64, _P, _P, _I32, _I32, _P, _P,
                                  _P, _SZ, _P]),
    "sfi_pack": (ctypes.c_int, [_SHP, _PRM, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _P, _I32, _P]),
    "sfi_slow_attn_window_ws": (_SZ, [_SHP, _I32, _I32, _I32]),
    "sfi_select_window_ws": (_SZ, [_SHP, _PRM, _I32, _I32, _I32]),
    "sfi_slow_attn_window": (ctypes.c_int, [_SHP, _I32, _P, _P, _P, _P, _P, _P, _I32, _I32, _P,
                                            _P, _I64, _P, _P, _P, _SZ, _P]),
    "sfi_select_window": (ctypes.c_int, [_SHP, _PRM, _I32, _P, _I64, _P, _P, _I64, _P, _P, _I32,
                                         _I32, _P, _P, _P, _SZ, _P]),
    "sfi_step_control": (ctypes.c_int, [_SHP, _PRM, _I32, _I32, _P, _P, _I32, _P, _P, _P, _P,
                                        _P, _P]),
    "sfi_kv_append": (ctypes.c_int, [_SHP, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _I64, _P]),
    "sfi_decode_attn_ws": (_SZ, [_SHP, _I32, _I32, _I32, _I32, _I32]),
    "sfi_decode_attn": (ctypes.c_int, [_SHP, _I32, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _P, _P,
                                       _P, _P, _I32, _I32, _I32, _P, _P, _I64, _P, _P, _P, _SZ,
                                       _P]),
    "sfi_pack_update_ws": (_SZ, [_SHP, _PRM, _I32]),
    "sfi_pack_update": (ctypes.c_int, [_SHP, _PRM, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _P, _I32,
                                       _P, _I64, _P, _P, _SZ, _P]),
    "sfi_fast_attn": (ctypes.c_int, [_SHP, _P, _P, _P, _P, _I32, _P, _P, _P, _P, _P, _P, _I32,
                                     _I32, _P, _P, _P, _P, _SZ, _P]),
    "sfi_fast_attn_noalloc": (ctypes.c_int, [_SHP, _P, _P, _P, _P, _I32, _P, _P, _P, _P, _P, _P,
                                             _I32, _I32, _P, _P, _P, _P]),
}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libsfi.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with sparse_kv_attention_decode_amd/build.py "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_str(code: int) -> str:
    return load().sfi_status_str(code).decode()


def _check(fn: str, rc: int):
    if rc != SFI_OK:
        raise SfiError(fn, rc, status_str(rc))


def make_shape(batch, num_q_heads, num_kv_heads, head_dim, max_pages_per_seq, dtype,
               page_size=16) -> SfiShape:
    dt = {"bf16": SFI_BF16, "f32": SFI_F32, torch.bfloat16: SFI_BF16, torch.float32: SFI_F32}
    return SfiShape(batch, num_q_heads, num_kv_heads, head_dim, page_size, max_pages_per_seq,
                    dt.get(dtype, dtype))


def make_params(n_sink, n_recent, top_k, nms_radius, lam, alpha_soft, alpha_cross,
                lambda_clip=-1.0, nms_greedy=False) -> SfiSelectParams:
    """lambda_clip < 0: fixed fusion weight lam; in [0, 1]: the clipped adaptive weight.
    nms_greedy: greedy soft-NMS instead of the one-pass reading."""
    return SfiSelectParams(n_sink, n_recent, top_k, nms_radius, lam, alpha_soft, alpha_cross,
                           lambda_clip, int(bool(nms_greedy)))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


# ----------------------------------------------------------------- workspace size queries
def sfi_slow_attn_ws(shape: SfiShape, n_seqs: int, max_seq_len: int) -> int:
    return load().sfi_slow_attn_ws(ctypes.byref(shape), n_seqs, max_seq_len)


def sfi_fast_attn_ws(shape: SfiShape, n_seqs: int, packed_cap: int, max_recent: int) -> int:
    return load().sfi_fast_attn_ws(ctypes.byref(shape), n_seqs, packed_cap, max_recent)


def sfi_select_ws(shape: SfiShape, params: SfiSelectParams, n_seqs: int, max_seq_len: int) -> int:
    return load().sfi_select_ws(ctypes.byref(shape), ctypes.byref(params), n_seqs, max_seq_len)


def sfi_slow_attn_window_ws(shape: SfiShape, window: int, n_seqs: int, max_seq_len: int) -> int:
    return load().sfi_slow_attn_window_ws(ctypes.byref(shape), window, n_seqs, max_seq_len)


def sfi_select_window_ws(shape: SfiShape, params: SfiSelectParams, window: int, n_seqs: int,
                         max_seq_len: int) -> int:
    return load().sfi_select_window_ws(ctypes.byref(shape), ctypes.byref(params), window, n_seqs,
                                       max_seq_len)


def sfi_packed_cap(params: SfiSelectParams) -> int:
    return load().sfi_packed_cap(ctypes.byref(params))


def sfi_abi_version() -> int:
    return load().sfi_abi_version()


def workspace(nbytes: int, device) -> torch.Tensor:
    """Device workspace of at least nbytes (256-byte aligned by the caching allocator)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------- entry points
def sfi_key_norms(shape, k_cache, block_table, seq_lens, seq_ids, n_seqs, pos_begin, pos_end,
                  key_norm, norm_stride, stream=None) -> None:
    rc = load().sfi_key_norms(ctypes.byref(shape), _ptr(k_cache), _ptr(block_table),
                              _ptr(seq_lens), _ptr(seq_ids), n_seqs, pos_begin, pos_end,
                              _ptr(key_norm), norm_stride, _stream(stream))
    _check("sfi_key_norms", rc)


def sfi_slow_attn(shape, q, k_cache, v_cache, block_table, seq_lens, seq_ids, n_seqs,
                  max_seq_len, out, logits, logits_stride, lse, ws, ws_bytes=None,
                  stream=None, status=None) -> None:
    ws_bytes = ws.numel() if ws_bytes is None else ws_bytes
    rc = load().sfi_slow_attn(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                              _ptr(block_table), _ptr(seq_lens), _ptr(seq_ids), n_seqs,
                              max_seq_len, _ptr(out), _ptr(logits), logits_stride, _ptr(lse),
                              _ptr(status), _ptr(ws), ws_bytes, _stream(stream))
    _check("sfi_slow_attn", rc)


def sfi_slow_attn_window(shape, window, q_win, k_cache, v_cache, block_table, seq_lens, seq_ids,
                         n_seqs, max_seq_len, out, logits, logits_stride, lse, ws, ws_bytes=None,
                         stream=None, status=None) -> None:
    ws_bytes = ws.numel() if ws_bytes is None else ws_bytes
    rc = load().sfi_slow_attn_window(ctypes.byref(shape), window, _ptr(q_win), _ptr(k_cache),
                                     _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
                                     _ptr(seq_ids), n_seqs, max_seq_len, _ptr(out), _ptr(logits),
                                     logits_stride, _ptr(lse), _ptr(status), _ptr(ws), ws_bytes,
                                     _stream(stream))
    _check("sfi_slow_attn_window", rc)


def sfi_select(shape, params, logits, logits_stride, lse, key_norm, norm_stride, seq_lens,
               seq_ids, n_seqs, max_seq_len, sel_idx, dbg_scores, ws, ws_bytes=None,
               stream=None) -> None:
    ws_bytes = ws.numel() if ws_bytes is None else ws_bytes
    rc = load().sfi_select(ctypes.byref(shape), ctypes.byref(params), _ptr(logits),
                           logits_stride, _ptr(lse), _ptr(key_norm), norm_stride,
                           _ptr(seq_lens), _ptr(seq_ids), n_seqs, max_seq_len, _ptr(sel_idx),
                           _ptr(dbg_scores), _ptr(ws), ws_bytes, _stream(stream))
    _check("sfi_select", rc)


def sfi_select_window(shape, params, window, logits, logits_stride, lse, key_norm, norm_stride,
                      seq_lens, seq_ids, n_seqs, max_seq_len, sel_idx, dbg_scores, ws,
                      ws_bytes=None, stream=None) -> None:
    ws_bytes = ws.numel() if ws_bytes is None else ws_bytes
    rc = load().sfi_select_window(ctypes.byref(shape), ctypes.byref(params), window,
                                  _ptr(logits), logits_stride, _ptr(lse), _ptr(key_norm),
                                  norm_stride, _ptr(seq_lens), _ptr(seq_ids), n_seqs,
                                  max_seq_len, _ptr(sel_idx), _ptr(dbg_scores), _ptr(ws),
                                  ws_bytes, _stream(stream))
    _check("sfi_select_window", rc)


def sfi_pack(shape, params, k_cache, v_cache, block_table, sel_idx, seq_ids, n_seqs, packed_k,
             packed_v, packed_pos, packed_len, packed_cap, stream=None) -> None:
    rc = load().sfi_pack(ctypes.byref(shape), ctypes.byref(params), _ptr(k_cache),
                         _ptr(v_cache), _ptr(block_table), _ptr(sel_idx), _ptr(seq_ids), n_seqs,
                         _ptr(packed_k), _ptr(packed_v), _ptr(packed_pos), _ptr(packed_len),
                         packed_cap, _stream(stream))
    _check("sfi_pack", rc)


def sfi_fast_attn(shape, q, packed_k, packed_v, packed_len, packed_cap, k_cache, v_cache,
                  block_table, recent_start, seq_lens, seq_ids, n_seqs, max_recent, out, lse,
                  ws, ws_bytes=None, stream=None, status=None) -> None:
    ws_bytes = ws.numel() if ws_bytes is None else ws_bytes
    rc = load().sfi_fast_attn(ctypes.byref(shape), _ptr(q), _ptr(packed_k), _ptr(packed_v),
                              _ptr(packed_len), packed_cap, _ptr(k_cache), _ptr(v_cache),
                              _ptr(block_table), _ptr(recent_start), _ptr(seq_lens),
                              _ptr(seq_ids), n_seqs, max_recent, _ptr(out), _ptr(lse),
                              _ptr(status), _ptr(ws), ws_bytes, _stream(stream))
    _check("sfi_fast_attn", rc)


def sfi_fast_attn_noalloc(shape, q, packed_k, packed_v, packed_len, packed_cap, k_cache,
                          v_cache, block_table, recent_start, seq_lens, seq_ids, n_seqs,
                          max_recent, out, lse, stream=None, status=None) -> None:
    rc = load().sfi_fast_attn_noalloc(ctypes.byref(shape), _ptr(q), _ptr(packed_k),
                                      _ptr(packed_v), _ptr(packed_len), packed_cap,
                                      _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                      _ptr(recent_start), _ptr(seq_lens), _ptr(seq_ids), n_seqs,
                                      max_recent, _ptr(out), _ptr(lse), _ptr(status),
                                      _stream(stream))
    _check("sfi_fast_attn_noalloc", rc)


def sfi_step_control(shape, params, refresh_budget, token_ids, boundary_tokens, n_boundary,
                     state_in, state_out, slow_ids, fast_ids, counts, sliding_recent=0,
                     stream=None) -> None:
    rc = load().sfi_step_control(ctypes.byref(shape), ctypes.byref(params), refresh_budget,
                                 int(sliding_recent), _ptr(token_ids), _ptr(boundary_tokens), n_boundary,
                                 _ptr(state_in), _ptr(state_out), _ptr(slow_ids),
                                 _ptr(fast_ids), _ptr(counts), _stream(stream))
    _check("sfi_step_control", rc)


def sfi_kv_append(shape, k_new, v_new, k_cache, v_cache, block_table, seq_lens, seq_ids, n_seqs,
                  key_norm, norm_stride, stream=None) -> None:
    rc = load().sfi_kv_append(ctypes.byref(shape), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                              _ptr(v_cache), _ptr(block_table), _ptr(seq_lens), _ptr(seq_ids),
                              n_seqs, _ptr(key_norm), norm_stride, _stream(stream))
    _check("sfi_kv_append", rc)


def sfi_decode_attn_ws(shape, window, n_seqs, packed_cap, max_recent, max_seq_len) -> int:
    return load().sfi_decode_attn_ws(ctypes.byref(shape), window, n_seqs, packed_cap, max_recent,
                                     max_seq_len)


def sfi_decode_attn(shape, window, q, q_win, packed_k, packed_v, packed_len, packed_cap, k_cache,
                    v_cache, block_table, recent_start, seq_lens, fast_ids, slow_ids, n_seqs,
                    max_recent, max_seq_len, out, logits, logits_stride, lse, ws, ws_bytes=None,
                    stream=None, status=None) -> None:
    ws_bytes = ws.numel() if ws_bytes is None else ws_bytes
    rc = load().sfi_decode_attn(ctypes.byref(shape), window, _ptr(q), _ptr(q_win),
                                _ptr(packed_k), _ptr(packed_v), _ptr(packed_len), packed_cap,
                                _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                _ptr(recent_start), _ptr(seq_lens), _ptr(fast_ids),
                                _ptr(slow_ids), n_seqs, max_recent, max_seq_len, _ptr(out),
                                _ptr(logits), logits_stride, _ptr(lse), _ptr(status), _ptr(ws),
                                ws_bytes, _stream(stream))
    _check("sfi_decode_attn", rc)


def sfi_pack_update_ws(shape, params, n_seqs) -> int:
    return load().sfi_pack_update_ws(ctypes.byref(shape), ctypes.byref(params), n_seqs)


def sfi_pack_update(shape, params, k_cache, v_cache, block_table, sel_idx, seq_ids, n_seqs,
                    packed_k, packed_v, packed_pos, packed_len, packed_cap, slot_map, map_stride,
                    ws, ws_bytes=None, stream=None, status=None) -> None:
    ws_bytes = ws.numel() if ws_bytes is None else ws_bytes
    rc = load().sfi_pack_update(ctypes.byref(shape), ctypes.byref(params), _ptr(k_cache),
                                _ptr(v_cache), _ptr(block_table), _ptr(sel_idx), _ptr(seq_ids),
                                n_seqs, _ptr(packed_k), _ptr(packed_v), _ptr(packed_pos),
                                _ptr(packed_len), packed_cap, _ptr(slot_map), map_stride,
                                _ptr(status), _ptr(ws), ws_bytes, _stream(stream))
    _check("sfi_pack_update", rc)
