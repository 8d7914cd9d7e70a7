"""Operation-level wrappers (include/er_ops.h) on torch device tensors.

Marshalling only: each call enqueues the library's kernel on the current
torch stream.
"""
from __future__ import annotations

import ctypes as C

from . import _lib
from ._lib import check


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else None


def _stream():
    import torch
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _act(t):
    import torch
    return _lib.ER_BF16 if t.dtype == torch.bfloat16 else _lib.ER_F32


def quantize(quant: str, w, codes, scale, zero=None):
    lib = _lib.load()
    q = _lib.ER_W4_G128_ASYM if quant == "w4" else _lib.ER_W8_PERCH_SYM
    N, K = w.shape
    check(lib.er_op_quantize(q, _act(w), _ptr(w), N, K, _ptr(codes), _ptr(scale), _ptr(zero), _stream()),
          None, "er_op_quantize")


def w4_kernel_order(canon, N: int, K: int, out):
    check(_lib.load().er_op_w4_kernel_order(_ptr(canon), N, K, _ptr(out), _stream()), None, "er_op_w4_kernel_order")


def linear(x, fmt: int, w, N: int, K: int, y, scale=None, zero=None, path: int = 0):
    M = x.shape[0]
    check(_lib.load().er_op_linear(_act(x), _ptr(x), x.stride(0), M, fmt, _ptr(w), _ptr(scale), _ptr(zero), N, K,
                                   _ptr(y), y.stride(0), path, _stream()), None, "er_op_linear")


def linear_fused(epi: int, x, M: int, fmt: int, w, N: int, K: int, y=None, scale=None, zero=None, *,
                 xnorm: bool = False, xrow=None, ssq_in=None, gnorm=None, eps: float = 1e-6, ssq_acc=None,
                 ssq_zero=None, qkv: dict | None = None, path: int = 0):
    """er_op_linear_fused; `qkv` holds hq, hkv, hd, pos, slot, cos_sin, q_out, kv_pool, layer, n_layers."""
    qa = None
    if qkv is not None:
        qa = _lib.QkvArgs(qkv["hq"], qkv["hkv"], qkv["hd"], qkv["pos"].data_ptr(), qkv["slot"].data_ptr(),
                          qkv["cos_sin"].data_ptr(), qkv["q_out"].data_ptr(), qkv["kv_pool"].data_ptr(),
                          qkv["layer"], qkv["n_layers"])
    check(_lib.load().er_op_linear_fused(epi, _ptr(x), x.stride(0), M, int(xnorm), _ptr(xrow), _ptr(ssq_in),
                                         _ptr(gnorm), eps, fmt, _ptr(w), _ptr(scale), _ptr(zero), N, K, _ptr(y),
                                         y.stride(0) if y is not None else 0, _ptr(ssq_acc), _ptr(ssq_zero),
                                         C.byref(qa) if qa is not None else None, path, _stream()),
          None, "er_op_linear_fused")


def attention(q, out, kv_pool, n_layers, layer, hq, hkv, hd, block_table, bt_row, q_row0, q_pos0, q_count,
              max_q_count, max_ctx):
    check(_lib.load().er_op_attention(_act(q), _ptr(q), _ptr(out), _ptr(kv_pool), n_layers, layer, hq, hkv, hd,
                                      _ptr(block_table), block_table.shape[1], _ptr(bt_row), _ptr(q_row0),
                                      _ptr(q_pos0), _ptr(q_count), bt_row.shape[0], max_q_count, max_ctx,
                                      _stream()), None, "er_op_attention")


def attention_noalloc(q, out, kv_pool, n_layers, layer, hq, hkv, hd, block_table, bt_row, q_row0, q_pos0, q_count,
                      max_q_count, max_ctx):
    check(_lib.load().er_op_attention_noalloc(_act(q), _ptr(q), _ptr(out), _ptr(kv_pool), n_layers, layer, hq, hkv,
                                              hd, _ptr(block_table), block_table.shape[1], _ptr(bt_row),
                                              _ptr(q_row0), _ptr(q_pos0), _ptr(q_count), bt_row.shape[0],
                                              max_q_count, max_ctx, _stream()), None, "er_op_attention_noalloc")


def stats_bytes(V: int) -> int:
    return int(_lib.load().er_op_stats_bytes(V))


def row_stats(logits, temperature: float, top_p: float, stats):
    rows, V = logits.shape
    check(_lib.load().er_op_row_stats(_ptr(logits), rows, V, logits.stride(0), temperature, top_p, _ptr(stats),
                                      _stream()), None, "er_op_row_stats")


def sample_rows(logits, stats, temperature: float, seed: int, seq_id, pos, draft_idx: int, purpose: int, out,
                out_stride: int = 1, top_p: float = 1.0):
    rows, V = logits.shape
    check(_lib.load().er_op_sample_rows(_ptr(logits), _ptr(stats), rows, V, logits.stride(0), temperature, top_p,
                                        seed, _ptr(seq_id), _ptr(pos), draft_idx, purpose, _ptr(out), out_stride,
                                        _stream()), None, "er_op_sample_rows")


def spec_decide(p_logits, p_stats, q_logits, q_stats, tokens, B: int, gamma: int, temperature: float, seed: int,
                seq_id, pos0, out_tok, n_acc, top_p: float = 1.0):
    V = p_logits.shape[-1]
    check(_lib.load().er_op_spec_decide(_ptr(p_logits), _ptr(p_stats), _ptr(q_logits), _ptr(q_stats), _ptr(tokens),
                                        B, gamma, V, temperature, top_p, seed, _ptr(seq_id), _ptr(pos0),
                                        _ptr(out_tok), _ptr(n_acc), _stream()), None, "er_op_spec_decide")


def philox_uniform(seed: int, ctr, u):
    n = ctr.shape[0]
    check(_lib.load().er_op_philox_uniform(seed, _ptr(ctr), n, _ptr(u), _stream()), None, "er_op_philox_uniform")
