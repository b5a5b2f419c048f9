"""Brute-force fp64 reference of the decoder for tiny shapes (test helper).

It recomputes the whole sequence from scratch at every step (no KV cache, no blocking),
with numpy/torch library routines for the storage formats, so that it shares neither
code nor evaluation order with the oracle.  The KV cache format is part of the model's
semantics, so keys and values are rounded into it (here from fp64) before attention.
"""
from __future__ import annotations

import numpy as np
import torch


def dec16(raw: np.ndarray, fmt: str) -> np.ndarray:
    raw = np.ascontiguousarray(raw)
    if fmt == "f16":
        return raw.view(np.float16).astype(np.float64)
    return (raw.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dec_e4m3(raw: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(raw)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def round_to(x: np.ndarray, fmt: str, scale: float = 1.0) -> np.ndarray:
    t = torch.from_numpy(np.asarray(x, dtype=np.float64))
    if fmt == "f16":
        return t.to(torch.float16).to(torch.float64).numpy()
    if fmt == "bf16":
        return t.to(torch.bfloat16).to(torch.float64).numpy()
    q = torch.clamp(t / scale, -448.0, 448.0).to(torch.float8_e4m3fn)
    return q.to(torch.float64).numpy() * scale


def int_codes(raw: np.ndarray, fmt: str) -> np.ndarray:
    """Two's-complement integer codes as fp64: int8 bytes, or int4 nibbles (even column low)."""
    raw = np.ascontiguousarray(raw)
    if fmt == "int8":
        return raw.view(np.int8).astype(np.float64)
    b = raw.view(np.uint8).astype(np.int64)
    q = np.stack([b & 15, b >> 4], axis=-1).reshape(raw.shape[0], -1)
    return np.where(q >= 8, q - 16, q).astype(np.float64)


def _dequant(raw, S, fmt):
    if fmt in ("int8", "int4"):
        q = int_codes(raw, fmt)
        return q * np.repeat(dec16(S, "bf16"), 128, 1)[:, : q.shape[1]]
    q = dec_e4m3(raw)
    S = S.astype(np.float64)
    return q * np.repeat(np.repeat(S, 128, 0), 128, 1)[: q.shape[0], : q.shape[1]]


def linear(weights, layer: int, kind: str) -> np.ndarray:
    w = weights.workload
    raw = weights.layers[layer][kind]
    if w.wdtype in ("f16", "bf16"):
        return dec16(raw, w.wdtype)
    return _dequant(raw, weights.scales[layer][kind], w.wdtype)


def lm_head(weights) -> np.ndarray:
    w = weights.workload
    if w.wdtype in ("f16", "bf16"):
        return dec16(weights.lm_head, w.wdtype)
    return _dequant(weights.lm_head, weights.lm_head_scale, w.wdtype)


def act(weights, X: np.ndarray) -> np.ndarray:
    """The activation operand of a linear layer: binary16 for the integer weight formats (A16)."""
    if weights.workload.wdtype in ("int8", "int4"):
        return np.asarray(X, np.float64).astype(np.float16).astype(np.float64)
    return X


def _rms(X, g, eps):
    return X / np.sqrt((X * X).mean(axis=-1, keepdims=True) + eps) * g


def _rope_rows(M, positions, hd, theta):
    """M: [T][heads*hd]; rotate-half per head with angle p * theta^(-2i/hd)."""
    T = M.shape[0]
    Mh = M.reshape(T, -1, hd).copy()
    i = np.arange(hd // 2)
    ang = np.asarray(positions, np.float64)[:, None] * theta ** (-2.0 * i / hd)[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = Mh[..., : hd // 2].copy(), Mh[..., hd // 2:].copy()
    Mh[..., : hd // 2] = a * c - b * s
    Mh[..., hd // 2:] = b * c + a * s
    return Mh.reshape(T, -1)


def logits_all(weights, tokens, kv_scales=None, cached_kv=None, attn_override=None, collect_kv=None,
               forced_last=None):
    """Logits at the LAST position of `tokens`, recomputing everything.

    cached_kv: optional (k, v) fp64 arrays [L][nkv][P0][hd] of already-dequantised cache
    contents for positions 0..P0-1 that precede `tokens` (then `tokens` sit at P0..).
    collect_kv: optional list; receives per layer the (k, v) fp64 values [T][nkv][hd] of `tokens`
    (k after RoPE) before they are rounded into the cache format.
    forced_last: optional (k, v) fp64 arrays [L][nkv][hd]: the already-dequantised cache row of the
    LAST token, used in place of its own rounded k and v.
    """
    w = weights.workload
    efmt = "bf16" if w.wdtype in ("fp8", "int8", "int4") else w.wdtype
    H, hd, nq, nkv = w.hidden, w.head_dim, w.n_q, w.n_kv
    grp = nq // nkv
    P0 = 0 if cached_kv is None else cached_kv[0].shape[2]
    toks = np.asarray(tokens)
    T = len(toks)
    pos = np.arange(P0, P0 + T)
    X = dec16(weights.embed, efmt)[toks]
    for l in range(w.layers):
        g1 = dec16(weights.layers[l]["attn_norm"], efmt)
        g2 = dec16(weights.layers[l]["ffn_norm"], efmt)
        Xn = _rms(X, g1, w.eps)
        Xa = act(weights, Xn)
        Q = _rope_rows(Xa @ linear(weights, l, "wq").T, pos, hd, w.theta)
        K = _rope_rows(Xa @ linear(weights, l, "wk").T, pos, hd, w.theta)
        Vv = Xa @ linear(weights, l, "wv").T
        K = K.reshape(T, nkv, hd)
        Vv = Vv.reshape(T, nkv, hd)
        if collect_kv is not None:
            collect_kv.append((K.copy(), Vv.copy()))
        Kr = np.empty_like(K)
        Vr = np.empty_like(Vv)
        for g in range(nkv):
            ks = 1.0 if kv_scales is None else float(kv_scales[l, g, 0])
            vs = 1.0 if kv_scales is None else float(kv_scales[l, g, 1])
            Kr[:, g] = round_to(K[:, g], w.kvdtype, ks)
            Vr[:, g] = round_to(Vv[:, g], w.kvdtype, vs)
            if forced_last is not None:
                Kr[-1, g] = forced_last[0][l, g]
                Vr[-1, g] = forced_last[1][l, g]
        if cached_kv is not None:
            Kr = np.concatenate([np.transpose(cached_kv[0][l], (1, 0, 2)), Kr], axis=0)
            Vr = np.concatenate([np.transpose(cached_kv[1][l], (1, 0, 2)), Vr], axis=0)
        O = np.zeros((T, nq * hd))
        for j in range(nq):
            g = j // grp
            s = Q[:, j * hd:(j + 1) * hd] @ Kr[:, g].T / np.sqrt(hd)  # [T][P0+T]
            mask = np.arange(P0 + T)[None, :] > pos[:, None]
            s = np.where(mask, -np.inf, s)
            if attn_override == "uniform":
                s = np.where(mask, -np.inf, 0.0)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p = p / p.sum(axis=1, keepdims=True)
            O[:, j * hd:(j + 1) * hd] = p @ Vr[:, g]
        X = X + act(weights, O) @ linear(weights, l, "wo").T
        Xn = act(weights, _rms(X, g2, w.eps))
        G = Xn @ linear(weights, l, "w_gate").T
        U = Xn @ linear(weights, l, "w_up").T
        Hh = G / (1.0 + np.exp(-G)) * U
        X = X + act(weights, Hh) @ linear(weights, l, "w_down").T
    xf = _rms(X[-1], dec16(weights.final_norm, efmt), w.eps)
    return lm_head(weights) @ act(weights, xf)
