"""Seeded synthetic inputs for the batch-1 decode workloads.

This module is shared by the CPU oracle's tests and by the GPU library's tests and
benchmark.  It produces data only (weights, prompts, KV contents, FP8 block
quantisation of the weights) and contains none of the decode arithmetic.  The
generator is counter based (SplitMix64 finaliser + Box-Muller in double), defined in
``synthgen.c``; every element depends only on (seed, tensor id, index).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional

import numpy as np

from .workloads import WORKLOADS, Workload  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synthgen.c")
_LIB = os.path.join(_HERE, "libsynthgen.so")
_lib = None

FMT_F16, FMT_BF16, FMT_F32 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile libsynthgen.so with gcc (OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        u64, i64, i32, u32, dbl, vp = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32,
                                       ctypes.c_double, ctypes.c_void_p)
        lib.sg_normal_fill.argtypes = [u64, u64, u64, dbl, dbl, i32, vp]
        lib.sg_uniform_int.argtypes = [u64, u64, u64, u32, vp]
        lib.sg_quant_e4m3_block.argtypes = [vp, i64, i64, vp, vp]
        lib.sg_quant_e4m3_scaled.argtypes = [vp, i64, ctypes.c_float, vp]
        lib.sg_quant_int_group.argtypes = [vp, i64, i64, i32, vp, vp]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def normal(seed: int, tensor: int, shape, std: float, fmt: int, mean: float = 0.0) -> np.ndarray:
    """N(mean, std) rounded (nearest even) into fmt; returns uint16 bits for 16-bit formats."""
    n = int(np.prod(shape))
    out = np.empty(shape, dtype=np.float32 if fmt == FMT_F32 else np.uint16)
    _load().sg_normal_fill(seed, tensor, n, mean, std, fmt, _ptr(out))
    return out


def uniform_int(seed: int, tensor: int, count: int, n: int) -> np.ndarray:
    out = np.empty(count, dtype=np.int32)
    _load().sg_uniform_int(seed, tensor, count, n, _ptr(out))
    return out


def quant_e4m3_block(w_bf16: np.ndarray):
    """128x128 block quantisation of a bf16 matrix into OCP E4M3FN codes + fp32 scales."""
    rows, cols = w_bf16.shape
    q = np.empty((rows, cols), dtype=np.uint8)
    s = np.empty(((rows + 127) // 128, (cols + 127) // 128), dtype=np.float32)
    _load().sg_quant_e4m3_block(_ptr(np.ascontiguousarray(w_bf16)), rows, cols, _ptr(q), _ptr(s))
    return q, s


def quant_int_group(w_bf16: np.ndarray, bits: int):
    """Symmetric per-row, per-128-column-group integer quantisation of a bf16 matrix.

    Returns (codes, scales): int8 codes as int8 [rows][cols], or int4 codes two per byte (even
    column in the low nibble) as uint8 [rows][cols // 2]; scales are bf16 bits
    [rows][ceil(cols / 128)] with s = bf16(max|w| / qmax) and q = clamp(rne(w / s), +-qmax),
    qmax = 127 or 7.
    """
    assert bits in (4, 8)
    rows, cols = w_bf16.shape
    assert bits == 8 or cols % 2 == 0
    q = np.empty((rows, cols if bits == 8 else cols // 2), dtype=np.int8 if bits == 8 else np.uint8)
    s = np.empty((rows, (cols + 127) // 128), dtype=np.uint16)
    _load().sg_quant_int_group(_ptr(np.ascontiguousarray(w_bf16)), rows, cols, bits, _ptr(q), _ptr(s))
    return q, s


def quant_e4m3_scaled(v: np.ndarray, scale: float) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    q = np.empty(v.shape, dtype=np.uint8)
    _load().sg_quant_e4m3_scaled(_ptr(v), v.size, float(scale), _ptr(q))
    return q


# ----------------------------------------------------------------------------------------------
# Model weights in the canonical layout: every linear weight is [out][in], row-major.
# ----------------------------------------------------------------------------------------------
LAYER_KINDS = ["wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down", "attn_norm", "ffn_norm"]
LINEAR_KINDS = ["wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"]


def _tensor_id(layer: int, kind: str) -> int:
    if layer < 0:
        return 1_000_000 + ["embed", "final_norm", "lm_head"].index(kind)
    return layer * 16 + LAYER_KINDS.index(kind)


def linear_shapes(w: "Workload") -> Dict[str, tuple]:
    qd, kvd = w.n_q * w.head_dim, w.n_kv * w.head_dim
    return {"wq": (qd, w.hidden), "wk": (kvd, w.hidden), "wv": (kvd, w.hidden), "wo": (w.hidden, qd),
            "w_gate": (w.ffn, w.hidden), "w_up": (w.ffn, w.hidden), "w_down": (w.hidden, w.ffn)}


@dataclass
class ModelWeights:
    """Host arrays of one synthetic model.  16-bit tensors hold raw bits (uint16)."""
    workload: Workload
    embed: np.ndarray
    final_norm: np.ndarray
    lm_head: np.ndarray
    layers: List[Dict[str, np.ndarray]]
    lm_head_scale: Optional[np.ndarray] = None  # fp8 / int8 / int4 only
    scales: List[Dict[str, np.ndarray]] = field(default_factory=list)  # fp8 / int8 / int4 only, per layer


def make_weights(w: "Workload", seed: Optional[int] = None, std: float = 0.02, gain_std: float = 0.0,
                 zero: tuple = ()) -> ModelWeights:
    """Generate the synthetic model of workload w.

    Linear and embedding weights ~ N(0, std) in the 16-bit storage format (bf16 for the
    fp8, int8 and int4 workloads, whose linear weights are then quantised: fp8 per 128x128
    block, int8 / int4 per row and 128-column group).  Norm gains are 1 (gain_std > 0 gives 1 + N(0, gain_std)).
    `zero` names linear kinds to set to zero (closed-form test variants).
    """
    seed = w.seed if seed is None else seed
    fmt = FMT_F16 if w.wdtype == "f16" else FMT_BF16
    gfmt = fmt
    H, V = w.hidden, w.vocab
    shapes = linear_shapes(w)

    def gain(layer, kind):
        if gain_std > 0:
            return normal(seed, _tensor_id(layer, kind), (H,), gain_std, gfmt, mean=1.0)
        one = np.float32(1.0)
        bits = np.frombuffer(np.float16(1.0).tobytes(), np.uint16)[0] if gfmt == FMT_F16 else \
            np.uint16(one.view(np.uint32) >> 16)
        return np.full((H,), bits, dtype=np.uint16)

    embed = normal(seed, _tensor_id(-1, "embed"), (V, H), std, fmt)
    lm = normal(seed, _tensor_id(-1, "lm_head"), (V, H), std, fmt)
    layers = []
    for l in range(w.layers):
        d = {}
        for k in LINEAR_KINDS:
            if k in zero:
                d[k] = np.zeros(shapes[k], dtype=np.uint16)
            else:
                d[k] = normal(seed, _tensor_id(l, k), shapes[k], std, fmt)
        d["attn_norm"] = gain(l, "attn_norm")
        d["ffn_norm"] = gain(l, "ffn_norm")
        layers.append(d)
    mw = ModelWeights(workload=w, embed=embed, final_norm=gain(-1, "final_norm"), lm_head=lm, layers=layers)
    if w.wdtype == "fp8":
        for d in layers:
            sc = {}
            for k in LINEAR_KINDS:
                q, s = quant_e4m3_block(d[k])
                d[k] = q
                sc[k] = s
            mw.scales.append(sc)
        mw.lm_head, mw.lm_head_scale = quant_e4m3_block(lm)
    elif w.wdtype in ("int8", "int4"):
        bits = 8 if w.wdtype == "int8" else 4
        for d in layers:
            sc = {}
            for k in LINEAR_KINDS:
                d[k], sc[k] = quant_int_group(d[k], bits)
            mw.scales.append(sc)
        mw.lm_head, mw.lm_head_scale = quant_int_group(lm, bits)
    return mw


def make_prompt(w: "Workload", length: Optional[int] = None, seed: Optional[int] = None) -> np.ndarray:
    seed = w.seed if seed is None else seed
    return uniform_int(seed, 2_000_000, w.prompt if length is None else length, w.vocab)


def make_kv(w: "Workload", positions: int, seed: Optional[int] = None, std: float = 1.0):
    """Synthetic KV cache contents [L][n_kv][positions][head_dim] in the KV storage format.

    Returns (k, v, kv_scales) where kv_scales is [L][n_kv][2] fp32 for the fp8 KV format
    (else None).  Values ~ N(0, std) (the spread of k and v in these synthetic models).
    """
    seed = w.seed if seed is None else seed
    shape = (w.layers, w.n_kv, positions, w.head_dim)
    if w.kvdtype in ("f16", "bf16"):
        fmt = FMT_F16 if w.kvdtype == "f16" else FMT_BF16
        return normal(seed, 3_000_000, shape, std, fmt), normal(seed, 3_000_001, shape, std, fmt), None
    kf = normal(seed, 3_000_000, shape, std, FMT_F32)
    vf = normal(seed, 3_000_001, shape, std, FMT_F32)
    scales = np.empty((w.layers, w.n_kv, 2), dtype=np.float32)
    kq = np.empty(shape, dtype=np.uint8)
    vq = np.empty(shape, dtype=np.uint8)
    for l in range(w.layers):
        for g in range(w.n_kv):
            for j, (src, dst) in enumerate(((kf, kq), (vf, vq))):
                # a fixed-headroom static scale: 4 sigma maps to 448
                s = np.float32(4.0 * std / 448.0)
                scales[l, g, j] = s
                dst[l, g] = quant_e4m3_scaled(src[l, g], float(s))
    return kq, vq, scales
