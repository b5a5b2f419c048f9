"""CPU oracle for batch-1 greedy decode (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this
package.  It is a plain, slow C++ implementation (``pmk_oracle.cpp``) of the decode step
with fp32 activations and fp32 accumulation in ascending index order, and it shares no
code with the GPU library.  Every function is pinned by ``tests/test_oracle_pins.py``.

Parity unpinned: none of its functions is without a pin; the whole-model GPU comparison
itself has no external reference value (the pages print no worked example).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pmk_oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

F16, BF16, E4M3, I8, I4 = 0, 1, 2, 3, 4
FMT = {"f16": F16, "bf16": BF16, "fp8": E4M3, "int8": I8, "int4": I4}


def build(force: bool = True) -> str:
    """Compile liboracle.so with g++ (OpenMP; no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["g++", "-std=c++17", "-O3", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


class _Config(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int), ("H", ctypes.c_int), ("nq", ctypes.c_int), ("nkv", ctypes.c_int),
                ("hd", ctypes.c_int), ("F", ctypes.c_int), ("V", ctypes.c_int), ("eps", ctypes.c_float),
                ("theta", ctypes.c_double), ("wfmt", ctypes.c_int), ("efmt", ctypes.c_int),
                ("kvfmt", ctypes.c_int), ("max_seq", ctypes.c_int)]


class _Weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("final_norm", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("lm_head_scale", ctypes.c_void_p), ("layer", ctypes.POINTER(ctypes.c_void_p)),
                ("layer_scale", ctypes.POINTER(ctypes.c_void_p))]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        vp, i32, i64, f32, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_double
        L.orc_decode.argtypes = [i32, vp, i64, vp]
        L.orc_encode.argtypes = [i32, vp, i64, vp]
        L.orc_rmsnorm.argtypes = [vp, vp, i32, f32, vp]
        L.orc_gemv.argtypes = [i32, vp, vp, i32, i32, vp, vp]
        L.orc_matmul_tokens.argtypes = [i32, vp, vp, i32, i32, vp, i32, vp]
        L.orc_weight_matrix.argtypes = [i32, vp, vp, i32, i32, vp]
        L.orc_rope.argtypes = [vp, i32, i32, f64]
        L.orc_attend.argtypes = [vp, vp, vp, i32, f32, f32, i32, i32, vp]
        L.orc_silu.argtypes = [f32]
        L.orc_silu.restype = f32
        L.orc_argmax.argtypes = [vp, i32]
        L.orc_create.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(_Weights)]
        L.orc_create.restype = vp
        L.orc_destroy.argtypes = [vp]
        L.orc_get_pos.argtypes = [vp]
        L.orc_set_kv_scales.argtypes = [vp, vp]
        L.orc_load_kv.argtypes = [vp, vp, vp, i32]
        L.orc_read_kv.argtypes = [vp, vp, vp, i32]
        L.orc_prefill.argtypes = [vp, vp, i32, i32, vp]
        L.orc_step.argtypes = [vp, i32, vp]
        L.orc_step_forced.argtypes = [vp, i32, vp, vp, vp, vp, vp]
        L.orc_num_threads.argtypes = []
        L.orc_set_threads.argtypes = [i32]
        L.orc_kv_amax.argtypes = [vp, vp]
        L.orc_reset_kv_amax.argtypes = [vp]
        L.orc_kv_scales_from_amax.argtypes = [vp, vp]
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be contiguous"
    return a.ctypes.data


# ---------------------------------------------------------------------------------------------
# single operations (numpy in, numpy out)
# ---------------------------------------------------------------------------------------------
def decode(fmt: int, raw: np.ndarray) -> np.ndarray:
    raw = np.ascontiguousarray(raw)
    out = np.empty(raw.shape, np.float32)
    lib().orc_decode(fmt, _p(raw), raw.size, _p(out))
    return out


def encode(fmt: int, x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint8 if fmt == E4M3 else np.uint16)
    lib().orc_encode(fmt, _p(x), x.size, _p(out))
    return out


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    g = np.ascontiguousarray(g, np.float32)
    y = np.empty_like(x)
    lib().orc_rmsnorm(_p(x), _p(g), x.size, eps, _p(y))
    return y


def _scales(fmt: int, scales: Optional[np.ndarray]):
    """fp8 block scales as fp32; int8 / int4 group scales stay bf16 bits (uint16)."""
    if scales is None:
        return None
    if fmt in (I8, I4):
        assert scales.dtype == np.uint16, "integer formats take bf16 scale bits"
        return np.ascontiguousarray(scales)
    return np.ascontiguousarray(scales, np.float32)


def _cols(fmt: int, W: np.ndarray) -> int:
    return W.shape[1] * 2 if fmt == I4 else W.shape[1]


def gemv(fmt: int, W: np.ndarray, x: np.ndarray, scales: Optional[np.ndarray] = None) -> np.ndarray:
    """y = W x (fp32, k ascending).  int4 W is [rows][cols / 2] packed bytes; the integer formats
    round x to binary16 first."""
    W = np.ascontiguousarray(W)
    x = np.ascontiguousarray(x, np.float32)
    rows, cols = W.shape[0], _cols(fmt, W)
    assert x.size == cols
    y = np.empty(rows, np.float32)
    S = _scales(fmt, scales)
    lib().orc_gemv(fmt, _p(W), _p(S), rows, cols, _p(x), _p(y))
    return y


def weight_matrix(fmt: int, W: np.ndarray, scales: Optional[np.ndarray] = None) -> np.ndarray:
    """The dequantised weights w(n, k) as fp32 [rows][cols]."""
    W = np.ascontiguousarray(W)
    rows, cols = W.shape[0], _cols(fmt, W)
    out = np.empty((rows, cols), np.float32)
    S = _scales(fmt, scales)
    lib().orc_weight_matrix(fmt, _p(W), _p(S), rows, cols, _p(out))
    return out


def rope(u: np.ndarray, pos: int, theta: float) -> np.ndarray:
    u = np.array(u, dtype=np.float32, copy=True)
    lib().orc_rope(_p(u), u.size, pos, theta)
    return u


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, fmt: int, ks: float = 1.0, vs: float = 1.0) -> np.ndarray:
    q = np.ascontiguousarray(q, np.float32)
    K = np.ascontiguousarray(K)
    V = np.ascontiguousarray(V)
    T, hd = K.shape
    out = np.empty(hd, np.float32)
    lib().orc_attend(_p(q), _p(K), _p(V), fmt, ks, vs, T, hd, _p(out))
    return out


def silu(z: float) -> float:
    return lib().orc_silu(z)


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops from now on."""
    lib().orc_set_threads(int(n))


def argmax(v: np.ndarray) -> int:
    v = np.ascontiguousarray(v, np.float32)
    return lib().orc_argmax(_p(v), v.size)


# ---------------------------------------------------------------------------------------------
# whole model
# ---------------------------------------------------------------------------------------------
class OracleModel:
    """The decoder over host weight arrays (canonical [out][in] layout, storage formats).

    `weights` is any object with attributes embed, final_norm, lm_head, lm_head_scale,
    layers (list of dicts with wq wk wv wo w_gate w_up w_down attn_norm ffn_norm) and scales
    (list of dicts of fp8 block scales or int8 / int4 group scales), and `workload` with the
    model shape.  The arrays are
    referenced, not copied: keep them alive while the model lives.
    """

    KINDS = ["wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down", "attn_norm", "ffn_norm"]
    LIN = ["wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"]

    def __init__(self, weights, max_seq: Optional[int] = None):
        w = weights.workload
        self.w = w
        self._keep = weights
        wfmt = FMT[w.wdtype]
        efmt = BF16 if w.wdtype in ("fp8", "int8", "int4") else wfmt
        self.cfg = _Config(w.layers, w.hidden, w.n_q, w.n_kv, w.head_dim, w.ffn, w.vocab, w.eps, w.theta,
                           wfmt, efmt, FMT[w.kvdtype], max_seq if max_seq is not None else w.max_seq)
        ptrs = []
        for d in weights.layers:
            ptrs += [_p(d[k]) for k in self.KINDS]
        self._layer = (ctypes.c_void_p * len(ptrs))(*ptrs)
        sc = None
        if w.wdtype in ("fp8", "int8", "int4"):
            sptrs = []
            for d in weights.scales:
                sptrs += [_p(d[k]) for k in self.LIN]
            self._scale = (ctypes.c_void_p * len(sptrs))(*sptrs)
            sc = ctypes.cast(self._scale, ctypes.POINTER(ctypes.c_void_p))
        self.wts = _Weights(_p(weights.embed), _p(weights.final_norm), _p(weights.lm_head),
                            _p(weights.lm_head_scale) if weights.lm_head_scale is not None else None,
                            ctypes.cast(self._layer, ctypes.POINTER(ctypes.c_void_p)), sc)
        self.h = lib().orc_create(ctypes.byref(self.cfg), ctypes.byref(self.wts))
        if not self.h:
            raise ValueError("oracle rejected the model shape")

    def __del__(self):
        if getattr(self, "h", None):
            lib().orc_destroy(self.h)
            self.h = None

    @property
    def pos(self) -> int:
        return lib().orc_get_pos(self.h)

    def set_kv_scales(self, s: np.ndarray):
        s = np.ascontiguousarray(s, np.float32)
        assert s.shape == (self.w.layers, self.w.n_kv, 2)
        lib().orc_set_kv_scales(self.h, _p(s))

    def kv_amax(self) -> np.ndarray:
        """Largest |k| (after RoPE) and |v| per (layer, kv head) appended since the last reset,
        before rounding to the cache format: [layers][n_kv][2]."""
        out = np.empty((self.w.layers, self.w.n_kv, 2), np.float32)
        lib().orc_kv_amax(self.h, _p(out))
        return out

    def reset_kv_amax(self):
        lib().orc_reset_kv_amax(self.h)

    def kv_scales_from_amax(self) -> np.ndarray:
        """Static FP8 KV scales from kv_amax(): amax / 448 in fp32, 1 where amax is 0."""
        out = np.empty((self.w.layers, self.w.n_kv, 2), np.float32)
        lib().orc_kv_scales_from_amax(self.h, _p(out))
        return out

    def load_kv(self, k: np.ndarray, v: np.ndarray, P: int):
        k = np.ascontiguousarray(k)
        v = np.ascontiguousarray(v)
        if lib().orc_load_kv(self.h, _p(k), _p(v), P) != 0:
            raise ValueError("bad KV length")

    def read_kv(self, P: int):
        w = self.w
        dt = np.uint8 if w.kvdtype == "fp8" else np.uint16
        k = np.empty((w.layers, w.n_kv, P, w.head_dim), dt)
        v = np.empty_like(k)
        lib().orc_read_kv(self.h, _p(k), _p(v), P)
        return k, v

    def prefill(self, tokens: np.ndarray, block: int = 64, want_logits: bool = True):
        t = np.ascontiguousarray(tokens, np.int32)
        lg = np.empty(self.w.vocab, np.float32) if want_logits else None
        tok = lib().orc_prefill(self.h, _p(t), t.size, block, _p(lg))
        if tok < 0:
            raise RuntimeError(f"oracle prefill failed ({tok})")
        return tok, lg

    def step_forced(self, tok: int, k_row: np.ndarray, v_row: np.ndarray):
        """One step that appends the given KV row (cache-format codes [layers][n_kv][head_dim]) instead
        of its own rounding of k and v, as a teacher-forced step takes a given token.  Returns
        (next token, logits, own k row, own v row): the codes this step itself would have appended."""
        w = self.w
        k_row = np.ascontiguousarray(k_row)
        v_row = np.ascontiguousarray(v_row)
        assert k_row.shape == (w.layers, w.n_kv, w.head_dim) and v_row.shape == k_row.shape
        own_k, own_v = np.empty_like(k_row), np.empty_like(v_row)
        lg = np.empty(w.vocab, np.float32)
        nxt = lib().orc_step_forced(self.h, int(tok), _p(k_row), _p(v_row), _p(own_k), _p(own_v), _p(lg))
        if nxt == -2:
            raise RuntimeError("oracle KV capacity exceeded")
        if nxt < 0:
            raise RuntimeError("oracle logits contain NaN")
        return nxt, lg, own_k, own_v

    def step(self, tok: int, want_logits: bool = True):
        lg = np.empty(self.w.vocab, np.float32) if want_logits else None
        nxt = lib().orc_step(self.h, int(tok), _p(lg))
        if nxt == -2:
            raise RuntimeError("oracle KV capacity exceeded")
        if nxt < 0:
            raise RuntimeError("oracle logits contain NaN")
        return nxt, lg
