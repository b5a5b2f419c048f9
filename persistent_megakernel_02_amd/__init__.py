"""Persistent batch-1 decode megakernel for MI355X (gfx950): Python binding of libpmk.so.

The binding only marshals arguments: PyTorch supplies device memory and the stream, and
every step of the decode path (weight repacking, prefill, decode, argmax) runs in the
library's HIP kernels.  The C names of include/pmk.h are available unchanged from
``persistent_megakernel_02_amd._lib``; ``Decoder`` wraps one context.
"""
from __future__ import annotations

import ctypes
from typing import Optional

from . import _lib
from ._lib import (PMK_DT_BF16, PMK_DT_F16, PMK_DT_FP8_E4M3, PMK_DT_INT4, PMK_DT_INT8,  # noqa: F401
                   PMK_MODE_GRAPH, PMK_MODE_MEGAKERNEL,
                   PMK_MODE_PER_OP, PMK_SYNC_COUNTERS, PMK_SYNC_FLAGS, PmkError, check, load, pmk_device_error,
                   pmk_model_config, pmk_schedule_config, pmk_schedule_info, pmk_sizes, pmk_task, pmk_tune_result,
                   pmk_weight_ptrs)

_DT = {"f16": PMK_DT_F16, "bf16": PMK_DT_BF16, "fp8": PMK_DT_FP8_E4M3, "int8": PMK_DT_INT8, "int4": PMK_DT_INT4}


def model_config(w, max_seq: Optional[int] = None) -> pmk_model_config:
    """pmk_model_config from any object with the workload attributes (layers, hidden, n_q, n_kv,
    head_dim, ffn, vocab, eps, theta, wdtype, kvdtype, max_seq)."""
    return pmk_model_config(w.layers, w.hidden, w.n_q, w.n_kv, w.head_dim, w.ffn, w.vocab,
                            max_seq if max_seq is not None else w.max_seq, w.eps, w.theta, _DT[w.wdtype],
                            _DT[w.kvdtype], 0, 0)


def schedule_config(n_cus: int = 0, sync_mode: int = PMK_SYNC_FLAGS, attn_splits: int = 0, prefetch: int = 0,
                    trace_steps: int = 0, spin_limit: int = 0, combine_parts: int = 0,
                    combine_o_share: int = 0, prefill_chunk: int = 0,
                    prefill_ksplit: int = 0, combine_o_copy: int = 0) -> pmk_schedule_config:
    return pmk_schedule_config(n_cus, sync_mode, attn_splits, prefetch, trace_steps, spin_limit, combine_parts,
                               combine_o_share, prefill_chunk, prefill_ksplit, combine_o_copy)


def _stream(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _aligned_empty(nbytes: int, device):
    import torch
    t = torch.empty(int(nbytes) + 256, dtype=torch.uint8, device=device)
    off = (-t.data_ptr()) % 256
    return t, t[off:off + int(nbytes)]


class DeviceWeights:
    """Canonical weight tensors on the device and the pmk_weight_ptrs that names them."""

    KINDS = ["wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down", "attn_norm", "ffn_norm"]
    LIN = ["wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"]

    def __init__(self, host, device="cuda:0"):
        import torch

        def up(a):
            return torch.from_numpy(a).to(device)

        self.embed = up(host.embed)
        self.final_norm = up(host.final_norm)
        self.lm_head = up(host.lm_head)
        self.lm_head_scale = up(host.lm_head_scale) if host.lm_head_scale is not None else None
        self.layers = [{k: up(d[k]) for k in self.KINDS} for d in host.layers]
        self.scales = [{k: up(d[k]) for k in self.LIN} for d in host.scales] if host.scales else []
        ptrs = [d[k].data_ptr() for d in self.layers for k in self.KINDS]
        self._layer_arr = (ctypes.c_void_p * len(ptrs))(*ptrs)
        sc = None
        if self.scales:
            sptrs = [d[k].data_ptr() for d in self.scales for k in self.LIN]
            self._scale_arr = (ctypes.c_void_p * len(sptrs))(*sptrs)
            sc = ctypes.cast(self._scale_arr, ctypes.POINTER(ctypes.c_void_p))
        self.ptrs = pmk_weight_ptrs(self.embed.data_ptr(), self.final_norm.data_ptr(), self.lm_head.data_ptr(),
                                    self.lm_head_scale.data_ptr() if self.lm_head_scale is not None else None,
                                    ctypes.cast(self._layer_arr, ctypes.POINTER(ctypes.c_void_p)), sc)


class Decoder:
    """One library context: caller-owned buffers (torch uint8 tensors), weights, KV state."""

    def __init__(self, cfg: pmk_model_config, device: int = 0, sched: Optional[pmk_schedule_config] = None,
                 allocate: bool = True, static_workspace: bool = False):
        import torch
        self.lib = load()
        self.cfg = cfg
        self.device = device
        ctx = ctypes.c_void_p()
        check(self.lib.pmk_create(ctypes.byref(cfg), ctypes.byref(sched) if sched is not None else None, device,
                                  ctypes.byref(ctx)))
        self.ctx = ctx
        s = pmk_sizes()
        check(self.lib.pmk_buffer_sizes(ctx, ctypes.byref(s)), ctx)
        self.sizes = s
        if allocate:
            dev = torch.device("cuda", device)
            self._arena_raw, self.arena = _aligned_empty(s.arena_bytes, dev)
            self._kv_raw, self.kv = _aligned_empty(s.kv_bytes, dev)
            if static_workspace:
                # the workspace is the library's static device array: no allocation for it here
                self.ws = None
                check(self.lib.pmk_bind_static_workspace(ctx, self.arena.data_ptr(), self.kv.data_ptr()), ctx)
            else:
                self._ws_raw, self.ws = _aligned_empty(s.workspace_bytes, dev)
                check(self.lib.pmk_bind(ctx, self.arena.data_ptr(), self.kv.data_ptr(), self.ws.data_ptr()), ctx)

    def close(self):
        if getattr(self, "ctx", None):
            self.lib.pmk_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- calls ----
    def load_weights(self, dw: DeviceWeights, stream=None):
        self._weights = dw
        check(self.lib.pmk_load_weights(self.ctx, ctypes.byref(dw.ptrs), _stream(stream)), self.ctx)

    def prefill(self, tokens, kv_scales=None, stream=None):
        import torch
        first = torch.empty(1, dtype=torch.int32, device=tokens.device)
        check(self.lib.pmk_prefill_kv(self.ctx, tokens.data_ptr(), tokens.numel(),
                                      kv_scales.data_ptr() if kv_scales is not None else None, first.data_ptr(),
                                      _stream(stream)), self.ctx)
        return first

    def kv_scales(self, stream=None):
        """The FP8 KV scales in force, [layers][n_kv][2] (K, V) fp32 on the device."""
        import torch
        out = torch.empty((self.cfg.n_layers, self.cfg.n_kv_heads, 2), dtype=torch.float32,
                          device=torch.device("cuda", self.device))
        check(self.lib.pmk_get_kv_scales(self.ctx, out.data_ptr(), _stream(stream)), self.ctx)
        return out

    def read_kv(self, P: int, stream=None):
        """KV cache positions 0..P-1 as device tensors [layers][n_kv][P][head_dim] (cache format)."""
        import torch
        dt = torch.uint8 if self.cfg.kv_dtype == PMK_DT_FP8_E4M3 else torch.int16
        shape = (self.cfg.n_layers, self.cfg.n_kv_heads, P, self.cfg.head_dim)
        dev = torch.device("cuda", self.device)
        k, v = torch.empty(shape, dtype=dt, device=dev), torch.empty(shape, dtype=dt, device=dev)
        check(self.lib.pmk_read_kv(self.ctx, k.data_ptr(), v.data_ptr(), P, _stream(stream)), self.ctx)
        return k, v

    def load_kv(self, k, v, P: int, next_token: int, kv_scales=None, stream=None):
        check(self.lib.pmk_load_kv(self.ctx, k.data_ptr() if k is not None else None,
                                   v.data_ptr() if v is not None else None, P, next_token,
                                   kv_scales.data_ptr() if kv_scales is not None else None, _stream(stream)), self.ctx)

    def rewind(self, pos: int, token, stream=None):
        check(self.lib.pmk_rewind(self.ctx, pos, token.data_ptr(), _stream(stream)), self.ctx)

    def decode(self, n: int, logits: bool = False, eos: int = -1, out_tokens=None, out_logits=None, n_done=None,
               stream=None):
        import torch
        dev = torch.device("cuda", self.device)
        if out_tokens is None:
            out_tokens = torch.full((n,), -1, dtype=torch.int32, device=dev)
        if logits and out_logits is None:
            out_logits = torch.empty((n, self.cfg.vocab), dtype=torch.float32, device=dev)
        if n_done is None:
            n_done = torch.zeros(1, dtype=torch.int32, device=dev)
        check(self.lib.pmk_decode_n_tokens(self.ctx, n, out_tokens.data_ptr(),
                                           out_logits.data_ptr() if out_logits is not None else None, eos,
                                           n_done.data_ptr(), _stream(stream)), self.ctx)
        return out_tokens, out_logits, n_done

    def set_mode(self, mode: int):
        check(self.lib.pmk_set_mode(self.ctx, mode), self.ctx)

    def position(self) -> int:
        p = ctypes.c_int32()
        check(self.lib.pmk_get_position(self.ctx, ctypes.byref(p)), self.ctx)
        return p.value

    def poll_error(self) -> pmk_device_error:
        e = pmk_device_error()
        self.lib.pmk_poll_error(self.ctx, ctypes.byref(e))
        return e

    def set_trace(self, on: bool):
        check(self.lib.pmk_set_trace(self.ctx, 1 if on else 0), self.ctx)

    def trace_stats(self):
        a, b = ctypes.c_double(), ctypes.c_double()
        check(self.lib.pmk_trace_stats(self.ctx, ctypes.byref(a), ctypes.byref(b)), self.ctx)
        return a.value, b.value

    def tune(self, steps: int = 0, stream=None) -> pmk_tune_result:
        """Keep-or-revert search over the schedule's knobs and GEMV row shares (pmk_tune): each
        candidate is validated, gated on the greedy tokens and largest logits of `steps` measured
        steps, timed, and kept only if faster.  Position and next token are restored."""
        r = pmk_tune_result()
        check(self.lib.pmk_tune(self.ctx, steps, ctypes.byref(r), _stream(stream)), self.ctx)
        return r

    def trace_export(self, path: str):
        check(self.lib.pmk_trace_export(self.ctx, path.encode()), self.ctx)

    def schedule_info(self) -> pmk_schedule_info:
        i = pmk_schedule_info()
        check(self.lib.pmk_schedule_get_info(self.ctx, ctypes.byref(i)), self.ctx)
        return i
