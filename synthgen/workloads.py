"""The decode workloads: model shapes, storage formats, prompt length and decode steps.

Pure data.  Values the workload statement leaves open use the Llama defaults
(RoPE theta 10000 and RMSNorm eps 1e-5 where unstated; KV stored in the weight format).
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    hidden: int
    n_q: int
    n_kv: int
    head_dim: int
    ffn: int
    vocab: int
    eps: float
    theta: float
    wdtype: str   # "f16" | "bf16" | "fp8" (E4M3 + 128x128 fp32 block scales) | "int8" | "int4"
                  # (two's-complement codes + one bf16 scale per row and 128-column group)
    kvdtype: str  # "f16" | "bf16" | "fp8" (E4M3 + per (layer, kv head, K|V) fp32 scale)
    prompt: int
    steps: int
    seed: int

    @property
    def max_seq(self) -> int:
        return self.prompt + self.steps

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    def weight_bytes(self) -> int:
        """Bytes of weights streamed per decode token: every GEMV weight (with its fp8 block scales
        or int8 / int4 group scales), the norm gains, one embedding row and the LM head."""
        H, F, V, L = self.hidden, self.ffn, self.vocab, self.layers
        qkv = (self.n_q + 2 * self.n_kv) * self.head_dim
        lin = L * (qkv * H + H * self.n_q * self.head_dim + 2 * F * H + H * F) + V * H
        bits = {"fp8": 8, "int8": 8, "int4": 4}.get(self.wdtype, 16)
        total = lin * bits // 8 + (2 * L + 1) * H * 2 + H * 2  # gains (16-bit) + one embedding row (16-bit)
        if self.wdtype == "fp8":
            def blocks(r, c):
                return ((r + 127) // 128) * ((c + 127) // 128)
            qd, kvd = self.n_q * self.head_dim, self.n_kv * self.head_dim
            per_layer = blocks(qd, H) + 2 * blocks(kvd, H) + blocks(H, qd) + 2 * blocks(F, H) + blocks(H, F)
            total += 4 * (L * per_layer + blocks(V, H))
        if self.wdtype in ("int8", "int4"):
            def groups(r, c):
                return r * ((c + 127) // 128)
            qd, kvd = self.n_q * self.head_dim, self.n_kv * self.head_dim
            per_layer = groups(qd, H) + 2 * groups(kvd, H) + groups(H, qd) + 2 * groups(F, H) + groups(H, F)
            total += 2 * (L * per_layer + groups(V, H))
        return total

    def kv_bytes_per_position(self) -> int:
        kb = 1 if self.kvdtype == "fp8" else 2
        return self.layers * self.n_kv * self.head_dim * 2 * kb

    def kv_bytes_read(self, step: int) -> int:
        """KV bytes read by decode step `step` (0-based): T = prompt + step + 1 positions."""
        return (self.prompt + step + 1) * self.kv_bytes_per_position()

    def mean_bytes_per_token(self) -> float:
        kv = sum(self.kv_bytes_read(i) for i in range(self.steps)) / self.steps
        return self.weight_bytes() + kv


SEED_BASE = 20260601

WORKLOADS = {
    "tiny": Workload("tiny", 2, 256, 4, 2, 64, 688, 1024, 1e-5, 10000.0, "f16", "f16", 16, 32, SEED_BASE + 0),
    "1b": Workload("1b", 16, 2048, 32, 8, 64, 8192, 32000, 1e-5, 10000.0, "bf16", "bf16", 512, 128, SEED_BASE + 1),
    "2b": Workload("2b", 26, 2560, 20, 4, 128, 6912, 32000, 1e-5, 10000.0, "f16", "f16", 1024, 256, SEED_BASE + 2),
    "8b": Workload("8b", 32, 4096, 32, 8, 128, 14336, 128256, 1e-5, 500000.0, "bf16", "bf16", 4096, 256,
                   SEED_BASE + 3),
    "8b_fp8": Workload("8b_fp8", 32, 4096, 32, 8, 128, 14336, 128256, 1e-5, 500000.0, "fp8", "fp8", 8192, 256,
                       SEED_BASE + 4),
    # weight-only integer variants of the 8B decode (W8A16 / W4A16, bf16 KV cache)
    "8b_int8": Workload("8b_int8", 32, 4096, 32, 8, 128, 14336, 128256, 1e-5, 500000.0, "int8", "bf16", 4096, 256,
                        SEED_BASE + 5),
    "8b_int4": Workload("8b_int4", 32, 4096, 32, 8, 128, 14336, 128256, 1e-5, 500000.0, "int4", "bf16", 4096, 256,
                        SEED_BASE + 6),
}
