"""The five synthetic workloads this library is tested and measured on.

Shapes follow the workloads the source pages motivate: KIVI's Llama / Mistral
(GQA) long-context decode ("Makale Bülteni -- KIVI", lead paragraph and
section "Kod ve Entegrasyon Haritası") and an MLA cache with a 2-bit content
latent and a 4-bit RoPE key ("QuantMLA ...", section "QuantMLA Mimarisi ve
Temel Bileşenleri").  The model names are shape templates only; every tensor
is seeded synthetic data (see ``synth.py``).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    index: int            # seed offset
    kind: str             # "kivi" or "mla"
    batch: int
    n_q_heads: int
    n_kv_heads: int
    T: int                # tokens in the cache at decode time
    kd: int               # key-stream dim (KIVI: head dim, MLA: RoPE dim)
    kG: int               # key token-group size G
    kbits: int
    vd: int               # value-stream dim (KIVI: head dim, MLA: latent dim)
    vG: int               # value channel-group size
    vbits: int
    outlier_scale: float  # factor on the 1% outlier key channels

    @property
    def qd(self) -> int:
        return self.kd if self.kind == "kivi" else self.vd + self.kd

    @property
    def sigma(self) -> float:
        """Softmax scale 1/sqrt(width of the q.k contraction)."""
        return 1.0 / math.sqrt(self.qd)

    @property
    def n_outlier(self) -> int:
        return max(1, math.ceil(0.01 * self.n_kv_heads * self.kd))

    @property
    def R(self) -> int:
        return self.T % self.kG

    @property
    def n_blocks(self) -> int:
        return self.T // self.kG

    def capacity(self, extra: int = 0) -> int:
        """Token capacity covering T + extra, rounded up to whole key blocks."""
        need = self.T + extra
        return ((need + self.kG - 1) // self.kG) * self.kG

    def with_T(self, T: int) -> "Workload":
        return replace(self, T=T)

    # algorithmic bytes of one decode call (cache read + q read + out write)
    def cache_bytes(self, T: int | None = None) -> int:
        T = self.T if T is None else T
        nb, R = T // self.kG, T % self.kG
        per_pair = (nb * self.kG * self.kd * self.kbits // 8      # key codes
                    + nb * self.kd * 4                             # key scale+zero
                    + R * self.kd * 2                              # fp16 residual
                    + T * self.vd * self.vbits // 8                # value codes
                    + T * (self.vd // self.vG) * 4)                # value scale+zero
        return per_pair * self.batch * self.n_kv_heads

    def qo_bytes(self) -> int:
        return self.batch * self.n_q_heads * (self.qd + self.vd) * 2

    def decode_bytes(self, T: int | None = None) -> int:
        return self.cache_bytes(T) + self.qo_bytes()

    def fp16_kv_bytes(self, T: int | None = None) -> int:
        T = self.T if T is None else T
        return self.batch * self.n_kv_heads * T * (self.kd + self.vd) * 2

    def decode_flops(self, T: int | None = None) -> int:
        T = self.T if T is None else T
        return 2 * self.batch * self.n_q_heads * T * (self.qd + self.vd)


def _kivi(name, index, B, Hq, Hkv, D, T, G):
    return Workload(name, index, "kivi", B, Hq, Hkv, T, D, G, 2, D, 32, 2, 50.0)


WORKLOADS = [
    _kivi("tiny_mha_d64_t250", 0, 1, 2, 2, 64, 250, 32),
    _kivi("llama2_7b_layer_mha_t4096", 1, 8, 32, 32, 128, 4096, 32),
    _kivi("mistral_7b_gqa_t32805", 2, 32, 32, 8, 128, 32768 + 37, 64),
    _kivi("longctx_gqa_t131072", 3, 4, 32, 8, 128, 131072, 32),
    Workload("mla_absorbed_b64_t16384", 4, "mla", 64, 128, 1, 16384,
             64, 64, 4, 512, 32, 2, 20.0),
]

# Prompt (prefill) workloads: causal attention over the prompt's fp16 K / V
# with the bulk quantize fused in.  Mistral-7B-shaped GQA layer, a 4096-token
# prompt per sequence.
PREFILL_WORKLOADS = [
    _kivi("mistral_7b_gqa_prefill_b4_t4096", 5, 4, 32, 8, 128, 4096, 64),
]

BY_NAME = {w.name: w for w in WORKLOADS + PREFILL_WORKLOADS}
