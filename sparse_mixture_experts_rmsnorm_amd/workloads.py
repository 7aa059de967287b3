"""The MoE-layer workloads: shapes, routing rule and expert kind, nothing else.

Five layer shapes are used throughout (tests, smoke check, benchmark):

  tiny_fp32          T=64, d=128, E=4 GELU experts of 256, top-2, fp32,
                     no capacity limit
  mixtral_bf16       T=4096, d=4096, E=8 SwiGLU experts of 14336, top-2,
                     capacity factor 1.25 (overflow dropped)
  variable_bcsr_bf16 T=8192, d=768, E=8 GELU experts of sizes
                     [(1,2048),(7,1024)], top-2, dropless, BCSR block 128,
                     router bias ~ N(0,1)
  finegrained_bf16   T=16384, d=2048, E=64 SwiGLU experts of 1408, top-6,
                     capacity factor 1.5, Zipf(1.1) router bias, plus two
                     always-on SwiGLU(1408) shared experts
  atomic_bf16        T=8192, d=1024, 2^20 atomic GELU experts behind a
                     1024 x 1024 Cartesian router, top-32, plus a dense
                     GELU shared MLP of 4096

and mixtral_mxfp8 / variable_bcsr_mxfp8, the Mixtral-shaped and the
variable-size BCSR layers with MXFP8 routed experts (OCP Microscaling: E4M3
elements, one E8M0 scale per 32 along K).

The variable-size expert spec follows the "Variable-size experts" nanoMOE
notes (configuration section: [(count, size), ...]); the capacity factor and
top-k follow the "Mixture of Experts (MoE)" glossary; the atomic experts and
the Cartesian router follow the OmniMoE summary, section 2.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    E: int
    k: int
    dtype: str = "bf16"            # "f32" or "bf16"
    act: str = "swiglu"            # "gelu", "gelu_tanh" or "swiglu"
    expert_sizes: tuple = ()       # [(count, size), ...]; () = uniform `ffn`
    ffn: int = 0                   # uniform expert width
    cf: float = 0.0                # capacity factor; <= 0: no limit
    bias: str = "none"             # "none", "normal" or "zipf"
    zipf_s: float = 1.1
    expert_kind: str = "grouped"   # "grouped", "bcsr" or "atomic"
    router: str = "dense"          # "dense" or "cartesian"
    Nr: int = 0
    Nc: int = 0
    shared_ffn: int = 0            # width of the always-on shared FFN (0: none)
    shared_act: str = "swiglu"
    renorm: int = 1
    eps: float = 1e-6
    gamma: bool = False            # draw a non-trivial RMSNorm gain
    seed: int = 0
    w_std: float = 0.02
    quant: str = "none"            # "none" or "mxfp8" (routed and shared grouped experts)

    @property
    def sizes(self) -> list:
        if self.router == "cartesian":
            return []
        if self.expert_sizes:
            out = []
            for count, size in self.expert_sizes:
                out += [((size + 127) // 128) * 128 if self.expert_kind == "bcsr" else size] * count
            if len(out) != self.E:
                raise ValueError("expert_sizes counts must sum to E")
            return out
        return [self.ffn] * self.E

    @property
    def f_offsets(self) -> list:
        off = [0]
        for s in self.sizes:
            off.append(off[-1] + s)
        return off

    @property
    def pad(self) -> int:
        return 128 if self.expert_kind == "bcsr" else 1

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", T=64, d=128, E=4, k=2, dtype="f32", act="gelu",
                          ffn=256, cf=0.0, seed=1001),
    "mixtral_bf16": Workload("mixtral_bf16", T=4096, d=4096, E=8, k=2, act="swiglu",
                             ffn=14336, cf=1.25, seed=1002),
    "mixtral_mxfp8": Workload("mixtral_mxfp8", T=4096, d=4096, E=8, k=2, act="swiglu",
                              ffn=14336, cf=1.25, quant="mxfp8", seed=1002),
    "variable_bcsr_bf16": Workload("variable_bcsr_bf16", T=8192, d=768, E=8, k=2, act="gelu",
                                   expert_sizes=((1, 2048), (7, 1024)), cf=0.0,
                                   bias="normal", expert_kind="bcsr", seed=1003),
    "variable_bcsr_mxfp8": Workload("variable_bcsr_mxfp8", T=8192, d=768, E=8, k=2,
                                    act="gelu", expert_sizes=((1, 2048), (7, 1024)), cf=0.0,
                                    bias="normal", expert_kind="bcsr", quant="mxfp8",
                                    seed=1003),
    "finegrained_bf16": Workload("finegrained_bf16", T=16384, d=2048, E=64, k=6, act="swiglu",
                                 ffn=1408, cf=1.5, bias="zipf", shared_ffn=2 * 1408,
                                 shared_act="swiglu", seed=1004),
    "atomic_bf16": Workload("atomic_bf16", T=8192, d=1024, E=1 << 20, k=32, act="gelu",
                            router="cartesian", Nr=1024, Nc=1024, expert_kind="atomic",
                            shared_ffn=4096, shared_act="gelu", seed=1005),
}


def flops_experts(wl: Workload, kept_per_expert) -> float:
    """Algorithmic expert-FFN FLOPs for the kept rows (no padding)."""
    mult = 3 if wl.act == "swiglu" else 2
    return float(sum(2.0 * mult * wl.d * f * m for f, m in zip(wl.sizes, kept_per_expert)))
