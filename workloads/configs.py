"""The five synthetic workloads of the modal-SSM Hyena hot path.

Shapes follow the workloads the pages talk about: a 1.3B-parameter-wide model
(width 2048) generating 512 tokens (Laughing Hyena Distillery review,
"主要发现"), and a 64k-token sequence for the long convolution (StripedHyena
article, section "面向更長的上下文").

Fields
------
B, D, H, d, L, S : batch rows, channels, heads (filters tied per head),
                   complex modes per head, prompt length, generated steps.
act              : activation dtype of q/k/v/y: "f32" or "bf16".
r_lo, r_hi       : pole radius ~ U(r_lo, r_hi); pole angle ~ U(0, pi).
layers           : > 0 only for the projected stack (in_proj D->3D, out_proj D->D
                   around the operator in every layer).
"""

from dataclasses import dataclass


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    B: int
    D: int
    H: int
    d: int
    L: int
    S: int
    act: str
    r_lo: float
    r_hi: float
    layers: int = 0
    w_std: float = 0.02

    @property
    def P(self) -> int:
        return self.D // self.H

    @property
    def act_bytes(self) -> int:
        return 2 if self.act == "bf16" else 4

    @property
    def seed(self) -> int:
        return 1000 + self.index

    def describe(self) -> str:
        s = (f"B={self.B} D={self.D} H={self.H} d={self.d} L={self.L} S={self.S} "
             f"act={self.act} r~U({self.r_lo},{self.r_hi})")
        if self.layers:
            s += f" layers={self.layers}"
        return s


CONFIGS = {
    1: Config(1, "tiny-f32", B=1, D=64, H=4, d=8, L=256, S=64, act="f32",
              r_lo=0.5, r_hi=0.99),
    2: Config(2, "width2048-bf16", B=16, D=2048, H=16, d=16, L=2048, S=512,
              act="bf16", r_lo=0.8, r_hi=0.999),
    3: Config(3, "batch256-decode-bf16", B=256, D=2048, H=16, d=16, L=512, S=512,
              act="bf16", r_lo=0.5, r_hi=0.99),
    4: Config(4, "long64k-f32", B=4, D=4096, H=32, d=32, L=65536, S=128,
              act="f32", r_lo=0.9, r_hi=0.9999),
    5: Config(5, "stack24-bf16", B=64, D=2048, H=16, d=16, L=2048, S=512,
              act="bf16", r_lo=0.8, r_hi=0.999, layers=24),
}


def get_config(i: int) -> Config:
    if i not in CONFIGS:
        raise KeyError(f"unknown workload {i}; known: {sorted(CONFIGS)}")
    return CONFIGS[i]
