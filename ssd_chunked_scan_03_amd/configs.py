"""Workload shapes for the SSD forward scan.

Each workload names its shape (batch b, sequence T, heads H, head dim P, state N,
B/C groups G, chunk Q), the dtype of x/B/C/y, the dt range, whether the decay is
scalar per head or diagonal (per head and state dimension), whether h0 is drawn,
and the seed.  The value distributions are produced by :mod:`.synth`.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk: int
    dtype: str            # "f32" or "bf16": dtype of x, B, C and y
    dt_lo: float
    dt_hi: float
    diag: bool = False    # per-(h, n) decay instead of per-h
    h0: bool = False      # draw a nonzero initial state h0 ~ N(0, 0.1^2)
    seed: int = 0

    @property
    def nchunks(self) -> int:
        return (self.seqlen + self.chunk - 1) // self.chunk

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    def shape(self) -> dict:
        return dict(b=self.batch, T=self.seqlen, H=self.nheads, P=self.headdim,
                    N=self.dstate, G=self.ngroups, Q=self.chunk)


TINY_F32 = Workload("tiny_f32_b1_T256_H2_P16_N16", 1, 256, 2, 16, 16, 1, 64, "f32",
                    1e-3, 0.1, seed=0)
M780 = Workload("mamba2_780m_layer_b2_T2048_H48_P64_N128", 2, 2048, 48, 64, 128, 1, 256,
                "bf16", 1e-3, 0.1, seed=1)
M2P7B = Workload("mamba2_2p7b_layer_b8_T4096_H80_P64_N128", 8, 4096, 80, 64, 128, 1, 256,
                 "bf16", 1e-3, 0.1, h0=True, seed=2)
LONG = Workload("long_b1_T65536_H32_P64_N256_G8", 1, 65536, 32, 64, 256, 8, 256, "bf16",
                1e-4, 1e-2, seed=3)
DIAG = Workload("diag_b4_T4096_H32_P64_N64_Q128", 4, 4096, 32, 64, 64, 1, 128, "bf16",
                1e-3, 0.1, diag=True, seed=4)

WORKLOADS = [TINY_F32, M780, M2P7B, LONG, DIAG]
HEADLINE = M2P7B
LONG_CHUNKS = (64, 128, 256)
