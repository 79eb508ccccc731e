"""The five synthetic KDA workloads, as plain data.

Each workload is named by what it is and its sizes. Shapes follow the
K3 layer geometry: 96 heads with 128-wide keys and values per head
("K3 Architecture Illustrated", section "A fixed state still has a cost",
FIG 24 capacity model, whose crossover points 2731 / 5461 tokens hold for
H = 96, dk = dv = 128), and long sequences ("Kimi K3 - Lesson 3 of 14 -
Sequence axis", the 8K -> 1M context curriculum).

Field meanings
--------------
B, T, H, dk, dv : batch, tokens, heads, key width, value width.
qkv, gate       : storage dtype of q/k/v/o ("f32" | "bf16") and of g/beta.
z_mu, z_sd      : the log-decay logits are z ~ N(z_mu, z_sd) and
                  g = -5 * sigmoid(z).
forced_channels : number of key channels per (b, h) whose logit is pinned
                  to forced_z at every token (0 = none).
s0_sd           : S0 ~ N(0, s0_sd) in fp32, or None for a zero state.
steps           : decode workloads only: consecutive single-token steps.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

CHUNK = 64   # tokens per chunk of the chunkwise form
TILE = 16    # tokens per tile inside a chunk
G_MIN = -5.0  # floor of the log-decay


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str          # "fwd" | "decode"
    B: int
    H: int
    dk: int
    dv: int
    T: int = 1
    qkv: str = "bf16"
    gate: str = "f32"
    z_mu: float = 0.0
    z_sd: float = 1.0
    forced_channels: int = 0
    forced_z: float = 0.0
    s0_sd: Optional[float] = None
    steps: int = 1
    note: str = field(default="", compare=False)

    def scaled(self, **kw) -> "Workload":
        """Same recipe at other sizes (used for reduced parity cases)."""
        name = kw.pop("name", None) or self.name + "_reduced"
        return replace(self, name=name, **kw)


# Tiny fp32 forward: every output checked, the oracle runs it in well under a second.
TINY_F32 = Workload(
    name="kda_fwd_B1_H2_T256_d64_f32", kind="fwd",
    B=1, H=2, T=256, dk=64, dv=64, qkv="f32", gate="f32",
    z_mu=0.0, z_sd=1.0, s0_sd=None,
)

# One head group, bf16 q/k/v, fp32 gates, random fp32 initial state.
HEADGROUP_BF16 = Workload(
    name="kda_fwd_B1_H8_T4096_d128_bf16", kind="fwd",
    B=1, H=8, T=4096, dk=128, dv=128, qkv="bf16", gate="f32",
    z_mu=0.0, z_sd=1.5, s0_sd=0.02,
)

# Training shape, all-bf16 inputs; the headline forward workload.
# Most channels retain (g near 0) and 5% of key channels sit at the decay
# floor (g close to -5) at every token, so every 16-token tile reaches a
# cumulative log-decay close to the 80 bound.  With g = -5*sigmoid(z) that
# intent needs z ~ N(-2, 1) and a forced logit of +6; the opposite signs
# (z ~ N(2, 1), forced -6) are kept as a second parity case, TRAIN_BF16_LITERAL.
TRAIN_BF16 = Workload(
    name="kda_fwd_B4_H32_T16384_d128_bf16", kind="fwd",
    B=4, H=32, T=16384, dk=128, dv=128, qkv="bf16", gate="bf16",
    z_mu=-2.0, z_sd=1.0, forced_channels=6, forced_z=6.0, s0_sd=None,
)
TRAIN_BF16_LITERAL = replace(
    TRAIN_BF16, name="kda_fwd_B4_H32_T16384_d128_bf16_literal",
    z_mu=2.0, forced_z=-6.0,
)

# Long single sequence: 96 heads over 131072 tokens (2048 chunks of 64).
LONG_BF16 = Workload(
    name="kda_fwd_B1_H96_T131072_d128_bf16", kind="fwd",
    B=1, H=96, T=131072, dk=128, dv=128, qkv="bf16", gate="bf16",
    z_mu=0.0, z_sd=1.0, s0_sd=None,
)

# One GPU's share of LONG_BF16 under 8-way head sharding (12 of its 96 heads):
# 24 workgroups of the plain forward for 256 CUs, the sequence-parallel case.
LONG_SHARE_BF16 = LONG_BF16.scaled(H=12, name="kda_fwd_B1_H12_T131072_d128_bf16")

# Batched single-token decode: 256 sequences x 96 heads of fp32 128x128 state.
DECODE_BF16 = Workload(
    name="kda_decode_B256_H96_d128_bf16_x64", kind="decode",
    B=256, H=96, dk=128, dv=128, qkv="bf16", gate="f32",
    z_mu=0.0, z_sd=1.0, s0_sd=0.02, steps=64,
)

ALL = [TINY_F32, HEADGROUP_BF16, TRAIN_BF16, TRAIN_BF16_LITERAL, LONG_BF16, DECODE_BF16]
BY_NAME = {w.name: w for w in ALL}
