"""The synthetic workloads the path is checked and measured on.

Shapes follow the OneLA operator suite (§4.1: R requests, W beams, T decode
steps, H heads, K = d_k, V = d_v) and the DeltaLog recurrent-kernel table
(Table 3: H/d_k/d_v = 32/128/128, FP32 state; GDN log with M = 8, KDA and
RWKV6 logs with M = 4).  Seeds: the tiny workload uses seed 0; the others use their index.
"""

from __future__ import annotations

from dataclasses import dataclass

from . import synth


@dataclass(frozen=True)
class BeamWorkload:
    name: str
    R: int
    H: int
    dk: int
    dv: int
    W: int
    L: int
    s0_std: float
    seed: int
    parents: str
    channel_decay: bool = False
    hot_frac: float = 0.3
    Hk: int | None = None  # key heads shared by the value heads (None: one each)

    @property
    def beam_steps(self) -> int:
        return self.R * self.W * self.L

    def inputs(self, **over):
        kw = dict(R=self.R, H=self.H, dk=self.dk, dv=self.dv, W=self.W, L=self.L,
                  s0_std=self.s0_std, seed=self.seed, parents=self.parents,
                  channel_decay=self.channel_decay, hot_frac=self.hot_frac, Hk=self.Hk)
        kw.update(over)
        return synth.make_inputs(**kw)


@dataclass(frozen=True)
class SequenceWorkload:
    """Bounded-log decoding of independent sequences (one beam each)."""
    name: str
    R: int
    H: int
    dk: int
    dv: int
    T: int
    M: int
    s0_std: float
    seed: int
    channel_decay: bool = False
    plain_update: bool = False  # the RWKV6 update pair (k_t, v_t); implies channel decay

    @property
    def rule(self) -> str:
        return "plain" if self.plain_update else "delta"

    @property
    def sequence_steps(self) -> int:
        return self.R * self.T

    def inputs(self, **over):
        kw = dict(R=self.R, H=self.H, dk=self.dk, dv=self.dv, T=self.T,
                  s0_std=self.s0_std, seed=self.seed, channel_decay=self.channel_decay)
        kw.update(over)
        return synth.make_sequence_inputs(**kw)


TINY = BeamWorkload("tiny_gdn_beam", R=1, H=2, dk=16, dv=16, W=4, L=3,
                    s0_std=0.1, seed=0, parents="uniform")
SINGLE = BeamWorkload("gdn_single_request", R=1, H=32, dk=128, dv=128, W=128, L=3,
                      s0_std=0.05, seed=1, parents="topk")
LARGE = BeamWorkload("gdn_large_beam", R=8, H=32, dk=128, dv=128, W=512, L=4,
                     s0_std=0.05, seed=2, parents="topk_hot", hot_frac=0.3)
DELTALOG = SequenceWorkload("deltalog_bounded_log", R=128, H=32, dk=128, dv=128,
                            T=64, M=8, s0_std=0.05, seed=3)
KDA = BeamWorkload("kda_channel_decay_beam", R=16, H=32, dk=128, dv=128, W=256, L=4,
                   s0_std=0.05, seed=4, parents="topk", channel_decay=True)

# 32 value heads reading 16 key heads (two value heads per key head)
SHARED_KEYS = BeamWorkload("gdn_large_beam_shared_key_heads", R=8, H=32, dk=128, dv=128, W=512, L=4,
                           s0_std=0.05, seed=6, parents="topk_hot", hot_frac=0.3, Hk=16)

# the widest recurrent state of the operator suite's range: K = 256, V = 512
WIDE = BeamWorkload("gdn_wide_state_beam", R=8, H=16, dk=256, dv=512, W=512, L=4,
                    s0_std=0.05, seed=7, parents="topk_hot", hot_frac=0.3)

# channel decay on a wide value state: d_k = 128, d_v = 512
KDA_WIDE = BeamWorkload("kda_wide_value_beam", R=8, H=16, dk=128, dv=512, W=256, L=4,
                        s0_std=0.05, seed=8, parents="topk", channel_decay=True)

# OneLA §4.1/§4.3 "Qwen geometry" (H_K = H_V = 16, K = V = 128) at W = 512 with six decode
# steps (O = 7 output tokens): R = 4 (the recurrent-path breakdown) and R = 16 (the largest shape)
QWEN_R4 = BeamWorkload("onela_qwen_geometry_r4", R=4, H=16, dk=128, dv=128, W=512, L=6,
                       s0_std=0.05, seed=9, parents="topk_hot", hot_frac=0.3)
QWEN_R16 = BeamWorkload("onela_qwen_geometry_r16", R=16, H=16, dk=128, dv=128, W=512, L=6,
                        s0_std=0.05, seed=10, parents="topk_hot", hot_frac=0.3)

RWKV6 = SequenceWorkload("rwkv6_bounded_log", R=128, H=32, dk=128, dv=128, T=64, M=4,
                         s0_std=0.05, seed=5, channel_decay=True, plain_update=True)

# the KDA row of DeltaLog Table 3: 32/128/128, FP32 state, BF16 K / FP32 U log, M = 4
KDA_LOG = SequenceWorkload("kda_bounded_log", R=128, H=32, dk=128, dv=128, T=64, M=4,
                           s0_std=0.05, seed=11, channel_decay=True)

ALL = (TINY, SINGLE, LARGE, DELTALOG, KDA, RWKV6, SHARED_KEYS, WIDE, KDA_WIDE, QWEN_R4, QWEN_R16, KDA_LOG)
BY_NAME = {w.name: w for w in ALL}
