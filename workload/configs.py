"""The five workload shapes of the Pi0/DM0.5-style action expert.

Shapes follow the pages' problem statement: a Gemma-style action expert
(DM0.5/OpenDM guide, section 5.2 "Suffix") fed a prefix KV cache (section 5.1
"Prefix"), an action chunk of 50 rows (section 7.3, chunk-size 50) and 10 Euler
steps (section 5.3 "Flow Matching"); the Pi0-scale sizes are those of the
300M-parameter expert timed on the "From 3ms to 2.5s" slides ("2x params ->
4.4x latency" table). The verification case follows the Realtime-VLA FLASH
article, section 03 ("multi-step parallel verification").
"""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class AEConfig:
    name: str
    n_layers: int
    width: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    mlp_dim: int
    action_dim: int
    horizon: int
    prefix_len: int
    max_batch: int = 1
    max_taus: int = 0
    rope_base: float = 10000.0
    rms_eps: float = 1e-6
    weight_dtype: str = "bf16"   # "f32" | "bf16": every linear except the MLP
    mlp_dtype: str = "bf16"      # "f32" | "bf16" | "fp8": gate / up / down
    kv_dtype: str = "bf16"       # "f32" | "bf16": prefix cache storage
    gripper_dim: int = -1        # action dim holding the +-1 gripper channel, -1 = none
    time_mode: int = 0           # 0: temb added to every action_in_proj row; 1: per-layer time modulation
    qk_norm: int = 0             # 1: RMSNorm of q and k per head (gains q_norm, k_norm) before RoPE
    draft: int = 0               # 1: draft model (one block, learnable queries over image features)
    prefill: int = 0             # 1: prefix prefill (the VLM's blocks over the prefix tokens -> KV cache)
    steps: int = 10
    batch: int = 1               # robots advanced together
    weight_std: float = 0.02
    weight_seed: int = 0
    kv_seed: int = 100
    noise_seed: int = 200

    def with_(self, **kw):
        return replace(self, **kw)

    @property
    def n_params(self):
        w, A, dh, F = self.width, self.action_dim, self.head_dim, self.mlp_dim
        per_layer = (self.n_q_heads + 2 * self.n_kv_heads) * dh * w + w * self.n_q_heads * dh + 3 * F * w + 2 * w
        per_layer += (6 * w * w + 6 * w if self.time_mode else 0) + (2 * dh if self.qk_norm else 0)
        final = (2 * w * w + 2 * w) if self.time_mode else 0
        if self.draft:  # queries replace the time MLP and action_in_proj
            return self.n_layers * per_layer + self.horizon * w + (A * w + A) + w
        if self.prefill:  # the blocks only: no time MLP, action projections or final norm
            return self.n_layers * per_layer
        return self.n_layers * per_layer + 2 * (w * w + w) + (w * A + w) + (A * w + A) + w + final


TINY = AEConfig(
    name="tiny_fp32", n_layers=2, width=256, n_q_heads=4, n_kv_heads=1, head_dim=64, mlp_dim=1024,
    action_dim=8, horizon=8, prefix_len=64, weight_dtype="f32", mlp_dtype="f32", kv_dtype="f32", steps=4,
)
PI0 = AEConfig(
    name="pi0_bf16", n_layers=18, width=1024, n_q_heads=8, n_kv_heads=1, head_dim=256, mlp_dim=4096,
    action_dim=32, horizon=50, prefix_len=816, steps=10,
)
PI0_FP8 = PI0.with_(name="pi0_fp8mlp_2view", prefix_len=560, mlp_dtype="fp8")
PI0_VERIFY = PI0.with_(name="pi0_verify", max_taus=4, gripper_dim=31)
PI0_BATCH16 = PI0.with_(name="pi0_batch16", max_batch=16, batch=16)

# DM0.5-style expert at the Pi0 shapes (DM0.5 guide, section 5.2: the time MLP conditions every
# layer, and the expert sits on a Gemma3 text stack, which normalises q and k per head)
DM05 = PI0.with_(name="dm05_bf16", time_mode=1, qk_norm=1)
# and its speculative verification (FLASH article, section 03) at the Pi0 verify shape
DM05_VERIFY = DM05.with_(name="dm05_verify", max_taus=4, gripper_dim=31)

# Draft model of the speculative round (FLASH article, section 03: one Gemma block and a linear action
# head, ~110M parameters; learnable action queries over the current image features): a 2B-class Gemma
# block (width 2048, 8q/1kv x 256, MLP 16384) over 3 views x 256 image tokens, 50 x 32 chunk
DRAFT = AEConfig(
    name="draft_bf16", n_layers=1, width=2048, n_q_heads=8, n_kv_heads=1, head_dim=256, mlp_dim=16384,
    action_dim=32, horizon=50, prefix_len=768, draft=1, steps=1,
)

# Prefix prefill (DM0.5 guide 5.1 and 6.3: the VLM prefix is encoded once into the per-layer KV cache
# the expert reads; the guide runs its MLP in FP8 E4M3): a 2B-class Gemma stack (18 layers, width
# 2048, 8q/1kv x 256 -- the expert's kv heads and head_dim --, MLP 16384) over the 816 prefix tokens
PREFILL = AEConfig(
    name="prefill_fp8mlp", n_layers=18, width=2048, n_q_heads=8, n_kv_heads=1, head_dim=256, mlp_dim=16384,
    action_dim=32, horizon=816, prefix_len=0, mlp_dtype="fp8", prefill=1, steps=1,
)

CONFIGS = [TINY, PI0, PI0_FP8, PI0_VERIFY, PI0_BATCH16, DM05, DM05_VERIFY, DRAFT, PREFILL]
VERIFY_TAUS = (0.2, 0.4, 0.6, 0.8)
VERIFY_DELTA = 0.05


def config_by_name(name):
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)
