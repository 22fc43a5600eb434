"""Shared test helpers: seeded inputs for both sides, tolerance metric."""
import numpy as np

from oracle import ae_oracle as O
from workload import configs as C
from workload import gen as G

# max |gpu - oracle| <= TOL * RMS(oracle) over every entry of the chunk
TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}


def tol_for(cfg):
    return TOL["fp8"] if cfg.mlp_dtype == "fp8" else TOL[cfg.weight_dtype]


def rel_err(got, ref):
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref)) / np.sqrt(np.mean(ref ** 2)))


# Small shapes the oracle finishes in well under a second that still span several
# tiles and leave ragged tails: 20 chunk rows (2 token tiles, 12 padding rows),
# 120 keys (2 attention chunks, last one partial), 24 action dims (2 output tiles,
# 8 padding rows), 2 kv heads (GQA groups of 2).
SMALL_BF16 = C.AEConfig(
    name="small_bf16", n_layers=2, width=256, n_q_heads=4, n_kv_heads=2, head_dim=64, mlp_dim=512,
    action_dim=24, horizon=20, prefix_len=100, max_batch=3, max_taus=3, gripper_dim=23, steps=3)
SMALL_FP8 = SMALL_BF16.with_(name="small_fp8", mlp_dtype="fp8")
SMALL_F32 = SMALL_BF16.with_(name="small_f32", weight_dtype="f32", mlp_dtype="f32", kv_dtype="f32")


class Case:
    """Weights, prefix caches and noise for one config, in storage and float64 forms."""

    def __init__(self, cfg, n_slots=None, weight_seed=None):
        self.cfg = cfg
        self.W = G.make_weights(cfg, weight_seed)
        self.Wd = O.dequantize_weights(cfg, self.W)
        n = cfg.max_batch if n_slots is None else n_slots
        self.kv = [G.make_prefix_kv(cfg, cfg.kv_seed + r) for r in range(n)]
        self.kvd = [O.decode_kv(cfg, k, v) for k, v in self.kv]

    def noise(self, batch, seed=None):
        return G.make_noise(self.cfg, self.cfg.noise_seed if seed is None else seed, batch)

    def oracle_denoise(self, noise, steps, robots=None):
        robots = range(noise.shape[0]) if robots is None else robots
        return np.stack([O.denoise(self.cfg, self.Wd, self.kvd[r][0], self.kvd[r][1], noise[r].astype(np.float64), steps)
                         for r in robots])

    def oracle_verify(self, slot, draft, noise, taus, delta, cfg=None):
        """cfg overrides the config when the weights are shared with another workload (e.g. gripper_dim)."""
        return O.verify(cfg or self.cfg, self.Wd, self.kvd[slot][0], self.kvd[slot][1], draft, noise, taus, delta)
