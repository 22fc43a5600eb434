"""Seeded input generators (weights, prefix KV cache, noise, verification drafts).

Every array is drawn with ``numpy.random.default_rng(seed)`` (PCG64) in the
order documented on each function, then stored in the format the library's
C-ABI takes:

* ``f32``  -> ``float32``
* ``bf16`` -> ``uint16`` bit patterns, rounded to nearest-even (torch CPU cast)
* ``fp8``  -> ``uint8`` OCP FP8 E4M3 bit patterns plus one ``float32`` scale per
  output channel (row), ``s_j = max_i |W_ji| / 448``, codes = RNE(W / s_j)

Nothing here computes any step of the method; the quantisers are the input
format, and each side decodes them with its own decoder.
"""
import numpy as np
import torch

from .configs import VERIFY_TAUS

FP8_MAX = 448.0


def _to_bf16_bits(a32):
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _to_fp8_rows(a32):
    """Per-output-channel (row) OCP E4M3 quantisation: returns (codes uint8, scales f32)."""
    a32 = np.ascontiguousarray(a32, dtype=np.float32)
    amax = np.abs(a32).max(axis=1)
    scale = np.where(amax > 0, amax / FP8_MAX, 1.0).astype(np.float32)
    scaled = np.clip(a32 / scale[:, None], -FP8_MAX, FP8_MAX)
    codes = torch.from_numpy(scaled).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def store(a32, dtype):
    """Cast a float32 array to the storage format ``dtype`` ("f32" | "bf16")."""
    if dtype == "f32":
        return np.ascontiguousarray(a32, dtype=np.float32)
    if dtype == "bf16":
        return _to_bf16_bits(a32)
    raise ValueError(dtype)


def weight_names(cfg):
    """(name, shape, kind) in draw order. Linear weights are row-major [out][in]."""
    w, A, dh, F = cfg.width, cfg.action_dim, cfg.head_dim, cfg.mlp_dim
    nq, nkv = cfg.n_q_heads, cfg.n_kv_heads
    if getattr(cfg, "draft", 0):  # learnable action queries instead of the time MLP and action_in_proj
        out = [("queries", (cfg.horizon, w), "query")]
    elif getattr(cfg, "prefill", 0):  # the VLM's blocks only
        out = []
    else:
        out = [
            ("time_in_w", (w, w), "lin"), ("time_in_b", (w,), "bias"),
            ("time_out_w", (w, w), "lin"), ("time_out_b", (w,), "bias"),
            ("action_in_w", (w, A), "lin"), ("action_in_b", (w,), "bias"),
        ]
    for l in range(cfg.n_layers):
        p = f"layers.{l}."
        out += [
            (p + "ln1", (w,), "gain"),
            (p + "wq", (nq * dh, w), "lin"), (p + "wk", (nkv * dh, w), "lin"), (p + "wv", (nkv * dh, w), "lin"),
            (p + "wo", (w, nq * dh), "lin"),
            (p + "ln2", (w,), "gain"),
            (p + "wg", (F, w), "mlp"), (p + "wu", (F, w), "mlp"), (p + "wd", (w, F), "mlp"),
        ]
        if cfg.time_mode:  # [scale1 | shift1 | gate1 | scale2 | shift2 | gate2] from temb
            out += [(p + "w_mod", (6 * w, w), "lin"), (p + "b_mod", (6 * w,), "modbias")]
        if cfg.qk_norm:
            out += [(p + "q_norm", (dh,), "normgain"), (p + "k_norm", (dh,), "normgain")]
    if not getattr(cfg, "prefill", 0):
        out += [("final_ln", (w,), "gain"), ("action_out_w", (A, w), "lin"), ("action_out_b", (A,), "bias")]
    if cfg.time_mode:  # [scale | shift] of the final norm
        out += [("final_mod_w", (2 * w, w), "lin"), ("final_mod_b", (2 * w,), "modbias")]
    return out


def make_weights(cfg, seed=None):
    """Random-init expert weights.

    Draw order: for each entry of ``weight_names`` that is not a gain or a
    modulation bias, one ``standard_normal(shape, float32) * weight_std`` draw
    ("normgain": ``1 + 0.1 * standard_normal``). Gains are 1; modulation biases
    are 0 except their gate thirds (1), so the modulated block starts near the
    plain one. Biases stay float32; "lin" tensors use ``weight_dtype``; "mlp"
    tensors use ``mlp_dtype`` (fp8 adds ``<name>.scale``).
    """
    rng = np.random.default_rng(cfg.weight_seed if seed is None else seed)
    W = {}
    for name, shape, kind in weight_names(cfg):
        if kind == "gain":
            W[name] = np.ones(shape, np.float32)
            continue
        if kind == "modbias":
            b = np.zeros(shape, np.float32)
            w = cfg.width
            if shape[0] == 6 * w:
                b[2 * w:3 * w] = 1.0
                b[5 * w:6 * w] = 1.0
            W[name] = b
            continue
        if kind == "query":  # N(0, 1) rows: an embedding table's scale
            W[name] = rng.standard_normal(shape, dtype=np.float32)
            continue
        if kind == "normgain":
            W[name] = (1.0 + 0.1 * rng.standard_normal(shape, dtype=np.float32)).astype(np.float32)
            continue
        a = rng.standard_normal(shape, dtype=np.float32) * np.float32(cfg.weight_std)
        if kind == "bias":
            W[name] = a.astype(np.float32)
        elif kind == "lin":
            W[name] = store(a, cfg.weight_dtype)
        elif cfg.mlp_dtype == "fp8":
            W[name], W[name + ".scale"] = _to_fp8_rows(a)
        else:
            W[name] = store(a, cfg.mlp_dtype)
    return W


def make_prefix_kv(cfg, seed=None):
    """Prefix cache K then V, each [L][P][n_kv][dh] N(0,1), stored in ``kv_dtype``.

    The cache holds keys as the prefix encoder leaves them (already position
    rotated), so it is used as given.
    """
    rng = np.random.default_rng(cfg.kv_seed if seed is None else seed)
    shape = (cfg.n_layers, cfg.prefix_len, cfg.n_kv_heads, cfg.head_dim)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    return store(k, cfg.kv_dtype), store(v, cfg.kv_dtype)


def make_prefix_embeddings(cfg, seed):
    """Prefix token embeddings [P][w] float32 N(0, 1) for the prefill (P = cfg.horizon rows)."""
    return np.random.default_rng(seed).standard_normal((cfg.horizon, cfg.width), dtype=np.float32)


def make_features(cfg, seed):
    """Image features [P][w] float32 N(0, 1) for the draft model (3 views x 256 tokens at the block's width)."""
    return np.random.default_rng(seed).standard_normal((cfg.prefix_len, cfg.width), dtype=np.float32)


def make_noise(cfg, seed=None, batch=None):
    """Initial noise [batch][H][A] float32; robot r draws from seed + r."""
    b = cfg.batch if batch is None else batch
    s0 = cfg.noise_seed if seed is None else seed
    return np.stack([
        np.random.default_rng(s0 + r).standard_normal((cfg.horizon, cfg.action_dim), dtype=np.float32)
        for r in range(b)
    ])


def make_draft(cfg, seed):
    """Smooth random-walk draft chunk [H][A] float32 with a +-1 gripper channel.

    Draw order from ``default_rng(seed)``: start row N(0, 0.5^2) over the
    non-gripper dims, increments N(0, 0.05^2) for rows 1..H-1, gripper sign
    (+1 / -1 with equal odds), and for odd seeds a switch row uniform in
    [1, H-1]. The walk is smoothed with a 3-tap moving average (edges
    replicated). Even seeds hold the gripper constant; odd seeds flip it once.
    """
    H, A = cfg.horizon, cfg.action_dim
    g = cfg.gripper_dim
    rng = np.random.default_rng(seed)
    cols = [c for c in range(A) if c != g]
    start = rng.standard_normal(len(cols)) * 0.5
    inc = rng.standard_normal((H - 1, len(cols))) * 0.05
    walk = np.vstack([start[None, :], start[None, :] + np.cumsum(inc, axis=0)])
    padded = np.vstack([walk[:1], walk, walk[-1:]])
    smooth = (padded[:-2] + padded[1:-1] + padded[2:]) / 3.0
    d = np.zeros((H, A), np.float64)
    d[:, cols] = smooth
    if g >= 0:
        sign = 1.0 if rng.random() < 0.5 else -1.0
        d[:, g] = sign
        if seed % 2 == 1:
            i_s = int(rng.integers(1, H))
            d[i_s:, g] = -sign
    return d.astype(np.float32)


def make_verify_case(cfg, seed):
    """(draft [H][A], noise [H][A], taus [n_tau]) for one verification seed; noise from 300 + seed."""
    draft = make_draft(cfg, seed)
    noise = np.random.default_rng(300 + seed).standard_normal((cfg.horizon, cfg.action_dim), dtype=np.float32)
    return draft, noise, np.asarray(VERIFY_TAUS, np.float32)
