"""Pins for the CPU oracle: each oracle function checked against something other
than itself (library routines, closed forms, invariants, brute force on tiny
inputs), so that a dropped term, a wrong sign or index, or a transposed
operand fails at least one test."""
import math

import numpy as np
import pytest
import scipy.special as sps
import torch

from oracle import ae_oracle as O
from workload import configs as C
from workload import gen as G


# ---------------------------------------------------------------- decoders

def test_bf16_decoder_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint32).astype(np.uint16)
    bits = np.concatenate([bits, np.array([0x0000, 0x8000, 0x3f80, 0xbf80, 0x7f7f, 0x0001], np.uint16)])
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = O.decode_bf16(bits)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (ref == got))


def test_e4m3_decoder_exhaustive_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.decode_e4m3(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    # OCP E4M3: largest finite 448, smallest subnormal 2^-9, NaN only at 0x7f / 0xff
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and np.sum(np.isnan(got)) == 2


def test_fp8_rows_roundtrip_within_half_ulp():
    rng = np.random.default_rng(2)
    w = rng.standard_normal((16, 64)).astype(np.float32) * 0.02
    codes, scale = G._to_fp8_rows(w)
    deq = O.decode(codes, "fp8", scale)
    # every row's max maps to +-448 exactly; relative error of E4M3 RNE is <= 2^-4
    assert np.allclose(np.abs(deq).max(axis=1), np.abs(w).max(axis=1), rtol=1e-6)
    big = np.abs(w) > scale[:, None] * 2.0 ** -6 * 8
    assert np.all(np.abs(deq - w)[big] <= np.abs(w)[big] * 2.0 ** -4 + 1e-12)


# An fp8-MLP config and its fp32 twin draw the same float32 weights (same seed, shapes and draw order;
# only the storage format differs), so the fp32 twin's tensors are the unquantised originals.
_FP8_CFG = C.TINY.with_(name="pin_fp8", n_layers=2, width=64, n_q_heads=2, n_kv_heads=1, head_dim=32, mlp_dim=128,
                        action_dim=8, horizon=6, prefix_len=10, weight_dtype="bf16", mlp_dtype="fp8",
                        kv_dtype="bf16")
_F32_TWIN = _FP8_CFG.with_(name="pin_f32", weight_dtype="f32", mlp_dtype="f32", kv_dtype="f32")


def test_dequantize_routes_mlp_through_e4m3_with_row_scales():
    """DM0.5 guide 6.3 (E4M3 MLP weights with scales): gate/up/down decode as E4M3 codes times one
    scale per output row, checked against torch's float8_e4m3fn decoder and against the unquantised
    draw within E4M3's half-ulp; every other linear decodes as weight_dtype (torch's bfloat16 view),
    and biases and gains stay as drawn."""
    W = G.make_weights(_FP8_CFG)
    Wd = O.dequantize_weights(_FP8_CFG, W)
    W32 = G.make_weights(_F32_TWIN)
    assert not any(n.endswith(".scale") for n in Wd)
    for l in range(_FP8_CFG.n_layers):
        for nm in ("wg", "wu", "wd"):
            key = f"layers.{l}.{nm}"
            codes, scale = W[key], W[key + ".scale"]
            assert codes.dtype == np.uint8 and scale.shape == (codes.shape[0],)
            ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy() * scale[:, None]
            assert np.array_equal(Wd[key], ref), key
            # against the float32 draw: relative error <= 2^-4 above the subnormal range, absolute
            # <= 2^-10 * scale below it (per row: a column scale or a bf16 decode of the codes fails)
            a = W32[key].astype(np.float64)
            bound = np.maximum(np.abs(a) * 2.0 ** -4, scale[:, None].astype(np.float64) * 2.0 ** -10) * (1 + 1e-6)
            assert np.all(np.abs(Wd[key] - a) <= bound), key
            # each row's largest magnitude lands on +-448 * scale
            assert np.allclose(np.abs(Wd[key]).max(axis=1), np.abs(a).max(axis=1), rtol=1e-6), key
        for nm in ("wq", "wk", "wv", "wo"):
            key = f"layers.{l}.{nm}"
            assert W[key].dtype == np.uint16, key
            ref = torch.from_numpy(W[key].view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
            assert np.array_equal(Wd[key], ref), key
            a = W32[key].astype(np.float64)
            assert np.all(np.abs(Wd[key] - a) <= np.abs(a) * 2.0 ** -8 * (1 + 1e-6)), key
        for nm in ("ln1", "ln2"):
            assert np.array_equal(Wd[f"layers.{l}.{nm}"], W[f"layers.{l}.{nm}"].astype(np.float64))
    for key in ("time_in_w", "time_out_w", "action_in_w", "action_out_w"):
        ref = torch.from_numpy(W[key].view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
        assert np.array_equal(Wd[key], ref), key
    for key in ("time_in_b", "time_out_b", "action_in_b", "action_out_b", "final_ln"):
        assert np.array_equal(Wd[key], W32[key].astype(np.float64)), key


def test_fp8_velocity_is_the_fp32_velocity_of_the_dequantised_weights():
    """The storage format enters the velocity only through dequantisation: the fp8 config's velocity
    equals the fp32 twin's velocity when the twin is fed the fp8 config's dequantised tensors, and
    differs from the twin's own (unquantised) velocity by about the E4M3 rounding."""
    W = G.make_weights(_FP8_CFG)
    Wd = O.dequantize_weights(_FP8_CFG, W)
    k, v = G.make_prefix_kv(_FP8_CFG, 100)
    kk, vv = O.decode_kv(_FP8_CFG, k, v)
    x = G.make_noise(_FP8_CFG, 200, 1)[0].astype(np.float64)
    got = O.velocity(_FP8_CFG, Wd, kk, vv, x, 0.3)
    twin = O.velocity(_F32_TWIN, dict(Wd), kk, vv, x, 0.3)
    assert np.array_equal(got, twin)
    own = O.velocity(_F32_TWIN, O.dequantize_weights(_F32_TWIN, G.make_weights(_F32_TWIN)), kk, vv, x, 0.3)
    rel = np.max(np.abs(got - own)) / np.sqrt(np.mean(own ** 2))
    assert 0 < rel < 6e-2, rel


# ---------------------------------------------------------------- elementwise

def test_gelu_tanh_against_erf_gelu():
    x = np.linspace(-6, 6, 2001)
    exact = 0.5 * x * (1.0 + sps.erf(x / math.sqrt(2.0)))
    assert np.max(np.abs(O.gelu_tanh(x) - exact)) < 5e-4
    assert O.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert abs(O.gelu_tanh(np.array([8.0]))[0] - 8.0) < 1e-9
    assert abs(O.gelu_tanh(np.array([-8.0]))[0]) < 1e-9


def test_silu_against_expit():
    x = np.linspace(-20, 20, 401)
    assert np.allclose(O.silu(x), x * sps.expit(x), rtol=1e-12, atol=1e-15)


def test_rmsnorm_output_rms_is_gain_and_scale_invariant():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 64)) * 3.0
    y = O.rmsnorm(x, np.full(64, 2.5), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 2.5)
    assert np.allclose(O.rmsnorm(7.0 * x, 1.0, 0.0), O.rmsnorm(x, 1.0, 0.0))
    # eps sits inside the root: a zero row stays zero, a tiny row is damped
    z = O.rmsnorm(np.zeros((1, 8)), 1.0, 1e-6)
    assert np.all(z == 0)


def test_linear_orientation():
    w = np.array([[1.0, 2.0, 3.0], [0.0, -1.0, 0.0]])  # [out=2][in=3]
    x = np.array([[1.0, 1.0, 1.0]])
    assert np.array_equal(O.linear(x, w, np.array([10.0, 20.0])), np.array([[16.0, 19.0]]))


# ---------------------------------------------------------------- time embedding

def test_sinusoid_special_values():
    w = 64
    half = w // 2
    phi0 = O.sinusoid(0.0, w)
    assert np.array_equal(phi0, np.concatenate([np.zeros(half), np.ones(half)]))
    phi1 = O.sinusoid(1.0, w)
    # slowest component has period 4: at t = 1 it is a quarter turn
    assert abs(phi1[half - 1] - 1.0) < 1e-12 and abs(phi1[w - 1]) < 1e-12
    # fastest component has period 4e-3: t = 1 is 250 full turns, t = 1e-3 a quarter turn
    assert abs(phi1[0]) < 1e-9 and abs(phi1[half] - 1.0) < 1e-9
    assert abs(O.sinusoid(1e-3, w)[0] - 1.0) < 1e-12
    t = 0.37
    p = O.sinusoid(t, w)
    assert np.allclose(p[:half] ** 2 + p[half:] ** 2, 1.0)
    # periods are geometric: log-frequencies equally spaced
    ang = np.arctan2(O.sinusoid(1e-4, w)[:half], O.sinusoid(1e-4, w)[half:])
    ratio = ang[:-1] / ang[1:]
    assert np.allclose(ratio, (4.0 / 4e-3) ** (1.0 / (half - 1)))


# ---------------------------------------------------------------- RoPE

def test_rope_closed_form_on_basis_vectors():
    dh, half, base = 16, 8, 10000.0
    for d in (0, 3, 7):
        e = np.zeros((1, 1, dh))
        e[0, 0, d] = 1.0
        pos = 5
        r = O.rope(e, np.array([pos]), base)[0, 0]
        theta = pos * base ** (-2.0 * d / dh)
        expect = np.zeros(dh)
        expect[d] = math.cos(theta)
        expect[d + half] = math.sin(theta)
        assert np.allclose(r, expect, atol=1e-15)


def test_rope_norm_and_relative_position():
    rng = np.random.default_rng(4)
    dh = 32
    q = rng.standard_normal((1, 1, dh))
    k = rng.standard_normal((1, 1, dh))
    for m in (0, 3, 50):
        assert np.isclose(np.linalg.norm(O.rope(q, np.array([m]), 10000.0)), np.linalg.norm(q))
    def dot(m, n):
        return float(np.sum(O.rope(q, np.array([m]), 10000.0) * O.rope(k, np.array([n]), 10000.0)))
    assert np.isclose(dot(10, 3), dot(817, 810))
    assert np.isclose(dot(0, 0), float(np.sum(q * k)))


# ---------------------------------------------------------------- attention

def _attention_bruteforce(q, k, v):
    """Scalar triple loop: out[r][h][:] = sum_j softmax_j(q.k_j / sqrt(dh)) v_j, kv head = h * n_kv // n_q."""
    n_rows, n_q, dh = q.shape
    n_keys, n_kv, _ = k.shape
    out = np.zeros_like(q)
    for r in range(n_rows):
        for h in range(n_q):
            g = (h * n_kv) // n_q
            scores = []
            for j in range(n_keys):
                s = 0.0
                for d in range(dh):
                    s += q[r, h, d] * k[j, g, d]
                scores.append(s / math.sqrt(dh))
            mx = max(scores)
            ws = [math.exp(s - mx) for s in scores]
            tot = sum(ws)
            for d in range(dh):
                out[r, h, d] = sum(ws[j] * v[j, g, d] for j in range(n_keys)) / tot
    return out


def test_attention_bruteforce_gqa():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((3, 4, 8))
    k = rng.standard_normal((7, 2, 8))
    v = rng.standard_normal((7, 2, 8))
    assert np.allclose(O.attention(q, k, v), _attention_bruteforce(q, k, v), atol=1e-12)


def test_attention_gqa_equals_mha_with_repeated_kv_and_shift_invariance():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((5, 8, 16))
    k = rng.standard_normal((11, 1, 16))
    v = rng.standard_normal((11, 1, 16))
    a = O.attention(q, k, v)
    assert np.allclose(a, O.attention(q, np.repeat(k, 8, axis=1), np.repeat(v, 8, axis=1)))
    c = rng.standard_normal(16)
    assert np.allclose(a, O.attention(q, k + c, v))          # constant key shift: softmax invariant
    z = O.attention(np.zeros_like(q), k, v)                   # zero query: uniform weights
    assert np.allclose(z, np.broadcast_to(v.mean(axis=0), z.shape))


# ---------------------------------------------------------------- Euler integration

@pytest.mark.parametrize("steps", [1, 2, 4, 10])
def test_euler_recovers_target_under_exact_linear_field(steps):
    rng = np.random.default_rng(7)
    a = rng.standard_normal((8, 8))
    eps = rng.standard_normal((8, 8))
    seen = []

    def exact(x, t):
        assert t < 1.0
        seen.append(t)
        return (a - x) / (1.0 - t)

    x = O.euler_integrate(eps, steps, exact)
    assert np.allclose(x, a, atol=1e-12)
    assert np.allclose(seen, np.arange(steps) / steps)


def test_interpolation_endpoints_and_exact_velocity():
    rng = np.random.default_rng(8)
    d = rng.standard_normal((6, 4))
    e = rng.standard_normal((6, 4))
    x = O.interpolate(d, e, [0.0, 1.0, 0.25])
    assert np.allclose(x[0], e) and np.allclose(x[1], d)
    # on the linear path the exact velocity is d - eps and the endpoint rebuild returns d
    a_hat = x[2] + (1 - 0.25) * (d - e)
    assert np.allclose(a_hat, d)


# ---------------------------------------------------------------- verification

def _exact_velocity(a, x_tau, taus):
    return np.stack([(a - x_tau[j]) / (1.0 - taus[j]) for j in range(len(taus))])


def test_verify_full_accept_when_draft_is_exact_target():
    rng = np.random.default_rng(9)
    H, A = 50, 32
    a = rng.standard_normal((H, A))
    a[:, 31] = 1.0
    eps = rng.standard_normal((H, A))
    taus = np.array([0.2, 0.4, 0.6, 0.8])
    x = O.interpolate(a, eps, taus)
    acc, sw, D = O.accept_from_velocity(a, x, _exact_velocity(a, x, taus), taus, 0.05, 31)
    assert acc == H and sw == 0 and np.max(D) < 1e-12
    acc0, _, _ = O.accept_from_velocity(a, x, _exact_velocity(a, x, taus), taus, 0.0, 31)
    assert acc0 == 0  # strict < delta


@pytest.mark.parametrize("k", [0, 1, 17, 49])
def test_verify_prefix_length_closed_form(k):
    rng = np.random.default_rng(10 + k)
    H, A = 50, 32
    a = rng.standard_normal((H, A))
    a[:, 31] = -1.0
    d = a.copy()
    d[k:, 0] += 0.1 + rng.random(H - k)  # distance >= 0.1 = 2 delta from row k on
    eps = rng.standard_normal((H, A))
    taus = np.array([0.2, 0.4, 0.6, 0.8])
    x = O.interpolate(d, eps, taus)
    acc, sw, D = O.accept_from_velocity(d, x, _exact_velocity(a, x, taus), taus, 0.05, 31)
    assert acc == k and sw == 0
    # the exact field makes every rebuilt endpoint a, so D is tau-independent ||a_i - d_i||
    assert np.allclose(D, np.linalg.norm(a - d, axis=1)[None, :].repeat(4, axis=0))


def test_verify_gripper_switch_forces_zero():
    rng = np.random.default_rng(11)
    H, A = 50, 32
    a = rng.standard_normal((H, A))
    a[:, 31] = 1.0
    a[30:, 31] = -1.0
    eps = rng.standard_normal((H, A))
    taus = np.array([0.2, 0.4, 0.6, 0.8])
    x = O.interpolate(a, eps, taus)
    acc, sw, _ = O.accept_from_velocity(a, x, _exact_velocity(a, x, taus), taus, 0.05, 31)
    assert sw == 1 and acc == 0
    assert O.gripper_switch(a, -1) == 0


def test_draft_generator_switches_on_odd_seeds_only():
    cfg = C.PI0_VERIFY
    for s in range(16):
        d = G.make_draft(cfg, s)
        assert set(np.unique(d[:, 31])) <= {-1.0, 1.0}
        assert O.gripper_switch(d, 31) == (s % 2)


# ---------------------------------------------------------------- whole-network composition

def _tiny_cfg(**kw):
    base = C.TINY.with_(n_layers=2, width=32, n_q_heads=4, n_kv_heads=1, head_dim=8, mlp_dim=64,
                        action_dim=4, horizon=5, prefix_len=6)
    return base.with_(**kw)


def _tiny_inputs(cfg, seed=0):
    W = G.make_weights(cfg, seed)
    Wd = O.dequantize_weights(cfg, W)
    k, v = G.make_prefix_kv(cfg, 100 + seed)
    kk, vv = O.decode_kv(cfg, k, v)
    noise = G.make_noise(cfg, 200 + seed, 1)[0].astype(np.float64)
    return Wd, kk, vv, noise


def test_zero_out_proj_gives_constant_velocity():
    cfg = _tiny_cfg()
    Wd, kk, vv, noise = _tiny_inputs(cfg)
    Wd["action_out_w"][:] = 0.0
    c = np.array([0.5, -1.0, 2.0, 0.25])
    Wd["action_out_b"] = c
    for steps in (1, 3, 10):
        x = O.denoise(cfg, Wd, kk, vv, noise, steps)
        assert np.allclose(x, noise + c, atol=1e-12)


def test_identity_layers_when_output_projections_are_zero():
    cfg = _tiny_cfg()
    Wd, kk, vv, noise = _tiny_inputs(cfg)
    for l in range(cfg.n_layers):
        Wd[f"layers.{l}.wo"][:] = 0.0
        Wd[f"layers.{l}.wd"][:] = 0.0
    v = O.velocity(cfg, Wd, kk, vv, noise, 0.3)
    h0 = O.linear(noise, Wd["action_in_w"], Wd["action_in_b"]) + O.time_embedding(Wd, 0.3, cfg.width)
    expect = O.linear(O.rmsnorm(h0, Wd["final_ln"], cfg.rms_eps), Wd["action_out_w"], Wd["action_out_b"])
    assert np.allclose(v, expect)
    kk2 = np.random.default_rng(1).standard_normal(kk.shape)
    assert np.allclose(O.velocity(cfg, Wd, kk2, vv, noise, 0.3), expect)


def test_attention_uses_prefix_and_suffix_keys_of_its_own_layer():
    """q = 0 and suffix v = 0 make every head output mean(prefix V) * P / (P + H)."""
    cfg = _tiny_cfg(n_layers=2)
    Wd, kk, vv, noise = _tiny_inputs(cfg)
    for l in range(cfg.n_layers):
        Wd[f"layers.{l}.wq"][:] = 0.0
        Wd[f"layers.{l}.wv"][:] = 0.0
        Wd[f"layers.{l}.wd"][:] = 0.0
    P, H = cfg.prefix_len, cfg.horizon
    h = O.linear(noise, Wd["action_in_w"], Wd["action_in_b"]) + O.time_embedding(Wd, 0.6, cfg.width)
    for l in range(cfg.n_layers):
        head_out = vv[l, :, 0, :].sum(axis=0) / (P + H)                  # [dh], single kv head
        o = np.tile(head_out, cfg.n_q_heads)                              # every query head, same kv head
        h = h + O.linear(o[None, :], Wd[f"layers.{l}.wo"])
    expect = O.linear(O.rmsnorm(h, Wd["final_ln"], cfg.rms_eps), Wd["action_out_w"], Wd["action_out_b"])
    assert np.allclose(O.velocity(cfg, Wd, kk, vv, noise, 0.6), expect)


def test_batched_robot_equals_robot_alone_and_verify_rows_equal_velocity():
    cfg = _tiny_cfg(gripper_dim=3, max_batch=2, batch=2)
    W = G.make_weights(cfg, 0)
    Wd = O.dequantize_weights(cfg, W)
    kvs = [O.decode_kv(cfg, *G.make_prefix_kv(cfg, 100 + r)) for r in range(2)]
    noise = G.make_noise(cfg, 200, 2).astype(np.float64)
    xb = O.denoise_batch(cfg, Wd, kvs, noise, 3)
    assert np.array_equal(xb[1], O.denoise(cfg, Wd, kvs[1][0], kvs[1][1], noise[1], 3))
    d = noise[0] * 0.1
    taus = np.array([0.2, 0.6])
    acc, sw, D = O.verify(cfg, Wd, kvs[0][0], kvs[0][1], d, noise[1], taus, 10.0)
    x1 = O.interpolate(d, noise[1], taus)[1]
    a1 = x1 + 0.4 * O.velocity(cfg, Wd, kvs[0][0], kvs[0][1], x1, 0.6)
    assert np.allclose(D[1], np.linalg.norm(a1 - d, axis=1))


def test_rmsnorm_eps_inside_root():
    c = 1e-4
    y = O.rmsnorm(np.full((1, 4), c), 1.0, 1e-6)
    assert np.allclose(y, c / math.sqrt(c * c + 1e-6))


def test_time_mlp_composition_order():
    """time_in -> SiLU -> time_out: with W_in = 0 the hidden layer is silu(b_in) for every t."""
    w = 8
    rng = np.random.default_rng(12)
    Wd = {"time_in_w": np.zeros((w, w)), "time_in_b": rng.standard_normal(w),
          "time_out_w": rng.standard_normal((w, w)), "time_out_b": rng.standard_normal(w)}
    expect = Wd["time_out_w"] @ (Wd["time_in_b"] * sps.expit(Wd["time_in_b"])) + Wd["time_out_b"]
    for t in (0.0, 0.5):
        assert np.allclose(O.time_embedding(Wd, t, w), expect)
    # with W_out = I and b = 0 the output is silu(W_in phi(t)): phi(0) = [0.., 1..]
    Wd = {"time_in_w": np.eye(w), "time_in_b": np.zeros(w), "time_out_w": np.eye(w), "time_out_b": np.zeros(w)}
    phi = np.concatenate([np.zeros(w // 2), np.ones(w // 2)])
    assert np.allclose(O.time_embedding(Wd, 0.0, w), phi * sps.expit(phi))


def _one_layer_weights(w, dh, nq, F):
    z = lambda *s: np.zeros(s)
    return {"layers.0.ln1": np.ones(w), "layers.0.ln2": np.ones(w),
            "layers.0.wq": z(nq * dh, w), "layers.0.wk": z(dh, w), "layers.0.wv": z(dh, w),
            "layers.0.wo": z(w, nq * dh), "layers.0.wg": z(F, w), "layers.0.wu": z(F, w), "layers.0.wd": z(w, F)}


def test_geglu_gate_is_the_gelu_branch():
    """h += W_d (gelu(W_g n) * (W_u n)): gate row reads n[0], up row reads n[1]."""
    cfg = _tiny_cfg(n_layers=1, width=4, n_q_heads=1, head_dim=4, mlp_dim=2, prefix_len=2, horizon=1)
    Wd = _one_layer_weights(4, 4, 1, 2)
    Wd["layers.0.wg"][0, 0] = 3.0
    Wd["layers.0.wu"][0, 1] = 2.0
    Wd["layers.0.wd"][2, 0] = 1.0
    h0 = np.array([[1.0, -0.5, 0.25, 2.0]])
    n2 = h0 / np.sqrt(np.mean(h0 ** 2) + cfg.rms_eps)
    kp = np.zeros((2, 1, 4))
    h1 = O.decoder_layer(cfg, Wd, 0, h0, kp, kp)
    g = 3.0 * n2[0, 0]
    erf_gelu = 0.5 * g * (1 + sps.erf(g / math.sqrt(2)))
    assert np.allclose(h1[0, [0, 1, 3]], h0[0, [0, 1, 3]])
    assert abs(h1[0, 2] - (h0[0, 2] + erf_gelu * 2.0 * n2[0, 1])) < 1e-3


@pytest.mark.parametrize("P", [1, 3])
def test_suffix_rope_position_is_prefix_len_plus_row(P):
    """One suffix row at position P attends a prefix key (0, kappa): its score is n0 kappa sin(P) / sqrt(2)."""
    cfg = _tiny_cfg(n_layers=1, width=2, n_q_heads=1, head_dim=2, mlp_dim=2, prefix_len=P, horizon=1, rope_base=10000.0)
    Wd = _one_layer_weights(2, 2, 1, 2)
    Wd["layers.0.wq"][0, 0] = 1.0          # q = (n0, 0); suffix k = v = 0
    Wd["layers.0.wo"][:] = np.eye(2)
    kappa = 3.0
    kp = np.zeros((P, 1, 2))
    kp[:, 0, 1] = kappa
    vp = np.zeros((P, 1, 2))
    vp[:, 0, 0], vp[:, 0, 1] = 1.0, 2.0
    h0 = np.array([[0.8, -0.3]])
    n0 = (h0 / np.sqrt(np.mean(h0 ** 2) + cfg.rms_eps))[0, 0]
    s = n0 * kappa * math.sin(P) / math.sqrt(2)
    w_pre = P * math.exp(s) / (P * math.exp(s) + 1.0)    # P equal prefix keys, one zero suffix key
    expect = h0 + w_pre * np.array([[1.0, 2.0]])             # every prefix value row is (1, 2)
    got = O.decoder_layer(cfg, Wd, 0, h0, kp, vp)
    assert np.allclose(got, expect)


def test_dual_path_round_branches_under_a_constant_velocity_field():
    """With action_out_w = 0 the expert's velocity is its bias c everywhere. Then a rebuilt endpoint is
    x_tau + (1 - tau) c = d + (1 - tau)(eps + c - d): noise eps = d - c rebuilds the draft exactly (every
    row accepted, fast path, the draft returned), any other noise far from it rejects row 0 (full path:
    Euler with constant velocity gives noise_full + c), and a gripper switch forces the full path."""
    cfg = _tiny_cfg(gripper_dim=3)
    Wd, kk, vv, noise_full = _tiny_inputs(cfg)
    Wd["action_out_w"][:] = 0.0
    c = np.array([0.5, -1.0, 2.0, 0.25])
    Wd["action_out_b"] = c
    taus = np.array([0.2, 0.5, 0.8])
    rng = np.random.default_rng(4)
    d = rng.standard_normal((cfg.horizon, cfg.action_dim))
    d[:, 3] = 1.0                                   # gripper open throughout
    act, acc, sw, full = O.dual_path_round(cfg, Wd, kk, vv, d, d - c, taus, 0.05, noise_full, 3)
    assert (acc, sw, full) == (cfg.horizon, 0, 0) and np.array_equal(act, d)
    far = d - c + 1.0                               # every rebuilt endpoint is (1 - tau) * 2 away from the draft
    act, acc, sw, full = O.dual_path_round(cfg, Wd, kk, vv, d, far, taus, 0.05, noise_full, 3)
    assert (acc, sw, full) == (0, 0, 1) and np.allclose(act, noise_full + c, atol=1e-12)
    ds = d.copy()
    ds[2:, 3] = -1.0                                # one switch: the full path although every row matches
    act, acc, sw, full = O.dual_path_round(cfg, Wd, kk, vv, ds, ds - c, taus, 0.05, noise_full, 3)
    assert (acc, sw, full) == (0, 1, 1) and np.allclose(act, noise_full + c, atol=1e-12)


# ---------------------------------------------------------------- time-modulated expert, QK-norm

def _mod_cfg(**kw):
    return _tiny_cfg(time_mode=1, **kw)


def test_modulated_expert_with_identity_modulation_is_the_additive_one_without_temb():
    """scale = shift = 0 and gate = 1 (zero modulation weights, bias thirds 0 / 0 / 1) leave every norm and
    residual as in the plain block, so the velocity equals the additive expert's with temb = 0."""
    cfg = _mod_cfg()
    Wd, kk, vv, x = _tiny_inputs(cfg)
    w = cfg.width
    for l in range(cfg.n_layers):
        Wd[f"layers.{l}.w_mod"][:] = 0.0
        b = np.zeros(6 * w)
        b[2 * w:3 * w] = b[5 * w:] = 1.0
        Wd[f"layers.{l}.b_mod"] = b
    Wd["final_mod_w"][:] = 0.0
    Wd["final_mod_b"][:] = 0.0
    base = cfg.with_(time_mode=0)
    Wb = {k: v for k, v in Wd.items() if "mod" not in k}
    Wb["time_out_w"] = np.zeros_like(Wd["time_out_w"])
    Wb["time_out_b"] = np.zeros_like(Wd["time_out_b"])
    for t in (0.0, 0.3, 0.9):
        assert np.allclose(O.velocity(cfg, Wd, kk, vv, x, t), O.velocity(base, Wb, kk, vv, x, t), atol=1e-12)


def test_modulation_gates_zero_make_every_layer_the_identity():
    cfg = _mod_cfg()
    Wd, kk, vv, x = _tiny_inputs(cfg)
    for l in range(cfg.n_layers):
        Wd[f"layers.{l}.w_mod"][:] = 0.0
        Wd[f"layers.{l}.b_mod"][:] = 0.0
    h0 = x @ Wd["action_in_w"].T + Wd["action_in_b"]
    temb = O.time_embedding(Wd, 0.4, cfg.width)
    fm = Wd["final_mod_w"] @ temb + Wd["final_mod_b"]
    scale, shift = fm[:cfg.width], fm[cfg.width:]
    n = h0 / np.sqrt(np.mean(h0 ** 2, axis=-1, keepdims=True) + cfg.rms_eps) * Wd["final_ln"]
    want = (n * (1.0 + scale) + shift) @ Wd["action_out_w"].T + Wd["action_out_b"]
    assert np.allclose(O.velocity(cfg, Wd, kk, vv, x, 0.4), want, atol=1e-12)


def test_modulation_scale_is_a_gain_on_the_norm():
    """A constant scale s on the attention norm equals the plain norm with gain ln1 * (1 + s)."""
    cfg = _mod_cfg(n_layers=1)
    Wd, kk, vv, x = _tiny_inputs(cfg)
    w = cfg.width
    s = np.linspace(-0.5, 0.7, w)
    Wd["layers.0.w_mod"][:] = 0.0
    b = np.zeros(6 * w)
    b[:w] = s
    b[2 * w:3 * w] = b[5 * w:] = 1.0
    Wd["layers.0.b_mod"] = b
    Wd["final_mod_w"][:] = 0.0
    Wd["final_mod_b"][:] = 0.0
    W2 = dict(Wd)
    W2["layers.0.ln1"] = Wd["layers.0.ln1"] * (1.0 + s)
    W2["layers.0.b_mod"] = b.copy()
    W2["layers.0.b_mod"][:w] = 0.0
    assert np.allclose(O.velocity(cfg, Wd, kk, vv, x, 0.2), O.velocity(cfg, W2, kk, vv, x, 0.2), atol=1e-12)


def test_modulation_shift_enters_after_the_norm():
    """With the MLP norm's gain 0 and scale 0, the MLP input is the shift alone: the MLP adds the
    constant gate2 * Wd (gelu(Wg b2) * (Wu b2)) to every row, whatever h is."""
    cfg = _mod_cfg(n_layers=1)
    Wd, kk, vv, x = _tiny_inputs(cfg)
    w = cfg.width
    rng = np.random.default_rng(3)
    b2 = rng.standard_normal(w)
    g2 = rng.standard_normal(w)
    Wd["layers.0.w_mod"][:] = 0.0
    b = np.zeros(6 * w)
    b[2 * w:3 * w] = 1.0
    b[4 * w:5 * w] = b2
    b[5 * w:] = g2
    Wd["layers.0.b_mod"] = b
    Wd["layers.0.ln2"] = np.zeros(w)
    const = g2 * (Wd["layers.0.wd"] @ (O.gelu_tanh(Wd["layers.0.wg"] @ b2) * (Wd["layers.0.wu"] @ b2)))
    W0 = dict(Wd)
    W0["layers.0.b_mod"] = b.copy()
    W0["layers.0.b_mod"][5 * w:] = 0.0   # no MLP branch
    h_mlp = O.decoder_layer(cfg, Wd, 0, x @ Wd["action_in_w"].T, kk[0], vv[0], np.split(b, 6))
    h_none = O.decoder_layer(cfg, W0, 0, x @ Wd["action_in_w"].T, kk[0], vv[0], np.split(W0["layers.0.b_mod"], 6))
    assert np.allclose(h_mlp - h_none, np.broadcast_to(const, h_mlp.shape), atol=1e-12)


@pytest.mark.parametrize("which", ["wq", "wk"])
def test_qk_norm_is_per_head_and_scale_free(which):
    """QK-norm normalises each head over head_dim: scaling the rows of one head of wq (or of the kv head of
    wk) by c > 0 leaves the velocity unchanged, and without QK-norm it does not."""
    cfg = _tiny_cfg(qk_norm=1, n_kv_heads=2, rms_eps=1e-30)  # eps would break exact scale invariance
    Wd, kk, vv, x = _tiny_inputs(cfg)
    dh = cfg.head_dim
    W2 = dict(Wd)
    W2[f"layers.0.{which}"] = Wd[f"layers.0.{which}"].copy()
    W2[f"layers.0.{which}"][dh:2 * dh] *= 3.7   # head 1 only
    v1, v2 = O.velocity(cfg, Wd, kk, vv, x, 0.5), O.velocity(cfg, W2, kk, vv, x, 0.5)
    assert np.allclose(v1, v2, atol=1e-10)
    off = cfg.with_(qk_norm=0)
    assert not np.allclose(O.velocity(off, Wd, kk, vv, x, 0.5), O.velocity(off, W2, kk, vv, x, 0.5), atol=1e-6)


# ---------------------------------------------------------------- draft model

def _draft_cfg():
    return C.DRAFT.with_(width=64, n_q_heads=4, n_kv_heads=1, head_dim=16, mlp_dim=128, horizon=6, prefix_len=9,
                         action_dim=4)


def test_draft_equals_one_block_over_features_and_queries():
    """The draft is one block over the whole sequence [features ; queries]: running that block on all P + H
    tokens (every token attends to every token, RoPE at 0..P+H-1) and reading the query rows gives the same
    chunk as the cached-feature form (features as prefix K/V, queries as suffix rows)."""
    cfg = _draft_cfg()
    Wd = O.dequantize_weights(cfg, G.make_weights(cfg, 5))
    feats = G.make_features(cfg, 6).astype(np.float64)
    P, H, nq, nkv, dh = cfg.prefix_len, cfg.horizon, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    seq = np.concatenate([feats, Wd["queries"]], axis=0)
    p = "layers.0."
    n = O.rmsnorm(seq, Wd[p + "ln1"], cfg.rms_eps)
    pos = np.arange(P + H)
    q = O.rope((n @ Wd[p + "wq"].T).reshape(P + H, nq, dh), pos, cfg.rope_base)
    k = O.rope((n @ Wd[p + "wk"].T).reshape(P + H, nkv, dh), pos, cfg.rope_base)
    v = (n @ Wd[p + "wv"].T).reshape(P + H, nkv, dh)
    # attention through torch's scaled-dot-product routine, kv head repeated per query head
    qt = torch.from_numpy(q.transpose(1, 0, 2))
    kt = torch.from_numpy(np.repeat(k, nq // nkv, axis=1).transpose(1, 0, 2))
    vt = torch.from_numpy(np.repeat(v, nq // nkv, axis=1).transpose(1, 0, 2))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).numpy().transpose(1, 0, 2).reshape(P + H, nq * dh)
    hs = seq + o @ Wd[p + "wo"].T
    n2 = O.rmsnorm(hs, Wd[p + "ln2"], cfg.rms_eps)
    hs = hs + (O.gelu_tanh(n2 @ Wd[p + "wg"].T) * (n2 @ Wd[p + "wu"].T)) @ Wd[p + "wd"].T
    want = O.rmsnorm(hs[P:], Wd["final_ln"], cfg.rms_eps) @ Wd["action_out_w"].T + Wd["action_out_b"]
    assert np.allclose(O.draft_chunk(cfg, Wd, feats), want, atol=1e-10)


def test_draft_head_zero_gives_bias_and_features_matter():
    cfg = _draft_cfg()
    Wd = O.dequantize_weights(cfg, G.make_weights(cfg, 5))
    f1, f2 = G.make_features(cfg, 6), G.make_features(cfg, 7)
    assert not np.allclose(O.draft_chunk(cfg, Wd, f1), O.draft_chunk(cfg, Wd, f2))
    Wd["action_out_w"][:] = 0.0
    assert np.allclose(O.draft_chunk(cfg, Wd, f1), np.broadcast_to(Wd["action_out_b"], (cfg.horizon, cfg.action_dim)))


# ---------------------------------------------------------------- prefix prefill

def _prefill_cfg(**kw):
    base = dict(n_layers=2, width=64, n_q_heads=4, n_kv_heads=2, head_dim=16, mlp_dim=128, horizon=7,
                mlp_dtype="f32", weight_dtype="f32", kv_dtype="f32")
    base.update(kw)
    return C.PREFILL.with_(**base)


def test_prefill_attention_is_unmasked():
    """Every prefix token attends to every prefix token: changing the last token's embedding changes the
    first token's layer-1 K and V (a causal mask would not), while layer 0's K and V of the first token,
    which come from its own embedding only, stay as they were."""
    cfg = _prefill_cfg()
    Wd = O.dequantize_weights(cfg, G.make_weights(cfg, 3))
    emb = G.make_prefix_embeddings(cfg, 4).astype(np.float64)
    e2 = emb.copy()
    e2[-1] += 1.0
    k, v = O.prefill_kv(cfg, Wd, emb)
    k2, v2 = O.prefill_kv(cfg, Wd, e2)
    assert np.allclose(k2[0, 0], k[0, 0], atol=1e-14) and np.allclose(v2[0, 0], v[0, 0], atol=1e-14)
    assert not np.allclose(k2[1, 0], k[1, 0], atol=1e-6) and not np.allclose(v2[1, 0], v[1, 0], atol=1e-6)


def test_prefill_first_layer_kv_and_single_token_closed_form():
    """Layer 0's K/V come from the embeddings alone (the block's norm, projections, K rotated at 0..P-1),
    and with one token the attention returns that token's V, so layer 1's input is closed form."""
    cfg = _prefill_cfg(horizon=1)
    Wd = O.dequantize_weights(cfg, G.make_weights(cfg, 3))
    e = G.make_prefix_embeddings(cfg, 4).astype(np.float64)
    k, v = O.prefill_kv(cfg, Wd, e)
    n = e / np.sqrt(np.mean(e ** 2) + cfg.rms_eps) * Wd["layers.0.ln1"]
    assert np.allclose(k[0].reshape(1, -1), n @ Wd["layers.0.wk"].T, atol=1e-12)  # position 0: no rotation
    assert np.allclose(v[0].reshape(1, -1), n @ Wd["layers.0.wv"].T, atol=1e-12)
    vh = np.repeat((n @ Wd["layers.0.wv"].T).reshape(cfg.n_kv_heads, -1), cfg.n_q_heads // cfg.n_kv_heads, axis=0)
    h1 = e + vh.reshape(1, -1) @ Wd["layers.0.wo"].T
    n2 = h1 / np.sqrt(np.mean(h1 ** 2) + cfg.rms_eps) * Wd["layers.0.ln2"]
    h1 = h1 + (O.gelu_tanh(n2 @ Wd["layers.0.wg"].T) * (n2 @ Wd["layers.0.wu"].T)) @ Wd["layers.0.wd"].T
    n1 = h1 / np.sqrt(np.mean(h1 ** 2) + cfg.rms_eps) * Wd["layers.1.ln1"]
    assert np.allclose(v[1].reshape(1, -1), n1 @ Wd["layers.1.wv"].T, atol=1e-12)
