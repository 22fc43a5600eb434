"""GPU path (libae.so through the C-ABI) against the CPU oracle, element by element.

Floating-point chunks must satisfy max|gpu - oracle| <= tol * RMS(oracle):
tol = 1e-4 (fp32), 2e-2 (bf16 weights, fp32 accumulate), 6e-2 (fp8 E4M3 MLP).
Integers (accepted prefix length, gripper-switch flag) must match exactly.
"""
import numpy as np
import pytest

from flow_matching_action_euler_amd import ActionExpert, AEError
from oracle import ae_oracle as O
from workload import configs as C
from workload import gen as G

from helpers import SMALL_BF16, SMALL_F32, SMALL_FP8, Case, rel_err, tol_for

pytestmark = pytest.mark.gpu


def _expert(case, slots=None):
    ex = ActionExpert(case.cfg, case.W)
    for r in range(case.cfg.max_batch if slots is None else slots):
        ex.load_prefix_kv(r, *case.kv[r])
    return ex


# ------------------------------------------------------------------ small shapes, several tiles, ragged tails

@pytest.mark.parametrize("cfg", [C.TINY, SMALL_F32, SMALL_BF16, SMALL_FP8], ids=lambda c: c.name)
def test_denoise_small_matches_oracle(cfg):
    case = Case(cfg)
    ex = _expert(case)
    B = cfg.max_batch
    noise = case.noise(B)
    for steps in (1, cfg.steps):
        got = ex.denoise(noise, steps)
        ref = case.oracle_denoise(noise, steps)
        err = rel_err(got, ref)
        print(f"{cfg.name} B={B} steps={steps} rel_err={err:.3e}")
        assert err <= tol_for(cfg), err
    ex.close()


@pytest.mark.parametrize("cfg", [SMALL_F32, SMALL_BF16, SMALL_FP8], ids=lambda c: c.name)
def test_verify_small_matches_oracle(cfg):
    case = Case(cfg)
    ex = _expert(case)
    for seed in range(4):
        draft = G.make_draft(cfg, seed)
        noise = case.noise(1, 300 + seed)[0]
        taus = np.array([0.2, 0.5, 0.8], np.float32)
        acc, sw, D = ex.verify(1, draft, noise, taus, 0.05)
        acc_o, sw_o, D_o = case.oracle_verify(1, draft, noise, taus, 0.05)
        assert sw == sw_o == seed % 2
        assert acc == acc_o
        assert rel_err(D, D_o) <= tol_for(cfg)
    ex.close()


def test_batched_robot_equals_robot_alone():
    case = Case(SMALL_BF16)
    ex = _expert(case)
    noise = case.noise(3)
    xb = ex.denoise(noise, 3)
    # robot 0 alone shares slot 0 and its noise
    x0 = ex.denoise(noise[:1], 3)
    assert rel_err(x0[0], xb[0]) <= 1e-3
    # repeated calls are bitwise reproducible (no float atomics anywhere)
    assert np.array_equal(ex.denoise(noise, 3), xb)
    ex.close()


def test_exchange_paths_agree(monkeypatch):
    """Split partials meet three ways: polled inside the launch (default), through arrival
    tickets (GEMM split-K, AE_EXCH_POLL=0) and in a merge launch (attention,
    AE_ATTN_CORESIDENT=0). A 1,100-token prefix gives the attention 5 key splits (2 without
    co-residency) and the down projection 2 k-splits. Every path matches the oracle; the GEMM
    paths add the same partials in the same order (bitwise equal), the attention paths split
    the keys differently (bf16-level agreement); per-kernel timing, whose
    graphs of one kernel alone leave partials unconsumed, leaves the next result unchanged."""
    cfg = SMALL_BF16.with_(name="small_bf16_long_prefix", prefix_len=1100)
    case = Case(cfg)
    noise = case.noise(cfg.max_batch)
    ref = case.oracle_denoise(noise, 3)
    outs = []
    for env in ({}, {"AE_EXCH_POLL": "0"}, {"AE_ATTN_CORESIDENT": "0"}):
        with monkeypatch.context() as m:
            for k, v in env.items():
                m.setenv(k, v)
            ex = _expert(case)
        got = ex.denoise(noise, 3)
        err = rel_err(got, ref)
        print(f"{env or 'default'} rel_err={err:.3e}")
        assert err <= tol_for(cfg), (env, err)
        for mode in (0, 2):  # isolated, then in place
            ex.kernel_times(mode, cfg.max_batch, 3, 1)
            assert np.array_equal(ex.denoise(noise, 3), got), (env, mode)
        outs.append(got)
        ex.close()
    assert np.array_equal(outs[0], outs[1])
    # 5 vs 2 key splits round the bf16 attention output differently: bf16-level agreement
    assert rel_err(outs[2], outs[0]) <= tol_for(cfg)


def test_zero_output_projection_gives_constant_velocity():
    """W_out = 0, b_out = c: every Euler step adds dt * c, so x_N = x_0 + c for any N."""
    cfg = SMALL_BF16
    case = Case(cfg)
    W = dict(case.W)
    W["action_out_w"] = np.zeros_like(W["action_out_w"])
    c = np.linspace(-1.0, 1.0, cfg.action_dim).astype(np.float32)
    W["action_out_b"] = c
    ex = ActionExpert(cfg, W)
    for r in range(cfg.max_batch):
        ex.load_prefix_kv(r, *case.kv[r])
    noise = case.noise(2)
    for steps in (1, 4, 10):
        x = ex.denoise(noise, steps)
        assert np.allclose(x, noise + c[None, None, :], atol=2e-6), steps
    ex.close()


def test_verify_closed_form_exact_endpoint():
    """v = c everywhere (W_out = 0): with noise = d0 - c the rebuilt endpoints equal d0,
    so a draft d0 + p (p = 0 before row k, |p| = 1 from row k) has D[j,i] = (1 - tau_j)|p_i|
    and the accepted length is exactly k; a gripper switch forces 0."""
    cfg = SMALL_BF16
    case = Case(cfg)
    W = dict(case.W)
    W["action_out_w"] = np.zeros_like(W["action_out_w"])
    c = np.linspace(-0.5, 0.5, cfg.action_dim).astype(np.float32)
    W["action_out_b"] = c
    ex = ActionExpert(cfg, W)
    ex.load_prefix_kv(0, *case.kv[0])
    H, A = cfg.horizon, cfg.action_dim
    rng = np.random.default_rng(0)
    d0 = rng.standard_normal((H, A)).astype(np.float32)
    d0[:, cfg.gripper_dim] = 1.0
    noise = (d0 - c[None, :]).astype(np.float32)
    taus = np.array([0.2, 0.5, 0.8], np.float32)
    for k in (0, 1, 7, H):
        d = d0.copy()
        d[k:, 0] += 1.0
        acc, sw, D = ex.verify(0, d, noise, taus, 0.05)
        assert (acc, sw) == (k, 0)
        expect = (1.0 - taus[:, None]) * np.where(np.arange(H) >= k, 1.0, 0.0)[None, :]
        assert np.allclose(D, expect, atol=1e-5)
    d = d0.copy()
    d[5:, cfg.gripper_dim] = -1.0
    noise_g = (d - c[None, :]).astype(np.float32)
    acc, sw, D = ex.verify(0, d, noise_g, taus, 0.05)
    assert (acc, sw) == (0, 1) and np.max(D) < 1e-5
    ex.close()


def test_error_codes():
    cfg = SMALL_BF16
    case = Case(cfg)
    ex = ActionExpert(cfg, case.W)
    noise = case.noise(1)
    with pytest.raises(AEError) as e:
        ex.denoise(noise, 3)  # slot 0 not loaded
    assert e.value.code == -3
    ex.load_prefix_kv(0, *case.kv[0])
    with pytest.raises(AEError) as e:
        ex.denoise(np.zeros((4, cfg.horizon, cfg.action_dim), np.float32), 3)  # batch > max_batch
    assert e.value.code == -1
    with pytest.raises(AEError) as e:
        ex.verify(0, noise[0], noise[0], np.zeros(4, np.float32), 0.05)  # n_tau > max_taus
    assert e.value.code == -1
    with pytest.raises(AEError) as e:
        ex.load_prefix_kv(5, *case.kv[0])
    assert e.value.code == -1
    ex.close()


SMALL_MAX = SMALL_BF16.with_(name="small_max", horizon=256, action_dim=64, prefix_len=64, max_batch=2, max_taus=1,
                             gripper_dim=63, steps=2)


def test_largest_chunk_and_action_width_match_oracle():
    """The largest suffix the kernels take (horizon 256, action_dim 64), two robots, then one flow
    time: delta 0 accepts nothing (the test is strict), a huge delta accepts every row of a draft
    without a switch."""
    cfg = SMALL_MAX
    case = Case(cfg)
    ex = _expert(case)
    noise = case.noise(2)
    got = ex.denoise(noise, cfg.steps)
    err = rel_err(got, case.oracle_denoise(noise, cfg.steps))
    print(f"small_max rel_err={err:.3e}")
    assert err <= tol_for(cfg), err
    draft = G.make_draft(cfg, 0)  # even seed: no gripper switch
    tau = np.array([0.5], np.float32)
    acc0, sw0, D = ex.verify(0, draft, noise[0], tau, 0.0)
    accH, swH, _ = ex.verify(0, draft, noise[0], tau, 1e30)
    assert (acc0, sw0) == (0, 0) and (accH, swH) == (cfg.horizon, 0)
    _, _, D_o = case.oracle_verify(0, draft, noise[0], tau, 0.0)
    assert rel_err(D, D_o) <= tol_for(cfg)
    ex.close()


@pytest.mark.parametrize("over", [dict(horizon=257), dict(action_dim=65)], ids=["horizon257", "action65"])
def test_sizes_past_the_kernels_are_rejected_at_create(over):
    cfg = SMALL_BF16.with_(**over)
    with pytest.raises(AEError) as e:
        ActionExpert(cfg, G.make_weights(cfg))
    assert e.value.code == -2


# ------------------------------------------------------------------ time-modulated expert with QK-norm

SMALL_DM05 = SMALL_BF16.with_(name="small_dm05", time_mode=1, qk_norm=1, max_taus=0)


@pytest.mark.parametrize("cfg", [SMALL_DM05, SMALL_DM05.with_(name="small_dm05_b7", max_batch=7),
                                 SMALL_BF16.with_(name="small_qknorm", qk_norm=1)], ids=lambda c: c.name)
def test_modulated_qknorm_denoise_matches_oracle(cfg):
    """Per-layer time modulation (scale / shift / gate of both norms and the final norm) and per-head
    QK-norm: 3 robots (one 64-token group) and 7 robots (the token-group loop), 1 and 3 steps."""
    case = Case(cfg)
    ex = _expert(case)
    noise = case.noise(cfg.max_batch)
    for steps in (1, cfg.steps):
        got = ex.denoise(noise, steps)
        ref = case.oracle_denoise(noise, steps)
        err = rel_err(got, ref)
        print(f"{cfg.name} steps={steps} rel_err={err:.3e}")
        assert err <= tol_for(cfg), err
    ex.close()


def test_qknorm_verify_matches_oracle():
    cfg = SMALL_BF16.with_(name="small_qknorm_v", qk_norm=1)
    case = Case(cfg)
    ex = _expert(case)
    taus = np.array([0.2, 0.5, 0.8], np.float32)
    for seed in range(2):
        draft = G.make_draft(cfg, seed)
        noise = case.noise(1, 300 + seed)[0]
        acc, sw, D = ex.verify(1, draft, noise, taus, 0.05)
        acc_o, sw_o, D_o = case.oracle_verify(1, draft, noise, taus, 0.05)
        assert (acc, sw) == (acc_o, sw_o)
        assert rel_err(D, D_o) <= tol_for(cfg)
    ex.close()


def _delta_sweep(ex, slot, draft, noise, taus, D, D_o, horizon):
    """Every accept length k whose deciding half-gap (between the running maxima of D over rows
    k - 1 and k) exceeds twice the largest measured |D - D_o|: the kernel must take each such
    decision exactly as the oracle does (FLASH article, section 03: a row is accepted only when every
    flow time reconstructs it within delta). Returns the lengths checked."""
    e = float(np.max(np.abs(D.astype(np.float64) - D_o)))
    run = np.maximum.accumulate(D_o.max(axis=0))
    checked = []
    for k in range(1, horizon):
        if 0.5 * (run[k] - run[k - 1]) > 2.0 * e:
            delta = float(0.5 * (run[k] + run[k - 1]))
            assert O.accept_from_distances(D_o, delta, 0) == k
            acc_k, _, _ = ex.verify(slot, draft, noise, taus, delta)
            assert acc_k == k, (k, acc_k)
            checked.append(k)
    return checked


def test_modulated_verify_matches_oracle():
    """Verification with the time-modulated QK-norm expert: each flow time's sequence takes the layer
    and final-norm modulation of its own tau (per-row vectors in every epilogue), against the oracle's
    independent velocity per tau; 3 flow times, two prefix slots, draft seeds with and without a
    gripper switch, and the accept decisions of a delta sweep."""
    cfg = SMALL_DM05.with_(name="small_dm05_v", max_taus=3)
    case = Case(cfg)
    ex = _expert(case)
    taus = np.array([0.15, 0.5, 0.85], np.float32)
    checked = []
    for slot in (0, 2):
        for seed in range(3):
            draft = G.make_draft(cfg, seed)
            noise = case.noise(1, 500 + seed)[0]
            acc, sw, D = ex.verify(slot, draft, noise, taus, 0.05)
            acc_o, sw_o, D_o = case.oracle_verify(slot, draft, noise, taus, 0.05)
            assert (acc, sw) == (acc_o, sw_o), (slot, seed)
            err = rel_err(D, D_o)
            print(f"dm05 verify slot {slot} seed {seed} D rel_err={err:.3e}")
            assert err <= tol_for(cfg), err
            if sw == 0:
                checked += _delta_sweep(ex, slot, draft, noise, taus, D, D_o, cfg.horizon)
    print(f"accept lengths checked: {sorted(set(checked))}")
    assert len(set(checked)) >= 3
    # a round: the fast path, or the full modulated denoise on a switching draft
    nf = case.noise(1, 600)[0]
    for seed in (0, 1):
        draft = G.make_draft(cfg, seed)
        nv = case.noise(1, 700 + seed)[0]
        _, _, D_o = case.oracle_verify(0, draft, nv, taus, 0.05)
        delta = float(D_o.max()) * 1.5 + 1e-3
        act, acc, sw, full = ex.round(0, draft, nv, taus, delta, nf, 2)
        act_o, acc_o, sw_o, full_o = O.dual_path_round(cfg, case.Wd, case.kvd[0][0], case.kvd[0][1], draft, nv, taus,
                                                       delta, nf, 2)
        assert (acc, sw, full) == (acc_o, sw_o, full_o), seed
        assert rel_err(act, act_o) <= tol_for(cfg) if full else np.array_equal(act, draft)
    ex.close()


def _strong_modulation(cfg, W, seed=7):
    """W with every modulation map scaled 30x and random shift biases: the generated maps move the
    norms by a few percent only, which would let a wrong row-to-sequence index or a lost shift bias
    pass at small widths."""
    rng = np.random.default_rng(seed)
    W = dict(W)
    w = cfg.width
    for name in [f"layers.{l}.w_mod" for l in range(cfg.n_layers)] + ["final_mod_w"]:
        W[name] = G.store(O.decode(W[name], cfg.weight_dtype).astype(np.float32) * np.float32(30.0), cfg.weight_dtype)
    for l in range(cfg.n_layers):
        b = W[f"layers.{l}.b_mod"].copy()
        b[w:2 * w] = 0.5 * rng.standard_normal(w)      # shift1
        b[4 * w:5 * w] = 0.5 * rng.standard_normal(w)  # shift2
        W[f"layers.{l}.b_mod"] = b.astype(np.float32)
    fb = W["final_mod_b"].copy()
    fb[w:] = 0.5 * rng.standard_normal(w)
    W["final_mod_b"] = fb.astype(np.float32)
    return W


@pytest.mark.parametrize("shape", [None, 1, 3], ids=lambda s: "modelled" if s is None else f"shape{s}")
def test_modulated_verify_strong_modulation(shape, monkeypatch):
    """Verification of a time-modulated expert whose modulation is large (30x maps, random shifts), so
    that every flow time's rows differ in their gains, gates and shift biases: the 64-token kernel and
    two token-tiled shapes against the oracle."""
    if shape is not None:
        monkeypatch.setenv("AE_TILED_SHAPE", str(shape))
    cfg = SMALL_DM05.with_(name="small_dm05_strong", max_taus=4)
    case = Case(cfg)
    case.W = _strong_modulation(cfg, case.W)
    case.Wd = O.dequantize_weights(cfg, case.W)
    ex = _expert(case)
    taus = np.array([0.1, 0.4, 0.6, 0.9], np.float32)
    for seed in range(2):
        draft = G.make_draft(cfg, seed)
        noise = case.noise(1, 800 + seed)[0]
        acc, sw, D = ex.verify(0, draft, noise, taus, 0.05)
        acc_o, sw_o, D_o = case.oracle_verify(0, draft, noise, taus, 0.05)
        assert (acc, sw) == (acc_o, sw_o), seed
        err = rel_err(D, D_o)
        print(f"strong modulation shape={shape} seed={seed} D rel_err={err:.3e}")
        assert err <= tol_for(cfg), err
    ex.close()


def test_dm05_full_matches_oracle():
    """DM0.5-style expert at the Pi0 shapes (18 layers, width 1024, 8q/1kv x 256, MLP 4096, P = 816), 10 steps."""
    cfg = C.DM05
    case = Case(cfg)
    ex = _expert(case)
    noise = case.noise(1)
    got = ex.denoise(noise, 10)
    ref = case.oracle_denoise(noise, 10)
    err = rel_err(got, ref)
    print(f"dm05 10 steps rel_err={err:.3e} gpu_ms={ex.last_gpu_ms():.3f}")
    assert err <= 2e-2
    ex.close()


def test_dm05_verify_full():
    """Verification with the DM0.5-style expert at the Pi0 verify shape (18 layers, width 1024, 8q/1kv x
    256, MLP 4096, P = 816, 4 flow times): accepted length, switch and distances against the oracle, and
    the accept decisions of a delta sweep."""
    cfg = C.DM05_VERIFY
    case = Case(cfg)
    ex = _expert(case)
    taus = np.asarray(C.VERIFY_TAUS, np.float32)
    checked = []
    for seed in range(8):
        draft, noise, _ = G.make_verify_case(cfg, seed)
        acc, sw, D = ex.verify(0, draft, noise, taus, C.VERIFY_DELTA)
        acc_o, sw_o, D_o = case.oracle_verify(0, draft, noise, taus, C.VERIFY_DELTA)
        assert (acc, sw) == (acc_o, sw_o), seed
        err = rel_err(D, D_o)
        print(f"dm05 verify seed {seed} D rel_err={err:.3e} gpu_ms={ex.last_gpu_ms():.3f}")
        assert err <= 2e-2, (seed, err)
        if sw == 0:
            checked += _delta_sweep(ex, 0, draft, noise, taus, D, D_o, cfg.horizon)
    print(f"{len(checked)} accept decisions checked, lengths {sorted(set(checked))}")
    assert len(set(checked)) >= 4
    ex.close()


# ------------------------------------------------------------------ draft model

SMALL_DRAFT = C.DRAFT.with_(name="small_draft", width=256, n_q_heads=4, n_kv_heads=2, head_dim=64, mlp_dim=512,
                            horizon=20, prefix_len=100, action_dim=24)


@pytest.mark.parametrize("cfg", [SMALL_DRAFT, C.DRAFT], ids=lambda c: c.name)
def test_draft_matches_oracle(cfg):
    """The draft's candidate chunk against the oracle: small (100 feature tokens: a partial last key block,
    2 kv heads) and full size (a 2B-class block, 768 feature tokens); two feature sets through one graph."""
    W = G.make_weights(cfg)
    Wd = O.dequantize_weights(cfg, W)
    ex = ActionExpert(cfg, W)
    for seed in (1, 2):
        feats = G.make_features(cfg, seed)
        got = ex.draft(feats)
        ref = O.draft_chunk(cfg, Wd, feats)
        err = rel_err(got, ref)
        print(f"{cfg.name} seed={seed} rel_err={err:.3e} gpu_ms={ex.last_gpu_ms():.3f}")
        assert err <= tol_for(cfg), err
    with pytest.raises(AEError) as e:
        ex.denoise(np.zeros((1, cfg.horizon, cfg.action_dim), np.float32), 1)
    assert e.value.code == -2
    ex.close()


def test_draft_entry_rejects_an_expert_handle():
    case = Case(SMALL_BF16)
    ex = _expert(case)
    with pytest.raises(AEError) as e:
        ex.draft(np.zeros((SMALL_BF16.prefix_len, SMALL_BF16.width), np.float32))
    assert e.value.code == -2
    ex.close()


# ------------------------------------------------------------------ prefix prefill

SMALL_PREFILL = C.PREFILL.with_(name="small_prefill", n_layers=2, width=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                                mlp_dim=512, horizon=100)


def _prefill_vs_oracle(cfg):
    W = G.make_weights(cfg)
    Wd = O.dequantize_weights(cfg, W)
    ex = ActionExpert(cfg, W)
    emb = G.make_prefix_embeddings(cfg, 11)
    k, v = ex.prefill(emb)
    k_o, v_o = O.prefill_kv(cfg, Wd, emb)
    kd, vd = O.decode_kv(cfg, k, v)
    for l in range(cfg.n_layers):
        ek, ev = rel_err(kd[l], k_o[l]), rel_err(vd[l], v_o[l])
        print(f"{cfg.name} layer {l}: K rel_err={ek:.3e} V rel_err={ev:.3e} gpu_ms={ex.last_gpu_ms():.3f}")
        assert ek <= tol_for(cfg) and ev <= tol_for(cfg), (l, ek, ev)
    ex.close()
    return k, v


def test_prefill_matches_oracle_small():
    """100 prefix tokens (a partial last key block), 2 kv heads, E4M3 MLP."""
    _prefill_vs_oracle(SMALL_PREFILL)


def test_prefill_full_width_first_two_layers():
    """The 2B-class stack's own per-layer shapes (width 2048, 8q/1kv x 256, E4M3 MLP 16384) over the 816
    prefix tokens; the first two layers of the 18 (a stack's first layers' K/V do not depend on the rest)."""
    _prefill_vs_oracle(C.PREFILL.with_(n_layers=2))


def test_expert_denoises_on_a_prefilled_cache():
    """The prefill output in ae_load_prefix_kv's format: an expert with the stack's kv heads, head_dim and
    depth denoises on it as the oracle does on the same cache."""
    pcfg = SMALL_PREFILL.with_(mlp_dtype="bf16")
    W = G.make_weights(pcfg)
    ex = ActionExpert(pcfg, W)
    k, v = ex.prefill(G.make_prefix_embeddings(pcfg, 12))
    ex.close()
    cfg = SMALL_BF16  # 2 layers, 2 kv heads x 64, prefix 100
    case = Case(cfg)
    exp = ActionExpert(cfg, case.W)
    exp.load_prefix_kv(0, k, v)
    noise = case.noise(1)
    got = exp.denoise(noise, 3)
    kk, vv = O.decode_kv(cfg, k, v)
    ref = O.denoise(cfg, case.Wd, kk, vv, noise[0].astype(np.float64), 3)
    assert rel_err(got[0], ref) <= tol_for(cfg)
    exp.close()


def test_prefill_to_slot_equals_the_host_round_trip():
    """ae_prefill_to_slot copies the stack's K/V on the device into an expert's slot: two robots with
    the same noise, one on a slot loaded through ae_prefill + ae_load_prefix_kv and one on a slot
    filled on the device from the same embeddings, denoise bit for bit alike (and as the oracle);
    mismatched shapes are rejected."""
    pcfg = SMALL_PREFILL.with_(mlp_dtype="bf16")
    pf = ActionExpert(pcfg, G.make_weights(pcfg))
    emb = G.make_prefix_embeddings(pcfg, 13)
    k, v = pf.prefill(emb)
    cfg = SMALL_BF16.with_(max_batch=2)
    case = Case(cfg, n_slots=0)
    exp = ActionExpert(cfg, case.W)
    exp.load_prefix_kv(0, k, v)
    pf.prefill_to_slot(emb, exp, 1)
    noise = case.noise(1)
    x = exp.denoise(np.concatenate([noise, noise]), 3)
    assert np.array_equal(x[0], x[1])
    kk, vv = O.decode_kv(cfg, k, v)
    assert rel_err(x[1], O.denoise(cfg, case.Wd, kk, vv, noise[0].astype(np.float64), 3)) <= tol_for(cfg)
    bcfg = SMALL_BF16.with_(prefix_len=96)
    bad = ActionExpert(bcfg, G.make_weights(bcfg))
    with pytest.raises(AEError) as e:
        pf.prefill_to_slot(emb, bad, 0)
    assert e.value.code == -2
    for h in (pf, exp, bad):
        h.close()


def test_prefill_entry_rejects_other_handles():
    case = Case(SMALL_BF16)
    ex = _expert(case)
    with pytest.raises(AEError) as e:
        ex.prefill(np.zeros((SMALL_BF16.horizon, SMALL_BF16.width), np.float32))
    assert e.value.code == -2
    ex.close()
    pf = ActionExpert(SMALL_PREFILL, G.make_weights(SMALL_PREFILL))
    with pytest.raises(AEError) as e:
        pf.denoise(np.zeros((1, SMALL_PREFILL.horizon, SMALL_PREFILL.action_dim), np.float32), 1)
    assert e.value.code == -2
    pf.close()


# ------------------------------------------------------------------ dual-path round

def test_dual_path_round_matches_oracle():
    """ae_round against the oracle's round: odd draft seeds switch the gripper (full path whatever
    delta is), even seeds take the fast path at a delta above every distance and the full path at
    delta 0 (nothing is < 0). Slot 0 and slot 2 (a graph of its own for that slot's prefix)."""
    cfg = SMALL_BF16
    case = Case(cfg)
    ex = _expert(case)
    taus = np.array([0.2, 0.5, 0.8], np.float32)
    seen = set()
    for slot in (0, 2):
        for seed in range(4):
            draft = G.make_draft(cfg, seed)
            nv = case.noise(1, 300 + seed)[0]
            nf = case.noise(1, 400 + seed)[0]
            _, _, D_o = case.oracle_verify(slot, draft, nv, taus, 0.05)
            for delta in (float(D_o.max()) * 1.5 + 1e-3, 0.0):
                act, acc, sw, full = ex.round(slot, draft, nv, taus, delta, nf, 2)
                act_o, acc_o, sw_o, full_o = O.dual_path_round(cfg, case.Wd, case.kvd[slot][0], case.kvd[slot][1],
                                                               draft, nv, taus, delta, nf, 2)
                assert (acc, sw, full) == (acc_o, sw_o, full_o), (slot, seed, delta)
                if full:
                    assert rel_err(act, act_o) <= tol_for(cfg)
                    assert rel_err(act, ex.denoise(np.stack([nf] * 3), 2)[0]) <= 1e-5 or slot != 0
                else:
                    assert np.array_equal(act, draft)
                seen.add(full)
    assert seen == {0, 1}
    ex.close()


# ------------------------------------------------------------------ token-tiled GEMMs (many tokens)

# 7 robots x 20 rows = 140 tokens (3 token groups). With a shape forced (AE_TILED_SHAPE) every GEMM
# but the output projection takes the token-tiled kernel: its 9 token tiles leave the last one
# ragged, and 8-tile token panels reach past the 12 tiles the buffers hold (those loads are
# clamped, their outputs dropped). The modelled choice keeps the 64-token kernel here (a tiled
# launch would fill too few compute units), which the full-size batched and verify tests cover.
SMALL_BF16_B7 = SMALL_BF16.with_(name="small_bf16_b7", max_batch=7)


@pytest.mark.parametrize("shape", [None, 0, 1, 2, 3], ids=lambda s: "modelled" if s is None else f"shape{s}")
def test_tiled_gemm_denoise_matches_oracle(shape, monkeypatch):
    if shape is not None:
        monkeypatch.setenv("AE_TILED_SHAPE", str(shape))
    case = Case(SMALL_BF16_B7)
    ex = _expert(case)
    noise = case.noise(7)
    got = ex.denoise(noise, 2)
    ref = case.oracle_denoise(noise, 2)
    err = rel_err(got, ref)
    print(f"tiled shape={shape} rel_err={err:.3e}")
    assert err <= tol_for(SMALL_BF16_B7), err
    ex.close()


SMALL_FP8_B7 = SMALL_FP8.with_(name="small_fp8_b7", max_batch=7)


@pytest.mark.parametrize("shape", [0, 1, 2, 3], ids=lambda s: f"shape{s}")
def test_tiled_gemm_fp8_mlp_denoise_matches_oracle(shape, monkeypatch):
    """E4M3 gate/up and down weights in the token-tiled kernel (widened to bf16 in LDS, scaled per
    output channel in the epilogue), every tile shape, 7 robots = 140 tokens."""
    monkeypatch.setenv("AE_TILED_SHAPE", str(shape))
    case = Case(SMALL_FP8_B7)
    ex = _expert(case)
    noise = case.noise(7)
    got = ex.denoise(noise, 2)
    ref = case.oracle_denoise(noise, 2)
    err = rel_err(got, ref)
    print(f"tiled fp8 shape={shape} rel_err={err:.3e}")
    assert err <= tol_for(SMALL_FP8_B7), err
    ex.close()


SMALL_DM05_B7 = SMALL_DM05.with_(name="small_dm05_b7t", max_batch=7)
SMALL_QKN_B7 = SMALL_BF16_B7.with_(name="small_qknorm_b7", qk_norm=1)


@pytest.mark.parametrize("shape", [0, 1, 2, 3], ids=lambda s: f"shape{s}")
@pytest.mark.parametrize("cfg", [SMALL_DM05_B7, SMALL_QKN_B7], ids=lambda c: c.name)
def test_tiled_gemm_modulated_qknorm_matches_oracle(cfg, shape, monkeypatch):
    """The token-tiled QKV and gate/up epilogues with the time-modulated expert's shift biases and the
    QK-norm sums of squares and gains (o_proj and down of a modulated expert keep the 64-token kernel),
    every tile shape, 7 robots = 140 tokens."""
    monkeypatch.setenv("AE_TILED_SHAPE", str(shape))
    case = Case(cfg)
    ex = _expert(case)
    noise = case.noise(7)
    got = ex.denoise(noise, 2)
    ref = case.oracle_denoise(noise, 2)
    err = rel_err(got, ref)
    print(f"tiled {cfg.name} shape={shape} rel_err={err:.3e}")
    assert err <= tol_for(cfg), err
    ex.close()


@pytest.mark.parametrize("shape", [1, 3], ids=lambda s: f"shape{s}")
def test_tiled_gemm_modulated_verify_matches_oracle(shape, monkeypatch):
    """A time-modulated verification pass of 8 flow times (160 rows) through the token-tiled QKV and
    gate/up epilogues: each row takes its own flow time's shift biases."""
    monkeypatch.setenv("AE_TILED_SHAPE", str(shape))
    cfg = SMALL_DM05.with_(name="small_dm05_t8", max_taus=8)
    case = Case(cfg)
    ex = _expert(case)
    taus = np.linspace(0.1, 0.9, 8).astype(np.float32)
    for seed in range(2):
        draft = G.make_draft(cfg, seed)
        noise = case.noise(1, 300 + seed)[0]
        acc, sw, D = ex.verify(1, draft, noise, taus, 0.05)
        acc_o, sw_o, D_o = case.oracle_verify(1, draft, noise, taus, 0.05)
        assert (acc, sw) == (acc_o, sw_o)
        err = rel_err(D, D_o)
        print(f"tiled dm05 verify shape={shape} seed={seed} D rel_err={err:.3e}")
        assert err <= tol_for(cfg), err
    ex.close()


def test_tiled_gemm_verify_matches_oracle(monkeypatch):
    """8 flow times x 20 rows = 160 tokens in one verification pass (token-tiled GEMMs)."""
    cfg = SMALL_BF16.with_(name="small_bf16_t8", max_taus=8)
    case = Case(cfg)
    ex = _expert(case)
    taus = np.linspace(0.1, 0.9, 8).astype(np.float32)
    for seed in range(2):
        draft = G.make_draft(cfg, seed)
        noise = case.noise(1, 300 + seed)[0]
        acc, sw, D = ex.verify(1, draft, noise, taus, 0.05)
        acc_o, sw_o, D_o = case.oracle_verify(1, draft, noise, taus, 0.05)
        assert (acc, sw) == (acc_o, sw_o)
        assert rel_err(D, D_o) <= tol_for(cfg)
    ex.close()


# ------------------------------------------------------------------ full Pi0-scale shapes

@pytest.fixture(scope="module")
def pi0_case():
    return Case(C.PI0_BATCH16, n_slots=16)


def test_pi0_bf16_denoise_full(pi0_case):
    cfg = C.PI0
    ex = ActionExpert(cfg, pi0_case.W)
    ex.load_prefix_kv(0, *pi0_case.kv[0])
    noise = pi0_case.noise(1)
    got = ex.denoise(noise, 10)
    ref = pi0_case.oracle_denoise(noise, 10)
    err = rel_err(got, ref)
    print(f"pi0 bf16 10 steps rel_err={err:.3e} gpu_ms={ex.last_gpu_ms():.3f}")
    assert err <= 2e-2
    ex.close()


def test_pi0_fp8_mlp_two_view_full():
    cfg = C.PI0_FP8
    case = Case(cfg)
    ex = _expert(case)
    noise = case.noise(1)
    got = ex.denoise(noise, 10)
    ref = case.oracle_denoise(noise, 10)
    err = rel_err(got, ref)
    print(f"pi0 fp8 10 steps rel_err={err:.3e} gpu_ms={ex.last_gpu_ms():.3f}")
    assert err <= 6e-2
    ex.close()


def test_pi0_verify_full(pi0_case):
    cfg = C.PI0_VERIFY
    ex = ActionExpert(cfg, pi0_case.W)
    ex.load_prefix_kv(0, *pi0_case.kv[0])
    taus = np.asarray(C.VERIFY_TAUS, np.float32)
    checked = []
    for seed in range(16):
        draft, noise, _ = G.make_verify_case(cfg, seed)
        acc, sw, D = ex.verify(0, draft, noise, taus, C.VERIFY_DELTA)
        acc_o, sw_o, D_o = pi0_case.oracle_verify(0, draft, noise, taus, C.VERIFY_DELTA, cfg)
        assert (acc, sw) == (acc_o, sw_o), seed
        assert sw == seed % 2
        err = rel_err(D, D_o)
        assert err <= 2e-2, (seed, err)
        # delta sweep: with a running max of D over rows, accept = k for any delta between the maxima
        # up to rows k-1 and k. Every k whose half-gap exceeds twice the largest measured |D - D_o|
        # is a decision the kernel must take exactly as the oracle does.
        if sw == 0:
            e = float(np.max(np.abs(D.astype(np.float64) - D_o)))
            run = np.maximum.accumulate(D_o.max(axis=0))
            for k in range(1, cfg.horizon):
                if 0.5 * (run[k] - run[k - 1]) > 2.0 * e:
                    delta = float(0.5 * (run[k] + run[k - 1]))
                    assert O.accept_from_distances(D_o, delta, 0) == k
                    acc_k, _, _ = ex.verify(0, draft, noise, taus, delta)
                    assert acc_k == k, (seed, k, acc_k)
                    checked.append(k)
    print(f"{len(checked)} accept decisions checked, lengths {sorted(set(checked))}")
    assert len(set(checked)) >= 10
    ex.close()


def test_pi0_verify_closed_form(pi0_case):
    """At the Pi0 verify shape, W_out = 0 and b_out = c make v = c: with noise = d0 - c the rebuilt
    endpoints equal d0, so a draft d0 + p (p = 0 before row k, p_0 = 1 from row k) has
    D[j, i] = (1 - tau_j) [i >= k] and the accepted length is exactly k for delta below 1 - max tau."""
    cfg = C.PI0_VERIFY
    W = dict(pi0_case.W)
    W["action_out_w"] = np.zeros_like(W["action_out_w"])
    c = np.linspace(-0.5, 0.5, cfg.action_dim).astype(np.float32)
    W["action_out_b"] = c
    ex = ActionExpert(cfg, W)
    ex.load_prefix_kv(0, *pi0_case.kv[0])
    H, A = cfg.horizon, cfg.action_dim
    rng = np.random.default_rng(3)
    d0 = rng.standard_normal((H, A)).astype(np.float32)
    d0[:, cfg.gripper_dim] = 1.0
    noise = (d0 - c[None, :]).astype(np.float32)
    taus = np.asarray(C.VERIFY_TAUS, np.float32)
    for k in (0, 1, 17, 49, 50):
        d = d0.copy()
        d[k:, 0] += 1.0
        acc, sw, D = ex.verify(0, d, noise, taus, C.VERIFY_DELTA)
        assert (acc, sw) == (k, 0), k
        expect = (1.0 - taus[:, None]) * (np.arange(H) >= k)[None, :]
        assert np.allclose(D, expect, atol=1e-5), k
    ex.close()


@pytest.mark.parametrize("robots", [range(0, 4), range(4, 8), range(8, 12), range(12, 16)],
                         ids=lambda r: f"robots{r.start}-{r.stop - 1}")
def test_pi0_batch16_every_robot(pi0_case, robots):
    """All 16 robots of one batch-16 pass, four per test so that each oracle run stays short."""
    ex = _expert(pi0_case, slots=16)
    noise = pi0_case.noise(16)
    got = ex.denoise(noise, 10)
    ref = pi0_case.oracle_denoise(noise, 10, robots)
    for i, r in enumerate(robots):
        err = rel_err(got[r], ref[i])
        print(f"batch16 robot {r} rel_err={err:.3e}")
        assert err <= 2e-2
    ex.close()


# ------------------------------------------------------------------ several robots at the Pi0 widths

# Pi0 widths, two layers, several robots (launch per phase: the step kernel is for batch 1): a 100-key
# prefix and a 1,100-key prefix (37 blocks), 50 rows x 8 heads = 25 query tiles
PI0W = [C.PI0.with_(name="pi0w_p100_b3", n_layers=2, prefix_len=100, max_batch=3, batch=3, steps=2),
          C.PI0.with_(name="pi0w_p1100_b2", n_layers=2, prefix_len=1100, max_batch=2, batch=2, steps=2)]


@pytest.mark.parametrize("cfg", PI0W, ids=lambda c: c.name)
def test_batched_robots_at_pi0_widths_match_oracle(cfg):
    case = Case(cfg)
    ex = _expert(case)
    noise = case.noise(cfg.max_batch)
    for steps in (1, 2):
        got = ex.denoise(noise, steps)
        ref = case.oracle_denoise(noise, steps)
        for r in range(cfg.max_batch):
            err = rel_err(got[r], ref[r])
            print(f"{cfg.name} steps={steps} robot {r} rel_err={err:.3e}")
            assert err <= tol_for(cfg), (steps, r, err)
    ex.close()


# Many robots at the Pi0 widths: more query tiles than compute units, so the attention takes two query
# tiles per workgroup. 32 robots x 17 rows: 9 query tiles per robot (odd: the last workgroup of each
# robot has one tile); 40 robots x 16 rows with an 850-key prefix: 8 tiles, 28 key blocks (the most the
# two-tile workgroup walks)
PAIRS = [C.PI0.with_(name="pi0w_h17_b32", n_layers=2, horizon=17, prefix_len=100, max_batch=32, batch=32, steps=2),
         C.PI0.with_(name="pi0w_h16_p850_b40", n_layers=2, horizon=16, prefix_len=850, max_batch=40, batch=40,
                     steps=2)]


@pytest.mark.parametrize("cfg", PAIRS, ids=lambda c: c.name)
def test_two_tile_attention_matches_oracle(cfg):
    case = Case(cfg)
    ex = _expert(case)
    noise = case.noise(cfg.max_batch)
    got = ex.denoise(noise, 2)
    ref = case.oracle_denoise(noise, 2)
    errs = [rel_err(got[r], ref[r]) for r in range(cfg.max_batch)]
    print(f"{cfg.name} worst robot rel_err={max(errs):.3e}")
    assert max(errs) <= tol_for(cfg), errs
    ex.close()
