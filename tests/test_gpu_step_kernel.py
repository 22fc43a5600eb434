"""The persistent step kernel (batch 1: one launch per Euler step, phases exchanging activations
through polled rings inside the launch) against the oracle, against the launch-per-phase path, and
its bounded waits: with AE_WAIT_TICKS=0 every wait gives up at once, the synchronous calls repeat
their pass on launches that wait for nothing inside a kernel, and an asynchronous call's give-up is
reported by the next call on the handle.

Tolerance as for every bf16 chunk: max|gpu - oracle| <= 2e-2 * RMS(oracle) (6e-2 with an fp8 MLP).
"""
import numpy as np
import pytest
import torch

from flow_matching_action_euler_amd import ActionExpert, AEError
from workload import configs as C

from helpers import SMALL_BF16, Case, rel_err, tol_for

pytestmark = pytest.mark.gpu

# Pi0 widths (the step kernel is built for them), two layers and short chunks so the oracle is quick:
# 20 rows (2 token tiles, 12 padding rows), 24 action dims, a 100-key prefix (one key split) and a
# 1,100-key prefix (several key splits, last block partial).
STEP_BF16 = C.PI0.with_(name="step_bf16", n_layers=2, horizon=20, prefix_len=100, action_dim=24, steps=3)
STEP_FP8 = STEP_BF16.with_(name="step_fp8", mlp_dtype="fp8")
STEP_LONG = STEP_BF16.with_(name="step_bf16_long_prefix", prefix_len=1100, horizon=50, action_dim=32)
STEP_H64 = STEP_BF16.with_(name="step_bf16_h64", horizon=64, prefix_len=300)
# time modulation and QK-norm (the DM0.5-style expert): per-step gains, shift biases and gates, and the
# per-head 1/rms of q and k exchanged between the QKV and attention phases
STEP_DM05 = STEP_BF16.with_(name="step_dm05", time_mode=1, qk_norm=1)
STEP_DM05_LONG = STEP_LONG.with_(name="step_dm05_long_prefix", time_mode=1, qk_norm=1)


def _uses_step_kernel(ex, steps):
    names = [n for n, _, _ in ex.kernel_times(0, 1, steps, 1)]
    return "fused_step" in names


def _expert(case):
    ex = ActionExpert(case.cfg, case.W)
    for r in range(case.cfg.max_batch):
        ex.load_prefix_kv(r, *case.kv[r])
    return ex


@pytest.mark.parametrize("cfg", [STEP_BF16, STEP_FP8, STEP_LONG, STEP_H64, STEP_DM05, STEP_DM05_LONG],
                         ids=lambda c: c.name)
def test_step_kernel_matches_oracle(cfg):
    case = Case(cfg)
    ex = _expert(case)
    assert _uses_step_kernel(ex, 2), "batch-1 denoise at these widths runs the persistent step kernel"
    noise = case.noise(1)
    # odd and even step counts in turn: the two activation rings alternate between launches and an
    # odd count ends with a ring reset, which the next call relies on
    for steps in (1, 2, 3, 1, 4):
        got = ex.denoise(noise, steps)
        err = rel_err(got, case.oracle_denoise(noise, steps))
        print(f"{cfg.name} steps={steps} rel_err={err:.3e} gpu_ms={ex.last_gpu_ms():.3f}")
        assert err <= tol_for(cfg), (steps, err)
        assert np.array_equal(ex.denoise(noise, steps), got), steps  # bitwise reproducible
    ex.close()


@pytest.mark.parametrize("cfg", [STEP_LONG, STEP_DM05_LONG], ids=lambda c: c.name)
def test_step_kernel_agrees_with_launch_per_phase(cfg, monkeypatch):
    """Same GEMM splits, different attention key splits and reduction order: bf16-level agreement."""
    case = Case(cfg)
    noise = case.noise(1)
    outs = {}
    for fused in ("1", "0"):
        with monkeypatch.context() as m:
            m.setenv("AE_FUSED", fused)
            ex = _expert(case)
        assert _uses_step_kernel(ex, 3) == (fused == "1")
        outs[fused] = ex.denoise(noise, 3)
        ex.close()
    ref = case.oracle_denoise(noise, 3)
    for k, v in outs.items():
        assert rel_err(v, ref) <= tol_for(cfg), k
    assert rel_err(outs["1"], outs["0"]) <= tol_for(cfg)


@pytest.mark.parametrize("cfg", [STEP_BF16, SMALL_BF16.with_(name="small_bf16_long_prefix", prefix_len=1100)],
                         ids=lambda c: c.name)
def test_zero_tick_waits_repeat_the_pass(cfg, monkeypatch):
    """Every in-kernel wait gives up at once: denoise (step kernel or launch per phase, batch 1 and
    the full batch) and verify still return the oracle's results, from the repeated pass."""
    monkeypatch.setenv("AE_WAIT_TICKS", "0")
    case = Case(cfg)
    ex = _expert(case)
    for batch in (1, cfg.max_batch):
        noise = case.noise(batch)
        ref = case.oracle_denoise(noise, 3)
        for _ in range(4):  # the step kernel is set aside after repeated give-ups; results stay right
            got = ex.denoise(noise, 3)
            assert rel_err(got, ref) <= tol_for(cfg), batch
    if cfg.max_taus:
        rng = np.random.default_rng(1)
        H, A = cfg.horizon, cfg.action_dim
        draft = rng.standard_normal((H, A)).astype(np.float32)
        noise = rng.standard_normal((H, A)).astype(np.float32)
        taus = np.array([0.2, 0.5, 0.8], np.float32)
        acc, sw, D = ex.verify(0, draft, noise, taus, 0.05)
        acc_o, sw_o, D_o = case.oracle_verify(0, draft, noise, taus, 0.05)
        assert (acc, sw) == (acc_o, sw_o)
        assert rel_err(D, D_o) <= tol_for(cfg)
    ex.close()


def test_zero_tick_async_give_up_is_reported_by_the_next_call(monkeypatch):
    monkeypatch.setenv("AE_WAIT_TICKS", "0")
    cfg = STEP_BF16
    case = Case(cfg)
    ex = _expert(case)
    noise = case.noise(1)
    ref = case.oracle_denoise(noise, 2)
    dev = torch.device("cuda:0")
    d_noise = torch.from_numpy(noise).to(dev)
    d_out = torch.empty_like(d_noise)
    reported = 0
    for _ in range(3):
        ex.denoise_async(1, d_noise.data_ptr(), 2, d_out.data_ptr())
        torch.cuda.synchronize()
        try:
            got = ex.denoise(noise, 2)
        except AEError as e:
            assert "gave up" in str(e)
            reported += 1
            got = ex.denoise(noise, 2)  # the exchange buffers were restored
        assert rel_err(got, ref) <= tol_for(cfg)
    assert reported >= 1, "a zero-tick wait inside the step kernel gives up"
    ex.close()


def test_step_kernel_on_another_prefix_slot():
    """A dual-path round on prefix slot 1 whose draft switches the gripper runs the full path: the
    batch-1 denoise of slot 1 on the persistent step kernel (its cache offset is the slot's)."""
    from oracle import ae_oracle as O
    from workload import gen as G
    cfg = STEP_BF16.with_(name="step_bf16_round", max_batch=2, max_taus=3, gripper_dim=23)
    case = Case(cfg)
    ex = _expert(case)
    taus = np.array([0.2, 0.5, 0.8], np.float32)
    draft = G.make_draft(cfg, 1)  # odd seeds switch the gripper
    nv = case.noise(1, 301)[0]
    nf = case.noise(1, 401)[0]
    for slot in (1, 0, 1):
        act, acc, sw, full = ex.round(slot, draft, nv, taus, 0.05, nf, 3)
        act_o, acc_o, sw_o, full_o = O.dual_path_round(cfg, case.Wd, case.kvd[slot][0], case.kvd[slot][1], draft, nv,
                                                       taus, 0.05, nf, 3)
        assert (acc, sw, full) == (acc_o, sw_o, full_o) == (0, 1, 1), slot
        err = rel_err(act, act_o)
        print(f"slot {slot} full-path rel_err={err:.3e}")
        assert err <= tol_for(cfg), (slot, err)
    ex.close()


# the work split's edge cases: 1 and 16 rows (one token tile, ntp 1), 17 and 33 rows (2 and 3 token tiles,
# ragged), a one-key prefix (one block, 31 masked keys), a 31-key prefix, and a 2,000-key prefix (65 blocks:
# 9 key splits of 8 blocks, more units than the XCD grouping covers)
EDGE = [STEP_BF16.with_(name=f"step_h{H}_p{P}", horizon=H, prefix_len=P, steps=2)
        for H, P in ((1, 100), (16, 1), (17, 31), (33, 2000))]


@pytest.mark.parametrize("cfg", EDGE, ids=lambda c: c.name)
def test_step_kernel_work_split_edges(cfg):
    case = Case(cfg)
    ex = _expert(case)
    assert _uses_step_kernel(ex, 2)
    noise = case.noise(1)
    for steps in (1, 2):
        got = ex.denoise(noise, steps)
        err = rel_err(got, case.oracle_denoise(noise, steps))
        print(f"{cfg.name} steps={steps} rel_err={err:.3e}")
        assert err <= tol_for(cfg), (steps, err)
    ex.close()
