"""Invariances of the GPU path through the C-ABI:
- a pass replayed from its captured hipGraph equals the same launches enqueued directly (AE_GRAPH=0), bit
  for bit (denoise on the launch-per-phase path and on the persistent step kernel, verification);
- the split-K factor of o_proj and down (AE_SPLITK=<o>,<down>: 1, 2 or 4 partial sums) changes the
  summation order only: every factor matches the oracle within the bf16 bar (max|gpu - oracle| <=
  2e-2 * RMS(oracle)), and the default (4, 4) is bitwise the forced (4, 4)."""
import numpy as np
import pytest

from flow_matching_action_euler_amd import ActionExpert
from workload import configs as C

from helpers import SMALL_BF16, Case, rel_err, tol_for

pytestmark = pytest.mark.gpu

STEP_BF16 = C.PI0.with_(name="step_bf16", n_layers=2, horizon=20, prefix_len=100, action_dim=24, steps=3)


def _expert(case, env, monkeypatch):
    with monkeypatch.context() as m:
        for k, v in env.items():
            m.setenv(k, v)
        ex = ActionExpert(case.cfg, case.W)
    for r in range(case.cfg.max_batch):
        ex.load_prefix_kv(r, *case.kv[r])
    return ex


@pytest.mark.parametrize("cfg", [SMALL_BF16, STEP_BF16], ids=lambda c: c.name)
def test_graph_replay_equals_eager_pass(cfg, monkeypatch):
    case = Case(cfg)
    graph = _expert(case, {}, monkeypatch)
    eager = _expert(case, {"AE_GRAPH": "0"}, monkeypatch)
    for batch in sorted({1, cfg.max_batch}):
        noise = case.noise(batch)
        for steps in (1, 3):
            a = graph.denoise(noise, steps)
            b = eager.denoise(noise, steps)
            assert np.array_equal(a, b), (batch, steps)
            assert rel_err(a, case.oracle_denoise(noise, steps)) <= tol_for(cfg)
    if cfg.max_taus:
        rng = np.random.default_rng(5)
        H, A = cfg.horizon, cfg.action_dim
        draft = rng.standard_normal((H, A)).astype(np.float32)
        noise = rng.standard_normal((H, A)).astype(np.float32)
        taus = np.array([0.2, 0.5, 0.8], np.float32)
        ra = graph.verify(0, draft, noise, taus, 0.05)
        rb = eager.verify(0, draft, noise, taus, 0.05)
        assert ra[:2] == rb[:2] and np.array_equal(ra[2], rb[2])
    graph.close()
    eager.close()


# o_proj K = 4 x 256 = 1024 and down K = 1024 (32 k-blocks each): every factor 1, 2, 4 leaves whole
# 8-wave k-slices; 20-row chunks, 3 robots = one token group (where o_proj and down split K)
SPLIT_BF16 = SMALL_BF16.with_(name="small_bf16_dh256", head_dim=256, mlp_dim=1024)


def test_split_k_factor_changes_only_the_summation_order(monkeypatch):
    cfg = SPLIT_BF16
    case = Case(cfg)
    noise = case.noise(cfg.max_batch)
    ref = case.oracle_denoise(noise, 3)
    outs = {}
    for sk in ("1,1", "2,2", "4,4", "1,4", "4,1", "2,4"):
        ex = _expert(case, {"AE_SPLITK": sk}, monkeypatch)
        outs[sk] = ex.denoise(noise, 3)
        err = rel_err(outs[sk], ref)
        print(f"AE_SPLITK={sk} rel_err={err:.3e}")
        assert err <= tol_for(cfg), (sk, err)
        ex.close()
    ex = _expert(case, {}, monkeypatch)
    assert np.array_equal(ex.denoise(noise, 3), outs["4,4"])
    ex.close()
    # the factors are really applied: 1, 2 and 4 partial sums round differently somewhere in the chunk
    assert not np.array_equal(outs["1,1"], outs["4,4"])
    assert not np.array_equal(outs["2,2"], outs["4,4"])
