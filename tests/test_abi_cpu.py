"""C-ABI checks that need no GPU: exported symbols, struct layouts, and the
argument validation that ae_create does before touching a device."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from flow_matching_action_euler_amd import binding as B
from workload import configs as C
from workload import gen as G

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ae.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ae_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = B.load_library()
    names = _declared()
    assert len(names) == 15
    assert sorted(B.EXPORTS) == names
    for n in names:
        assert hasattr(lib, n), n


def test_struct_layouts_match_the_header(tmp_path):
    prog = tmp_path / "layout.c"
    prog.write_text(r'''
#include <stdio.h>
#include <stddef.h>
#include "ae.h"
int main(void) {
  printf("%zu %zu %zu %zu\n", sizeof(ae_config), sizeof(ae_layer_weights), sizeof(ae_weights), sizeof(ae_kernel_stat));
  printf("%zu %zu %zu %zu\n", offsetof(ae_config, rope_base), offsetof(ae_config, gripper_dim),
         offsetof(ae_weights, layers), offsetof(ae_kernel_stat, total_ms));
  return 0;
}
''')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.dirname(HEADER), str(prog), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()
    got = [int(x) for x in out]
    exp = [ctypes.sizeof(B.ae_config), ctypes.sizeof(B.ae_layer_weights), ctypes.sizeof(B.ae_weights),
           ctypes.sizeof(B.ae_kernel_stat), B.ae_config.rope_base.offset, B.ae_config.gripper_dim.offset,
           B.ae_weights.layers.offset, B.ae_kernel_stat.total_ms.offset]
    assert got == exp


def _create_rc(cfg, W):
    lib = B.load_library()
    keep = []

    def p(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        keep.append(a)
        return a.ctypes.data

    L = cfg.n_layers
    layers = (B.ae_layer_weights * L)()
    for l in range(L):
        for f in ("ln1", "wq", "wk", "wv", "wo", "ln2", "wg", "wu", "wd"):
            setattr(layers[l], f, p(W.get(f"layers.{l}.{f}")))
        for f in ("wg", "wu", "wd"):
            setattr(layers[l], f + "_scale", p(W.get(f"layers.{l}.{f}.scale")))
    w = B.ae_weights(time_in_w=p(W["time_in_w"]), time_in_b=p(W["time_in_b"]), time_out_w=p(W["time_out_w"]),
                     time_out_b=p(W["time_out_b"]), action_in_w=p(W["action_in_w"]), action_in_b=p(W["action_in_b"]),
                     layers=layers, final_ln=p(W["final_ln"]), action_out_w=p(W["action_out_w"]),
                     action_out_b=p(W["action_out_b"]))
    c = B.make_config(cfg)
    h = ctypes.c_void_p()
    rc = lib.ae_create(ctypes.byref(c), ctypes.byref(w), ctypes.byref(h))
    msg = lib.ae_last_error(None).decode()
    if rc == 0:
        lib.ae_destroy(h)
    return rc, msg


@pytest.fixture(scope="module")
def tiny_weights():
    return G.make_weights(C.TINY)


@pytest.mark.parametrize("change,code", [
    (dict(width=0), -1),
    (dict(n_kv_heads=3), -1),           # does not divide n_q_heads
    (dict(gripper_dim=8), -1),           # outside action_dim
    (dict(width=200), -2),               # not a multiple of 256
    (dict(head_dim=48), -2),             # not one of 32, 64, 128, 256
    (dict(action_dim=65), -2),
    (dict(kv_dtype="bf16"), -2),         # cache type differs from the attention weights
    (dict(mlp_dtype="fp8"), -2),         # fp8 MLP needs bf16 attention weights
])
def test_create_rejects_bad_config_before_any_device_call(tiny_weights, change, code):
    rc, msg = _create_rc(C.TINY.with_(**change), tiny_weights)
    assert rc == code and msg


def test_create_rejects_missing_weight(tiny_weights):
    W = dict(tiny_weights)
    W["layers.1.wd"] = None
    rc, msg = _create_rc(C.TINY, W)
    assert rc == -1 and "null" in msg


def test_binding_raises_without_library(tmp_path):
    with pytest.raises(OSError):
        B._lib, saved = None, B._lib
        try:
            B.load_library(str(tmp_path / "missing.so"))
        finally:
            B._lib = saved


def test_bench_work_figures_match_the_closed_forms():
    """bench.py's algorithmic bytes and FLOPs per step, against the per-layer arithmetic of the
    Pi0-scale shapes: 17.30 M weights per layer (qkv 2560 x 1024, o 1024 x 2048, gate/up
    2 x 4096 x 1024, down 1024 x 4096), Q.K^T and P.V of 8 x 50 query rows over 866 keys x 256."""
    import bench
    per_layer = 2560 * 1024 + 1024 * 2048 + 2 * 4096 * 1024 + 1024 * 4096
    assert per_layer == 17_301_504
    attn = 4 * 8 * 50 * 866 * 256
    io = 2 * 2 * 1024 * 32 * 50
    assert bench.step_flops(C.PI0, 1) == 18 * (2 * 50 * per_layer + attn) + io
    assert bench.step_flops(C.PI0_BATCH16, 16) == 16 * bench.step_flops(C.PI0, 1)
    # bytes: bf16 weights once per step + the prefix K and V of every robot (suffix K/V excluded)
    kv = 2 * 816 * 256 * 2
    assert bench.step_bytes(C.PI0, 1) == 18 * (2 * per_layer + kv) + 2 * 2 * 1024 * 32
    assert bench.step_bytes(C.PI0, 16) - bench.step_bytes(C.PI0, 1) == 15 * 18 * kv
    # one persistent step-kernel launch is one whole Euler step of one robot
    assert bench.kernel_bytes(C.PI0)["fused_step"] == bench.step_bytes(C.PI0, 1)
    assert bench.kernel_flops(C.PI0, 1)["fused_step"] == bench.step_flops(C.PI0, 1)
    # the attention of one robot: 354.7 MFLOP over 886,784 B of K/V = 400 FLOP/B, above the bf16
    # ridge (2.5 PFLOP/s over 8 TB/s = 312.5 FLOP/B): its roof is the MFMA one; a GEMM's is HBM
    e = bench.annotate({}, bench.kernel_bytes(C.PI0)["attn"], bench.kernel_flops(C.PI0, 1)["attn"], 10.0)
    assert e["alg_bytes"] == 886_784 and e["alg_flops"] == attn and e["bound"] == "mfma"
    assert e["frac"] == e["mfma_frac"] == round(attn / 10e-6 / 2.5e15, 4)
    e = bench.annotate({}, bench.kernel_bytes(C.PI0)["down_resid"], bench.kernel_flops(C.PI0, 1)["down_resid"], 10.0)
    assert e["bound"] == "hbm" and e["frac"] == e["hbm_frac"]


def test_prefill_flops_match_the_closed_form():
    """The 2B-class prefill stack: 110.1 M weights per layer (qkv 2560 x 2048, o 2048 x 2048, gate/up/down
    3 x 16384 x 2048), 2 FLOPs per weight per token over 816 tokens, Q.K^T and P.V of 8 x 816 query rows
    over 816 keys x 256; the weights are the stack's parameters less its two norm gains per layer."""
    import bench
    per_layer = 2560 * 2048 + 2048 * 2048 + 3 * 16384 * 2048
    assert per_layer == 110_100_480
    assert per_layer == C.PREFILL.n_params // 18 - 2 * 2048
    assert bench.prefill_flops(C.PREFILL) == 18 * (2 * 816 * per_layer + 4 * 8 * 816 * 816 * 256)


def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    """The library's host code (config checks, weight packing, prefix-cache repacking: csrc/ae_host.hpp)
    built with g++ -fsanitize=address,undefined and run by tests/host/ae_host_check.cpp on varied
    shapes and on configs whose sizes would overflow int; any sanitizer report or layout mismatch fails."""
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = tmp_path / "ae_host_check"
    src = os.path.join(ROOT, "tests", "host", "ae_host_check.cpp")
    build = subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                            "-fno-omit-frame-pointer", src, "-o", str(exe)], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0 and run.stdout.strip() == "ok", (run.stdout[-2000:], run.stderr[-2000:])
