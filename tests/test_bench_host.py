"""Host logic of the benchmark (no GPU): the assignment of profiled kernel
dispatches to the library calls of a step, the kernel classification, the
GEMM shape table of the matrix-core summary, and the parser of the GPU clock
and power sample."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _dispatches(recipe, steps, reduce_after_wgrad=True):
    """A synthetic dispatch list: `steps` steps of the bench's call sequence,
    each kernel tagged with its step and stage."""
    out = []
    for s in range(steps):
        for stage, kinds in bench.step_sequence(bench.SHAPES, recipe):
            for kd in kinds:
                out.append((kd, "k", (s, stage)))
            if stage.startswith("gemm_wgrad") and reduce_after_wgrad:
                out.append(("reduce", "r", (s, stage)))
    return out


def test_walk_steps_assigns_every_dispatch_to_its_call():
    disp = _dispatches("tensor", 5)
    steps = bench.walk_steps(disp, 3, 2)
    assert len(steps) == 3
    for i, st in enumerate(steps):
        for stage, kind, name, (s, orig) in st:
            assert s == i + 2 and orig == stage
        # 2 layers x (2 two-kernel quantizes (X with W, then dY) + 3 GEMMs
        # + 1 split-K reduce)
        assert len(st) == 2 * (2 * 2 + 3 + 1)


def test_walk_steps_block_recipe_starts_at_the_first_weight_block_cast():
    tensor = _dispatches("tensor", 2)
    block = [(k, "cast_kernel<0, 2>" if (k == "cast" and st[1].startswith("quant_w")) else n, st)
             for k, n, st in _dispatches("block", 3)]
    steps = bench.walk_steps(tensor + block, 2, 1, "block")
    assert len(steps) == 2
    assert all(kind != "amax" for st in steps for _, kind, _, _ in st)


def test_walk_steps_rejects_a_trace_out_of_order():
    disp = _dispatches("tensor", 2)
    disp[3] = ("gemm", "k", disp[3][2])        # a GEMM where a cast belongs
    with pytest.raises(SystemExit):
        bench.walk_steps(disp, 1, 1)


def test_kernel_kind():
    assert bench.kernel_kind("void fp8k::cast_kernel<1, 0>(fp8k::CastArgs)") == "cast"
    assert bench.kernel_kind("void fp8k::amax_partial_kernel<true>(HIP_vector_type<unsigned int, 4u> const*)") == "amax"
    assert bench.kernel_kind("void fp8k::tensor::gemm_tensor_kernel<0, 0, true>(fp8k::tensor::Args)") == "gemm"
    assert bench.kernel_kind("fp8k::splitk_reduce_kernel(float const*, int)") == "reduce"
    assert bench.kernel_kind("void at::native::vectorized_elementwise_kernel<4>") is None


def test_gemm_shapes_cover_the_bench_workloads():
    shapes = bench._bench_gemm_shapes()
    for N, K, M in ((131072, 512, 2048), (131072, 2048, 512), (16384, 8192, 8192), (262144, 512, 8192)):
        assert (N, M, K) in shapes and (N, K, M) in shapes and (M, K, N) in shapes
    assert (8192, 8192, 16384) in shapes


_SAMPLE = """GPU: 0
    POWER:
        SOCKET_POWER: 1397 W
        GFX_VOLTAGE: N/A
    CLOCK:
        GFX_0:
            CLK: 1787 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
        GFX_1:
            CLK: 1710 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
        MEM_0:
            CLK: 2000 MHz
"""


def test_amd_smi_sample_parser(monkeypatch):
    class R:
        stdout = _SAMPLE

    monkeypatch.setattr(subprocess, "run", lambda *a, **k: R())
    s = bench._amd_smi_sample()
    assert s == {"gfx_mhz": [1787, 1710], "socket_power_w": 1397}


def test_amd_smi_sample_missing_tool(monkeypatch):
    def boom(*a, **k):
        raise FileNotFoundError("amd-smi")

    monkeypatch.setattr(subprocess, "run", boom)
    assert bench._amd_smi_sample() is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) and not r.stdout.strip().startswith("{")
