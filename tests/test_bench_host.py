"""Host-side checks of the benchmark: its FLOP and byte arithmetic, and that it
refuses a multi-GPU run before touching any device."""
from __future__ import annotations

import os
import subprocess
import sys
from types import SimpleNamespace

import pytest

import bench
from causal_self_attention_amd.inputs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (workload, forward FLOP, backward FLOP): 4*D and 10*D per visible (query,
# key) pair, B*H*T(T+1)/2 pairs per launch.
FLOPS = [
    ("shakespeare_char_f32_b1_h6_t256", 50_528_256, 126_320_640),
    ("shakespeare_char_bf16_b64_h6_t256", 3_233_808_384, 8_084_520_960),
    ("gpt2_124m_bf16_b12_h12_t1024", 19_346_227_200, 48_365_568_000),
    ("gpt2_350m_bf16_b12_h16_t1024", 25_794_969_600, 64_487_424_000),
    ("gpt2_774m_sharp_bf16_b8_h20_t1024", 21_495_808_000, 53_739_520_000),
    ("gpt2_1558m_bf16_b4_h25_t1024", 13_434_880_000, 33_587_200_000),
    ("gpt2_1558m_long_bf16_b2_h25_t2048", 26_856_652_800, 67_141_632_000),
]


@pytest.mark.parametrize("name,fwd,bwd", FLOPS)
def test_flop_counts(name, fwd, bwd):
    assert bench.flops(WORKLOADS[name]) == (fwd, bwd)


def test_decode_bytes_counts_rows_up_to_each_length():
    w = SimpleNamespace(B=2, H=3, D=64, dtype="bf16")
    # cache rows 5 + 7 per head, K and V, 2 bytes; q and O 2 bytes; LSE 4 bytes
    expect = (5 + 7) * 3 * 64 * 2 * 2 + 2 * 2 * 3 * 64 * 2 + 4 * 2 * 3
    assert bench.decode_bytes(w, [5, 7]) == expect
    w32 = SimpleNamespace(B=1, H=1, D=32, dtype="f32")
    assert bench.decode_bytes(w32, [0]) == 2 * 32 * 4 + 4


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused(args, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       env={**os.environ, **env}, capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_committed_traffic_record_matches_the_kernel_source():
    # The HBM-traffic record under profiles/ is keyed by a hash of the
    # backward-main sources; a record taken on other source is reported as
    # null by the benchmark, so the committed one must match the tree.
    rec = bench.load_traffic(0)
    assert rec is not None and rec > 0


def test_data_set_rotation_count():
    # Enough copies of a step's data to reach 1 GiB (four times the 256 MB
    # Infinity Cache), at most 16; an explicit count is taken as given.
    assert bench.n_sets(0, 227_600_000) == 5   # GPT-2 124M training step
    assert bench.n_sets(0, 201_326_592) == 6   # its 201 MB decode cache
    assert bench.n_sets(0, 3 << 30) == 1
    assert bench.n_sets(0, 1000) == 16
    assert bench.n_sets(1, 227_600_000) == 1
    assert bench.n_sets(3, 10) == 3


def test_host_cpu_description():
    info = bench.host_cpu()
    assert info["logical_cpus"] >= 1
    assert isinstance(info["cpu_model"], str) and info["cpu_model"]
    assert info["physical_cores"] is None or 1 <= info["physical_cores"] <= info["logical_cpus"]
    assert 1 <= bench.default_threads() <= 16


def test_every_benchmark_configuration_is_a_workload():
    for name in bench.ALL_CONFIGS:
        assert name in WORKLOADS
    assert bench.DEFAULT_WORKLOAD in bench.ALL_CONFIGS


def test_clock_probe_library_exports_its_launch():
    # Built beside the attention library by causal_self_attention_amd.build;
    # loading it needs no GPU.
    import ctypes
    assert os.path.exists(bench.PROBE_LIB), "build the libraries first"
    lib = ctypes.CDLL(bench.PROBE_LIB)
    assert hasattr(lib, "sclk_probe_launch")
