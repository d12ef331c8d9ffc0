"""Host-side arithmetic of bench.py (CPU): the algorithmic byte and flop
counts its rooflines divide by, the profile staleness check, and the refusal
of a multi-GPU run.

The byte counts are pinned to the per-unit figures stated for the path, worked
out by hand here: the K-pass Newton forward reads xproj once per iteration
(K G values), reads and writes the iterate between iterations (2 (K - 1) S)
and writes h (1) per channel-token; the backward reads xproj (G), the
previous state (S) and dL/dh (1) and writes dL/dxproj (G)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from workloads import WORKLOADS  # noqa: E402


def test_newton_bytes_of_the_long_lstm():
    # 2 x 131072 tokens x 256 channels x (2*4 + 2*1*2 + 1 = 13 values) x 4 bytes
    w = WORKLOADS["lstm_t131k"]
    assert bench.algorithmic_newton_bytes(w) == 2 * 131072 * 256 * 13 * 4 == 3489660928


@pytest.mark.parametrize("name,values,elt", [
    ("gru_tiny", 3 * 3 + 2 * 2 * 1 + 1, 4),
    ("gru_d256", 3 * 3 + 2 * 2 * 1 + 1, 4),
    ("gru_bf16", 3 * 3 + 2 * 2 * 1 + 1, 2),
    ("gru_ragged", 3 * 3 + 2 * 2 * 1 + 1, 4),
])
def test_newton_bytes_of_the_gru_workloads(name, values, elt):
    w = WORKLOADS[name]
    assert bench.algorithmic_newton_bytes(w) == w.tokens * w.d_h * values * elt


def test_backward_bytes():
    w = WORKLOADS["lstm_t131k"]   # (2*4 + 2 + 1) values of 4 bytes: 44 bytes per channel-token
    assert bench.algorithmic_backward_bytes(w) == 2 * 131072 * 256 * 44
    g = WORKLOADS["gru_bf16"]     # (2*3 + 1 + 1) values of 2 bytes
    assert bench.algorithmic_backward_bytes(g) == g.tokens * g.d_h * 8 * 2


def test_projection_flops():
    w = WORKLOADS["lstm_t131k"]
    assert bench.proj_flops(w) == 2 * 262144 * 1024 * 256


def test_headmix_flops_count_the_block_products():
    # one (step, head): per iteration three 16 x 16 x 16 block products
    # (3 * 2 * 16^3) and four sets of three block matrix-vector products
    # (4 * 3 * 2 * 16^2); the final residual pass three more matrix-vector
    # products
    per_iter = 3 * 2 * 16 ** 3 + 4 * 3 * 2 * 16 ** 2
    assert bench.headmix_flops(8, 4096, 256, 3) == 8 * 4096 * 16 * (3 * per_iter + 3 * 2 * 16 ** 2)


def test_profiles_are_checked_against_their_sources():
    # every committed summary names the hash of the sources it was taken
    # from; a missing summary yields no fields
    assert bench.profile_fields("k_proj", "no_such_workload") == {}
    h = bench.kernel_source_hash("k_newton_sp")
    assert len(h) == 16 and h == bench.kernel_source_hash("k_newton_sp")
    assert h != bench.kernel_source_hash("k_proj")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
