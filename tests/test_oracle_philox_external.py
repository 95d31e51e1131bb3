"""External pin of the oracle's Philox4x32-10: rocRAND's Philox engine (compiled from its
public header for the host CPU) on random keys and counters, including the counter layout
(j >> 3, i, t, layer) the stochastic rounding uses."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import qgalore_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    hipcc = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")
    if not hipcc or not os.path.exists("/opt/rocm/include/rocrand/rocrand_kernel.h"):
        pytest.skip("hipcc or rocRAND headers not available")
    exe = str(tmp_path_factory.mktemp("rr") / "rocrand_philox_ref")
    res = subprocess.run([hipcc, "-O1", os.path.join(HERE, "rocrand_philox_ref.cpp"), "-o", exe],
                         capture_output=True, text=True)
    if res.returncode != 0:
        pytest.skip("could not build the rocRAND reference: " + res.stderr[-400:])
    return exe


def test_philox_matches_rocrand_engine(rocrand_ref):
    rng = np.random.default_rng(2024)
    n = 2000
    seeds = rng.integers(0, 2 ** 63, size=n, dtype=np.int64).astype(np.uint64)
    seeds[:3] = [0, 1234, 2 ** 64 - 1]
    ctr = rng.integers(0, 2 ** 32, size=(n, 4), dtype=np.uint64)
    # rocRAND addresses counter words 0-1 through a 64-bit element offset (4 per counter),
    # so word 1 must stay below 2^30 to be reachable
    ctr[:, 1] >>= np.uint64(2)
    ctr[:3] = 0
    lines = "\n".join(f"{int(s)} {c[0]} {c[1]} {c[2]} {c[3]}" for s, c in zip(seeds, ctr))
    out = subprocess.run([rocrand_ref], input=lines, capture_output=True, text=True, check=True)
    got = np.array([[int(v) for v in ln.split()] for ln in out.stdout.strip().splitlines()],
                   dtype=np.uint64)
    want = np.stack([O.philox4x32_10(c[None, :], (int(s) & 0xFFFFFFFF, int(s) >> 32))[0]
                     for s, c in zip(seeds, ctr)]).astype(np.uint64)
    assert got.shape == want.shape
    assert np.array_equal(got, want)


def test_sr_uniform_counter_layout_matches_rocrand(rocrand_ref):
    """u(seed, t, layer, i, j) is half of word (j >> 1) & 3 of Philox at counter
    (j >> 3, i, t, layer): checked through rocRAND's engine."""
    rng = np.random.default_rng(7)
    seed, t, layer = 1234, 17, 42
    i = rng.integers(0, 11008, size=300)
    j = rng.integers(0, 11008, size=300)
    lines = "\n".join(f"{seed} {jj >> 3} {ii} {t} {layer}" for ii, jj in zip(i, j))
    out = subprocess.run([rocrand_ref], input=lines, capture_output=True, text=True, check=True)
    words = np.array([[int(v) for v in ln.split()] for ln in out.stdout.strip().splitlines()],
                     dtype=np.uint64)
    w = words[np.arange(300), (j >> 1) & 3]
    bits = np.where(j & 1, w >> 16, w & 0xFFFF)
    want = bits.astype(np.float64) / 65536.0
    got = O.sr_uniform(seed, t, layer, i, j).astype(np.float64)
    assert np.array_equal(got, want)
