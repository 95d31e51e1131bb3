"""The adaptive refresh schedule on the drifting 7B workload, from its closed form.

Layer k of the 224-layer set turns its gradient's column space at rho_k = 0.05 k / 223 radians
per step, so the noise-free subspace similarity of refreshes at steps t and s is
|cos(rho_k (t - s))| (AIMech Q-GaLore page, mechanism claim "layer-adaptive subspace cosine
schedule", paper Section 3.1: the interval doubles while the similarity exceeds gamma = 0.4).
Run through the oracle's schedule over 200 steps from an interval of 25, the closed form fixes
the SVD count the GPU run must reproduce: 1037 refreshes against 1792 for the fixed interval
(42.1% saved), with 134 layers refreshed 4 times, 73 five times and 17 eight times."""
import math
from collections import Counter

from oracle import qgalore_oracle as O
from quantized_rank_gradient_amd import workloads as WL


def closed_form_counts():
    cfg = WL.CONFIGS["schedule7b"]
    counts = []
    for k in range(len(cfg.layers)):
        rho = WL.drift_rate(cfg, k)
        steps, _ = O.simulate_schedule(lambda t, s: abs(math.cos(rho * (t - s))),
                                       WL.SCHEDULE_DELTA0, cfg.steps, WL.SCHEDULE_GAMMA)
        counts.append(len(steps))
    return counts


def test_schedule_svd_count_from_the_closed_form():
    counts = closed_form_counts()
    fixed = len(counts) * O.fixed_interval_refreshes(WL.SCHEDULE_DELTA0, 200)
    assert len(counts) == 224
    assert fixed == 1792
    assert sum(counts) == 1037
    assert Counter(counts) == {4: 134, 5: 73, 8: 17}
    assert round(1 - sum(counts) / fixed, 3) == 0.421


def test_slow_layers_double_every_time_and_fast_layers_never():
    """Layer 0 does not drift: every test passes, intervals 25, 50, 100 give refreshes at
    0, 25, 75, 175. The fastest layer (0.05 rad/step) has |cos(1.25)| = 0.315 < 0.4 at a gap
    of 25, so it keeps the fixed interval: 8 refreshes."""
    cfg = WL.CONFIGS["schedule7b"]
    s0, d0 = O.simulate_schedule(lambda t, s: 1.0, 25, 200)
    assert s0 == [0, 25, 75, 175] and d0 == 200
    rho = WL.drift_rate(cfg, 223)
    assert abs(rho - 0.05) < 1e-15
    s1, d1 = O.simulate_schedule(lambda t, s: abs(math.cos(rho * (t - s))), 25, 200)
    assert s1 == list(range(0, 200, 25)) and d1 == 25
