"""The adaptive refresh schedule on LLaMA-7B shapes (224 layers, rank 128, 200 steps) over
drifting low-rank gradients (workloads: layer k turns its subspace at 0.05 k / 223 rad per
step; the refresh interval starts at 25 and doubles when CosSim > 0.4).

Checked against the oracle: every similarity test the GPU makes (same INT4 projections, to
1e-4, with the same decision unless the oracle's value lies within 1e-4 of gamma), each layer's
refresh count replayed through the oracle's schedule with the oracle's similarity values, and
one optimizer step of three layers at a few steps (from the GPU's state at that step). The
similarities also follow the workload's closed form |cos(rho (t - s))| up to the INT4
quantization and the noise. Prints the SVDs saved against the fixed interval of 25.
"""
import math

import numpy as np
import pytest

from oracle import qgalore_oracle as O
from quantized_rank_gradient_amd import workloads as WL
from tests import parity as PAR

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

SAMPLED = (0, 4, 223)          # q of block 0, gate of block 0, down of the last block
CHECK_STEPS = (0, 25, 199)     # first step, the first refresh test, the last step


def test_adaptive_schedule_on_drifting_7b_gradients():
    from quantized_rank_gradient_amd.schedule_run import ScheduleRun
    cfg = WL.CONFIGS["schedule7b"]
    r = cfg.r
    h = O.Hyper(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.alpha)
    run = ScheduleRun(cfg, debug_layers=SAMPLED)
    tests = {}                 # (layer, t) -> (gpu value, oracle value, step of the old P)

    def on_test(k, t, cs, new, old, t_old):
        L = cfg.layers[k]
        qn, sn = (x.cpu().numpy() for x in new)
        qo, so = (x.cpu().numpy() for x in old)
        tests[(k, t)] = (cs, O.cossim(qn, sn, qo, so, L.m, r), t_old)

    snaps = {}

    def before_step(t):
        if t in CHECK_STEPS:
            for k in SAMPLED:
                Lt = run.layers[k]
                snaps[(k, t)] = dict(
                    G=Lt.G.view(torch.int16).cpu().numpy().view(np.uint16),
                    **{a: getattr(Lt, a).cpu().numpy().copy()
                       for a in ("Wq", "Ws", "Pq", "Ps", "Mq", "Ms", "Vq", "Vs")})

    results = []

    def after_step(t):
        if t not in CHECK_STEPS:
            return
        rng = np.random.default_rng(t)
        for k in SAMPLED:
            L = cfg.layers[k]
            s = snaps.pop((k, t))
            st = O.LayerState(L.m, L.n, r, L.layer_id, s["Wq"], s["Ws"], s["Pq"], s["Ps"],
                              s["Mq"], s["Ms"], s["Vq"], s["Vs"])
            st0 = st.copy()
            rows = np.sort(rng.choice(L.m, size=32, replace=False))
            res = O.qgalore_step(st, s["G"], t + 1, WL.SR_SEED, h, rows=rows)
            Lt = run.layers[k]
            out = dict(R=run.R_out[k].cpu().numpy(), U=run.U_out[k].cpu().numpy(),
                       **{a: getattr(Lt, a).cpu().numpy() for a in ("Wq", "Mq", "Ms", "Vq", "Vs")})
            results.append(PAR.check_step(st0, res, st, out, hp=h, rows=rows, t=t + 1))

    summary = run.run(on_test=on_test, before_step=before_step, after_step=after_step)
    run.close()
    assert len(results) == len(SAMPLED) * len(CHECK_STEPS)

    # every similarity test against the oracle on the same INT4 projections
    assert tests, "no similarity tests ran"
    worst = 0.0
    for (k, t), (cs, want, _) in tests.items():
        worst = max(worst, abs(cs - want))
        assert abs(cs - want) <= 1e-4, (k, t, cs, want)
        if abs(want - WL.SCHEDULE_GAMMA) > 1e-4:
            assert (cs > WL.SCHEDULE_GAMMA) == (want > WL.SCHEDULE_GAMMA), (k, t, cs, want)

    # each layer's refresh count, replayed through the oracle's schedule on the oracle's values
    for k in range(len(cfg.layers)):
        def cs_fn(t_new, t_old, k=k):
            return tests[(k, t_new)][1]
        steps, _ = O.simulate_schedule(cs_fn, WL.SCHEDULE_DELTA0, cfg.steps, WL.SCHEDULE_GAMMA)
        assert len(steps) == summary["per_layer_counts"][k], k

    # the workload's closed form, up to INT4 quantization and the gradient noise
    dev_cf = max(abs(cs - abs(math.cos(WL.drift_rate(cfg, k) * (t - t_old))))
                 for (k, t), (cs, _, t_old) in tests.items())
    assert dev_cf <= 0.05, dev_cf
    print(f"\nadaptive schedule: {summary['svds']} SVDs vs {summary['svds_fixed_interval']} at a "
          f"fixed interval ({100 * summary['svds_saved']:.1f}% saved), "
          f"{summary['similarity_tests']} tests, max |GPU - oracle| {worst:.2e}, "
          f"max deviation from |cos(rho dt)| {dev_cf:.3f}, times {summary['seconds']}")
