"""The projection stored as INT8 codes or as bf16 values instead of INT4 codes (the
comparison formats of the Q-GaLore pages: the 8-bit projection of the Q-GaLore baseline and
GaLore's 16-bit one), through the same step and similarity kernels, against the oracle."""
import numpy as np
import pytest

from oracle import qgalore_oracle as O
from quantized_rank_gradient_amd import workloads as WL
from tests import parity as PAR

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

from tests.test_gpu_step import custom_cfg, gpu_step, snapshot   # noqa: E402


@pytest.mark.parametrize("m,r", [(256, 32), (1376, 128), (7, 8), (4096, 1024)])
def test_quantize_proj_int8_bit_exact(m, r):
    from quantized_rank_gradient_amd import binding as B
    P = (np.random.default_rng(m + r).standard_normal((m, r)) / np.sqrt(m)).astype(np.float32)
    Pq, Ps = B.quantize_proj(torch.from_numpy(P).cuda(), fmt="int8")
    want_q, want_s = O.quantize_proj(P, "int8")
    assert np.array_equal(Pq.cpu().numpy(), want_q)
    assert np.array_equal(Ps.cpu().numpy(), want_s)


CASES = [
    (512, 512, 128, "zero", 1),       # Adam in the projection kernel
    (300, 200, 64, "random", 3),      # ragged rows: separate Adam pass, element-wise rounding
    (4096, 256, 1024, "random", 2),   # rank 1024
]


@pytest.mark.parametrize("fmt", ["int8", "bf16"])
@pytest.mark.parametrize("m,n,r,moments,t", CASES)
def test_step_with_projection_format(fmt, m, n, r, moments, t):
    cfg = custom_cfg(m, n, r)
    L = cfg.layers[0]
    st, P = PAR.host_state(cfg, L, r, moments, fmt=fmt)
    G = WL.gradient_bf16(cfg, L, t)
    Lt = PAR.to_device(st, G, P, quantize_on_gpu=False)
    before = st.copy()
    res = O.qgalore_step(st, G, t, WL.SR_SEED)
    out = gpu_step(Lt, t)
    PAR.check_step(before, res, st, out, t=t)


def test_plan_mixing_projection_formats():
    from quantized_rank_gradient_amd import binding as B
    shapes = [(512, 512, "int4"), (512, 1376, "int8"), (1376, 512, "bf16"), (300, 200, "bf16")]
    r = 64
    cfg = WL.Config("formats", 8, tuple(WL.LayerShape(k, "l", m, n)
                                        for k, (m, n, _) in enumerate(shapes)), r=r, sigma=1e-3)
    t = 2
    states, devs, Gs = [], [], []
    for L, (_, _, fmt) in zip(cfg.layers, shapes):
        st, P = PAR.host_state(cfg, L, r, "random", fmt=fmt)
        G = WL.gradient_bf16(cfg, L, t)
        states.append(st)
        devs.append(PAR.to_device(st, G, P, quantize_on_gpu=False))
        Gs.append(G)
    Rs = [torch.empty((r, L.n), dtype=torch.float32, device="cuda") for L in cfg.layers]
    Us = [torch.empty((L.m, L.n), dtype=torch.float32, device="cuda") for L in cfg.layers]
    plan = B.Plan(devs, hp=dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, alpha=0.25),
                  R_out=Rs, U_out=Us)
    plan.step(t, WL.SR_SEED)
    torch.cuda.synchronize()
    for st, Lt, G, Ro, Uo in zip(states, devs, Gs, Rs, Us):
        before = st.copy()
        res = O.qgalore_step(st, G, t, WL.SR_SEED)
        PAR.check_step(before, res, st, snapshot(Lt, Ro, Uo), t=t)
    plan.close()


@pytest.mark.parametrize("fmt", ["int8", "bf16"])
@pytest.mark.parametrize("m,r", [(512, 64), (4096, 128), (2048, 512)])
def test_cossim_with_projection_format(fmt, m, r):
    from quantized_rank_gradient_amd import binding as B
    rng = np.random.default_rng(m * 3 + r)
    full = np.linalg.qr(rng.standard_normal((m, 2 * r)))[0]
    A0, A1 = full[:, :r], full[:, r:]
    cases = (A0, A0 * np.cos(1.159) + A1 * np.sin(1.159),
             np.linalg.qr(rng.standard_normal((m, r)))[0])

    def dev(x):
        if x is None:
            return None
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:       # bf16 bit patterns
            return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(x).cuda()

    qa, sa = O.quantize_proj(A0.astype(np.float32), fmt)
    for Pb in cases:
        qb, sb = O.quantize_proj(Pb.astype(np.float32), fmt)
        want = O.cossim(qa, sa, qb, sb, m, r, fmt)
        got = B.cossim(dev(qa), dev(sa), dev(qb), dev(sb), m, r, fmt=fmt)
        assert abs(got - want) <= 1e-4, (fmt, got, want)
