"""The back-projection's alpha fold on the GPU. A step that does not write U, with alpha a
power of two no larger than one, rounds with S * fl(alpha / s) in place of fl(alpha S) / s;
outside the subnormal range the two are the same number (tests/test_kernel_numerics.py), so
the INT8 codes must come out bit for bit as in the same step with U requested (which takes
the unfolded path), and R, M and V are untouched by the choice. The folded codes are also
checked against the oracle with the unfolded run's U."""
import numpy as np
import pytest

from oracle import qgalore_oracle as O
from quantized_rank_gradient_amd import workloads as WL
from tests import parity as PAR

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

KEYS = ("Wq", "Mq", "Ms", "Vq", "Vs")


def _B():
    from quantized_rank_gradient_amd import binding as B
    return B


def _cfg(m, n, r, sigma=1e-3, layer_id=3):
    return WL.Config("custom", 9, (WL.LayerShape(layer_id, f"{m}x{n}", m, n),), r=r, sigma=sigma)


def _run(st, G, P, t, hp, with_u):
    B = _B()
    Lt = PAR.to_device(st, G, P)
    R_out = torch.empty((st.r, st.n), dtype=torch.float32, device="cuda")
    U_out = torch.empty((st.m, st.n), dtype=torch.float32, device="cuda") if with_u else None
    B.step(Lt, t, WL.SR_SEED, hp=hp, R_out=R_out, U_out=U_out)
    torch.cuda.synchronize()
    out = {k: getattr(Lt, k).cpu().numpy() for k in KEYS}
    out["R"] = R_out.cpu().numpy()
    if with_u:
        out["U"] = U_out.cpu().numpy()
    return out


@pytest.mark.parametrize("m,n,r,alpha", [
    (512, 512, 128, 0.25),     # small back-projection tile, vector rounding path
    (1376, 512, 128, 0.25),    # row tail of the tile grid
    (2048, 5461, 64, 0.25),    # odd n: element-wise rounding path
    (300, 200, 64, 0.5),       # ragged everywhere, groups straddling rows
    (640, 512, 256, 1.0),      # large tile; alpha = 1 folds as well
    (4096, 256, 1024, 0.25),   # rank 1024: 32 back-projection stages
    (512, 512, 128, 0.3),      # not a power of two: both runs take the unfolded path
    (512, 512, 128, 2.0),      # above one: not folded either
])
def test_step_without_u_gives_the_same_codes(m, n, r, alpha):
    print(f"[alpha fold] step {m}x{n} r={r} alpha={alpha}", flush=True)
    cfg = _cfg(m, n, r)
    L = cfg.layers[0]
    st, P = PAR.host_state(cfg, L, r, "random")
    t = 3
    G = WL.gradient_bf16(cfg, L, t)
    hp = dict(lr=1e-3, alpha=alpha)
    with_u = _run(st, G, P, t, hp, True)
    without_u = _run(st, G, P, t, hp, False)
    for k in KEYS + ("R",):
        assert np.array_equal(with_u[k].view(np.uint8), without_u[k].view(np.uint8)), k
    before = st.copy()
    res = O.qgalore_step(st, G, t, WL.SR_SEED, O.Hyper(alpha=alpha))
    PAR.check_step(before, res, st, dict(without_u, U=with_u["U"]), hp=O.Hyper(alpha=alpha), t=t)


def test_non_finite_rounding_inputs_folded():
    """The non-finite cases of the rounding (scales 1e-45, 3e-39 and 1.5e-38 in the first three
    groups, |U| of order 1) give the same codes with and without U: where fl(alpha S) / s is not
    finite, S * fl(alpha / s) is not finite either, and both keep the old code."""
    for n in (256, 200):
        cfg = _cfg(256, n, 32, sigma=1e-2)
        L = cfg.layers[0]
        st, P = PAR.host_state(cfg, L, 32, "zero")
        st.Ws[:] = 1.0
        st.Ws[0] = 1e-45
        st.Ws[1] = 3e-39
        st.Ws[2] = 1.5e-38
        G = WL.gradient_bf16(cfg, L, 1)
        hp = dict(lr=10.0, alpha=0.25)
        a = _run(st, G, P, 1, hp, True)
        b = _run(st, G, P, 1, hp, False)
        assert np.array_equal(a["Wq"], b["Wq"]), n
        assert np.array_equal(a["Wq"].ravel()[:256], st.Wq.ravel()[:256])


def test_plan_without_u_gives_the_same_codes():
    """A grouped step over mixed shapes (both back-projection tiles' rounding paths) without U
    against the same plan with U."""
    B = _B()
    shapes = [(512, 512), (1376, 512), (512, 1376), (300, 200)]
    r = 64
    cfg = WL.Config("mixed", 8, tuple(WL.LayerShape(k, "l", m, n)
                                       for k, (m, n) in enumerate(shapes)), r=r, sigma=1e-3)
    t = 2
    outs = []
    for with_u in (True, False):
        devs = []
        for L in cfg.layers:
            st, P = PAR.host_state(cfg, L, r, "random")
            devs.append(PAR.to_device(st, WL.gradient_bf16(cfg, L, t), P))
        Us = ([torch.empty((L.m, L.n), dtype=torch.float32, device="cuda") for L in cfg.layers]
              if with_u else None)
        plan = B.Plan(devs, hp=dict(lr=1e-3, alpha=0.25), U_out=Us)
        plan.step(t, WL.SR_SEED)
        torch.cuda.synchronize()
        outs.append([{k: getattr(Lt, k).cpu().numpy() for k in KEYS} for Lt in devs])
        plan.close()
    for a, b in zip(*outs):
        for k in KEYS:
            assert np.array_equal(a[k], b[k]), k
