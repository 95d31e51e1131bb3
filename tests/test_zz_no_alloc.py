"""The no-alloc step (qgalore_step_noalloc: the scratch is the library's fixed device array,
not a caller workspace) against the workspace step (qgalore_step), through the C ABI, on two
calls in a row, the second with a smaller layer: every output bit-identical. Also the size
limit, checked on the host before any HIP call."""
import ctypes

import numpy as np
import pytest

from oracle import qgalore_oracle as O
from quantized_rank_gradient_amd import workloads as WL
from tests import parity as PAR

torch = pytest.importorskip("torch")


def _B():
    from quantized_rank_gradient_amd import binding as B
    return B


def _outputs(Lt, R_out, U_out):
    out = {k: getattr(Lt, k).cpu().numpy() for k in ("Wq", "Mq", "Ms", "Vq", "Vs")}
    out["R"] = R_out.cpu().numpy()
    out["U"] = U_out.cpu().numpy()
    return out


@pytest.mark.gpu
def test_noalloc_step_matches_the_workspace_step_twice():
    B = _B()
    assert torch.cuda.is_available()
    # each call smaller than the one before; the last has odd rows (N~ rows padded in the scratch)
    for (m, n, r, t) in [(2048, 1536, 256, 2), (640, 392, 64, 3), (300, 333, 32, 4)]:
        cfg = WL.Config("custom", 9, (WL.LayerShape(5, f"{m}x{n}", m, n),), r=r, sigma=1e-3)
        L = cfg.layers[0]
        st, P = PAR.host_state(cfg, L, r, "random")
        G = WL.gradient_bf16(cfg, L, t)
        outs = {}
        for which in ("workspace", "noalloc"):
            Lt = PAR.to_device(st, G, P)
            R_out = torch.empty((r, n), dtype=torch.float32, device="cuda")
            U_out = torch.empty((m, n), dtype=torch.float32, device="cuda")
            hp = dict(lr=1e-3, alpha=0.25)
            if which == "workspace":
                B.step(Lt, t, WL.SR_SEED, hp=hp, R_out=R_out, U_out=U_out)
            else:
                B.step_noalloc(Lt, t, WL.SR_SEED, hp=hp, R_out=R_out, U_out=U_out)
            torch.cuda.synchronize()
            outs[which] = _outputs(Lt, R_out, U_out)
        for k in outs["workspace"]:
            assert np.array_equal(outs["noalloc"][k].view(np.uint8),
                                  outs["workspace"][k].view(np.uint8)), (m, n, r, k)
        before = st.copy()
        res = O.qgalore_step(st, G, t, WL.SR_SEED)
        PAR.check_step(before, res, st, outs["noalloc"], t=t)


@pytest.mark.gpu
def test_noalloc_step_without_u_matches_the_workspace_step():
    """Both entry points without U (the rounding's alpha-folded path), two calls in a row, the
    second smaller: every output bit-identical between them."""
    B = _B()
    assert torch.cuda.is_available()
    for (m, n, r, t) in [(1376, 512, 128, 2), (333, 517, 40, 3)]:
        cfg = WL.Config("custom", 9, (WL.LayerShape(6, f"{m}x{n}", m, n),), r=r, sigma=1e-3)
        L = cfg.layers[0]
        st, P = PAR.host_state(cfg, L, r, "random")
        G = WL.gradient_bf16(cfg, L, t)
        outs = {}
        for which in ("workspace", "noalloc"):
            Lt = PAR.to_device(st, G, P)
            R_out = torch.empty((r, n), dtype=torch.float32, device="cuda")
            hp = dict(lr=1e-3, alpha=0.25)
            if which == "workspace":
                B.step(Lt, t, WL.SR_SEED, hp=hp, R_out=R_out)
            else:
                B.step_noalloc(Lt, t, WL.SR_SEED, hp=hp, R_out=R_out)
            torch.cuda.synchronize()
            outs[which] = {k: getattr(Lt, k).cpu().numpy() for k in ("Wq", "Mq", "Ms", "Vq", "Vs")}
            outs[which]["R"] = R_out.cpu().numpy()
        for k in outs["workspace"]:
            assert np.array_equal(outs["noalloc"][k].view(np.uint8),
                                  outs["workspace"][k].view(np.uint8)), (m, n, r, k)


def test_noalloc_step_rejects_a_layer_beyond_its_scratch():
    """A layer whose scratch exceeds the fixed array: QG_ERR_WORKSPACE before any HIP call."""
    B = _B()
    d = B.LayerDesc()
    d.m, d.n, d.r, d.layer_id = 16384, 32768, 1024, 0   # N~ alone is 64 MiB
    d.lr, d.beta1, d.beta2, d.eps, d.alpha = 1e-3, 0.9, 0.999, 1e-8, 0.25
    fake = 0x10000
    d.M_scale = d.V_scale = fake
    need = B.lib().qgalore_layer_workspace_bytes(ctypes.byref(d))
    assert need > B.NOALLOC_SCRATCH_BYTES
    st = B.lib().qgalore_step_noalloc(ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake,
                                      1, 1234)
    assert st == 4
    assert b"scratch" in B.lib().qgalore_last_error()
