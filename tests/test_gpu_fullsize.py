"""Parity at full LLaMA-7B size in the launch configuration the benchmark times: one grouped
plan over all 224 layers. Sampled layers (one of each shape) are checked against the oracle:
the projected gradient R and the requantized moments in full, the back-projection and the
stochastic rounding on sampled weight rows. Step 1 starts from zero moments; step 3 runs on
the moments two earlier steps with other gradients left (INT8 codes with real scales). Step 1
also runs as the benchmark launches it (no U written anywhere) and must give the same codes."""
import numpy as np
import pytest

from oracle import qgalore_oracle as O
from quantized_rank_gradient_amd import workloads as WL
from tests import parity as PAR

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

SAMPLED = (0, 4, 223)        # q of block 0, gate of block 0, down of block 31


@pytest.mark.parametrize("key", ["llama7b_r128", "llama7b_r1024"])
def test_full_7b_plan_sampled_layers(key):
    from quantized_rank_gradient_amd import binding as B
    cfg = WL.CONFIGS[key]
    r = cfg.r
    dev = torch.device("cuda:0")
    layers, Ps_float = [], {}
    Rs, Us = [], []
    for k, L in enumerate(cfg.layers):
        G = WL.gradient_bf16_device(cfg, L, 1, device=dev)
        W = WL.weights_int8_device(cfg, L, device=dev)
        P = WL.orthonormal_device(cfg, L, r, device=dev)
        Pq, Ps = B.quantize_proj(P)
        if k in SAMPLED:
            Ps_float[k] = P.cpu().numpy()
        del P
        ng = B.n_groups(r * L.n)
        layers.append(B.LayerTensors(
            L.layer_id, G, W, torch.full((B.n_groups(L.m * L.n),), cfg.w_scale, device=dev),
            Pq, Ps, torch.zeros((r, L.n), dtype=torch.int8, device=dev),
            torch.zeros(ng, device=dev), torch.zeros((r, L.n), dtype=torch.int8, device=dev),
            torch.zeros(ng, device=dev), r))
        Rs.append(torch.empty((r, L.n), device=dev) if k in SAMPLED else None)
        Us.append(torch.empty((L.m, L.n), device=dev) if k in SAMPLED else None)
    # host copies of the sampled layers' inputs before the step changes them
    before = {}
    for k in SAMPLED:
        Lt = layers[k]
        before[k] = dict(G=Lt.G.view(torch.int16).cpu().numpy().view(np.uint16),
                         W=Lt.Wq.cpu().numpy(), Pq=Lt.Pq.cpu().numpy(), Ps=Lt.Ps.cpu().numpy())
    hp = dict(lr=cfg.lr, beta1=cfg.beta1, beta2=cfg.beta2, eps=cfg.eps, alpha=cfg.alpha)
    # First the benchmark's own launch: no layer writes U, so the rounding takes its
    # alpha-folded path. The sampled layers are then reset, and the step below (which writes
    # their U and takes the unfolded path) must give the same codes bit for bit.
    keys = ("Wq", "Mq", "Ms", "Vq", "Vs")
    saved = {k: {a: getattr(layers[k], a).clone() for a in keys} for k in SAMPLED}
    plan0 = B.Plan(layers, hp=hp)
    plan0.step(1, WL.SR_SEED)
    torch.cuda.synchronize()
    folded = {k: {a: getattr(layers[k], a).cpu().numpy() for a in keys} for k in SAMPLED}
    plan0.close()
    del plan0
    for k in SAMPLED:
        for a in keys:
            getattr(layers[k], a).copy_(saved[k][a])
    del saved
    plan = B.Plan(layers, hp=hp, R_out=Rs, U_out=Us)
    plan.step(1, WL.SR_SEED)
    torch.cuda.synchronize()
    for k in SAMPLED:
        for a in keys:
            assert np.array_equal(getattr(layers[k], a).cpu().numpy(), folded[k][a]), (k, a)
    rng = np.random.default_rng(0)
    for k in SAMPLED:
        L = cfg.layers[k]
        b = before[k]
        Pq_o, Ps_o = O.quantize_proj(Ps_float[k])
        assert np.array_equal(b["Pq"], Pq_o) and np.array_equal(b["Ps"], Ps_o)
        Mq, Ms, Vq, Vs = WL.zero_moments(r, L.n)
        st = O.LayerState(L.m, L.n, r, L.layer_id, b["W"].copy(), WL.weight_scales(cfg, L),
                          Pq_o, Ps_o, Mq, Ms, Vq, Vs)
        st0 = st.copy()
        rows = np.sort(rng.choice(L.m, size=48, replace=False))
        res = O.qgalore_step(st, b["G"], 1, WL.SR_SEED, rows=rows)
        Lt = layers[k]
        out = dict(R=Rs[k].cpu().numpy(), U=Us[k].cpu().numpy(), Wq=Lt.Wq.cpu().numpy(),
                   Mq=Lt.Mq.cpu().numpy(), Ms=Lt.Ms.cpu().numpy(), Vq=Lt.Vq.cpu().numpy(),
                   Vs=Lt.Vs.cpu().numpy())
        PAR.check_step(st0, res, st, out, rows=rows)

    # Steps 2 and 3 on fresh gradients, so that the moments hold INT8 codes with real group
    # scales: step 3 is checked from the state the GPU left after step 2.
    for t in (2, 3):
        for k, L in enumerate(cfg.layers):
            layers[k].G.copy_(WL.gradient_bf16_device(cfg, L, t, device=dev))
        if t == 3:
            for k in SAMPLED:
                Lt = layers[k]
                before[k] = dict(G=Lt.G.view(torch.int16).cpu().numpy().view(np.uint16),
                                 W=Lt.Wq.cpu().numpy(), Mq=Lt.Mq.cpu().numpy(),
                                 Ms=Lt.Ms.cpu().numpy(), Vq=Lt.Vq.cpu().numpy(),
                                 Vs=Lt.Vs.cpu().numpy())
        plan.step(t, WL.SR_SEED)
    torch.cuda.synchronize()
    for k in SAMPLED:
        L = cfg.layers[k]
        b = before[k]
        assert np.abs(b["Mq"]).max() > 1 and np.abs(b["Ms"]).max() > 0
        Pq_o, Ps_o = O.quantize_proj(Ps_float[k])
        st = O.LayerState(L.m, L.n, r, L.layer_id, b["W"].copy(), WL.weight_scales(cfg, L),
                          Pq_o, Ps_o, b["Mq"].copy(), b["Ms"].copy(), b["Vq"].copy(),
                          b["Vs"].copy())
        st0 = st.copy()
        rows = np.sort(rng.choice(L.m, size=48, replace=False))
        res = O.qgalore_step(st, b["G"], 3, WL.SR_SEED, rows=rows)
        Lt = layers[k]
        out = dict(R=Rs[k].cpu().numpy(), U=Us[k].cpu().numpy(), Wq=Lt.Wq.cpu().numpy(),
                   Mq=Lt.Mq.cpu().numpy(), Ms=Lt.Ms.cpu().numpy(), Vq=Lt.Vq.cpu().numpy(),
                   Vs=Lt.Vs.cpu().numpy())
        PAR.check_step(st0, res, st, out, rows=rows, t=3)
    plan.close()
