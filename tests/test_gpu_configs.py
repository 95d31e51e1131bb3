"""Parity of one grouped optimizer step over whole LLaMA-shaped layer sets.

* LLaMA-60M shapes (8 blocks x {q, k, v, o 512x512; gate, up 1376x512; down 512x1376},
  rank 128): every one of the 56 layers is checked against the oracle in full (R, U, the
  moments and every weight).
* LLaMA-1B shapes (24 blocks x {2048x2048 x4; 5461x2048 x2; 2048x5461}, rank 512): one layer
  of each shape is checked, the moments in full and the weights on sampled rows. The down
  projection (n = 5461) has ragged rows, so this one plan mixes layers whose Adam runs in the
  projection kernel with layers that go through the separate Adam pass and the element-wise
  rounding path.
"""
import numpy as np
import pytest

from oracle import qgalore_oracle as O
from quantized_rank_gradient_amd import workloads as WL
from tests import parity as PAR

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _hp(cfg):
    return dict(lr=cfg.lr, beta1=cfg.beta1, beta2=cfg.beta2, eps=cfg.eps, alpha=cfg.alpha)


def test_llama60m_full_set_every_layer():
    from quantized_rank_gradient_amd import binding as B
    cfg = WL.CONFIGS["llama60m"]
    r = cfg.r
    states, devs, Gs = [], [], []
    for L in cfg.layers:
        st, P = PAR.host_state(cfg, L, r, "zero")
        G = WL.gradient_bf16(cfg, L, 1)
        states.append(st)
        devs.append(PAR.to_device(st, G, P, quantize_on_gpu=False))
        Gs.append(G)
    Rs = [torch.empty((r, L.n), dtype=torch.float32, device="cuda") for L in cfg.layers]
    Us = [torch.empty((L.m, L.n), dtype=torch.float32, device="cuda") for L in cfg.layers]
    plan = B.Plan(devs, hp=_hp(cfg), R_out=Rs, U_out=Us)
    plan.step(1, WL.SR_SEED)
    torch.cuda.synchronize()
    h = O.Hyper(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.alpha)
    for st, Lt, G, Ro, Uo in zip(states, devs, Gs, Rs, Us):
        before = st.copy()
        res = O.qgalore_step(st, G, 1, WL.SR_SEED, h)
        out = {k: getattr(Lt, k).cpu().numpy() for k in ("Wq", "Mq", "Ms", "Vq", "Vs")}
        out["R"] = Ro.cpu().numpy()
        out["U"] = Uo.cpu().numpy()
        PAR.check_step(before, res, st, out, hp=h)
    plan.close()


SAMPLED_1B = (0, 4, 167)     # q of block 0 (2048x2048), gate of block 0 (5461x2048), last down


def test_llama1b_plan_sampled_layers():
    from quantized_rank_gradient_amd import binding as B
    cfg = WL.CONFIGS["llama1b"]
    r = cfg.r
    dev = torch.device("cuda:0")
    layers, P_float, Rs, Us = [], {}, [], []
    for k, L in enumerate(cfg.layers):
        G = WL.gradient_bf16_device(cfg, L, 1, device=dev)
        W = WL.weights_int8_device(cfg, L, device=dev)
        P = WL.orthonormal_device(cfg, L, r, device=dev)
        Pq, Ps = B.quantize_proj(P)
        if k in SAMPLED_1B:
            P_float[k] = P.cpu().numpy()
        del P
        ng = B.n_groups(r * L.n)
        layers.append(B.LayerTensors(
            L.layer_id, G, W, torch.full((B.n_groups(L.m * L.n),), cfg.w_scale, device=dev),
            Pq, Ps, torch.zeros((r, L.n), dtype=torch.int8, device=dev),
            torch.zeros(ng, device=dev), torch.zeros((r, L.n), dtype=torch.int8, device=dev),
            torch.zeros(ng, device=dev), r))
        Rs.append(torch.empty((r, L.n), device=dev) if k in SAMPLED_1B else None)
        Us.append(torch.empty((L.m, L.n), device=dev) if k in SAMPLED_1B else None)
    before = {}
    for k in SAMPLED_1B:
        Lt = layers[k]
        before[k] = dict(G=Lt.G.view(torch.int16).cpu().numpy().view(np.uint16),
                         W=Lt.Wq.cpu().numpy(), Pq=Lt.Pq.cpu().numpy(), Ps=Lt.Ps.cpu().numpy())
    plan = B.Plan(layers, hp=_hp(cfg), R_out=Rs, U_out=Us)
    plan.step(1, WL.SR_SEED)
    torch.cuda.synchronize()
    h = O.Hyper(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.alpha)
    rng = np.random.default_rng(1)
    for k in SAMPLED_1B:
        L = cfg.layers[k]
        b = before[k]
        Pq_o, Ps_o = O.quantize_proj(P_float[k])
        assert np.array_equal(b["Pq"], Pq_o) and np.array_equal(b["Ps"], Ps_o)
        Mq, Ms, Vq, Vs = WL.zero_moments(r, L.n)
        st = O.LayerState(L.m, L.n, r, L.layer_id, b["W"].copy(), WL.weight_scales(cfg, L),
                          Pq_o, Ps_o, Mq, Ms, Vq, Vs)
        st0 = st.copy()
        rows = np.sort(rng.choice(L.m, size=48, replace=False))
        res = O.qgalore_step(st, b["G"], 1, WL.SR_SEED, h, rows=rows)
        Lt = layers[k]
        out = dict(R=Rs[k].cpu().numpy(), U=Us[k].cpu().numpy(), Wq=Lt.Wq.cpu().numpy(),
                   Mq=Lt.Mq.cpu().numpy(), Ms=Lt.Ms.cpu().numpy(), Vq=Lt.Vq.cpu().numpy(),
                   Vs=Lt.Vs.cpu().numpy())
        PAR.check_step(st0, res, st, out, hp=h, rows=rows)
    plan.close()
