"""GPU parity of the Q-GaLore step: the library's HIP kernels against the CPU oracle on the
same seeded inputs, through the C ABI. Rules are in tests/parity.py."""
import numpy as np
import pytest

from oracle import qgalore_oracle as O
from quantized_rank_gradient_amd import workloads as WL
from tests import parity as PAR

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _B():
    from quantized_rank_gradient_amd import binding as B
    return B


def gpu_step(Lt, t, seed=WL.SR_SEED, hp=None):
    B = _B()
    R_out = torch.empty((Lt.r, Lt.n), dtype=torch.float32, device="cuda")
    U_out = torch.empty((Lt.m, Lt.n), dtype=torch.float32, device="cuda")
    h = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, alpha=0.25)
    h.update(hp or {})
    B.step(Lt, t, seed, hp=h, R_out=R_out, U_out=U_out)
    torch.cuda.synchronize()
    return snapshot(Lt, R_out, U_out)


def snapshot(Lt, R_out=None, U_out=None):
    out = {k: getattr(Lt, k).cpu().numpy() for k in ("Wq", "Mq", "Ms", "Vq", "Vs")}
    if R_out is not None:
        out["R"] = R_out.cpu().numpy()
    if U_out is not None:
        out["U"] = U_out.cpu().numpy()
    return out


def custom_cfg(m, n, r, sigma=1e-3):
    return WL.Config("custom", 9, (WL.LayerShape(3, f"{m}x{n}", m, n),), r=r, sigma=sigma)


# ------------------------------------------------------------------ INT4 quantizer ---

@pytest.mark.parametrize("m,r", [(256, 32), (1376, 128), (5461, 512), (7, 9), (4096, 1024)])
def test_quantize_proj_bit_exact(m, r):
    B = _B()
    rng = np.random.default_rng(m * 131 + r)
    P = np.linalg.qr(rng.standard_normal((m, min(r, m))))[0]
    if P.shape[1] < r:
        P = np.concatenate([P, rng.standard_normal((m, r - P.shape[1])) * 0.1], axis=1)
    P = P.astype(np.float32)
    P[: min(m, 3)] = 0.0                         # a zero run: a zero-scale group when r is small
    Pq_o, Ps_o = O.quantize_proj(P)
    Pq_g, Ps_g = B.quantize_proj(torch.from_numpy(P).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(Ps_g.cpu().numpy(), Ps_o)
    assert np.array_equal(Pq_g.cpu().numpy(), Pq_o)


# ------------------------------------------------------------------- step parity ---

CASES = [
    # m, n, r, moments, t
    (512, 512, 128, "zero", 1),        # LLaMA-60M attention shape, first step
    (1376, 512, 128, "random", 3),     # gate/up shape: m not a multiple of the 128 tile
    (512, 1376, 128, "random", 2),     # down shape: n ragged, scale groups straddle rows
    (300, 200, 64, "random", 5),       # ragged everywhere, short last groups
    (2048, 5461, 64, "random", 2),     # odd n: unaligned rows take the element-wise path
    (384, 1378, 64, "random", 2),      # n = 2 (mod 8): G rows 4-byte aligned, N~ rows padded
    (333, 517, 40, "random", 3),       # odd m and n, rank not a multiple of 32
    (5461, 256, 32, "zero", 1),        # odd m: K tail of the projection, row tail of W
    (64, 40, 8, "random", 2),          # smallest rank
    (24, 13, 16, "random", 3),         # tiny, odd n, a single short group
    (128, 96, 128, "random", 2),       # full rank r = m
    (4096, 256, 1024, "random", 4),    # rank 1024: eight projection row tiles
    # back-projection K loops (K = r, 32 per stage) ending at each position of the LDS ring:
    (256, 512, 96, "random", 3),       # small tile, two buffers, 3 stages
    (384, 768, 192, "zero", 1),        # large tile, three buffers, 6 stages
    (640, 512, 224, "random", 2),      # large tile, 7 stages
]


@pytest.mark.parametrize("m,n,r,moments,t", CASES)
def test_step_matches_oracle(m, n, r, moments, t):
    cfg = custom_cfg(m, n, r)
    L = cfg.layers[0]
    st, P = PAR.host_state(cfg, L, r, moments)
    G = WL.gradient_bf16(cfg, L, t)
    Lt = PAR.to_device(st, G, P)
    assert np.array_equal(Lt.Pq.cpu().numpy(), st.Pq)
    before = st.copy()
    res = O.qgalore_step(st, G, t, WL.SR_SEED)
    out = gpu_step(Lt, t)
    PAR.check_step(before, res, st, out, t=t)


def test_single256_ten_steps_each_from_the_oracle_state():
    """The 256 x 256, rank-32 layer for ten steps. Before every step the GPU state is reset to
    the oracle's, so every step is compared on identical inputs (moments non-zero from t = 2)."""
    cfg = WL.CONFIGS["single256"]
    L = cfg.layers[0]
    st, P = PAR.host_state(cfg, L, cfg.r, "zero")
    flips = 0
    for t in range(1, cfg.steps + 1):
        G = WL.gradient_bf16(cfg, L, t)
        Lt = PAR.to_device(st, G, P)
        before = st.copy()
        res = O.qgalore_step(st, G, t, WL.SR_SEED)
        out = gpu_step(Lt, t)
        flips += PAR.check_step(before, res, st, out, t=t)
    assert flips <= max(1, 1e-4 * cfg.steps * L.m * L.n)


def test_zero_gradient_leaves_weights_and_moments_unchanged():
    cfg = custom_cfg(512, 384, 64)
    L = cfg.layers[0]
    st, P = PAR.host_state(cfg, L, 64, "zero")
    Lt = PAR.to_device(st, np.zeros((L.m, L.n), np.uint16), P)
    out = gpu_step(Lt, 1)
    assert np.array_equal(out["Wq"], st.Wq)
    assert not out["Mq"].any() and not out["Vq"].any() and not out["Ms"].any()


def test_step_is_deterministic():
    cfg = custom_cfg(1376, 512, 128)
    L = cfg.layers[0]
    st, P = PAR.host_state(cfg, L, 128, "random")
    G = WL.gradient_bf16(cfg, L, 2)
    a = gpu_step(PAR.to_device(st, G, P), 2)
    b = gpu_step(PAR.to_device(st, G, P), 2)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_clamp_and_zero_scale_groups():
    """A large update saturates at +-127; a zero weight scale leaves its group untouched."""
    cfg = custom_cfg(256, 256, 32, sigma=1e-2)
    L = cfg.layers[0]
    st, P = PAR.host_state(cfg, L, 32, "zero")
    st.Ws[:] = 1e-7                    # tiny scales: |U|/s >> 127
    st.Ws[5] = 0.0
    G = WL.gradient_bf16(cfg, L, 1)
    Lt = PAR.to_device(st, G, P)
    before = st.copy()
    res = O.qgalore_step(st, G, 1, WL.SR_SEED)
    out = gpu_step(Lt, 1)
    PAR.check_step(before, res, st, out)
    assert np.all(np.abs(out["Wq"]).max() == 127)
    assert np.array_equal(out["Wq"].ravel()[5 * 256:6 * 256], before.Wq.ravel()[5 * 256:6 * 256])


# --------------------------------------------------------------------- grouped step ---

def test_plan_matches_oracle_over_mixed_layers():
    B = _B()
    shapes = [(512, 512), (1376, 512), (512, 1376), (300, 200)]
    r = 64
    cfg = WL.Config("mixed", 8, tuple(WL.LayerShape(k, "l", m, n) for k, (m, n) in enumerate(shapes)),
                    r=r, sigma=1e-3)
    t = 2
    states, devs, Gs = [], [], []
    for L in cfg.layers:
        st, P = PAR.host_state(cfg, L, r, "random")
        G = WL.gradient_bf16(cfg, L, t)
        states.append(st)
        devs.append(PAR.to_device(st, G, P))
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


def test_plans_in_turn_share_one_workspace():
    """Two plans over windows of a layer set, stepped one after the other on one stream with
    one workspace of the larger size (no synchronization between them): every layer matches
    the oracle."""
    B = _B()
    shapes = [(512, 1376), (1376, 512), (300, 200), (512, 512)]
    r = 64
    cfg = WL.Config("mixed", 8, tuple(WL.LayerShape(k, "l", m, n) for k, (m, n) in enumerate(shapes)),
                    r=r, sigma=1e-3)
    t = 2
    states, devs, Gs = [], [], []
    for L in cfg.layers:
        st, P = PAR.host_state(cfg, L, r, "random")
        G = WL.gradient_bf16(cfg, L, t)
        states.append(st)
        devs.append(PAR.to_device(st, G, P))
        Gs.append(G)
    Rs = [torch.empty((r, L.n), dtype=torch.float32, device="cuda") for L in cfg.layers]
    Us = [torch.empty((L.m, L.n), dtype=torch.float32, device="cuda") for L in cfg.layers]
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, alpha=0.25)
    plans = [B.Plan(devs[a:b], hp=hp, R_out=Rs[a:b], U_out=Us[a:b]) for a, b in ((0, 2), (2, 4))]
    ws = B.alloc_workspace(max(p.workspace_bytes for p in plans))
    for p in plans:
        p.step(t, WL.SR_SEED, ws)
    torch.cuda.synchronize()
    for st, Lt, G, Ro, Uo in zip(states, devs, Gs, Rs, Us):
        before = st.copy()
        res = O.qgalore_step(st, G, t, WL.SR_SEED)
        PAR.check_step(before, res, st, snapshot(Lt, Ro, Uo), t=t)
    for p in plans:
        p.close()


def test_plan_kept_projections_match_fresh_dequant():
    """With dequantized projections kept between steps, three steps in which one layer's P is
    replaced (and reported) before the third give the same state, bit for bit, as a plan that
    dequantizes every projection at every step."""
    B = _B()
    shapes = [(512, 512), (1376, 512), (512, 1376)]
    r = 64
    cfg = WL.Config("mixed", 8, tuple(WL.LayerShape(k, "l", m, n) for k, (m, n) in enumerate(shapes)),
                    r=r, sigma=1e-3)
    runs = []
    for keep in (False, True):
        devs = []
        for L in cfg.layers:
            st, P = PAR.host_state(cfg, L, r, "random")
            devs.append(PAR.to_device(st, WL.gradient_bf16(cfg, L, 1), P))
        plan = B.Plan(devs, hp=dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, alpha=0.25))
        if keep:
            plan.cache_proj(True)
        ws = B.alloc_workspace(plan.workspace_bytes)
        for t in (1, 2, 3):
            if t == 3:   # a refresh replaces layer 1's projection
                rng = np.random.default_rng(77)
                Pn = np.linalg.qr(rng.standard_normal((shapes[1][0], r)))[0].astype(np.float32)
                q, sc = B.quantize_proj(torch.from_numpy(Pn).cuda())
                devs[1].Pq.copy_(q)
                devs[1].Ps.copy_(sc)
                if keep:
                    plan.proj_changed(1)
            plan.step(t, WL.SR_SEED, ws)
        torch.cuda.synchronize()
        runs.append([snapshot(Lt) for Lt in devs])
        plan.close()
    for a, b in zip(*runs):
        for k in a:
            assert np.array_equal(a[k], b[k]), k


# ------------------------------------------------------------------------- CosSim ---

def test_cossim_batch_of_mixed_row_counts():
    """One batched call over pairs with different m (same r) equals the oracle per pair."""
    B = _B()
    r = 128
    pairs, want = [], []
    for k, m in enumerate((512, 4096, 1376, 11008, 4096)):
        rng = np.random.default_rng(100 + k)
        A = np.linalg.qr(rng.standard_normal((m, r)))[0].astype(np.float32)
        Bm = np.linalg.qr(A + 0.6 * k * rng.standard_normal((m, r)) / np.sqrt(m))[0].astype(np.float32)
        qa, sa = O.quantize_proj(Bm)
        qb, sb = O.quantize_proj(A)
        want.append(O.cossim(qa, sa, qb, sb, m, r))
        pairs.append(tuple(torch.from_numpy(x).cuda() for x in (qa, sa, qb, sb)) + (m,))
    out = torch.full((len(pairs),), -1.0, device="cuda")
    B.cossim_batch(pairs, r, out)
    got = out.cpu().numpy()
    assert np.all(np.abs(got - np.array(want)) <= 1e-4), (got, want)

@pytest.mark.parametrize("r", [1024, 968])
def test_cossim_batch_large_rank(r):
    """A batch of eight pairs at rank 1024, and at 968 (ragged edge tiles): the cross product
    on 128-edge tiles with split-K; similarities from near 0 to 1."""
    B = _B()
    m = r + 8 * 44
    pairs, want = [], []
    for k in range(8):
        rng = np.random.default_rng(500 + k)
        A = np.linalg.qr(rng.standard_normal((m, r)))[0].astype(np.float32)
        Bm = np.linalg.qr(A + 0.25 * k * rng.standard_normal((m, r)) / np.sqrt(m))[0].astype(np.float32)
        qa, sa = O.quantize_proj(Bm)
        qb, sb = O.quantize_proj(A)
        want.append(O.cossim(qa, sa, qb, sb, m, r))
        pairs.append(tuple(torch.from_numpy(x).cuda() for x in (qa, sa, qb, sb)) + (m,))
    out = torch.full((len(pairs),), -1.0, device="cuda")
    B.cossim_batch(pairs, r, out)
    got = out.cpu().numpy()
    assert np.all(np.abs(got - np.array(want)) <= 1e-4), (got, want)


@pytest.mark.parametrize("m,r", [(600, 40), (512, 64), (1000, 96), (4096, 128), (2048, 512),
                                 (1376, 264), (4096, 1024)])
def test_cossim_matches_oracle(m, r):
    B = _B()
    rng = np.random.default_rng(m + r)
    full = np.linalg.qr(rng.standard_normal((m, 2 * r)))[0]
    A0, A1 = full[:, :r], full[:, r:]
    Prand = np.linalg.qr(rng.standard_normal((m, r)))[0]
    half = np.concatenate([A0[:, : r // 2], A1[:, r // 2:]], axis=1)   # half the spectrum ~0
    cases = ((None, A0), (1.159, None), (0.5, None), (None, Prand), (None, half), (None, A1))
    for theta, other in cases:
        Pb = other if theta is None else A0 * np.cos(theta) + A1 * np.sin(theta)
        qa, sa = O.quantize_proj(A0.astype(np.float32))
        qb, sb = O.quantize_proj(Pb.astype(np.float32))
        want = O.cossim(qa, sa, qb, sb, m, r)
        got = B.cossim(*(torch.from_numpy(x).cuda() for x in (qa, sa, qb, sb)), m, r)
        assert abs(got - want) <= 1e-4, (theta, got, want)
        if abs(want - 0.4) > 1e-4:
            assert (got > 0.4) == (want > 0.4)


@pytest.mark.parametrize("m,n", [(256, 256), (256, 200)])
def test_non_finite_rounding_inputs_keep_the_old_code(m, n):
    """Group scales chosen so that the rounding input d = W + U/s + u is not finite, or so
    large that it clamps. n = 256 takes the 16-wide vector path (whose fast branch tests the
    sum of a 16-element run), n = 200 the element-wise path.
      group 0: s = 1e-45 (subnormal): 1/s = inf, so d = +-inf (or NaN where U = 0) and every
               code is kept;
      group 1: s = 3e-39 (subnormal): 1/s = 3.3e38 is finite, U/s overflows for |U| > ~1 and
               stays finite below: kept and clamped codes side by side;
      group 2: s = 1.5e-38: every d is finite (|d| < 0.6 * FLT_MAX) but a run's fp32 sum can
               overflow, which sends the vector path to its element-by-element branch;
      other groups: s = 1, ordinary rounding.
    Both sides must keep the old code exactly where d is not finite."""
    cfg = custom_cfg(m, n, 32, sigma=1e-2)
    L = cfg.layers[0]
    st, P = PAR.host_state(cfg, L, 32, "zero")
    st.Ws[:] = 1.0
    st.Ws[0] = 1e-45
    st.Ws[1] = 3e-39
    st.Ws[2] = 1.5e-38
    hp = O.Hyper(lr=10.0)                  # |N| ~ 10, so |U| is of order 1
    G = WL.gradient_bf16(cfg, L, 1)
    Lt = PAR.to_device(st, G, P)
    before = st.copy()
    with np.errstate(over="ignore", invalid="ignore"):
        res = O.qgalore_step(st, G, 1, WL.SR_SEED, hp)
    out = gpu_step(Lt, 1, hp=dict(lr=10.0))
    with np.errstate(over="ignore", invalid="ignore"):
        PAR.check_step(before, res, st, out, hp=hp)

    d = res.d.ravel()
    w0 = before.Wq.ravel()
    g0, g1, g2 = slice(0, 256), slice(256, 512), slice(512, 768)
    assert not np.isfinite(d[g0]).any()
    assert np.array_equal(out["Wq"].ravel()[g0], w0[g0])
    fin1 = np.isfinite(d[g1])
    assert fin1.any() and (~fin1).any(), "group 1 should mix finite and infinite d"
    assert np.array_equal(out["Wq"].ravel()[g1][~fin1], w0[g1][~fin1])
    big = fin1 & (np.abs(np.nan_to_num(d[g1])) > 128)
    assert big.any() and np.all(np.abs(out["Wq"].ravel()[g1][big]) == 127)
    assert np.isfinite(d[g2]).all()
    if n % 16 == 0:
        # the vector path's test: the run's values added one after another in fp32
        sums = np.zeros(16, np.float32)
        runs = d[g2].reshape(16, 16).astype(np.float32)
        with np.errstate(over="ignore", invalid="ignore"):
            for t in range(16):
                sums = (sums + runs[:, t]).astype(np.float32)
        assert (~np.isfinite(sums)).any(), "no 16-element run of group 2 overflows its sum"


# ------------------------------------------- where the INT4 projection is dequantized ---

@pytest.mark.parametrize("m,n,r", [
    (512, 512, 128),      # small back-projection tile, vector paths
    (1376, 512, 128),     # row tail of the projection's K loop
    (2048, 5461, 64),     # odd n: register-staged paths of both kernels
    (5461, 256, 32),      # odd m, rank 32 (one projection tile covers the whole rank)
    (4096, 256, 1024),    # rank 1024: eight projection row tiles, 32 back-projection stages
    (640, 512, 256),      # rank 256, large back-projection tile
])
def test_inline_and_pass_dequant_give_identical_steps(m, n, r):
    """The INT4 projection dequantized inside the MFMA kernels' stagers and by the separate
    pass into the workspace: the same bf16 P~ enters the same products in the same order, so
    every output is bit-identical; the inline step also matches the oracle."""
    cfg = custom_cfg(m, n, r)
    L = cfg.layers[0]
    st, P = PAR.host_state(cfg, L, r, "random")
    G = WL.gradient_bf16(cfg, L, 2)
    outs = {}
    for mode in ("inline", "pass"):
        Lt = PAR.to_device(st, G, P)
        R_out = torch.empty((r, n), dtype=torch.float32, device="cuda")
        U_out = torch.empty((m, n), dtype=torch.float32, device="cuda")
        _B().step(Lt, 2, WL.SR_SEED, hp=dict(lr=1e-3, alpha=0.25), R_out=R_out, U_out=U_out,
                  dequant=mode)
        torch.cuda.synchronize()
        outs[mode] = snapshot(Lt, R_out, U_out)
    for k in outs["pass"]:
        assert np.array_equal(outs["inline"][k].view(np.uint8), outs["pass"][k].view(np.uint8)), k
    before = st.copy()
    res = O.qgalore_step(st, G, 2, WL.SR_SEED)
    PAR.check_step(before, res, st, outs["inline"], t=2)


def test_workspace_without_a_bf16_projection_copy():
    """A layer whose INT4 projection is dequantized inline needs no bf16 copy of P in its
    workspace: the size query drops m * r * 2 bytes against the separate pass."""
    B = _B()
    import ctypes
    d = B.LayerDesc()
    d.m, d.n, d.r, d.p_format = 4096, 4096, 1024, 0
    d.dequant_mode = B.DEQUANT_MODES["pass"]
    with_copy = B.lib().qgalore_layer_workspace_bytes(ctypes.byref(d))
    d.dequant_mode = B.DEQUANT_MODES["inline"]
    inline = B.lib().qgalore_layer_workspace_bytes(ctypes.byref(d))
    assert with_copy - inline == 4096 * 1024 * 2
    d.r = 96                                          # no inline path at this rank
    assert B.lib().qgalore_layer_workspace_bytes(ctypes.byref(d)) >= 4096 * 96 * 2


def test_mixed_plan_of_inline_and_pass_layers():
    """One grouped launch over layers dequantized inline, by the pass, and at a rank that has
    only the pass: every layer matches the oracle."""
    B = _B()
    shapes = [(512, 512, 128, "inline"), (512, 512, 128, "pass"), (300, 200, 64, "auto"),
              (256, 512, 96, "auto"), (1376, 512, 128, "inline")]
    states, devs, Gs, Rs, Us, modes = [], [], [], [], [], []
    for k, (m, n, r, mode) in enumerate(shapes):
        cfg = WL.Config("custom", 9, (WL.LayerShape(20 + k, f"{m}x{n}", m, n),), r=r,
                        sigma=1e-3)
        L = cfg.layers[0]
        st, P = PAR.host_state(cfg, L, r, "random")
        G = WL.gradient_bf16(cfg, L, 3)
        states.append(st)
        devs.append(PAR.to_device(st, G, P))
        Gs.append(G)
        Rs.append(torch.empty((r, n), dtype=torch.float32, device="cuda"))
        Us.append(torch.empty((m, n), dtype=torch.float32, device="cuda"))
        modes.append(mode)
    plan = B.Plan(devs, hp=dict(lr=1e-3, alpha=0.25), R_out=Rs, U_out=Us, dequant=modes)
    plan.step(3, WL.SR_SEED)
    torch.cuda.synchronize()
    for st, Lt, G, Ro, Uo in zip(states, devs, Gs, Rs, Us):
        before = st.copy()
        res = O.qgalore_step(st, G, 3, WL.SR_SEED)
        PAR.check_step(before, res, st, snapshot(Lt, Ro, Uo), t=3)
    plan.close()
