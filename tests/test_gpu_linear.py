"""Products of a linear layer with an INT8-stored weight (forward, data gradient, weight
gradient) against the oracle.

Both sides form W~ = bf16(q * s) the same way; the GPU accumulates in fp32 where the oracle
sums in float64 and rounds once, and both round to bf16. An output may therefore differ by
one bf16 ulp where the fp32 sum lands on the other side of a rounding boundary, plus the fp32
accumulation error itself (bounded here by 2^-20 times the sum of |products|, far above its
typical size and far below a bf16 ulp of a typical entry)."""
import numpy as np
import pytest

from oracle import qgalore_oracle as O

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def bf16_host(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def ulp_bf16(bits):
    v = O.bf16_bits_to_f32(bits).astype(np.float64)
    nxt = O.bf16_bits_to_f32((bits.astype(np.uint32) + 1).astype(np.uint16)).astype(np.float64)
    return np.abs(nxt - v)


def check(got_bits, want_bits, absprod, what):
    got = O.bf16_bits_to_f32(got_bits).astype(np.float64)
    want = O.bf16_bits_to_f32(want_bits).astype(np.float64)
    bound = ulp_bf16(want_bits) * 1.0001 + 2.0 ** -20 * absprod
    bad = np.abs(got - want) > bound
    assert not bad.any(), (what, int(bad.sum()), float(np.abs(got - want).max()))
    return float(np.mean(got_bits != want_bits))


def make(T, m, n, seed):
    rng = np.random.default_rng(seed)
    Wq = rng.integers(-127, 128, size=(m, n)).astype(np.int8)
    Ws = (rng.uniform(0.5, 2.0, size=O.n_groups(m * n)) * 1e-3).astype(np.float32)
    X = O.f32_to_bf16_bits(rng.standard_normal((T, n)).astype(np.float32))
    dY = O.f32_to_bf16_bits(rng.standard_normal((T, m)).astype(np.float32))
    return Wq, Ws, X, dY


@pytest.mark.parametrize("T,m,n", [
    (256, 512, 512),
    (200, 1376, 512),    # T and m not multiples of the tile
    (136, 384, 1376),
    (8, 8, 8),           # a single partial tile, K of one chunk
    (77, 264, 40),
    (300, 264, 1408),    # n % 128 == 0: both weight products stage the codes by LDS DMA,
                         # with ragged token and weight-row tiles
    (520, 136, 256),     # one full and one partial weight-side tile, three token tiles
])
def test_int8_linear_products(T, m, n):
    from quantized_rank_gradient_amd import binding as B
    Wq, Ws, X, dY = make(T, m, n, T + m + n)
    Wt = np.abs(O.dequant_weight(Wq, Ws, m, n).astype(np.float64))
    Xa = np.abs(O.bf16_bits_to_f32(X).astype(np.float64))
    dYa = np.abs(O.bf16_bits_to_f32(dY).astype(np.float64))
    Wd, Sd = torch.from_numpy(Wq).cuda(), torch.from_numpy(Ws).cuda()
    Xd, dYd = bf16_dev(X), bf16_dev(dY)
    Y = B.int8_linear_fwd(Xd, Wd, Sd)
    dX = B.int8_linear_bwd_data(dYd, Wd, Sd)
    G = B.linear_bwd_weight(dYd, Xd)
    torch.cuda.synchronize()
    check(bf16_host(Y), O.linear_forward(X, Wq, Ws, m, n), Xa @ Wt.T, "Y")
    check(bf16_host(dX), O.linear_backward_data(dY, Wq, Ws, m, n), dYa @ Wt, "dX")
    check(bf16_host(G), O.linear_backward_weight(dY, X), dYa.T @ Xa, "G")


def test_int8_linear_7b_gate_shape_sampled():
    """LLaMA-7B gate projection (m = 11008, n = 4096) at 512 tokens; the oracle computes the
    full products in float64."""
    from quantized_rank_gradient_amd import binding as B
    T, m, n = 512, 11008, 4096
    Wq, Ws, X, dY = make(T, m, n, 9)
    Wd, Sd = torch.from_numpy(Wq).cuda(), torch.from_numpy(Ws).cuda()
    Xd, dYd = bf16_dev(X), bf16_dev(dY)
    Y = bf16_host(B.int8_linear_fwd(Xd, Wd, Sd))
    dX = bf16_host(B.int8_linear_bwd_data(dYd, Wd, Sd))
    G = bf16_host(B.linear_bwd_weight(dYd, Xd))
    Wt = np.abs(O.dequant_weight(Wq, Ws, m, n).astype(np.float64))
    Xa = np.abs(O.bf16_bits_to_f32(X).astype(np.float64))
    dYa = np.abs(O.bf16_bits_to_f32(dY).astype(np.float64))
    rows = np.random.default_rng(1).choice(T, size=32, replace=False)
    check(Y[rows], O.linear_forward(X[rows], Wq, Ws, m, n), Xa[rows] @ Wt.T, "Y")
    check(dX[rows], O.linear_backward_data(dY[rows], Wq, Ws, m, n), dYa[rows] @ Wt, "dX")
    orows = np.random.default_rng(2).choice(m, size=48, replace=False)
    check(G[orows], O.linear_backward_weight(dY[:, orows], X), dYa[:, orows].T @ Xa, "G")


def test_weight_gradient_feeds_the_step():
    """G from the weight-gradient kernel is the bf16 gradient a step takes: one step on it
    matches the oracle (same check as the other step tests)."""
    from quantized_rank_gradient_amd import binding as B
    from quantized_rank_gradient_amd import workloads as WL
    from tests import parity as PAR
    from tests.test_gpu_step import custom_cfg, gpu_step
    T, m, n, r = 384, 512, 768, 64
    _, _, X, dY = make(T, m, n, 21)
    G = bf16_host(B.linear_bwd_weight(bf16_dev(dY), bf16_dev(X)))
    cfg = custom_cfg(m, n, r)
    L = cfg.layers[0]
    st, P = PAR.host_state(cfg, L, r, "random")
    Lt = PAR.to_device(st, G, P, quantize_on_gpu=False)
    before = st.copy()
    res = O.qgalore_step(st, G, 2, WL.SR_SEED)
    PAR.check_step(before, res, st, gpu_step(Lt, 2), t=2)
