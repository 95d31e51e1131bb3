"""Pins for the CPU oracle: each test ties an oracle function to something other than the
oracle itself (a library routine, a closed form, an invariant, brute force, or a value the
pages print), so that a dropped term, a wrong sign or index, or a transposed operand fails.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import qgalore_oracle as O

F32 = np.float32
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- bf16 ---

def test_bf16_rounding_matches_torch_cpu_including_ties():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    # force exact ties (low half == 0x8000) on a quarter of them, with both kept-bit parities
    bits[::4] = (bits[::4] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    specials = np.array([0x7F7FFFFF, 0xFF7FFFFF, 0x7F800000, 0xFF800000, 0x00000001,
                         0x80000000, 0x00000000, 0x3F808000, 0x3F818000, 0x7F7F8000],
                        dtype=np.uint32)
    x = np.concatenate([bits, specials]).view(F32)
    ours = O.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all(np.isnan(O.bf16_bits_to_f32(ours[nan])))


def test_bf16_round_trip_is_exact_for_bf16_values():
    rng = np.random.default_rng(8)
    b = rng.integers(0, 2 ** 16, size=100_000, dtype=np.uint32).astype(np.uint16)
    v = O.bf16_bits_to_f32(b)
    keep = ~np.isnan(v)
    assert np.array_equal(O.f32_to_bf16_bits(v)[keep], b[keep])


# ------------------------------------------------------------------------ quantizers ---

def test_rne_is_half_to_even_like_torch_round():
    x = np.array([-2.5, -1.5, -0.5, 0.5, 1.5, 2.5, 126.5, -126.5], dtype=F32)
    assert np.array_equal(np.rint(x), torch.round(torch.from_numpy(x)).numpy())
    q, s = O.absmax_quantize(np.array([0.5, 1.5, 2.5] + [0.0] * 253 + [127.0], F32)[:256], 127)
    # scale 1 exactly only when absmax is 127: build that group explicitly
    g = np.zeros(256, F32)
    g[:4] = [0.5, 1.5, 2.5, 127.0]
    q, s = O.absmax_quantize(g, 127)
    assert s[0] == F32(1.0)
    assert list(q[:4]) == [0, 2, 2, 127]


@pytest.mark.parametrize("qmax", [7, 127])
def test_quantizer_properties(qmax):
    rng = np.random.default_rng(qmax)
    x = rng.standard_normal(256 * 37 + 100).astype(F32)   # short last group
    x[256 * 5:256 * 6] = 0.0                              # an all-zero group
    q, s = O.absmax_quantize(x, qmax)
    assert s.shape == (38,)
    assert s[5] == 0 and np.all(q[256 * 5:256 * 6] == 0)
    assert q.min() >= -qmax and q.max() <= qmax
    g = np.arange(x.size) // 256
    # the absmax element of every non-zero group maps to +-qmax
    for k in range(38):
        sl = slice(256 * k, min(256 * (k + 1), x.size))
        if s[k] > 0:
            i = np.argmax(np.abs(x[sl]))
            assert abs(int(q[sl][i])) == qmax
    # error bound |deq - x| <= s/2 (plus a few ulp of rounding)
    deq = O.dequantize(q, s)
    assert np.all(np.abs(deq - x) <= s[g] * F32(0.5) * F32(1 + 1e-5) + 1e-30)
    # idempotent: quantizing the dequantized values returns the same codes and scales
    q2, s2 = O.absmax_quantize(deq, qmax)
    assert np.array_equal(q2, q)
    assert np.allclose(s2, s, rtol=1e-6, atol=0)


def test_int4_packing_layout_and_round_trip():
    assert O.pack_int4(np.array([1, -1], np.int8)).tolist() == [0xF1]
    assert O.pack_int4(np.array([-8, 7, 3], np.int8)).tolist() == [0x78, 0x03]
    rng = np.random.default_rng(3)
    q = rng.integers(-7, 8, size=1001).astype(np.int8)
    assert np.array_equal(O.unpack_int4(O.pack_int4(q), q.size), q)


def test_int4_projection_memory_matches_pages():
    """INT4 P takes a quarter of BF16 P's bytes (the pages: 75% less projection memory)."""
    gold = json.load(open(os.path.join(GOLDEN, "pages_constants.json")))
    m, r = 4096, 128
    P = np.linalg.qr(np.random.default_rng(0).standard_normal((m, r)))[0].astype(F32)
    Pq, Ps = O.quantize_proj(P)
    bf16_bytes = 2 * m * r
    assert 1 - Pq.nbytes / bf16_bytes == pytest.approx(gold["int4_projection_memory_cut_vs_bf16"]["value"])
    assert Ps.size == m * r // 256


def test_projection_formats():
    """The three stores of P: INT4 and INT8 dequantize to bf16(code * scale) with the group
    quantizer's codes; bf16 is torch's bf16 cast of P; every format's P~ is bf16-exact and
    within its quantization error of P."""
    torch = pytest.importorskip("torch")
    m, r = 512, 64
    P = np.linalg.qr(np.random.default_rng(5).standard_normal((m, r)))[0].astype(F32)
    g = np.arange(m * r) // 256
    for fmt, qmax in (("int4", 7), ("int8", 127)):
        Pq, Ps = O.quantize_proj(P, fmt)
        q, s = O.absmax_quantize(P, qmax)
        codes = O.unpack_int4(Pq, m * r) if fmt == "int4" else Pq
        assert np.array_equal(codes, q.ravel()) and np.array_equal(Ps, s)
        Pt = O.dequant_proj(Pq, Ps, m, r, fmt)
        want = torch.from_numpy(q.ravel().astype(F32) * s[g]).to(torch.bfloat16).float().numpy()
        assert np.array_equal(Pt.ravel(), want)
        # |q s - P| <= s/2, and the bf16 rounding of q s adds at most half an ulp of |q s|
        # (<= 2^-8 |q s|, with |q s| <= |P| + s/2)
        half = s[g].astype(np.float64) * 0.5
        bound = half + (np.abs(P.ravel()).astype(np.float64) + half) * 2.0 ** -8
        assert np.all(np.abs(Pt.ravel().astype(np.float64) - P.ravel()) <= bound * (1 + 1e-6))
    Pq, Ps = O.quantize_proj(P, "bf16")
    assert Ps is None and Pq.dtype == np.uint16 and Pq.size == m * r
    Pt = O.dequant_proj(Pq, None, m, r, "bf16")
    assert np.array_equal(Pt, torch.from_numpy(P).to(torch.bfloat16).float().numpy())


# ------------------------------------------------------------------------ projection ---

def test_full_rank_projection_reconstructs_gradient():
    rng = np.random.default_rng(11)
    G = rng.standard_normal((12, 9))
    U, _, _ = np.linalg.svd(G)                 # m x m, full rank
    back = O.backproject(U, O.project(U, G))
    assert np.allclose(back, G, rtol=0, atol=1e-12 * np.abs(G).max())


def test_projection_recovers_coefficients_in_subspace():
    """G = P B with orthonormal P (m x r, r < m) gives R = P^T G = B exactly: fails for a
    transposed operand or a wrong side."""
    rng = np.random.default_rng(12)
    P = np.linalg.qr(rng.standard_normal((10, 4)))[0]
    B = rng.standard_normal((4, 7))
    assert np.allclose(O.project(P, P @ B), B, atol=1e-12)
    # back-projection of a unit coefficient is the corresponding column of P
    for k in range(4):
        e = np.zeros((4, 1)); e[k] = 1.0
        assert np.allclose(O.backproject(P, e)[:, 0], P[:, k], atol=0)


def test_qr_projection_is_orthonormal():
    rng = np.random.default_rng(13)
    P = np.linalg.qr(rng.standard_normal((64, 16)))[0]
    assert np.allclose(P.T @ P, np.eye(16), atol=1e-12)


def test_projection_rounds_once_to_fp32():
    """Brute force with exact rationals on tiny inputs: R is the exact sum rounded to fp32."""
    rng = np.random.default_rng(14)
    m, n, r = 6, 5, 3
    P = O.bf16_round(rng.standard_normal((m, r)).astype(F32))
    G = O.bf16_round(rng.standard_normal((m, n)).astype(F32) * F32(1e-3))
    R = O.project(P, G).astype(F32)
    for i in range(r):
        for j in range(n):
            exact = sum(Fraction(float(P[k, i])) * Fraction(float(G[k, j])) for k in range(m))
            ulp = np.spacing(np.abs(F32(float(exact))))
            assert abs(Fraction(float(R[i, j])) - exact) <= Fraction(float(ulp)) / 2


# ------------------------------------------------------------------------------ Adam ---

def test_adam_first_step_closed_form():
    """From M = V = 0 at t = 1: m^ = R, v^ = R^2, so N = -lr * R / (|R| + eps)."""
    h = O.Hyper()
    rng = np.random.default_rng(21)
    R = (rng.standard_normal(5000) * 1e-3).astype(F32)
    R[:10] = 0.0
    R[10:20] = 1e-9                   # comparable to eps
    _, _, N = O.adam_core(R, np.zeros_like(R), np.zeros_like(R), 1, h)
    R64 = R.astype(np.float64)
    want = -h.lr * R64 / (np.abs(R64) + h.eps)
    assert np.allclose(N, want, rtol=2e-6, atol=1e-12)
    assert np.all(np.sign(N[R != 0]) == -np.sign(R[R != 0]))


def test_adam_multi_step_matches_torch_optim_adam():
    """With fp32 moments (INT8 storage bypassed), N_t equals torch.optim.Adam's parameter
    change on the same gradient sequence."""
    h = O.Hyper(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
    rng = np.random.default_rng(22)
    shape = (64, 33)
    p = torch.zeros(shape, dtype=torch.float32, requires_grad=True)
    opt = torch.optim.Adam([p], lr=h.lr, betas=(h.beta1, h.beta2), eps=h.eps, weight_decay=0)
    m = np.zeros(shape, F32)
    v = np.zeros(shape, F32)
    for t in range(1, 8):
        R = (rng.standard_normal(shape) * 1e-3).astype(F32)
        before = p.detach().clone()
        p.grad = torch.from_numpy(R.copy())
        opt.step()
        delta = (p.detach() - before).numpy()
        m, v, N = O.adam_core(R, m, v, t, h)
        assert np.allclose(N, delta, rtol=2e-5, atol=1e-9), t


def test_adam_int8_state_round_trip():
    h = O.Hyper()
    rng = np.random.default_rng(23)
    r, n = 8, 96
    R = (rng.standard_normal((r, n)) * 1e-3).astype(F32)
    Mq, Ms = np.zeros((r, n), np.int8), np.zeros(3, F32)
    Vq, Vs = np.zeros((r, n), np.int8), np.zeros(3, F32)
    N, Mq2, Ms2, Vq2, Vs2, m1, v1 = O.adam_int8(R, Mq, Ms, Vq, Vs, 1, h)
    # stored moments dequantize to the fresh fp32 moments within half a step of the scale
    g = np.arange(r * n) // 256
    assert np.all(np.abs(O.dequantize(Mq2, Ms2).ravel() - m1.ravel()) <= Ms2[g] * 0.5 * (1 + 1e-5))
    assert np.all(Vq2 >= 0)


# --------------------------------------------------------------------------- Philox ---

def test_philox_uniforms_are_uniform():
    i = np.repeat(np.arange(256), 512)
    j = np.tile(np.arange(512), 256)
    u = O.sr_uniform(1234, 5, 3, i, j).astype(np.float64)
    N = u.size
    assert np.all((u >= 0) & (u < 1))
    assert abs(u.mean() - 0.5) < 3 * math.sqrt(1 / 12 / N)
    assert abs(u.var() - 1 / 12) < 3 * math.sqrt(1 / 180 / N)
    hist = np.bincount((u * 256).astype(int), minlength=256)
    chi2 = np.sum((hist - N / 256) ** 2 / (N / 256))
    assert chi2 < 255 + 5 * math.sqrt(2 * 255)      # ~5 sigma of a chi^2(255)


def test_philox_streams_differ_by_step_layer_and_seed():
    i = np.repeat(np.arange(64), 64)
    j = np.tile(np.arange(64), 64)
    base = O.sr_uniform(1234, 1, 0, i, j)
    for other in (O.sr_uniform(1234, 2, 0, i, j), O.sr_uniform(1234, 1, 1, i, j),
                  O.sr_uniform(1235, 1, 0, i, j), O.sr_uniform(1234 + (1 << 32), 1, 0, i, j)):
        c = np.corrcoef(base, other)[0, 1]
        assert abs(c) < 5 / math.sqrt(base.size)
        assert np.mean(base == other) < 0.01
    # the 8 elements of one counter block take 8 distinct 16-bit halves of one Philox output
    w = O.philox4x32_10(np.array([[0, 7, 1, 0]]), (1234, 0))[0]
    halves = [w[k >> 1] & 0xFFFF if k % 2 == 0 else w[k >> 1] >> 16 for k in range(8)]
    got = O.sr_uniform(1234, 1, 0, np.full(8, 7), np.arange(8)) * 65536
    assert [int(x) for x in got] == [int(x) for x in halves]


def test_philox_bijective_on_counters_for_fixed_key():
    ctr = np.zeros((4096, 4), np.uint32)
    ctr[:, 0] = np.arange(4096)
    out = O.philox4x32_10(ctr, (99, 7))
    assert len({tuple(row) for row in out.tolist()}) == 4096


# -------------------------------------------------------------- stochastic rounding ---

@pytest.mark.parametrize("frac", [0.001, 0.1, 0.5, 0.75, 0.999])
def test_stochastic_rounding_is_unbiased(frac):
    """Mean over 1e5 draws (varying step) equals the input within 3 sigma."""
    T = 100_000
    w0 = np.int8(3)
    Ws = np.array([1.0], F32)
    U = np.full((1, 1), F32(frac), F32)
    outs = np.empty(T)
    # vectorise over steps: one element, many t
    for t0 in range(0, T, 20_000):
        ts = np.arange(t0 + 1, t0 + 20_001)
        i = np.zeros(ts.size, np.int64)
        j = np.zeros(ts.size, np.int64)
        key = (99, 0)
        ctr = np.stack([j >> 3, i, ts, np.zeros_like(ts)], axis=1)
        words = O.philox4x32_10(ctr, key)[:, 0] & 0xFFFF
        uu = words.astype(F32) * F32(2 ** -16)
        d = (F32(w0) + U[0, 0]) + uu
        outs[t0:t0 + ts.size] = np.floor(d.astype(F32))
    # the vectorised path above must agree with the oracle's own SR on a few steps
    for t in (1, 2, 777):
        W1, _ = O.stochastic_round(np.full((1, 1), w0, np.int8), Ws, U, t, 99, 0)
        assert W1[0, 0] == outs[t - 1]
    mean = outs.mean() - float(w0)
    sigma = math.sqrt(frac * (1 - frac) / T)
    assert abs(mean - frac) <= 3 * sigma + 2 ** -16


def test_stochastic_rounding_special_cases():
    rng = np.random.default_rng(31)
    m, n = 4, 512
    W = rng.integers(-127, 128, size=(m, n), dtype=np.int8)
    Ws = np.full(8, 1e-3, F32)
    # zero update leaves W bit-identical for every draw
    for t in (1, 2, 3):
        W1, _ = O.stochastic_round(W, Ws, np.zeros((m, n), F32), t, 5, 0)
        assert np.array_equal(W1, W)
    # an integer number of LSBs is applied exactly (no rounding decision left)
    Ws1 = np.full(8, 1.0, F32)
    U = rng.integers(-3, 4, size=(m, n)).astype(F32)
    W1, _ = O.stochastic_round(W, Ws1, U, 1, 5, 0)
    assert np.array_equal(W1, np.clip(W.astype(int) + U.astype(int), -127, 127))
    # output is always floor or floor + 1 of the pre-round value
    U = (rng.standard_normal((m, n)) * 3e-3).astype(F32)
    W1, _ = O.stochastic_round(W, Ws, U, 2, 5, 0)
    tp = W.astype(F32) + U * (F32(1) / F32(1e-3))
    assert np.all((W1 == np.clip(np.floor(tp), -127, 127)) | (W1 == np.clip(np.floor(tp) + 1, -127, 127)))
    # clamping at +-127
    Wc = np.array([[127, -127, 126, -126]], np.int8)
    Uc = np.array([[5.0, -5.0, 5.0, -5.0]], F32)
    W1, _ = O.stochastic_round(Wc, np.array([1.0], F32), Uc, 1, 5, 0)
    assert W1.tolist() == [[127, -127, 127, -127]]
    # non-finite pre-round values leave W unchanged; a zero scale means no update
    Un = np.array([[np.inf, -np.inf, np.nan, 1.0]], F32)
    W1, _ = O.stochastic_round(Wc, np.array([1.0], F32), Un, 1, 5, 0)
    assert W1.tolist() == [[127, -127, 126, -125]]
    W1, _ = O.stochastic_round(Wc, np.array([0.0], F32), Uc, 1, 5, 0)
    assert np.array_equal(W1, Wc)


# --------------------------------------------------------------------------- CosSim ---

def test_cossim_pins():
    rng = np.random.default_rng(41)
    m, r = 96, 12
    P = np.linalg.qr(rng.standard_normal((m, r)))[0]
    assert O.cossim_float(P, P) == pytest.approx(1.0, abs=1e-12)
    Q = np.linalg.qr(rng.standard_normal((r, r)))[0]
    assert O.cossim_float(P, P @ Q) == pytest.approx(1.0, abs=1e-12)
    full = np.linalg.qr(rng.standard_normal((m, 2 * r)))[0]
    A0, A1 = full[:, :r], full[:, r:]
    assert O.cossim_float(A0, A1) == pytest.approx(0.0, abs=1e-12)
    # equals the mean cosine of the principal angles (library routine)
    B = np.linalg.qr(rng.standard_normal((m, r)))[0]
    want = np.mean(np.cos(scipy.linalg.subspace_angles(P, B)))
    assert O.cossim_float(P, B) == pytest.approx(want, abs=1e-10)
    # rotation closed form: P(theta) = A0 cos + A1 sin gives |cos theta|
    for theta in (0.3, 1.159, 2.0, 3.0):
        Pt = A0 * math.cos(theta) + A1 * math.sin(theta)
        assert O.cossim_float(A0, Pt) == pytest.approx(abs(math.cos(theta)), abs=1e-12)


def test_cossim_of_stored_int4_projection():
    """CosSim(P~, P~) = ||P~||_F^2 / r for the dequantized bf16 operand (not exactly 1)."""
    rng = np.random.default_rng(42)
    m, r = 512, 64
    P = np.linalg.qr(rng.standard_normal((m, r)))[0].astype(F32)
    Pq, Ps = O.quantize_proj(P)
    Pt = O.dequant_proj(Pq, Ps, m, r).astype(np.float64)
    cs = O.cossim(Pq, Ps, Pq, Ps, m, r)
    # sum of singular values of the PSD matrix Pt^T Pt is its trace
    assert cs == pytest.approx(np.sum(Pt * Pt) / r, rel=1e-12)
    assert abs(cs - 1.0) < 0.05


# ------------------------------------------------------------------------- schedule ---

def test_schedule_hand_traces():
    gold = json.load(open(os.path.join(GOLDEN, "pages_constants.json")))
    gamma = gold["gamma_default"]["value"]
    # a subspace that never moves: every test passes, the interval doubles each time
    steps, delta = O.simulate_schedule(lambda a, b: 1.0, 25, 200, gamma)
    assert steps == [0, 25, 75, 175] and delta == 25 * gold["interval_growth_factor"]["value"] ** 3
    # a subspace that always moves: the fixed-interval schedule
    steps, delta = O.simulate_schedule(lambda a, b: 0.1, 25, 200, gamma)
    assert steps == list(range(0, 200, 25)) and delta == 25
    assert O.fixed_interval_refreshes(25, 200) == 8
    # the threshold is strict: CosSim == gamma does not double
    steps, _ = O.simulate_schedule(lambda a, b: gamma, 25, 200, gamma)
    assert len(steps) == 8
    # pass, fail, pass: 0 (first), 25 pass -> 50, 75 fail -> 50, 125 pass -> 100, next 225
    seq = iter([0.9, 0.1, 0.9])
    steps, delta = O.simulate_schedule(lambda a, b: next(seq), 25, 200, gamma)
    assert steps == [0, 25, 75, 125] and delta == 100


def test_schedule_drifting_subspace_closed_form():
    """Noise-free drift P_t = A0 cos(rho t) + A1 sin(rho t): CosSim(P_t, P_s) = |cos(rho (t - s))|.
    The oracle schedule driven by the oracle CosSim on real matrices matches the one driven by
    the closed form."""
    rng = np.random.default_rng(43)
    m, r = 64, 8
    full = np.linalg.qr(rng.standard_normal((m, 2 * r)))[0]
    A0, A1 = full[:, :r], full[:, r:]
    for rho in (0.0, 0.01, 0.03, 0.05):
        def P(t):
            return A0 * math.cos(rho * t) + A1 * math.sin(rho * t)
        s_mat, d_mat = O.simulate_schedule(lambda a, b: O.cossim_float(P(a), P(b)), 25, 200)
        s_cf, d_cf = O.simulate_schedule(lambda a, b: abs(math.cos(rho * (a - b))), 25, 200)
        assert s_mat == s_cf and d_mat == d_cf


# -------------------------------------------------------------------------- refresh ---

def _hadamard(n):
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def test_refresh_projection_closed_form_bf16_exact():
    """G = A diag(s) B^T with orthonormal Hadamard columns (entries +-1/4) and s = 8, 4, 2, 1:
    every entry of G is a multiple of 1/16 below 1, so G is exact in bf16, and its leading
    left singular vectors are A's columns. All |entries| tie, so the first row fixes the
    sign."""
    H = _hadamard(16) / 4.0
    A, B = H[:, [1, 2, 3, 5]], H[:, [4, 6, 7, 9]]
    s = np.array([8.0, 4.0, 2.0, 1.0])
    G = (A * s) @ B.T
    bits = O.f32_to_bf16_bits(G.astype(np.float32))
    assert np.array_equal(O.bf16_bits_to_f32(bits).astype(np.float64), G)
    P, S = O.refresh_projection(bits, 3)
    want = A[:, :3] * np.sign(A[0, :3])
    np.testing.assert_allclose(P, want, atol=1e-12)
    np.testing.assert_allclose(S, s[:3], rtol=1e-12)
    assert np.all(P[0] > 0)


def test_refresh_projection_properties():
    """Random G: orthonormal columns, the eigen-equation G G^T p = sigma^2 p, the sign rule,
    and invariance under G -> -G (singular vectors flip, the convention flips them back)."""
    rng = np.random.default_rng(7)
    m, n, r = 40, 56, 6
    G = rng.standard_normal((m, n)).astype(np.float32)
    bits = O.f32_to_bf16_bits(G)
    Gd = O.bf16_bits_to_f32(bits).astype(np.float64)
    P, S = O.refresh_projection(bits, r)
    np.testing.assert_allclose(P.T @ P, np.eye(r), atol=1e-12)
    np.testing.assert_allclose(Gd @ (Gd.T @ P), P * S ** 2, rtol=0, atol=1e-9 * S[0] ** 2)
    assert np.all(np.diff(S) <= 0)
    idx = np.argmax(np.abs(P), axis=0)
    assert np.all(P[idx, np.arange(r)] > 0)
    Pn, Sn = O.refresh_projection(O.f32_to_bf16_bits(-G), r)
    np.testing.assert_allclose(Pn, P, atol=1e-12)
    np.testing.assert_allclose(Sn, S, rtol=1e-12)
    # library routine: the same subspace as numpy's eigh of G G^T
    w, V = np.linalg.eigh(Gd @ Gd.T)
    top = V[:, np.argsort(w)[::-1][:r]]
    np.testing.assert_allclose(np.abs(top.T @ P), np.eye(r), atol=1e-8)


def test_column_sign_rule_by_hand():
    P = np.array([[0.5, -0.2, 0.3], [-0.7, 0.2, -0.3], [0.1, 0.1, 0.0]])
    out = O.normalize_column_signs(P)
    # column 0: max |.| at row 1 (negative) -> flipped; column 1: tie at rows 0/1, row 0 is
    # negative -> flipped; column 2: tie, row 0 positive -> kept
    np.testing.assert_array_equal(out, P * np.array([-1.0, -1.0, 1.0]))


# --------------------------------------------------------------- INT8-weight linear ---

def test_int8_linear_exact_integer_case():
    """Small integers everywhere (codes, a power-of-two scale, activations): every product
    and sum is exact, so the three products equal integer matrix products, checked by
    brute force on Python integers."""
    rng = np.random.default_rng(3)
    T, m, n = 5, 6, 256
    Wq = rng.integers(-3, 4, size=(m, n)).astype(np.int8)
    Ws = np.full(O.n_groups(m * n), 0.5, dtype=np.float32)
    X = rng.integers(-2, 3, size=(T, n)).astype(np.float32)
    dY = rng.integers(-2, 3, size=(T, m)).astype(np.float32)
    Xb, dYb = O.f32_to_bf16_bits(X), O.f32_to_bf16_bits(dY)
    Wi = [[int(v) for v in row] for row in Wq]
    Xi = [[int(v) for v in row] for row in X]
    dYi = [[int(v) for v in row] for row in dY]
    Y = O.bf16_bits_to_f32(O.linear_forward(Xb, Wq, Ws, m, n))
    want = [[sum(Xi[t][i] * Wi[o][i] for i in range(n)) / 2 for o in range(m)] for t in range(T)]
    np.testing.assert_array_equal(Y, np.array(want, dtype=np.float32))
    dX = O.bf16_bits_to_f32(O.linear_backward_data(dYb, Wq, Ws, m, n))
    want = [[sum(dYi[t][o] * Wi[o][i] for o in range(m)) / 2 for i in range(n)] for t in range(T)]
    np.testing.assert_array_equal(dX, np.array(want, dtype=np.float32))
    G = O.bf16_bits_to_f32(O.linear_backward_weight(dYb, Xb))
    want = [[sum(dYi[t][o] * Xi[t][i] for t in range(T)) for i in range(n)] for o in range(m)]
    np.testing.assert_array_equal(G, np.array(want, dtype=np.float32))


def test_int8_linear_transpose_identities():
    """With one scale for every group, the data gradient is the forward product with the
    transposed weight, and the weight gradient's transpose is the product with the roles of
    X and dY exchanged; both catch a transposed or swapped operand."""
    rng = np.random.default_rng(4)
    T, m, n = 7, 256, 512
    Wq = rng.integers(-127, 128, size=(m, n)).astype(np.int8)
    Ws = np.full(O.n_groups(m * n), 3e-3, dtype=np.float32)
    dYb = O.f32_to_bf16_bits(rng.standard_normal((T, m)).astype(np.float32))
    Xb = O.f32_to_bf16_bits(rng.standard_normal((T, n)).astype(np.float32))
    WqT = np.ascontiguousarray(Wq.T)
    np.testing.assert_array_equal(O.linear_backward_data(dYb, Wq, Ws, m, n),
                                  O.linear_forward(dYb, WqT, Ws, n, m))
    np.testing.assert_array_equal(O.linear_backward_weight(dYb, Xb).T,
                                  O.linear_backward_weight(Xb, dYb))
    # the dequantized weight is the per-group q * s rounded to bf16
    Wt = O.dequant_weight(Wq, Ws, m, n)
    np.testing.assert_array_equal(Wt, O.bf16_round(Wq.astype(np.float32) * np.float32(3e-3)))
