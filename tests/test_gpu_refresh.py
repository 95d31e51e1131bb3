"""The GPU subspace refresh (randomized range finder, qgalore_refresh_proj) against the
oracle's definition: the r leading left singular vectors of G by a float64 SVD, with the
same column sign convention.

The library's result approximates the SVD. Its error has two parts:
  * the range finder: the captured subspace misses a fraction of about
    (sigma_{k+1} / sigma_r)^(2q+1) (q power iterations; Halko, Martinsson and Tropp 2011,
    Section 10). The test spectra drop tenfold after the r-th value, so this is below 1e-6;
  * rounding: the products with G use bf16 hi + lo parts of each fp32 basis (about 2^-16
    relative), and the k x k eigenproblem runs in fp32. A perturbation of relative size
    eps moves an individual singular vector by about eps / (relative gap of sigma_i^2 to its
    neighbours); the spectra below keep that gap at 1.5% or more at r = 32 and 0.8% at
    r = 128, so vectors move by well under 1e-3.
Sketches wider than 136 (ranks 192 to 1024 here) take the library's wide path (block
Gram-Schmidt and a block Jacobi eigensolver in fp64); the spectra below keep the relative gap
of sigma_i^2 at 0.2% or more up to rank 1024, so vectors still move by well under 1e-3.
Gradients whose column count is not a multiple of 8 are padded with zero columns inside the
library, which leaves every product unchanged.
Checks: each column within 2e-3 of the oracle's (max abs entry difference, unit vectors),
the subspace (1 - the smallest singular value of P*^T P below 1e-5), orthonormality, the
singular values (relative 1e-4 of sigma_1), and the INT4 codes equal to the oracle's
quantization of the GPU's own fp32 P (bit-exact)."""
import numpy as np
import pytest

from oracle import qgalore_oracle as O
from quantized_rank_gradient_amd import workloads as WL

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def spectrum_gradient(m, n, r, extra, seed, noise=1e-4):
    """bf16 G = A diag(s) B^T + noise: s falls linearly from 1 to 0.5 over the first r values,
    then drops tenfold and decays by 0.9 per value over `extra` more."""
    rng = np.random.default_rng(seed)
    q = min(r + extra, m, n)
    extra = q - r
    A = np.linalg.qr(rng.standard_normal((m, q)))[0]
    B = np.linalg.qr(rng.standard_normal((n, q)))[0]
    s = np.concatenate([np.linspace(1.0, 0.5, r), 0.05 * 0.9 ** np.arange(extra)])
    G = (A * s) @ B.T + noise * rng.standard_normal((m, n)) / np.sqrt(max(m, n))
    return O.f32_to_bf16_bits(G.astype(np.float32))


def gpu_refresh(bits, r, k, iters=2, seed=5):
    from quantized_rank_gradient_amd import binding as B
    m, n = bits.shape
    G = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    Om = torch.randn((n, k), generator=gen, device="cuda").to(torch.bfloat16)
    P = torch.empty((m, r), dtype=torch.float32, device="cuda")
    sig = torch.empty(r, dtype=torch.float32, device="cuda")
    Pq, Ps = B.refresh_proj(G, r, Om, power_iters=iters, P_out=P, sigma_out=sig)
    torch.cuda.synchronize()
    return P.cpu().numpy(), sig.cpu().numpy(), Pq.cpu().numpy(), Ps.cpu().numpy()


def check(bits, r, P, sig, Pq, Ps, col_tol=2e-3):
    m = bits.shape[0]
    Pw, Sw = O.refresh_projection(bits, r)
    Pg = P.astype(np.float64)
    np.testing.assert_allclose(Pg.T @ Pg, np.eye(r), atol=1e-4, err_msg="orthonormal")
    sv = np.linalg.svd(Pw.T @ Pg, compute_uv=False)
    assert 1.0 - sv.min() < 1e-5, f"subspace: 1 - min cos = {1.0 - sv.min():.3g}"
    err = np.abs(Pg - Pw).max(axis=0)
    assert err.max() < col_tol, f"columns: worst {err.max():.3g} at {int(err.argmax())}"
    np.testing.assert_allclose(sig, Sw, rtol=0, atol=1e-4 * Sw[0], err_msg="singular values")
    want_q, want_s = O.quantize_proj(P, "int4")
    assert np.array_equal(Pq, want_q) and np.array_equal(Ps, want_s), "INT4 codes of P"
    return err.max(), 1.0 - sv.min()


@pytest.mark.parametrize("m,n,r,k", [
    (512, 384, 32, 40),
    (1376, 512, 64, 72),     # rows not a multiple of the 128-row tile
    (200, 136, 64, 136),     # k = n: the widest sketch the shape allows
    (4096, 4096, 128, 136),
])
def test_refresh_matches_svd(m, n, r, k):
    bits = spectrum_gradient(m, n, r, k - r + 24, seed=m + n + r)
    check(bits, r, *gpu_refresh(bits, r, k))


@pytest.mark.parametrize("m,n,r,k", [
    (600, 400, 192, 200),     # the narrowest wide sketch: 7 blocks of 32 padded to 8
    (1376, 520, 256, 264),    # 3 blocks of 128 columns in the Gram-Schmidt, the last of 8
    (512, 389, 32, 40),       # n % 8 != 0 on the one-workgroup path
    (700, 333, 200, 208),     # n % 8 != 0 on the wide path, k close to n
])
def test_refresh_matches_svd_wide_and_ragged(m, n, r, k):
    bits = spectrum_gradient(m, n, r, k - r + 24, seed=m + n + r)
    check(bits, r, *gpu_refresh(bits, r, k))


def test_refresh_1b_down_shape_rank_512():
    """2048 x 5461 (the 1B down projection, 5461 columns), rank 512, k = 520."""
    bits = spectrum_gradient(2048, 5461, 512, 32, seed=17)
    check(bits, 512, *gpu_refresh(bits, 512, 520))


def test_refresh_7b_rank_1024():
    """4096 x 4096 (the 7B attention projections), rank 1024, k = 1032."""
    bits = spectrum_gradient(4096, 4096, 1024, 32, seed=19)
    check(bits, 1024, *gpu_refresh(bits, 1024, 1032))


def test_refresh_7b_gate_shape():
    """11008 x 4096 (the 7B gate and up projections), rank 128."""
    bits = spectrum_gradient(11008, 4096, 128, 32, seed=3)
    check(bits, 128, *gpu_refresh(bits, 128, 136))


def test_refresh_drifting_workload_subspace():
    """A gradient of the drifting-subspace workload (7B q shape, rank 128): its spectrum is
    nearly flat over the leading 128 values (1.5 to 0.5 times a scale, gaps of 0.8%), so
    individual vectors are compared only as a subspace, and CosSim with the SVD's P is 1."""
    cfg = WL.CONFIGS["schedule7b"]
    L = cfg.layers[0]
    dev = torch.device("cuda:0")
    basis = WL.drift_basis_device(cfg, L, device=dev)
    G = WL.drift_gradient_device(cfg, L, basis, WL.drift_rate(cfg, 0), 7)
    bits = G.view(torch.int16).cpu().numpy().view(np.uint16)
    P, sig, Pq, Ps = gpu_refresh(bits, cfg.r, cfg.r + 8)
    Pw, Sw = O.refresh_projection(bits, cfg.r)
    sv = np.linalg.svd(Pw.T @ P.astype(np.float64), compute_uv=False)
    assert 1.0 - sv.min() < 1e-4
    assert O.cossim_float(Pw, P) > 1.0 - 1e-5
    np.testing.assert_allclose(sig, Sw, rtol=1e-4)


def test_refresh_power_iterations_help():
    """With a slowly decaying tail, more power iterations capture more of the subspace."""
    rng = np.random.default_rng(11)
    m, n, r, k = 1024, 768, 32, 40
    A = np.linalg.qr(rng.standard_normal((m, 96)))[0]
    Bm = np.linalg.qr(rng.standard_normal((n, 96)))[0]
    s = 0.97 ** np.arange(96)
    bits = O.f32_to_bf16_bits(((A * s) @ Bm.T).astype(np.float32))
    Pw, _ = O.refresh_projection(bits, r)
    miss = []
    for q in (0, 1, 3):
        P = gpu_refresh(bits, r, k, iters=q)[0].astype(np.float64)
        miss.append(1.0 - np.linalg.svd(Pw.T @ P, compute_uv=False).min())
    assert miss[0] > miss[1] > miss[2], miss


@pytest.mark.parametrize("m,n,r,k", [
    (512, 384, 32, 40),      # one-workgroup orthonormalization
    (600, 400, 192, 200),    # block Gram-Schmidt and block Jacobi
])
def test_refresh_rank_deficient_gradient(m, n, r, k):
    """A gradient of rank 16 < r (16 nonzero columns, exactly zero elsewhere): the sketch's
    Gram matrices are singular and the orthonormalization raises pivots to its floor. The
    leading 16 vectors span the oracle's, their singular values match, the others are about
    zero, and everything is finite (the columns past the rank are not unique, so they are
    not compared)."""
    rk = 16
    rng = np.random.default_rng(m + r)
    G = np.zeros((m, n), np.float32)
    cols = rng.choice(n, rk, replace=False)
    G[:, cols] = rng.standard_normal((m, rk)) * np.linspace(1.0, 0.5, rk)
    bits = O.f32_to_bf16_bits(G)
    P, sig, Pq, Ps = gpu_refresh(bits, r, k)
    assert np.isfinite(P).all() and np.isfinite(sig).all() and np.isfinite(Ps).all()
    Pw, Sw = O.refresh_projection(bits, r)
    Pg = P.astype(np.float64)
    np.testing.assert_allclose(Pg[:, :rk].T @ Pg[:, :rk], np.eye(rk), atol=1e-4)
    sv = np.linalg.svd(Pw[:, :rk].T @ Pg[:, :rk], compute_uv=False)
    assert 1.0 - sv.min() < 1e-5, f"subspace: 1 - min cos = {1.0 - sv.min():.3g}"
    np.testing.assert_allclose(sig[:rk], Sw[:rk], rtol=0, atol=1e-4 * Sw[0])
    assert np.all(np.abs(sig[rk:]) < 1e-3 * Sw[0])
    want_q, want_s = O.quantize_proj(P, "int4")
    assert np.array_equal(Pq, want_q) and np.array_equal(Ps, want_s), "INT4 codes of P"


def test_refresh_zero_gradient():
    """G = 0: nothing to project. The library's result is finite with zero singular values
    (its P is not compared: any orthonormal basis is an SVD of the zero matrix)."""
    bits = np.zeros((512, 384), np.uint16)
    P, sig, Pq, Ps = gpu_refresh(bits, 32, 40)
    assert np.isfinite(P).all() and np.isfinite(Ps).all()
    assert np.all(sig == 0.0)
    want_q, want_s = O.quantize_proj(P, "int4")
    assert np.array_equal(Pq, want_q) and np.array_equal(Ps, want_s), "INT4 codes of P"
