"""Helpers shared by the GPU parity tests: building one layer's state on both sides from the
seeded generators, and the comparison rules.

Comparison rules (GPU against the oracle, same seeded inputs):
  * fp32 R and U: |gpu - oracle| <= 2e-3 * |oracle| + 2e-3 * rms(oracle) elementwise. U is
    compared at that bound with the oracle's back-projection of the N~ that the GPU's own R
    gives. End to end, N~ elements that the two R round to different bf16 values are allowed
    only as flips the R difference explains (explained_n_flips: the GPU's N~ is the rounding
    of the N its R gives, the oracle's N lies within the R difference's reach of a rounding
    boundary, and there are no more flips than that difference explains), and the bound
    grows by alpha * |P~| |delta N~| in the columns that hold such a flip.
  * R as a whole: rms(gpu - oracle) <= 2e-5 rms(oracle), the scale of an fp32 sum's
    rounding; a sum in a lower precision, or with terms lost, fails it.
  * INT8 codes (W, M, V): identical, except +-1 differences at elements whose rounding input
    sits at a decision boundary within the reach of the tolerated fp32 difference. For W the
    rounding input is d = W + U/s + u and the boundary an integer; for M and V it is x * inv
    and the boundary a half-integer. An element's allowed reach is
        1e-5 + |input_gpu - input_oracle| estimated from the fp32 difference of its source
    (U for W, R for M and V). At most 1e-4 of the compared elements may differ (at least one
    element is allowed, so that a tensor under 10^4 elements can show one explained flip).
  * Group scales of M and V: relative difference <= 1e-5.
"""
from __future__ import annotations

import numpy as np

from oracle import qgalore_oracle as O
from quantized_rank_gradient_amd import workloads as WL

F32 = np.float32

# R differences of an fp32 sum of exact bf16 products over K terms grow like 2^-24 sqrt(K)
# relative to rms(R) (about 4e-6 at K = 11008): 2e-5 leaves that margin five times over and
# is still fifty times below what a single bf16 rounding of R would leave (2^-9 / sqrt(3)).
R_ACCUM_RMS = 2e-5


def host_state(cfg, L, r, moments="zero", P=None, fmt="int4"):
    """Oracle-side state of one layer (numpy) and the float projection it was made from."""
    if P is None:
        P = WL.orthonormal_f32(cfg, L, r)
    Pq, Ps = O.quantize_proj(P, fmt)
    if moments == "zero":
        Mq, Ms, Vq, Vs = WL.zero_moments(r, L.n)
    else:
        Mq, Ms, Vq, Vs = WL.random_moments(cfg, L, r)
    st = O.LayerState(L.m, L.n, r, L.layer_id, WL.weights_int8(cfg, L), WL.weight_scales(cfg, L),
                      Pq, Ps, Mq, Ms, Vq, Vs, p_format=fmt)
    return st, P


def to_device(st, G_bits, P_float=None, quantize_on_gpu=True):
    """GPU-side tensors for the library. The projection is quantized by the library's own
    kernel from the same float P when `quantize_on_gpu` (the caller checks it against the
    oracle's codes)."""
    import torch
    from quantized_rank_gradient_amd import binding as B
    dev = torch.device("cuda:0")

    def t(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    fmt = st.p_format
    if quantize_on_gpu and P_float is not None:
        Pq, Ps = B.quantize_proj(t(P_float.astype(F32)), fmt=fmt)
    elif fmt == "bf16":
        Pq, Ps = t(st.Pq.view(np.int16)).view(torch.bfloat16), None
    else:
        Pq, Ps = t(st.Pq), t(st.Ps)
    G = t(G_bits.view(np.int16)).view(torch.bfloat16).reshape(st.m, st.n)
    return B.LayerTensors(layer_id=st.layer_id, G=G, Wq=t(st.Wq), Ws=t(st.Ws), Pq=Pq, Ps=Ps,
                          Mq=t(st.Mq), Ms=t(st.Ms), Vq=t(st.Vq), Vs=t(st.Vs), r=st.r,
                          p_format=fmt)


def assert_close_f32(gpu, ref, name, rtol=2e-3, extra=0.0):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    err = np.abs(gpu - ref)
    bound = rtol * np.abs(ref) + rtol * rms + extra
    bad = err > bound
    assert not bad.any(), (f"{name}: {int(bad.sum())} of {ref.size} outside tolerance; worst "
                           f"{float(err.max()):.3e} vs rms {rms:.3e}")


def assert_fp32_accumulation(gpu, ref, name, rel_rms=R_ACCUM_RMS):
    """The difference of a product that the GPU accumulates in fp32 from the oracle's, as a
    whole: rms(gpu - oracle) <= rel_rms * rms(oracle)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64).reshape(gpu.shape)
    if ref.size == 0:
        return
    rms = float(np.sqrt(np.mean(ref ** 2)))
    d = float(np.sqrt(np.mean((gpu - ref) ** 2)))
    print(f"{name}: rms difference {d / rms if rms else 0.0:.2e} of rms")
    assert d <= rel_rms * rms, f"{name}: rms difference {d:.3e} above {rel_rms} of rms {rms:.3e}"


def assert_codes(gpu, ref, x_ref, boundary, reach, name, cap=1e-4):
    """INT8 code parity. x_ref: the oracle's rounding input; boundary: 'int' (floor) or 'half'
    (round-half-even); reach: per-element allowed distance from the boundary."""
    gpu = np.asarray(gpu).astype(np.int32).ravel()
    ref = np.asarray(ref).astype(np.int32).ravel()
    x = np.asarray(x_ref, np.float64).ravel()
    diff = gpu - ref
    bad = diff != 0
    if not bad.any():
        return 0
    assert np.all(np.abs(diff) <= 1), f"{name}: a code differs by more than 1"
    if boundary == "int":
        margin = np.abs(x - np.rint(x))
    else:
        margin = np.abs(np.abs(x - np.floor(x)) - 0.5)
    reach = np.broadcast_to(np.asarray(reach, np.float64), x.shape)
    unexplained = bad & ~(margin <= reach)
    assert not unexplained.any(), (
        f"{name}: {int(unexplained.sum())} differing codes away from a rounding boundary "
        f"(margins {margin[unexplained][:5]}, reach {reach[unexplained][:5]})")
    frac = bad.mean()
    assert bad.sum() <= max(1.0, cap * bad.size), (
        f"{name}: {int(bad.sum())} differing codes ({frac:.2e} > {cap})")
    return int(bad.sum())




def _bf16_step(b, up):
    """The bf16 value next to the bf16-exact fp32 values b (bit patterns as int64), one unit
    up (towards +inf) where `up`, else down."""
    o = np.where(b < 0, -(b & 0x7FFFFFFF), b) >> 16          # sign-magnitude to integer line
    o = o + np.where(up, 1, -1)
    bits = np.where(o >= 0, o << 16, ((-o) << 16) | 0x80000000)
    return bits.astype(np.uint32).view(F32)


def _bf16_spacing(b):
    """Distance between consecutive bf16 values around the bf16-exact fp32 values b."""
    a = np.abs(np.asarray(b, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def expected_n_flips(N_g, N_o):
    """Expected number of bf16 rounding flips between N_g and N_o: an element whose two values
    lie delta apart, at a position that a rounding boundary does not favour, straddles one of
    the boundaries (bf16 spacing u apart) with probability min(1, delta / u)."""
    d = np.abs(np.asarray(N_g, np.float64) - np.asarray(N_o, np.float64))
    u = _bf16_spacing(O.bf16_round(np.asarray(N_o, F32)))
    return float(np.minimum(1.0, d / u).sum())


def explained_n_flips(N_g, Nb_g, N_o, Nb_o, P_rows, alpha):
    """The N~ elements that the GPU's R and the oracle's R round to different bf16 values, each
    checked to be a flip that the R difference explains, and the effect those flips carry
    into U.

    N_g is the oracle's Adam on the GPU's own fp32 R (which the caller has checked against the
    R bound), N_o the oracle's end to end (both fp32, before rounding); Nb_g, Nb_o their bf16
    roundings. Where N is steep in R (first step, R near zero: N = -lr R / (|R| + eps)) a
    tolerated R difference can move N across several bf16 values, so the rule is:
      * Nb_g is the rounding of N_g (the GPU's N~ is the one its R gives);
      * the oracle's N lies within reach of the rounding boundary next to it in the direction
        of N_g, the reach being |N_g - N_o| (what the R difference moves N by) plus 4 fp32
        ulps of N (given the two roundings, a consistency check);
      * the number of flips is what the N difference explains: at most 2 E + 4, E being
        expected_n_flips(N_g, N_o) (the flips are a sum of independent events of mean E, so
        2 E + 4 is far in the tail; more flips than that point to boundaries the two sides
        place differently, not to the R difference).
    Returns the bound extension for the end-to-end U check: alpha * |P~| |Nb_g - Nb_o|, which
    is non-zero only in the columns of N~ that hold a flip."""
    from oracle import qgalore_oracle as O
    Nb_g = np.asarray(Nb_g, F32)
    Nb_o = np.asarray(Nb_o, F32)
    assert np.array_equal(O.bf16_round(np.asarray(N_g, F32)), Nb_g), "GPU N~ is not bf16(N) of its R"
    assert np.array_equal(O.bf16_round(np.asarray(N_o, F32)), Nb_o), "oracle N~ is not bf16(N)"
    flips = Nb_g != Nb_o
    nflip = int(flips.sum())
    if nflip == 0:
        return 0.0
    E = expected_n_flips(N_g, N_o)
    print(f"N~ flips: {nflip} of {flips.size}, {E:.1f} expected from the N difference")
    assert nflip <= 2.0 * E + 4.0, (
        f"N~: {nflip} of {flips.size} elements round to another bf16 value, more than the "
        f"N difference explains ({E:.1f} expected)")
    ng = np.asarray(N_g, F32)[flips].astype(np.float64)
    no = np.asarray(N_o, F32)[flips].astype(np.float64)
    bo = Nb_o[flips].view(np.int32).astype(np.int64)
    nxt = _bf16_step(bo, ng > no).astype(np.float64)
    mid = (Nb_o[flips].astype(np.float64) + nxt) / 2
    reach = np.abs(ng - no) + 4 * np.spacing(np.abs(np.asarray(N_o, F32)[flips])).astype(np.float64)
    margin = np.abs(no - mid)
    assert np.all(margin <= reach), (
        f"N~: flips away from a bf16 rounding boundary (margins {margin[margin > reach][:4]}, "
        f"reach {reach[margin > reach][:4]})")
    dNb = np.abs(Nb_g.astype(np.float64) - Nb_o.astype(np.float64))
    cols = np.flatnonzero(flips.any(axis=0))
    carried = np.zeros((np.asarray(P_rows).shape[0], Nb_g.shape[1]), np.float64)
    carried[:, cols] = np.float64(alpha) * (np.abs(np.asarray(P_rows, np.float64)) @ dNb[:, cols])
    return carried


def check_step(st_before, res, st_after, gpu_out, hp=O.Hyper(), rows=None, t=1):
    """Compare one GPU step (gpu_out: dict of numpy arrays R, U, Wq, Mq, Ms, Vq, Vs) with the
    oracle's step `res` at step t that took `st_before` to `st_after`.

    U is checked stage by stage. The oracle's Adam and back-projection run once more on the
    GPU's own R (fp32, as the GPU holds it): that reproduces the GPU's N~ exactly (Adam is
    elementwise fp32 arithmetic), and U must match that back-projection to the tolerance.
    Against the oracle's end-to-end U, the only further difference allowed is what the
    N~ elements that round differently (bf16 neighbours, because R came out of a different
    summation order) carry through the back-projection."""
    assert_close_f32(gpu_out["R"], res.R, "R")
    assert_fp32_accumulation(gpu_out["R"], res.R, "R")
    U_gpu = gpu_out["U"] if rows is None else gpu_out["U"][np.asarray(rows)]
    m, r = st_before.m, st_before.r
    Pt = O.dequant_proj(st_before.Pq, st_before.Ps, m, r, st_before.p_format)
    P_rows = Pt if rows is None else Pt[np.asarray(rows)]
    R_gpu = np.asarray(gpu_out["R"], F32).reshape(res.R.shape)
    N_g = O.adam_int8(R_gpu, st_before.Mq, st_before.Ms, st_before.Vq, st_before.Vs, t, hp)[0]
    Nb_g = O.bf16_round(N_g)
    U_same_n = (F32(hp.alpha) * O.backproject(P_rows, Nb_g).astype(F32)).astype(F32)
    assert_close_f32(U_gpu, U_same_n, "U (back-projection of the GPU's N~)")
    carried = explained_n_flips(N_g, Nb_g, res.N, res.Nb, P_rows, hp.alpha)
    if np.any(carried):
        rms_u = float(np.sqrt(np.mean(np.asarray(res.U, np.float64) ** 2)))
        print(f"N~ flips carried into U: largest {float(np.max(carried)) / rms_u:.3e} of rms(U)")
    assert_close_f32(U_gpu, res.U, "U", extra=carried)

    # M and V: the rounding input is m1 * inv; the GPU's differs through R (and the scale)
    g = np.arange(res.m1.size) // O.GROUP
    invM = O.reciprocal_or_zero(st_after.Ms)[g]
    invV = O.reciprocal_or_zero(st_after.Vs)[g]
    c1, c2, _, _ = O.adam_constants(1, hp)
    dR = np.abs(gpu_out["R"].astype(np.float64) - res.R.astype(np.float64)).ravel()
    R64 = np.abs(res.R.astype(np.float64)).ravel()
    xm = res.m1.astype(np.float64).ravel() * invM
    xv = res.v1.astype(np.float64).ravel() * invV
    invM_g = O.reciprocal_or_zero(gpu_out["Ms"])[g].astype(np.float64)
    invV_g = O.reciprocal_or_zero(gpu_out["Vs"])[g].astype(np.float64)
    with np.errstate(invalid="ignore", divide="ignore"):
        rel_m = np.where(invM > 0, np.abs(invM_g / invM - 1.0), 0.0)
        rel_v = np.where(invV > 0, np.abs(invV_g / invV - 1.0), 0.0)
    reach_m = 1e-5 + 2 * np.float64(c1) * dR * invM + np.abs(xm) * (rel_m + 2e-7)
    reach_v = 1e-5 + 2 * np.float64(c2) * 2 * R64 * dR * invV + np.abs(xv) * (rel_v + 2e-7)
    assert np.allclose(gpu_out["Ms"], st_after.Ms, rtol=1e-5, atol=0), "M scales"
    assert np.allclose(gpu_out["Vs"], st_after.Vs, rtol=1e-5, atol=0), "V scales"
    assert_codes(gpu_out["Mq"], st_after.Mq, xm, "half", reach_m, "M")
    assert_codes(gpu_out["Vq"], st_after.Vq, xv, "half", reach_v, "V")

    # W: rounding input d = W + U * inv_s + u
    Wg = gpu_out["Wq"] if rows is None else gpu_out["Wq"][np.asarray(rows)]
    Wr = st_after.Wq if rows is None else st_after.Wq[np.asarray(rows)]
    n = st_before.n
    rows_idx = np.arange(Wr.shape[0]) if rows is None else np.asarray(rows)
    e = (rows_idx[:, None] * n + np.arange(n)[None, :]).ravel()
    inv = O.reciprocal_or_zero(st_before.Ws)[e // O.GROUP].astype(np.float64)
    dU = np.abs(U_gpu.astype(np.float64) - res.U.astype(np.float64)).ravel()
    reach_w = 1e-5 + dU * inv + 2 * np.spacing(np.float32(128.0))
    return assert_codes(Wg, Wr, res.d, "int", reach_w, "W")
