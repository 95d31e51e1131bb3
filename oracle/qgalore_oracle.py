"""Q-GaLore optimizer step: the CPU oracle.

TEST INFRASTRUCTURE ONLY. This module is the plain, slow, obviously-correct definition of
what the GPU library computes. Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import it. The product path (the HIP library and its
Python binding) never imports, calls or links anything here, and this module imports
nothing from the product path.

Sources (pages about the method; cited by title and locator):
  [QG-abs]  "Q-GaLore: Quantized GaLore with INT4 Projection and Layer-Adaptive Low-Rank
            Gradients", abstract (codewithpapers.app entry for arXiv 2407.08296).
  [QG-def]  AIMech curated page "Q-GaLore (Quantized GaLore with INT4 Projection and
            Layer-Adaptive Low-Rank Gradients)", definition paragraph.
  [QG-cos]  same page, mechanism claim "layer-adaptive subspace cosine schedule"
            (paper Section 3.1, Equation (5)).
  [QG-int]  same page, mechanism claim "INT4 projection and INT8 stochastic rounding"
            (paper Section 3.2, Figure 3).
  [QG-lim]  same page, limitation claim "simulated weight quantization throughput" and
            the curated-limitations list (paper Section 3.2, Section 4.4).
  [Philox]  Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
            SC'11, Section 3 (the Philox round function and key schedule).

Numeric contract (the pages fix the method, not the number formats; these readings are
this library's, and the GPU side implements the same contract independently):
  * fl(.) rounds to fp32 nearest-even after every single operation; no fused multiply-add.
    NumPy float32 arithmetic is exactly that.
  * bf(.) rounds fp32 to bf16 nearest-even. It is applied exactly twice in a step: to the
    dequantized projection (P~) and to the Adam update (N~). The gradient G arrives as bf16.
  * Group quantization: symmetric absmax over groups of 256 consecutive elements of the
    flattened row-major tensor (the last group may be short). s = fl(absmax / qmax),
    inv = fl(1 / s) (0 when s == 0), q = clamp(rne(fl(x * inv)), -qmax, qmax) with
    qmax = 127 (INT8: W, M, V) or 7 (INT4: P). rne is round-half-to-even.
  * INT4 packing: flat element 2k in the low nibble of byte k, 2k+1 in the high nibble,
    two's complement.
  * Projection is on the left: P is m x r, R = P~^T G (r x n), U = alpha * P~ N~ (m x n).
    Contractions are evaluated in float64 and rounded once to fp32.
  * Adam (Kingma-Ba with bias correction, eps = 1e-8 by default, no weight decay) runs on
    R with moments stored as INT8; the update uses the fresh fp32 moments, which are then
    requantized for storage.
  * Stochastic rounding of the weight update in units of the weight's group scale, with a
    16-bit uniform drawn from Philox4x32-10 keyed by (seed, step, layer, element).
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

GROUP = 256
QMAX_INT8 = 127
QMAX_INT4 = 7

F32 = np.float32
F64 = np.float64


# ---------------------------------------------------------------------------------------
# bf16
# ---------------------------------------------------------------------------------------

def f32_to_bf16_bits(x) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest, ties to even. NaN stays NaN (quiet).

    bf16 is the top half of an fp32 word; rounding adds 0x7FFF plus the lowest kept bit
    and truncates. Overflow carries into the exponent and gives inf, as IEEE requires.
    """
    x = np.ascontiguousarray(x, dtype=F32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    quiet_nan = ((u >> 16) | 0x0040) & 0xFFFF
    out = np.where(np.isnan(x), quiet_nan, rounded)
    return out.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """bf16 bit pattern -> fp32 value (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(F32)


def bf16_round(x) -> np.ndarray:
    """bf(x): the fp32 value of x rounded to bf16."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


# ---------------------------------------------------------------------------------------
# Group absmax quantization  [QG-def], [QG-int]: W, M, V in INT8 and P in INT4.
# ---------------------------------------------------------------------------------------

def n_groups(numel: int) -> int:
    return -(-int(numel) // GROUP)


def _grouped(x: np.ndarray) -> np.ndarray:
    flat = np.ascontiguousarray(x, dtype=F32).ravel()
    ng = n_groups(flat.size)
    padded = np.zeros(ng * GROUP, dtype=F32)
    padded[: flat.size] = flat
    return padded.reshape(ng, GROUP)


def group_scales(x, qmax: int) -> np.ndarray:
    """Per-group scale s = fl(absmax / qmax) (fp32, one per 256 flat elements)."""
    a = np.max(np.abs(_grouped(x)), axis=1)            # exact: max of fp32 magnitudes
    return (a / F32(qmax)).astype(F32)


def reciprocal_or_zero(s) -> np.ndarray:
    """inv = fl(1 / s), and 0 where s == 0."""
    s = np.asarray(s, dtype=F32)
    safe = np.where(s == 0, F32(1), s)
    return np.where(s == 0, F32(0), F32(1) / safe).astype(F32)


def absmax_quantize(x, qmax: int):
    """Symmetric absmax quantization over groups of 256 flat elements.

    Returns (codes int8 of x's shape, scales fp32[n_groups]).
    """
    x = np.asarray(x, dtype=F32)
    s = group_scales(x, qmax)
    inv = reciprocal_or_zero(s)
    flat = x.ravel()
    g = np.arange(flat.size) // GROUP
    scaled = (flat * inv[g]).astype(F32)
    q = np.clip(np.rint(scaled), -qmax, qmax).astype(np.int8)
    return q.reshape(x.shape), s


def dequantize(q, s) -> np.ndarray:
    """x = fl(float(q) * s[g]) for every flat element."""
    q = np.asarray(q)
    flat = q.ravel().astype(F32)
    g = np.arange(flat.size) // GROUP
    return (flat * np.asarray(s, dtype=F32)[g]).astype(F32).reshape(q.shape)


def pack_int4(q) -> np.ndarray:
    """Pack int codes in [-8, 7] two per byte: element 2k low nibble, 2k+1 high nibble."""
    flat = np.asarray(q).ravel().astype(np.int16)
    if flat.size % 2:
        flat = np.concatenate([flat, np.zeros(1, np.int16)])
    nib = (flat & 0xF).astype(np.uint8)
    return (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)


def unpack_int4(packed, numel: int) -> np.ndarray:
    """Inverse of pack_int4: returns int8 codes (two's-complement nibbles)."""
    b = np.asarray(packed, dtype=np.uint8).ravel()
    nib = np.empty(b.size * 2, dtype=np.int16)
    nib[0::2] = b & 0xF
    nib[1::2] = b >> 4
    nib = np.where(nib >= 8, nib - 16, nib)
    return nib[:numel].astype(np.int8)


# Projection storage formats. INT4 is the method's store [QG-int]; the same page sets it
# against GaLore's 16-bit projection and the 8-bit projection of the Q-GaLore baseline
# (identity notes), which these formats reproduce for comparison.
P_FORMATS = ("int4", "int8", "bf16")


def quantize_proj(P, fmt: str = "int4"):
    """Store an fp32 m x r projection in format fmt: INT4 (packed uint8[ceil(m*r/2)], fp32
    group scales), INT8 (int8[m*r], fp32 group scales) or bf16 (bit patterns uint16[m*r],
    no scales)."""
    if fmt == "int4":
        q, s = absmax_quantize(P, QMAX_INT4)
        return pack_int4(q), s
    if fmt == "int8":
        q, s = absmax_quantize(P, QMAX_INT8)
        return q.ravel().astype(np.int8), s
    if fmt == "bf16":
        return f32_to_bf16_bits(np.asarray(P, dtype=F32).ravel()), None
    raise ValueError(f"unknown projection format {fmt!r}")


def dequant_proj(Pq, Ps, m: int, r: int, fmt: str = "int4") -> np.ndarray:
    """P~ = bf(fl(q * s)) (or the stored bf16 values) as an m x r fp32 array whose values are
    bf16-exact."""
    if fmt == "int4":
        q = unpack_int4(Pq, m * r)
    elif fmt == "int8":
        q = np.asarray(Pq, dtype=np.int8).ravel()[: m * r]
    elif fmt == "bf16":
        return bf16_bits_to_f32(np.asarray(Pq).view(np.uint16).ravel()[: m * r]).reshape(m, r)
    else:
        raise ValueError(f"unknown projection format {fmt!r}")
    return bf16_round(dequantize(q, Ps)).reshape(m, r)


# ---------------------------------------------------------------------------------------
# Projection and back-projection  [QG-def], [QG-int]: R = P^T G and U = alpha * P N~.
# ---------------------------------------------------------------------------------------

def project(P, G) -> np.ndarray:
    """R = P^T G with the sum taken in float64 (the caller rounds to fp32)."""
    return np.asarray(P, dtype=F64).T @ np.asarray(G, dtype=F64)


def backproject(P, N) -> np.ndarray:
    """S = P N with the sum taken in float64 (the caller rounds to fp32 and scales)."""
    return np.asarray(P, dtype=F64) @ np.asarray(N, dtype=F64)


# ---------------------------------------------------------------------------------------
# Adam on the projected gradient with INT8 moments  [QG-def], [QG-int].
# ---------------------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Hyper:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    alpha: float = 0.25


def adam_constants(t: int, h: Hyper):
    """c1 = 1-b1, c2 = 1-b2, bc1 = 1-b1^t, bc2 = 1-b2^t: computed in double from the fp32
    hyperparameters (pow from the C library), then rounded once to fp32."""
    b1 = float(F32(h.beta1))
    b2 = float(F32(h.beta2))
    c1 = F32(1.0 - b1)
    c2 = F32(1.0 - b2)
    bc1 = F32(1.0 - math.pow(b1, float(t)))
    bc2 = F32(1.0 - math.pow(b2, float(t)))
    return c1, c2, bc1, bc2


def adam_core(R, m0, v0, t: int, h: Hyper):
    """One Adam update on fp32 moments, one fp32 rounding per operation.

    m1 = b1*m0 + c1*R ; v1 = b2*v0 + c2*(R*R) ; m^ = m1/bc1 ; v^ = v1/bc2 ;
    N = -(lr*m^) / (sqrt(v^) + eps).   Returns (m1, v1, N), all fp32.
    """
    c1, c2, bc1, bc2 = adam_constants(t, h)
    R = np.asarray(R, dtype=F32)
    b1, b2 = F32(h.beta1), F32(h.beta2)
    lr, eps = F32(h.lr), F32(h.eps)
    m1 = (b1 * np.asarray(m0, F32) + c1 * R).astype(F32)
    v1 = (b2 * np.asarray(v0, F32) + c2 * (R * R)).astype(F32)
    mh = (m1 / bc1).astype(F32)
    vh = (v1 / bc2).astype(F32)
    N = (-((lr * mh) / (np.sqrt(vh) + eps))).astype(F32)
    return m1, v1, N


def adam_int8(R, Mq, Ms, Vq, Vs, t: int, h: Hyper):
    """Adam with INT8 moment storage: dequantize, update, requantize.

    Returns (N, Mq', Ms', Vq', Vs', m1, v1).
    """
    m0 = dequantize(Mq, Ms)
    v0 = dequantize(Vq, Vs)
    m1, v1, N = adam_core(R, m0, v0, t, h)
    Mq2, Ms2 = absmax_quantize(m1, QMAX_INT8)
    Vq2, Vs2 = absmax_quantize(v1, QMAX_INT8)
    return N, Mq2, Ms2, Vq2, Vs2, m1, v1


# ---------------------------------------------------------------------------------------
# Philox4x32-10  [Philox]
# ---------------------------------------------------------------------------------------

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9   # golden ratio
PHILOX_W1 = 0xBB67AE85   # sqrt(3) - 1
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(counters, key):
    """Philox4x32 with 10 rounds on an (N, 4) array of 32-bit counters.

    One round: multiply words 0 and 2 by the two round multipliers into 64-bit products;
    the new words are (hi(M1*x2) ^ x1 ^ k0, lo(M1*x2), hi(M0*x0) ^ x3 ^ k1, lo(M0*x0)).
    The key (k0, k1) is bumped by the two Weyl constants between rounds.
    """
    c = np.asarray(counters, dtype=np.uint64).reshape(-1, 4) & _MASK32
    x0, x1, x2, x3 = (c[:, i].copy() for i in range(4))
    k0 = np.uint64(int(key[0]) & 0xFFFFFFFF)
    k1 = np.uint64(int(key[1]) & 0xFFFFFFFF)
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    for _ in range(10):
        p0 = x0 * m0
        p1 = x2 * m1
        x0, x1, x2, x3 = ((p1 >> np.uint64(32)) ^ x1 ^ k0,
                          p1 & _MASK32,
                          (p0 >> np.uint64(32)) ^ x3 ^ k1,
                          p0 & _MASK32)
        k0 = (k0 + np.uint64(PHILOX_W0)) & _MASK32
        k1 = (k1 + np.uint64(PHILOX_W1)) & _MASK32
    return np.stack([x0, x1, x2, x3], axis=1).astype(np.uint32)


def sr_uniform(seed: int, t: int, layer_id: int, i, j) -> np.ndarray:
    """The stochastic-rounding uniform for weight element (i, j) at step t of a layer.

    key = (seed mod 2^32, seed >> 32); counter = (j >> 3, i, t mod 2^32, layer_id).
    Word (j >> 1) & 3 of the Philox output holds elements 2w and 2w+1 of the 8-wide column
    block: the low 16 bits for even j, the high 16 bits for odd j. u = bits16 * 2^-16.
    """
    i = np.asarray(i, dtype=np.int64).ravel()
    j = np.asarray(j, dtype=np.int64).ravel()
    key = (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    ctr = np.stack([j >> 3, i, np.full_like(i, t & 0xFFFFFFFF),
                    np.full_like(i, layer_id & 0xFFFFFFFF)], axis=1)
    words = philox4x32_10(ctr, key)
    w = words[np.arange(i.size), (j >> 1) & 3].astype(np.uint32)
    bits = np.where((j & 1) == 1, w >> 16, w & 0xFFFF).astype(np.uint32)
    return (bits.astype(F32) * F32(2.0 ** -16)).astype(F32)


# ---------------------------------------------------------------------------------------
# Stochastic rounding into INT8 weights  [QG-def], [QG-int]: W <- W + xi(alpha P N~).
# ---------------------------------------------------------------------------------------

def stochastic_round(Wq, Ws, U, t: int, seed: int, layer_id: int, rows=None):
    """W' = clamp(floor(fl(fl(W + fl(U * inv_g)) + u)), -127, 127); W unchanged where the
    pre-floor value d is not finite.  With u uniform on [0, 1) the expectation of
    floor(w + a + u) is w + a, so the rounding is unbiased.

    `rows` (optional) restricts the computation to those weight rows; Wq and U then hold
    only those rows (used to check sampled rows of large layers).
    Returns (W', d) with d the pre-floor fp32 value (for margin accounting).
    """
    Wq = np.asarray(Wq, dtype=np.int8)
    U = np.asarray(U, dtype=F32)
    k, n = Wq.shape
    row_idx = np.arange(k) if rows is None else np.asarray(rows, dtype=np.int64)
    ii = np.repeat(row_idx, n)
    jj = np.tile(np.arange(n, dtype=np.int64), k)
    g = (ii * n + jj) // GROUP
    inv = reciprocal_or_zero(np.asarray(Ws, F32))[g]
    a = (U.ravel() * inv).astype(F32)
    tp = (Wq.ravel().astype(F32) + a).astype(F32)
    u = sr_uniform(seed, t, layer_id, ii, jj)
    d = (tp + u).astype(F32)
    with np.errstate(invalid="ignore"):
        new = np.clip(np.floor(d), -QMAX_INT8, QMAX_INT8)
        out = np.where(np.isfinite(d), new, Wq.ravel().astype(F32)).astype(np.int8)
    return out.reshape(k, n), d.reshape(k, n)


# ---------------------------------------------------------------------------------------
# The whole per-layer step
# ---------------------------------------------------------------------------------------

@dataclasses.dataclass
class LayerState:
    """One linear layer's optimizer state (all arrays host-side, row-major)."""
    m: int
    n: int
    r: int
    layer_id: int
    Wq: np.ndarray      # int8 m x n
    Ws: np.ndarray      # fp32 [groups(m*n)]   (fixed during the step)
    Pq: np.ndarray      # INT4: uint8 [ceil(m*r/2)] packed; INT8: int8 [m*r]; bf16: uint16
    Ps: np.ndarray      # fp32 [groups(m*r)] (None for bf16)
    Mq: np.ndarray      # int8 r x n
    Ms: np.ndarray      # fp32 [groups(r*n)]
    Vq: np.ndarray      # int8 r x n
    Vs: np.ndarray      # fp32 [groups(r*n)]
    p_format: str = "int4"

    def copy(self) -> "LayerState":
        return dataclasses.replace(self, **{f: (None if getattr(self, f) is None
                                                else getattr(self, f).copy()) for f in
                                            ("Wq", "Ws", "Pq", "Ps", "Mq", "Ms", "Vq", "Vs")})


@dataclasses.dataclass
class StepResult:
    R: np.ndarray       # fp32 r x n
    N: np.ndarray       # fp32 r x n (before bf16 rounding)
    Nb: np.ndarray      # fp32 r x n, bf16-exact
    m1: np.ndarray      # fp32 moments before requantization
    v1: np.ndarray
    U: np.ndarray       # fp32 m x n (or the sampled rows)
    d: np.ndarray       # fp32 pre-floor stochastic-rounding values


def qgalore_step(st: LayerState, G_bits, t: int, seed: int, h: Hyper = Hyper(),
                 rows=None) -> StepResult:
    """One Q-GaLore optimizer step for one layer, updating `st` in place.

    Follows the update rule of [QG-int] in the order the method runs it:
      1. P~ = bf(dequant(P_q))                       (INT4 projection, bf16 operand)
      2. R  = fl(P~^T G)                              (low-rank projected gradient)
      3. Adam on R with INT8 M, V -> N, new M, V      (moments requantized per group)
      4. N~ = bf(N)
      5. U  = fl(alpha * fl(P~ N~))                   (back-projection)
      6. W  <- SR(W + U / s_W)                        (unbiased stochastic rounding)
    `rows`: compute steps 5-6 only for those weight rows (W rows outside are untouched).
    """
    assert 1 <= t < 2 ** 32
    m, n, r = st.m, st.n, st.r
    Pt = dequant_proj(st.Pq, st.Ps, m, r, st.p_format)
    G = bf16_bits_to_f32(np.asarray(G_bits, dtype=np.uint16).reshape(m, n))
    R = project(Pt, G).astype(F32)
    N, Mq, Ms, Vq, Vs, m1, v1 = adam_int8(R, st.Mq, st.Ms, st.Vq, st.Vs, t, h)
    Nb = bf16_round(N)
    P_rows = Pt if rows is None else Pt[np.asarray(rows)]
    S = backproject(P_rows, Nb).astype(F32)
    U = (F32(h.alpha) * S).astype(F32)
    W_rows = st.Wq if rows is None else st.Wq[np.asarray(rows)]
    W_new, d = stochastic_round(W_rows, st.Ws, U, t, seed, st.layer_id, rows=rows)
    if rows is None:
        st.Wq = W_new
    else:
        st.Wq[np.asarray(rows)] = W_new
    st.Mq, st.Ms, st.Vq, st.Vs = Mq, Ms, Vq, Vs
    return StepResult(R=R, N=N, Nb=Nb, m1=m1, v1=v1, U=U, d=d)


# ---------------------------------------------------------------------------------------
# Subspace similarity and the layer-adaptive refresh schedule  [QG-cos]
# ---------------------------------------------------------------------------------------

GAMMA_DEFAULT = 0.4      # [QG-cos]: default threshold


def cossim_float(A, B) -> float:
    """CosSim(A, B) = (1/r) * sum_i sigma_i(A^T B) for m x r A and B (float64)."""
    C = np.asarray(A, dtype=F64).T @ np.asarray(B, dtype=F64)
    r = C.shape[0]
    return float(np.sum(np.linalg.svd(C, compute_uv=False)) / r)


def cossim(Pq_new, Ps_new, Pq_old, Ps_old, m: int, r: int, fmt: str = "int4") -> float:
    """CosSim between two stored projections (format fmt), each dequantized and bf16-rounded
    as the step uses it."""
    return cossim_float(dequant_proj(Pq_new, Ps_new, m, r, fmt),
                        dequant_proj(Pq_old, Ps_old, m, r, fmt))


@dataclasses.dataclass
class LayerSchedule:
    """Per-layer refresh bookkeeping of [QG-cos].

    A refresh (new P from an SVD of the current gradient) falls due at t == next_refresh.
    At every refresh after the first, the new projection is compared with the previous
    one; a similarity above gamma doubles the interval. The next refresh is then scheduled
    with the (possibly doubled) interval. Moments are kept across refreshes.
    """
    delta: int
    gamma: float = GAMMA_DEFAULT
    next_refresh: int = 0
    count: int = 0
    last_cossim: float = float("nan")

    def due(self, t: int) -> bool:
        return t >= self.next_refresh

    def refresh(self, t: int, cs: float | None) -> bool:
        """Record a refresh at step t. `cs` is CosSim(P_new, P_old) (ignored for the first
        refresh). Returns True when the interval doubled."""
        doubled = False
        if self.count > 0:
            if cs is None:
                raise ValueError("a refresh after the first needs the similarity value")
            self.last_cossim = float(cs)
            if cs > self.gamma:
                self.delta *= 2
                doubled = True
        self.count += 1
        self.next_refresh = t + self.delta
        return doubled


def simulate_schedule(cossim_fn, delta0: int, T: int, gamma: float = GAMMA_DEFAULT):
    """Run one layer's schedule over steps 0..T-1. cossim_fn(t_new, t_old) gives the
    similarity of the projections computed at those two steps. Returns (refresh steps, final
    interval)."""
    s = LayerSchedule(delta=delta0, gamma=gamma)
    steps = []
    last = None
    for t in range(T):
        if s.due(t):
            cs = None if last is None else cossim_fn(t, last)
            s.refresh(t, cs)
            steps.append(t)
            last = t
    return steps, s.delta


def fixed_interval_refreshes(delta0: int, T: int) -> int:
    """Refresh count of the fixed-interval baseline (an SVD every delta0 steps)."""
    return len(range(0, T, delta0))


# ---------------------------------------------------------------------------------------
# The refresh itself  [QG-def], [QG-int]: a layer's projection holds the r leading
# singular vectors of its gradient, recomputed by an SVD (projection on the left: the
# left singular vectors, P is m x r).
# ---------------------------------------------------------------------------------------

def normalize_column_signs(P) -> np.ndarray:
    """Singular vectors are defined up to sign; this library's convention makes each
    column's entry of largest magnitude positive (the first such row on ties)."""
    P = np.array(P, dtype=F64, copy=True)
    idx = np.argmax(np.abs(P), axis=0)
    neg = P[idx, np.arange(P.shape[1])] < 0
    P[:, neg] *= -1.0
    return P


def refresh_projection(G_bits, r: int):
    """P = the r leading left singular vectors of G (bf16 bit patterns, m x n), by a full
    SVD in float64, with the sign convention above; also returns the r leading singular
    values."""
    G = bf16_bits_to_f32(G_bits).astype(F64)
    U, S, _ = np.linalg.svd(G, full_matrices=False)
    return normalize_column_signs(U[:, :r]), S[:r]


# ---------------------------------------------------------------------------------------
# A linear layer whose weight is stored as INT8  [QG-lim]: activations stay 16-bit, and the
# INT8 weight (with its group scales, the format of W_q / W_s above) is dequantized to bf16
# inside the forward and backward products. Shapes: X is T x n (tokens x inputs), W is m x n
# (outputs x inputs, as the optimizer holds it), Y and dY are T x m. Products are summed in
# float64, rounded once to fp32 and then to bf16 (the activation format).
# ---------------------------------------------------------------------------------------

def dequant_weight(Wq, Ws, m: int, n: int) -> np.ndarray:
    """W~ = bf(fl(q * s)) as an m x n fp32 array of bf16-exact values."""
    q = np.asarray(Wq, dtype=np.int8).ravel()[: m * n]
    return bf16_round(dequantize(q, Ws)).reshape(m, n)


def _to_bf16_bits(x64) -> np.ndarray:
    return f32_to_bf16_bits(np.asarray(x64, dtype=F64).astype(F32))


def linear_forward(X_bits, Wq, Ws, m: int, n: int) -> np.ndarray:
    """Y = X W~^T (T x m), bf16 bit patterns."""
    X = bf16_bits_to_f32(X_bits).astype(F64).reshape(-1, n)
    return _to_bf16_bits(X @ dequant_weight(Wq, Ws, m, n).astype(F64).T)


def linear_backward_data(dY_bits, Wq, Ws, m: int, n: int) -> np.ndarray:
    """dX = dY W~ (T x n), bf16 bit patterns."""
    dY = bf16_bits_to_f32(dY_bits).astype(F64).reshape(-1, m)
    return _to_bf16_bits(dY @ dequant_weight(Wq, Ws, m, n).astype(F64))


def linear_backward_weight(dY_bits, X_bits) -> np.ndarray:
    """G = dY^T X (m x n), bf16 bit patterns: the weight gradient the optimizer step takes."""
    dY = bf16_bits_to_f32(dY_bits).astype(F64)
    X = bf16_bits_to_f32(X_bits).astype(F64)
    return _to_bf16_bits(dY.T @ X)
