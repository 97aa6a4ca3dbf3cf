"""Plain, slow, float64 CPU oracle of the Muon and Dimuon optimizer steps.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, never by the product path.  It
shares no code, header, table or constant with the HIP library.

Sources (cited by page title and section):

* "Muon Optimizer 정리" (dongju923.github.io): section "업데이트 규칙",
  eqs. (1)-(3): momentum, orthogonalisation, weight update; the unrolled
  momentum sum below eq. (1); section "Newton-Schulz 직교화": the odd
  quintic f(x) = a x + b x^3 + c x^5 with (a, b, c) = (3.4445, -4.7750,
  2.0315) and the polar identity (M M^T)^(-1/2) M = U V^T; section
  "참고: 대규모 학습으로의 확장": weight decay and a per-parameter update
  scale.
* "Muon. ինչ է լինում, երբ LLM-ի օպտիմիզատորը ..." (sitech.ge), section
  "SVD-ի փոխարեն՝ Newton–Schulz": divide by the Frobenius norm, then apply
  X <- aX + b(XX^T)X + c(XX^T)^2 X, usually five times, in bfloat16.
* "Dimuon: LoRA 에 맞춰 다시 짠 Muon" (optim-book, "Dimuon diagonal
  conditioning"): sections "양쪽에서 −1/4 제곱" (the same diagonal factors
  multiply the momentum before and after orthogonalisation; energy is the
  square of the entry size), "왜 「지난」 모멘텀인가" (the factors come from
  the previous step's momentum; a zero previous momentum turns them off),
  "문제 4. 감쇠 10⁻⁴ 는 무엇을 막는가" (factor = (relative energy + 1e-4)^(-1/4);
  the norm is fixed afterwards).
* "From PCG to Muon" (hwan-h-heo.github.io), section "6. Muon Reshaping /
  Muon's Gram Matrix": for an N x 2 matrix the Gram matrix taken is the 2 x 2
  one, G^T G.

Readings where the pages are silent or garbled (each is listed with its
evidence in the design notes):

* The Dimuon display formula did not survive extraction.  Reading:
  O ∝ D_R · NS(D_R M D_C) · D_C with the same D_R, D_C on both sides.
* "Relative energy" is relative to the largest row (column) energy.
* Energies are sums of squares of the previous momentum as stored, summed in
  float32 by the pairwise tree of :func:`pairwise_sum_f32`.
* After the post-scale, the step is rescaled so that ||O||_F = ||Z||_F
  ("the norm is fixed afterwards").
* Wide or square matrices iterate on X, tall ones on X^T, so the Gram matrix
  is min(m, n) square.
* The momentum buffer is stored in its own dtype (float32 or bfloat16); the
  orthogonaliser reads the stored value.
* Nesterov input (not printed on the pages): G + mu * M_t.
* Weight decay and update scale: W <- W - lr * (scale * O + wd * W).
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

import numpy as np

# "Muon Optimizer 정리", section "Newton-Schulz 직교화": the quintic's coefficients.
NS5_COEFFS: Tuple[float, float, float] = (3.4445, -4.7750, 2.0315)

# "Dimuon: LoRA 에 맞춰 다시 짠 Muon", "문제 4": the 1e-4 floor added to the
# relative energy.
DIMUON_EPS: float = 1e-4


# ----------------------------------------------------------------------------
# Storage rounding (what a float32 / bfloat16 tensor can hold)
# ----------------------------------------------------------------------------

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def _round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even).

    bfloat16 keeps 8 significant bits and float32's exponent range; the
    rounding is done once, straight from float64.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    finite = np.isfinite(x) & (x != 0.0)
    xf = x[finite]
    _, e = np.frexp(xf)                    # xf = m * 2**e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                # below 2**-126: fixed subnormal quantum
    quantum = np.ldexp(1.0, e - 8)         # 8 significant bits
    r = np.rint(xf / quantum) * quantum    # np.rint rounds half to even
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, r), r)
    out[finite] = r
    return out


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Value a tensor of ``dtype`` ('f32', 'bf16' or 'f64') would hold."""
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return _round_bf16(x)
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------
# Momentum ("Muon Optimizer 정리", eq. (1))
# ----------------------------------------------------------------------------

def momentum_update(m_prev: np.ndarray, g: np.ndarray, mu: float,
                    mom_dtype: str = "f64") -> np.ndarray:
    """M_t = mu * M_{t-1} + grad, stored in the momentum buffer's dtype.

    No (1 - mu) factor and no dampening: eq. (1) adds the raw gradient.
    """
    m = mu * np.asarray(m_prev, dtype=np.float64) + np.asarray(g, dtype=np.float64)
    return round_to_dtype(m, mom_dtype)


def nesterov_input(m_t: np.ndarray, g: np.ndarray, mu: float) -> np.ndarray:
    """Input to the orthogonaliser under Nesterov momentum: G + mu * M_t.

    "From PCG to Muon", "DL Optimizer w/ Line Search", names Nesterov momentum
    for Muon without printing it; this is the look-ahead reading.
    """
    return np.asarray(g, dtype=np.float64) + mu * np.asarray(m_t, dtype=np.float64)


# ----------------------------------------------------------------------------
# Dimuon energies and conditioning ("Dimuon: LoRA 에 맞춰 다시 짠 Muon")
# ----------------------------------------------------------------------------

def energies_f64(m_prev: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Row and column energies (sums of squared entries) in float64."""
    sq = np.asarray(m_prev, dtype=np.float64) ** 2
    return sq.sum(axis=1), sq.sum(axis=0)


def pairwise_sum_f32(p: np.ndarray) -> np.float32:
    """Float32 sum of ``p`` (1-D) by the stated pairwise tree.

    The sequence is padded with zeros to a power-of-two length; then, level by
    level, element 2i of the next level is (element 2i) + (element 2i+1) of
    this one, each addition rounded to float32.  Every addend is >= 0 here, so
    the amount of zero padding does not change the result.
    """
    a = np.asarray(p, dtype=np.float32).ravel()
    if a.size == 0:
        return np.float32(0.0)
    size = 1
    while size < a.size:
        size *= 2
    buf = np.zeros(size, dtype=np.float32)
    buf[: a.size] = a
    while buf.size > 1:
        buf = (buf[0::2] + buf[1::2]).astype(np.float32)
    return np.float32(buf[0])


def energies_f32_tree(m_prev: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Row energies R (length m) and column energies C (length n) in float32.

    Each square is fl32(x * x) of the stored value x; each sum is
    :func:`pairwise_sum_f32` over the row (for R) or the column (for C) in
    increasing index order.
    """
    x = np.asarray(m_prev, dtype=np.float64)
    # The product of two float32 values is exact in float64, so one float32
    # rounding gives the correctly rounded float32 square.
    sq = (x * x).astype(np.float32)
    m, n = sq.shape
    r = np.array([pairwise_sum_f32(sq[i, :]) for i in range(m)], dtype=np.float32)
    c = np.array([pairwise_sum_f32(sq[:, j]) for j in range(n)], dtype=np.float32)
    return r, c


def conditioning(energy: np.ndarray, eps: float = DIMUON_EPS) -> np.ndarray:
    """Diagonal factor (relative energy + eps)^(-1/4), in float64.

    Relative energy is energy / max(energy).  When every energy is zero (the
    first step, where the previous momentum is zero) the factor is 1: the
    conditioning is off.
    """
    e = np.asarray(energy, dtype=np.float64)
    if e.size == 0:
        return e.copy()
    emax = e.max()
    if not emax > 0.0:
        return np.ones_like(e)
    rho = e / emax
    return (rho + eps) ** -0.25


# ----------------------------------------------------------------------------
# Newton-Schulz orthogonalisation
# ----------------------------------------------------------------------------

def _coeffs_for(t: int, coeffs, schedule) -> Tuple[float, float, float]:
    if schedule is not None:
        a, b, c = schedule[t]
        return float(a), float(b), float(c)
    a, b, c = coeffs
    return float(a), float(b), float(c)


def newton_schulz(m: np.ndarray, steps: int = 5,
                  coeffs: Tuple[float, float, float] = NS5_COEFFS,
                  schedule: Optional[Sequence[Tuple[float, float, float]]] = None
                  ) -> np.ndarray:
    """NS5(M): Frobenius-normalise, then ``steps`` quintic iterations.

    sitech.ge Muon blog, "SVD-ի փոխարեն՝ Newton–Schulz": X = M / ||M||_F, then
    X <- aX + b(XX^T)X + c(XX^T)^2 X.  A tall matrix is iterated as its
    transpose so the Gram matrix XX^T is min(m, n) square ("From PCG to
    Muon", "Muon's Gram Matrix"), and the result is transposed back.
    ``schedule`` (one (a, b, c) per iteration) replaces the fixed triple.
    A zero matrix maps to zero.
    """
    x = np.asarray(m, dtype=np.float64)
    nu = np.sqrt(np.sum(x * x))
    if nu == 0.0:
        return np.zeros_like(x)
    x = x / nu
    tall = x.shape[0] > x.shape[1]
    if tall:
        x = x.T
    for t in range(steps):
        a, b, c = _coeffs_for(t, coeffs, schedule)
        gram = x @ x.T                       # XX^T
        x = a * x + b * (gram @ x) + c * ((gram @ gram) @ x)
    if tall:
        x = x.T
    return np.ascontiguousarray(x)


# ----------------------------------------------------------------------------
# Whole steps
# ----------------------------------------------------------------------------

@dataclass
class StepResult:
    w: np.ndarray          # updated weight, rounded to the weight dtype
    m: np.ndarray          # new momentum as stored
    o: np.ndarray          # orthogonalised step O (before the learning rate)
    r: Optional[np.ndarray] = None    # float32 row energies of M_prev (Dimuon)
    c: Optional[np.ndarray] = None    # float32 column energies of M_prev
    d_r: Optional[np.ndarray] = None  # row factors
    d_c: Optional[np.ndarray] = None  # column factors


def _apply_update(w, o, lr, scale, weight_decay, w_dtype):
    """W_t = W_{t-1} - lr * (scale * O + weight_decay * W_{t-1}).

    "Muon Optimizer 정리", eq. (3) with the weight decay and per-parameter
    update scale of section "참고: 대규모 학습으로의 확장" (both default off).
    """
    w = np.asarray(w, dtype=np.float64)
    w_new = w - lr * (scale * o + weight_decay * w)
    return round_to_dtype(w_new, w_dtype)


def muon_step(w, g, m_prev, *, lr: float, mu: float, steps: int = 5,
              coeffs=NS5_COEFFS, schedule=None, mom_dtype: str = "f64",
              w_dtype: str = "f64", nesterov: bool = False,
              weight_decay: float = 0.0, scale: float = 1.0) -> StepResult:
    """One Muon step on one matrix ("Muon Optimizer 정리", eqs. (1)-(3))."""
    m_t = momentum_update(m_prev, g, mu, mom_dtype)
    v = nesterov_input(m_t, g, mu) if nesterov else m_t
    o = newton_schulz(v, steps, coeffs, schedule)
    w_new = _apply_update(w, o, lr, scale, weight_decay, w_dtype)
    return StepResult(w=w_new, m=m_t, o=o)


def dimuon_step(w, g, m_prev, *, lr: float, mu: float, steps: int = 5,
                coeffs=NS5_COEFFS, schedule=None, eps: float = DIMUON_EPS,
                mom_dtype: str = "f64", w_dtype: str = "f64",
                nesterov: bool = False, weight_decay: float = 0.0,
                scale: float = 1.0) -> StepResult:
    """One Dimuon step on one matrix ("Dimuon: LoRA 에 맞춰 다시 짠 Muon").

    1. Row/column energies of the previous momentum (before it is updated).
    2. Factors d = (relative energy + eps)^(-1/4), identity if all are zero.
    3. Momentum update as in Muon.
    4. Z = NS(D_R M D_C).
    5. P = D_R Z D_C, rescaled so that ||O||_F = ||Z||_F (O = 0 if P = 0).
    6. Weight update as in Muon.
    """
    r32, c32 = energies_f32_tree(m_prev)
    d_r = conditioning(r32, eps)
    d_c = conditioning(c32, eps)
    m_t = momentum_update(m_prev, g, mu, mom_dtype)
    v = nesterov_input(m_t, g, mu) if nesterov else m_t
    y = d_r[:, None] * v * d_c[None, :]
    z = newton_schulz(y, steps, coeffs, schedule)
    p = d_r[:, None] * z * d_c[None, :]
    norm_p = np.sqrt(np.sum(p * p))
    if norm_p > 0.0:
        o = p * (np.sqrt(np.sum(z * z)) / norm_p)
    else:
        o = np.zeros_like(p)
    w_new = _apply_update(w, o, lr, scale, weight_decay, w_dtype)
    return StepResult(w=w_new, m=m_t, o=o, r=r32, c=c32, d_r=d_r, d_c=d_c)
