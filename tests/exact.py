"""Exact-arithmetic brute force used to pin the oracle (no GPU, no oracle code).

Moments are exact rationals (``fractions.Fraction``).  Parameters need a
square root, so they are carried as ``decimal.Decimal`` at 60 significant
digits, far below any double rounding.

The formulas are those of the optimizer page (docs.rs optirs_gpu
sparse_optimizer): sections "LazyAdamMode::Lazy" and
"LazyAdamMode::DormancyDecay" and the closing remark on the global step.
Dense Adam here is the textbook recursion run on every step, with an explicit
zero gradient for an untouched coordinate.
"""
from __future__ import annotations

from decimal import Decimal, getcontext
from fractions import Fraction

getcontext().prec = 60


def D(x) -> Decimal:
    if isinstance(x, Fraction):
        return Decimal(x.numerator) / Decimal(x.denominator)
    return Decimal(x)


def dense_adam_moments(grads_per_step, beta1: Fraction, beta2: Fraction):
    """Dense Adam moments for one coordinate, fed g_t on every step t = 1..T.

    grads_per_step: list of Fraction (0 on dormant steps).
    Returns lists m[t], v[t] for t = 1..T (index t-1)."""
    m = Fraction(0)
    v = Fraction(0)
    ms, vs = [], []
    for g in grads_per_step:
        m = beta1 * m + (1 - beta1) * g
        v = beta2 * v + (1 - beta2) * g * g
        ms.append(m)
        vs.append(v)
    return ms, vs


def lazy_moments(touches, beta1: Fraction, beta2: Fraction):
    """Lazy mode: m <- beta1*m + (1-beta1)*g at each touch, whatever the gap.

    touches: list of (t, g).  Returns the list of (m, v) after each touch."""
    m = Fraction(0)
    v = Fraction(0)
    out = []
    for _, g in touches:
        m = beta1 * m + (1 - beta1) * g
        v = beta2 * v + (1 - beta2) * g * g
        out.append((m, v))
    return out


def param_step(p: Decimal, m: Fraction, v: Fraction, t: int, lr, beta1: Fraction, beta2: Fraction,
               eps) -> Decimal:
    """p - lr * m_hat / (sqrt(v_hat) + eps) with global-step bias correction."""
    m_hat = m / (1 - beta1 ** t)
    v_hat = v / (1 - beta2 ** t)
    return p - D(lr) * D(m_hat) / (D(v_hat).sqrt() + D(eps))


def sparse_adam_exact(p0, touches, beta1: Fraction, beta2: Fraction, lr, eps, mode: str):
    """One coordinate of sparse / lazy Adam in exact arithmetic.

    touches: list of (t, g) with strictly increasing global steps t >= 1.
    Returns (p, m, v, last_step) after the last touch."""
    p = D(p0)
    m = Fraction(0)
    v = Fraction(0)
    s = 0
    for t, g in touches:
        gap = t - s
        d1 = beta1 ** gap if mode == "dormancy" else beta1
        d2 = beta2 ** gap if mode == "dormancy" else beta2
        m = d1 * m + (1 - beta1) * g
        v = d2 * v + (1 - beta2) * g * g
        p = param_step(p, m, v, t, lr, beta1, beta2, eps)
        s = t
    return p, m, v, s
