"""How far the library's LayerNorm + per-token INT8 may sit from the plain
fp64 definition (oracle.layernorm_quant_plain), derived from the arithmetic
the library states for it (the fixed-point row statistics, then fp32
normalisation; page "4.2 W8A8 量化与 SmoothQuant" section 6 gives the formula
but not its arithmetic).

Per row, with A = max |x_j|, 2^(E-1) <= A < 2^E, u = 2^-53 and v = 2^-24:

  statistics  every x_j is truncated to a multiple of g1 = 2^(E-39) and every
              x_j^2 to one of g2 = 2^(2E-39) before exact integer sums, so the
              grid mean is within g1 of mu and the grid mean square within g2
              of mean(x^2); the fp64 division by K rounds once:
                e_mu  = g1 + u (|mu| + g1)         (+ 2u |mu| for the
                                                     definition's own rounding)
                e_var = g2 (1 + 2^-40) + u Q + e_mu (2 |mu| + e_mu)
                        + u mu^2 + u var            (var = Q - mu^2, biased);
  rounding    mu32 = fl32(mu_hat) lies in [fl32(mu - e_mu), fl32(mu + e_mu)]
  to fp32     (fl32 is monotonic), and rstd32 = fl32(1 / sqrt(var_hat + eps))
              in [fl32(lo), fl32(hi)] with lo, hi the extremes of
              1 / sqrt(var + eps +- e_var), widened by the three fp64
              roundings; this gives e_mu32 and the relative error rho of
              rstd32 exactly as far as they depend on fp32 rounding;
  element j   d = fl(x - mu32), n = fl(d rstd32), t = fl(n gamma),
              z = fl(t + beta), each a single fp32 rounding:
                Dd = e_mu32 + v (D + e_mu32),             D = |x_j - mu|
                Dn = Dd rstd (1 + rho)(1 + v) + D rstd (rho + v + rho v)
                Dt = |gamma| (Dn + v (D rstd + Dn))
                Dz = Dt + v (|z*| + Dt)                    (no v term without beta);
  codes       with Dm = max_j Dz and m* = max_j |z*_j| (so |m - m*| <= Dm),
              x_scale = fl(m / 127) and q = fl(z fl(127 / m)):
                |x_scale - m*/127| <= (Dm + v (m* + Dm)) / 127 + 2u m*/127
                |q - q*| <= Dz 127/m_lo (1 + v)
                            + |z*| (127 Dm / (m_lo m*) + v 127 / m_lo)
                            + v (|q*| + 1),                m_lo = m* - Dm.

These are first-order bounds; the checks below double them to cover the
second-order products left out.  A code may differ from the definition's only
where q* lies within the bound of a rounding boundary (a half-integer), and
then by one.
"""
from __future__ import annotations

import numpy as np

U64 = 2.0 ** -53
U32 = 2.0 ** -24


def _f32(a):
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def bounds(x_f64: np.ndarray, gamma, beta, eps: float, plain: dict):
    """Per-element bound on |q - q*| and per-row bound on |x_scale - m*/127|
    for rows x_f64 [M, K] (the bf16 values in fp64), the folded gamma/beta (fp32
    values), eps (fp32) and the definition's results `plain`."""
    M, K = x_f64.shape
    g = np.abs(np.asarray(gamma, dtype=np.float32).astype(np.float64))
    has_beta = beta is not None
    e = float(np.float32(eps))
    mu, var, z, q, m = plain["mu"], plain["var"], plain["z"], plain["q"], plain["m"]

    A = np.abs(x_f64).max(axis=1)
    E = np.where(A > 0, np.frexp(np.where(A > 0, A, 1.0))[1], 0).astype(np.float64)
    g1 = np.where(A > 0, np.ldexp(1.0, (E - 39).astype(int)), 0.0)
    g2 = np.where(A > 0, np.ldexp(1.0, (2 * E - 39).astype(int)), 0.0)
    Q = var + mu * mu
    e_mu = g1 + U64 * (np.abs(mu) + g1) + 2 * U64 * np.abs(mu)
    e_var = g2 * (1 + 2.0 ** -40) + U64 * Q + e_mu * (2 * np.abs(mu) + e_mu) + U64 * mu * mu + U64 * var

    mu32_lo, mu32_hi = _f32(mu - e_mu), _f32(mu + e_mu)
    e_mu32 = np.maximum(mu - mu32_lo, mu32_hi - mu)

    v = var + e
    rstd = 1.0 / np.sqrt(v)
    ev = e_var + U64 * (v + e_var)
    v_lo = np.maximum(v - ev, np.finfo(np.float64).tiny)
    hi = 1.0 / np.sqrt(v_lo) * (1 + 4 * U64)
    lo = 1.0 / np.sqrt(v + ev) * (1 - 4 * U64)
    rho = np.maximum(rstd - _f32(lo), _f32(hi) - rstd) / rstd

    D = np.abs(x_f64 - mu[:, None])
    em = e_mu32[:, None]
    rs = rstd[:, None]
    rh = rho[:, None]
    Dd = em + U32 * (D + em)
    Dn = Dd * rs * (1 + rh) * (1 + U32) + D * rs * (rh + U32 + rh * U32)
    Dt = g[None, :] * (Dn + U32 * (D * rs + Dn))
    Dz = Dt + (U32 * (np.abs(z) + Dt) if has_beta else 0.0)
    Dm = Dz.max(axis=1)

    scale_bound = (Dm + U32 * (m + Dm)) / 127.0 + 2 * U64 * m / 127.0
    m_lo = np.maximum(m - Dm, np.finfo(np.float64).tiny)[:, None]
    mm = np.where(m > 0, m, 1.0)[:, None]
    dq = (Dz * 127.0 / m_lo * (1 + U32) + np.abs(z) * (127.0 * Dm[:, None] / (m_lo * mm) + U32 * 127.0 / m_lo)
          + U32 * (np.abs(q) + 1.0))
    dq = np.where(m[:, None] > 0, dq, 0.0)
    return 2.0 * dq, 2.0 * scale_bound


def check(codes, x_scale, x_f64, gamma, beta, eps, plain, max_boundary_frac=1e-3):
    """Assert that library codes / scales (numpy) are within the derived bound
    of the definition: scales within the scale bound; codes equal to the
    definition's wherever q* is farther than the bound from a half-integer, and
    within one elsewhere.  Returns the fraction of elements near a boundary,
    which must stay below max_boundary_frac (otherwise the bound is too loose
    to say anything)."""
    dq, sb = bounds(x_f64, gamma, beta, eps, plain)
    m = plain["m"]
    ds = np.abs(np.asarray(x_scale, dtype=np.float64) - m / 127.0)
    bad = np.nonzero(ds > sb)[0]
    assert bad.size == 0, (f"x_scale off the definition beyond the bound in rows {bad[:8].tolist()}: "
                           f"{ds[bad[:8]].tolist()} > {sb[bad[:8]].tolist()}")
    q = plain["q"]
    dist = np.abs(q - np.floor(q) - 0.5)  # distance from the nearest half-integer
    near = dist <= dq
    diff = np.abs(np.asarray(codes, dtype=np.int64) - plain["codes"].astype(np.int64))
    far_bad = np.nonzero((diff > 0) & ~near)
    assert far_bad[0].size == 0, (f"{far_bad[0].size} codes differ from the definition away from a rounding "
                                  f"boundary, e.g. at {list(zip(far_bad[0][:4].tolist(), far_bad[1][:4].tolist()))}")
    assert diff.max(initial=0) <= 1, "a code differs from the definition by more than one"
    frac = float(near.mean()) if near.size else 0.0
    assert frac < max_boundary_frac, f"bound too loose: {frac:.2e} of the codes sit within it of a boundary"
    return frac
