"""A plain FP32 evaluation of the multi-query read's backward (dvalues), for the precision floor
of narrow keys: every contraction is a sequential float32 sum over its index (no blocking, no
pairwise summation), elementwise steps in float32 ("Fast Attention Residuals" PyPI page, section
"Multi-query AttnRes": p_{m,s} = softmax_s(scale * rho_s * <t_s, q_m>), y_m = sum_s p_{m,s} v_s,
rho_s = 1 / sqrt(mean(t_s^2) + eps) over the key slice t_s = v_s[D - R:]). Test infrastructure:
it shares nothing with the GPU library and is not the oracle (which evaluates in FP64)."""
import numpy as np


def _seqdot(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Sequential float32 dot products over the last axis (broadcast over the others)."""
    prod = (a * b).astype(np.float32)
    return np.cumsum(prod, axis=-1, dtype=np.float32)[..., -1]


def multi_dvalues_fp32(V: np.ndarray, Q: np.ndarray, G: np.ndarray, eps: float = 2.0 ** -23,
                       scale: float = 1.0) -> np.ndarray:
    """V [S, N, D], Q [M, R], G [M, N, D] (query-major dY), all float32. Returns dvalues [S, N, D]
    (summed over the queries) evaluated in float32."""
    f = np.float32
    V, Q, G = (np.asarray(x, dtype=f) for x in (V, Q, G))
    S, N, D = V.shape
    M, R = Q.shape
    lo = D - R
    T = V[:, :, lo:]                                               # [S, N, R]
    ss = _seqdot(T, T)                                             # [S, N]
    rho = (f(1.0) / np.sqrt(ss / f(R) + f(eps))).astype(f)        # [S, N]
    c = _seqdot(T[None, :, :, :], Q[:, None, None, :])            # [M, S, N]
    z = (f(scale) * rho[None] * c).astype(f)
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax).astype(f)
    den = np.zeros((M, 1, N), dtype=f)
    for s in range(S):                                             # sequential over sources
        den = (den + e[:, s:s + 1, :]).astype(f)
    p = (e / den).astype(f)                                        # [M, S, N]
    dp = _seqdot(G[:, None, :, :], V[None, :, :, :])               # [M, S, N]
    delta = np.zeros((M, N), dtype=f)
    for s in range(S):
        delta = (delta + p[:, s, :] * dp[:, s, :]).astype(f)
    a = (f(scale) * p * (dp - delta[:, None, :]) * rho[None]).astype(f)   # [M, S, N]
    B = np.zeros((S, N), dtype=f)
    for m in range(M):
        B = (B + a[m] * c[m]).astype(f)
    B = (-(rho * rho) / f(R) * B).astype(f)
    dv = np.zeros((S, N, D), dtype=f)
    for m in range(M):
        dv = (dv + p[m][:, :, None] * G[m][None, :, :]).astype(f)
    slice_ = np.zeros((S, N, R), dtype=f)
    for m in range(M):
        slice_ = (slice_ + a[m][:, :, None] * Q[m][None, None, :]).astype(f)
    slice_ = (slice_ + B[:, :, None] * T).astype(f)
    dv[:, :, lo:] = (dv[:, :, lo:] + slice_).astype(f)
    return dv


def fp32_floor(V, Q, G, ref_dvalues: np.ndarray, **kw) -> float:
    """max |dvalues_fp32 - ref| / rms(ref): what a straightforward FP32 evaluation reaches."""
    dv = multi_dvalues_fp32(V, Q, G, **kw).astype(np.float64)
    r = np.asarray(ref_dvalues, dtype=np.float64)
    return float(np.abs(dv - r).max() / np.sqrt(np.mean(r * r)))
