"""Host-side comparison of verify-budget rules by the quantity the pages
compare schedulers by, Theta = tau * SPS(B) ("DSpark, la bozza ...", section
"Verificare meglio, non di più"): tau = expected tokens a round emits, B =
tokens in the verify batch."""

from __future__ import annotations

import numpy as np


def expected_theta(conf, budget, sps_B, sps_val):
    """(tau, N, Theta): tau = sum_b (1 + sum_{j < L_b} a_{b,j}) with a the fp32
    prefix products of the scores, N = sum_b (1 + L_b), Theta = tau / t(N),
    t = 1/SPS as the scheduler reads the table: linear between the points, the
    first value below the first point, the last segment extended beyond the
    last one."""
    c = np.asarray(conf, dtype=np.float32)
    a = np.cumprod(c, axis=1, dtype=np.float32).astype(np.float64)
    L = np.asarray(budget, dtype=np.int64)
    mask = np.arange(c.shape[1])[None, :] < L[:, None]
    tau = float(c.shape[0]) + float((a * mask).sum())
    N = float(c.shape[0] + L.sum())
    Bs = np.asarray(sps_B, np.float64)
    ts = 1.0 / np.asarray(sps_val, np.float64)
    if N <= Bs[0]:
        t = ts[0]
    else:
        i = min(int(np.searchsorted(Bs, N, side="right")) - 1, len(Bs) - 2)
        t = ts[i] + (ts[i + 1] - ts[i]) * (N - Bs[i]) / (Bs[i + 1] - Bs[i])
    return tau, N, tau / float(t)
