"""Rounding noise of a bf16 layer's attention operands, propagated through the float64 oracle.

Model: a bf16 layer stores the attention's operands q, k, v (forward and backward) and dO
(backward) in bf16, so each element reaches the attention as x (1 + d) with |d| <= 2^-8 (round to
nearest with 8 significant bits), the errors of different elements independent.  One token's errors
enter every pair of that token, so a sum over many pairs (a bias-table bin) or over few pairs (the
gradients of a short sequence) does not average them out; the oracle, evaluated with such
perturbed operands, carries exactly that correlation.  sigma, per output element, is the RMS over
seeded samples of (perturbed - exact) with d uniform in [-2^-8, 2^-8]: the RMS of a real rounding
error, 2^-8 / (m sqrt 3) for a mantissa m in [1, 2), is at most that of the model."""
from __future__ import annotations

import numpy as np

U_BF16 = 2.0 ** -8


def operand_noise(run, samples: int = 24, seed: int = 0, u: float = U_BF16):
    """run(attn_operands) -> dict of float64 arrays (run(None) is the exact evaluation).
    Returns (exact, sigma) with sigma[name] the per-element RMS deviation over `samples` runs whose
    operands are multiplied elementwise by 1 + d, d uniform in [-u, u]."""
    base = run(None)
    acc = {k: np.zeros(np.shape(v)) for k, v in base.items()}
    rng = np.random.default_rng(seed)

    def perturb(name, a):
        return a * (1.0 + rng.uniform(-u, u, np.shape(a)))

    for _ in range(samples):
        out = run(perturb)
        for k in acc:
            acc[k] += (np.asarray(out[k], np.float64) - base[k]) ** 2
    return base, {k: np.sqrt(v / samples) for k, v in acc.items()}
