"""Attention difference as a mean squared error.

PAB article, Figure 1 caption: the difference between the attention output of
the current diffusion step and that of the previous step is quantified by the
MSE.  The oracle takes the plain definition over all elements:

    mse(a, b) = (1/n) * sum_k (a_k - b_k)^2

in fp64 on exactly widened inputs.
"""

from __future__ import annotations

import numpy as np


def mse(a, b) -> float:
    """Mean of squared elementwise differences of two same-sized tensors."""
    if hasattr(a, "detach"):
        import torch

        a = a.detach().to("cpu").to(torch.float64).numpy()
        b = b.detach().to("cpu").to(torch.float64).numpy()
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    if a.size != b.size:
        raise ValueError("mse: size mismatch")
    if a.size == 0:
        raise ValueError("mse: empty input")
    d = a - b
    return float(np.dot(d, d) / a.size)
