"""E1: initial Mamba-2 state from the target's last-token hidden state.

H-Spec (Abstract; review page, Summary): each Mamba module's recurrent state
is initialised from a *projection* of the target model's hidden state at the
last input position.  The pages print no formula; the plainest reading is a
linear map with no bias and no nonlinearity:

    h0[b, s] = sum_i u[b, i] * W[i, s]          u: [C, d], W: [d, S]

and the flat state index s enumerates the Mamba-2 state [H, P, N] row-major,
s = (h*P + p)*N + n.
"""
import numpy as np


def init_state(u: np.ndarray, w: np.ndarray) -> np.ndarray:
    """u [C, d] and W [d, S] in float64 -> h0 [C, S] float64 (one matmul)."""
    u = np.asarray(u, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    if u.ndim != 2 or w.ndim != 2 or u.shape[1] != w.shape[0]:
        raise ValueError(f"shape mismatch u{u.shape} W{w.shape}")
    return u @ w
