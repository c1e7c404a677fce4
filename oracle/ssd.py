"""E2 / E3: the Mamba-2 (SSD) scan over the K-token draft block.

H-Spec (Abstract) drafts a whole block at once: the Mamba module is a
recurrence, yet its parallel scan evaluates all K positions together.  The
arithmetic is Mamba-2's selective state-space recurrence with a scalar decay
per head (Dao & Gu 2024, "Transformers are SSMs", the SSD layer):

    H_t = exp(delta_t * A) * H_{t-1} + delta_t * x_t (outer) B_t     (P x N)
    y_t = H_t @ Cm_t  (+ Dskip * x_t)
    H_{-1} = h0  (the projected last-token state, E1)

per request b and head h; B and Cm are shared by the heads of one group
(group of head h = h // (H / ng)).

ssd_recurrence is that definition, stepped one position at a time.
ssd_chunked is the chunked (block-parallel) restatement of the same
recurrence -- within a chunk: cumulative log-decay, the masked decay matrix
exp(segsum), the C.B^T products, the diagonal-block output and the
contribution of the incoming state; between chunks: state passing.  It is kept
in the oracle only so the tests can show, in float64, that the decomposition
the GPU uses reaches the recurrence's result.
"""
import numpy as np


def _groups(H: int, ng: int) -> np.ndarray:
    if H % ng:
        raise ValueError("ng must divide H")
    return np.arange(H) // (H // ng)


def _check(x, delta, A, B, Cm):
    C, K, H, P = x.shape
    if delta.shape != (C, K, H) or A.shape != (H,):
        raise ValueError("delta/A shape")
    if B.shape[:2] != (C, K) or Cm.shape != B.shape:
        raise ValueError("B/Cm shape")
    return C, K, H, P, B.shape[2], B.shape[3]


def ssd_recurrence(x, delta, A, B, Cm, h0=None, Dskip=None):
    """Literal recurrence.  Returns (y [C,K,H,P], h_final [C,H,P,N]) in float64.

    x [C,K,H,P], delta [C,K,H] (>0), A [H] (<0), B/Cm [C,K,ng,N],
    h0 [C,H,P,N] or None (zero state), Dskip [H] or None (no skip term).
    """
    x, delta, A, B, Cm = (np.asarray(v, dtype=np.float64) for v in (x, delta, A, B, Cm))
    C, K, H, P, ng, N = _check(x, delta, A, B, Cm)
    grp = _groups(H, ng)
    state = (np.zeros((C, H, P, N)) if h0 is None
             else np.array(h0, dtype=np.float64).reshape(C, H, P, N))
    y = np.zeros((C, K, H, P))
    for t in range(K):
        decay = np.exp(delta[:, t, :] * A[None, :])                    # [C,H]
        bt = B[:, t][:, grp, :]                                        # [C,H,N]
        ct = Cm[:, t][:, grp, :]                                       # [C,H,N]
        inject = (delta[:, t, :, None] * x[:, t])[..., None] * bt[:, :, None, :]
        state = decay[:, :, None, None] * state + inject               # [C,H,P,N]
        y[:, t] = np.einsum("chpn,chn->chp", state, ct)
        if Dskip is not None:
            y[:, t] += np.asarray(Dskip, np.float64)[None, :, None] * x[:, t]
    return y, state


def ssd_chunked(x, delta, A, B, Cm, h0=None, chunk=None, Dskip=None):
    """Chunked SSD restatement.  Same arguments and results as ssd_recurrence.

    chunk: chunk length Q (the last chunk may be shorter).  None = K.
    """
    x, delta, A, B, Cm = (np.asarray(v, dtype=np.float64) for v in (x, delta, A, B, Cm))
    C, K, H, P, ng, N = _check(x, delta, A, B, Cm)
    grp = _groups(H, ng)
    Q = K if chunk is None else int(chunk)
    Hs = (np.zeros((C, H, P, N)) if h0 is None
          else np.array(h0, dtype=np.float64).reshape(C, H, P, N))
    y = np.zeros((C, K, H, P))
    for c0 in range(0, K, Q):
        c1 = min(K, c0 + Q)
        q = c1 - c0
        a = delta[:, c0:c1, :] * A[None, None, :]                     # [C,q,H]
        lam = np.cumsum(a, axis=1)                                     # in-chunk cumulative log-decay
        tri = np.tril(np.ones((q, q), dtype=bool))                     # s <= t
        seg = lam[:, :, None, :] - lam[:, None, :, :]                  # [C,t,s,H] = sum_{s<r<=t} a_r
        L = np.where(tri[None, :, :, None], np.exp(np.where(tri[None, :, :, None], seg, 0.0)), 0.0)
        bc = B[:, c0:c1][:, :, grp, :]                                 # [C,q,H,N]
        cc = Cm[:, c0:c1][:, :, grp, :]
        G = np.einsum("cthn,cshn->ctsh", cc, bc)                       # C_t . B_s
        dx = delta[:, c0:c1, :, None] * x[:, c0:c1]                    # [C,q,H,P]
        y_diag = np.einsum("ctsh,cshp->cthp", L * G, dx)
        y_off = np.exp(lam)[..., None] * np.einsum("chpn,cthn->cthp", Hs, cc)
        y[:, c0:c1] = y_diag + y_off
        if Dskip is not None:
            y[:, c0:c1] += np.asarray(Dskip, np.float64)[None, None, :, None] * x[:, c0:c1]
        lam_end = lam[:, -1, :]                                        # [C,H]
        w_s = np.exp(lam_end[:, None, :] - lam)                        # [C,q,H]
        S_c = np.einsum("csh,cshp,cshn->chpn", w_s, dx, bc)
        Hs = np.exp(lam_end)[:, :, None, None] * Hs + S_c
    return y, Hs
