"""Oracle for in-model consensus: greedy (T=0) and rejection sampling (T>0).

TEST INFRASTRUCTURE ONLY -- never imported by the product path.

Sources (the Orthrus pages):

* Paper notes on Orthrus (zhangshuibai.github.io paper-notes), §4.1 step 3
  (left-to-right match over k = 1..K; at the first mismatch j the first j-1
  candidates are kept and one correction token is drawn from the AR
  distribution at position j), §4.2 (greedy: accept a candidate iff it equals
  the AR argmax; the correction is the AR argmax), §4.3 and §7.2 (T>0: accept
  with probability min(1, p_AR/q_diff), on rejection resample from the
  normalised max(0, p_AR - q_diff), the Leviathan/Chen rule), §9.1 (both modes
  are lossless: token-for-token at T=0, in distribution at T>0).
* hotdry.top blog post on Orthrus, section on parallel block projection and
  in-model consensus (same facts).

Readings of points the pages leave open:

* R2 -- logits row i is the AR distribution checked against cand[i].
* R3 -- no bonus token when all K candidates match: accept_len = K and
  correction = -1, so tokens per cycle = a + [a < K] lies in [1, K].
* R6 -- argmax ties go to the lowest index; NaN counts as greater than every
  number (first NaN wins); -0 equals +0.
* R7 -- the caller applies the temperature and passes probabilities for T>0.
* R8 -- the accept test is the strict ``u * q < p`` evaluated exactly in
  float64 (u and q carry at most 24 significant bits each, so the product is
  exact).
* R9 -- the residual is drawn by an integer inverse CDF: weights
  w_v = max(0, F(p_v) - F(q_v)) with F(x) = floor(clamp(x, 0, 1) * 2**60),
  total S, target T = floor(m * S / 2**24) with m = u_K * 2**24, pick the
  smallest v whose inclusive prefix sum of w exceeds T.
* R10 -- if S == 0, the same rule runs on w_v = F(p_v); if that is 0 too,
  the correction is token 0.
* R11 -- uniforms are [B, K+1] float32 on the 2**-24 grid in [0, 1):
  u[0..K-1] for the accept tests, u[K] for the residual draw.
* R28 -- a candidate outside [0, V) is not a token of the vocabulary: the
  target gives it probability 0, so it is rejected like any p = 0 token.

Inputs must be finite probability rows for the sampler (each row sums to at
most 8, which keeps every 64-bit prefix sum exact); outside that contract
results are unspecified.
"""
from __future__ import annotations

import numpy as np

FIXED_POINT_BITS = 60
UNIFORM_BITS = 24


def _np(x, dtype=None) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x) if dtype is None else np.asarray(x, dtype=dtype)


# ----------------------------------------------------------------- greedy --
def row_argmax(row) -> int:
    """Index of the largest entry; lowest index on ties; first NaN wins."""
    r = _np(row, np.float64)
    nan = np.isnan(r)
    if nan.any():
        return int(np.flatnonzero(nan)[0])
    top = r.max()
    return int(np.flatnonzero(r == top)[0])   # -0.0 == +0.0 in this compare


def greedy_consensus(logits, cand):
    """Greedy consensus for every sequence.

    logits [B, K, V] (float), cand [B, K] (int).
    Returns (accept_len [B], row_argmax [B, K], correction [B]) as int64.
    accept_len a = number of leading rows whose candidate equals the row
    argmax; correction = argmax of row a if a < K, else -1.
    """
    lg = _np(logits, np.float64)
    cd = _np(cand, np.int64)
    B, K, _ = lg.shape
    am = np.zeros((B, K), dtype=np.int64)
    acc = np.zeros(B, dtype=np.int64)
    corr = np.zeros(B, dtype=np.int64)
    for b in range(B):
        for i in range(K):
            am[b, i] = row_argmax(lg[b, i])
        a = 0
        while a < K and cd[b, a] == am[b, a]:
            a += 1
        acc[b] = a
        corr[b] = am[b, a] if a < K else -1
    return acc, am, corr


# --------------------------------------------------------------- sampling --
def fixed_point_weight(x) -> np.ndarray:
    """F(x) = floor(clamp(x, 0, 1) * 2**60) as exact int64 (NaN -> 0).

    x is float32; x * 2**60 is exact in float64 and so is its floor.
    """
    xd = _np(x, np.float64)
    xd = np.where(np.isnan(xd), 0.0, np.clip(xd, 0.0, 1.0))
    return np.floor(xd * float(2 ** FIXED_POINT_BITS)).astype(np.int64)


def uniform_to_grid_int(u) -> np.ndarray:
    """m = floor(u * 2**24) clamped to [0, 2**24 - 1] (NaN -> 0), as int64."""
    ud = _np(u, np.float64)
    ud = np.where(np.isnan(ud), 0.0, ud)
    m = np.floor(ud * float(2 ** UNIFORM_BITS))
    return np.clip(m, 0, 2 ** UNIFORM_BITS - 1).astype(np.int64)


def accepts(u, q_at_cand, p_at_cand):
    """Accept test of one draft token: u * q < p, in float64 (elementwise).

    u is on the 2**-24 grid and q is float32, so the product is exact; the
    compare is strict, so a token the target gives probability 0 is never
    accepted.  NaN anywhere rejects.
    """
    return _np(u, np.float64) * _np(q_at_cand, np.float64) < _np(p_at_cand, np.float64)


def accept_prefix(p_at_cand, q_at_cand, u) -> int:
    """Leading accepted count, scanning rows left to right.

    All three arguments are length-K vectors (float32 values).  Returns the
    first rejected index, or K if every row is accepted.
    """
    p = _np(p_at_cand, np.float64)
    q = _np(q_at_cand, np.float64)
    uu = _np(u, np.float64)
    for i in range(len(p)):
        if not accepts(uu[i], q[i], p[i]):
            return i
    return len(p)


def residual_weights(p_row, q_row) -> np.ndarray:
    """Integer residual weights max(0, F(p) - F(q)); F(p) if those sum to 0."""
    fp = fixed_point_weight(p_row)
    fq = fixed_point_weight(q_row)
    w = np.maximum(fp - fq, 0)
    if int(w.sum()) == 0:
        w = fp
    return w


def inverse_cdf_pick(w, m):
    """Smallest v with sum_{t <= v} w_t > floor(m * S / 2**24), S = sum w.

    ``m`` may be a Python int or an int64 array (vectorised over m).  The
    product m * S can exceed 64 bits, so it is split as
    m * (S >> 24) + floor(m * (S mod 2**24) / 2**24), an exact identity whose
    two terms fit in int64 for m < 2**24 and S < 2**63.  Returns 0 when S == 0.
    """
    w = np.asarray(w, dtype=np.int64)
    S = int(w.sum())
    if S == 0:
        return np.zeros_like(np.asarray(m)) if np.ndim(m) else 0
    cum = np.cumsum(w)
    hi, lo = S >> UNIFORM_BITS, S & ((1 << UNIFORM_BITS) - 1)
    if np.ndim(m) == 0:
        T = (int(m) * S) >> UNIFORM_BITS          # Python ints: exact
        return int(np.searchsorted(cum, T, side="right"))
    mm = np.asarray(m, dtype=np.int64)
    T = mm * np.int64(hi) + ((mm * np.int64(lo)) >> UNIFORM_BITS)
    return np.searchsorted(cum, T, side="right").astype(np.int64)


def sample_consensus(p_target, q_draft, cand, uniforms):
    """T>0 consensus for every sequence (exact rejection sampling).

    p_target, q_draft [B, K, V] float32 probabilities; cand [B, K] int;
    uniforms [B, K+1] float32.  Returns (accept_len [B], correction [B]).
    """
    P = _np(p_target, np.float32)
    Q = _np(q_draft, np.float32)
    cd = _np(cand, np.int64)
    U = _np(uniforms, np.float32)
    B, K, V = P.shape
    acc = np.zeros(B, dtype=np.int64)
    corr = np.zeros(B, dtype=np.int64)
    for b in range(B):
        # R28: a candidate outside the vocabulary [0, V) is a token the target
        # gives probability 0, so the strict accept test rejects it (R8); its
        # draft probability is then irrelevant and is taken as 0.
        inside = [0 <= cd[b, i] < V for i in range(K)]
        pc = np.array([P[b, i, cd[b, i]] if inside[i] else 0.0 for i in range(K)], dtype=np.float32)
        qc = np.array([Q[b, i, cd[b, i]] if inside[i] else 0.0 for i in range(K)], dtype=np.float32)
        a = accept_prefix(pc, qc, U[b, :K])
        acc[b] = a
        if a == K:
            corr[b] = -1
            continue
        w = residual_weights(P[b, a], Q[b, a])
        m = int(uniform_to_grid_int(U[b, K]))
        corr[b] = inverse_cdf_pick(w, m)
    return acc, corr


def tokens_committed(accept_len, block_k: int):
    """Tokens one cycle commits: the accepted prefix plus the correction."""
    a = _np(accept_len, np.int64)
    return a + (a < block_k).astype(np.int64)

