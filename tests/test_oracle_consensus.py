"""Pins for the consensus oracle (CPU only).

Greedy: a pure-Python brute force (different code: explicit loops and
comparisons, no numpy reductions), planted first-mismatch indices and ties,
NaN / signed-zero rules, and the page-fixed bounds on tokens per cycle.

Sampling: exact enumeration of every uniform on the 2**-24 grid on tiny
vocabularies.  The law of the first committed token must equal the target
distribution p (losslessness of Leviathan/Chen rejection sampling, which the
paper notes' §4.3 and §7.2 invoke) up to the grid and fixed-point quantisation,
plus the special cases that reduce the rule to a fixed answer.
"""
import math
import random

import numpy as np
import pytest
import torch

import oracle
from oracle.consensus import (accept_prefix, accepts, fixed_point_weight, inverse_cdf_pick,
                              residual_weights, uniform_to_grid_int)
from synth import Workload, greedy_inputs, sample_inputs

GRID = 1 << 24


# --------------------------------------------------------------- greedy ----
def _brute_argmax(row):
    best = 0
    for v in range(1, len(row)):
        x, y = row[v], row[best]
        if math.isnan(y):
            break
        if math.isnan(x) or x > y:
            best = v
    return best


def _brute_greedy(logits, cand):
    B, K = len(logits), len(logits[0])
    out = []
    for b in range(B):
        am = [_brute_argmax(list(map(float, logits[b][i]))) for i in range(K)]
        a = 0
        for i in range(K):
            if int(cand[b][i]) != am[i]:
                break
            a += 1
        out.append((a, am, am[a] if a < K else -1))
    return out


@pytest.mark.parametrize("ties", [False, True])
def test_greedy_matches_brute_force(ties):
    w = Workload("g", 1, 6, 1, 1, 1, 1, 7, 50, 4.0, 11)
    logits, cand, jstar = greedy_inputs(w, ties=ties)
    acc, am, corr = oracle.greedy_consensus(logits, cand)
    bf = _brute_greedy(logits.tolist(), cand.tolist())
    for b in range(6):
        assert acc[b] == bf[b][0] == jstar[b]
        assert list(am[b]) == bf[b][1]
        assert corr[b] == bf[b][2]


@pytest.mark.parametrize("j", [0, 1, 16, 31, 32])
def test_planted_first_mismatch(j):
    w = Workload("g", 1, 2, 1, 1, 1, 1, 32, 997, 3.0, 12)
    logits, cand, _ = greedy_inputs(w, first_mismatch=j, ties=True)
    acc, am, corr = oracle.greedy_consensus(logits, cand)
    assert (acc == j).all()
    assert oracle.tokens_committed(acc, 32).min() >= 1
    assert oracle.tokens_committed(acc, 32).max() <= 32
    for b in range(2):
        assert corr[b] == (-1 if j == 32 else am[b, j])


def test_all_match_and_first_row_mismatch():
    logits = torch.tensor([[[0.0, 3.0, 1.0], [2.0, 0.0, 2.0]]])
    acc, am, corr = oracle.greedy_consensus(logits, torch.tensor([[1, 0]]))
    assert (acc[0], corr[0]) == (2, -1) and list(am[0]) == [1, 0]
    acc, am, corr = oracle.greedy_consensus(logits, torch.tensor([[2, 0]]))
    assert (acc[0], corr[0]) == (0, 1)


def test_nan_and_signed_zero_rules():
    nan = float("nan")
    assert oracle.row_argmax(np.array([1.0, nan, 5.0, nan], dtype=np.float32)) == 1
    assert oracle.row_argmax(np.array([-1.0, -0.0, 0.0], dtype=np.float32)) == 1
    assert oracle.row_argmax(np.array([-np.inf, -np.inf], dtype=np.float32)) == 0
    assert oracle.row_argmax(np.array([3.0, np.inf, np.inf], dtype=np.float32)) == 1


# ------------------------------------------------------------- sampling ----
def _first_token_law(p, q):
    """Exact law of the first committed token, enumerating every uniform.

    The candidate y ~ q is enumerated with its probability q(y); the accept
    uniform and the residual uniform each range over the whole 2**-24 grid.
    """
    p = np.asarray(p, dtype=np.float32)
    q = np.asarray(q, dtype=np.float32)
    V = len(p)
    u = (np.arange(GRID, dtype=np.float64) / GRID).astype(np.float32)
    acc_prob = np.array([accepts(u, np.float32(q[y]), np.float32(p[y])).mean() for y in range(V)])
    w = residual_weights(p, q)
    picks = inverse_cdf_pick(w, uniform_to_grid_int(u))
    res_law = np.bincount(picks, minlength=V) / GRID
    qn = q.astype(np.float64) / q.astype(np.float64).sum()
    reject = float((qn * (1.0 - acc_prob)).sum())
    return qn * acc_prob + reject * res_law


def test_sampler_is_lossless_dyadic():
    """p, q dyadic (sum exactly 1): the law equals p within the grid error."""
    p = [0.5, 0.25, 0.125, 0.0625, 0.0625]
    q = [0.125, 0.125, 0.25, 0.25, 0.25]
    law = _first_token_law(p, q)
    assert np.abs(law - np.array(p)).max() <= 2.0 / GRID


def test_sampler_is_lossless_generic():
    """Softmax-made float32 p, q on V = 7, including a token with q > 0, p ~ 0."""
    rng = np.random.default_rng(3)
    zp, zq = rng.normal(0, 2, 7), rng.normal(0, 2, 7)
    zp[4] = -60.0
    p = (np.exp(zp) / np.exp(zp).sum()).astype(np.float32)
    q = (np.exp(zq) / np.exp(zq).sum()).astype(np.float32)
    law = _first_token_law(p, q)
    target = p.astype(np.float64) / p.astype(np.float64).sum()
    assert np.abs(law - target).max() <= 2.0 / GRID + 7 * 2.0 ** -23


def test_accept_is_strict_and_exact():
    # p(y) = 0 is never accepted, even with u = 0 (strict compare)
    assert accept_prefix([0.0, 0.5], [0.3, 0.5], [0.0, 0.0]) == 0
    # q == p: accepted for every u < 1
    assert accept_prefix([0.25] * 3, [0.25] * 3, [0.0, 0.5, 1.0 - 2.0 ** -24]) == 3
    # boundary: u * q == p exactly -> reject
    assert accept_prefix([0.25], [0.5], [0.5]) == 0
    assert accept_prefix([0.25], [0.5], [0.5 - 2.0 ** -24]) == 1


def test_one_hot_target_always_corrects_to_its_token():
    p = np.zeros(9, dtype=np.float32)
    p[6] = 1.0
    q = np.full(9, 1.0 / 9, dtype=np.float32)
    w = residual_weights(p, q)
    m = np.arange(0, GRID, 4099, dtype=np.int64)
    assert (inverse_cdf_pick(w, m) == 6).all()


def test_degenerate_residual_falls_back_to_target():
    p = np.array([0.25, 0.25, 0.5], dtype=np.float32)
    w = residual_weights(p, p)                       # max(0, p - q) == 0 everywhere
    assert list(w) == list(fixed_point_weight(p))
    assert inverse_cdf_pick(w, 0) == 0
    assert inverse_cdf_pick(w, GRID - 1) == 2
    assert inverse_cdf_pick(np.zeros(4, dtype=np.int64), 123) == 0


def _brute_pick(w, m):
    S = sum(int(x) for x in w)
    T = (m * S) // GRID
    run = 0
    for v, x in enumerate(w):
        run += int(x)
        if run > T:
            return v
    raise AssertionError("no pick")


def test_inverse_cdf_matches_big_integer_brute_force():
    rng = random.Random(5)
    for trial in range(40):
        V = rng.randint(1, 30)
        w = np.array([rng.choice([0, rng.randint(0, 2 ** 58)]) for _ in range(V)], dtype=np.int64)
        if w.sum() == 0:
            w[rng.randrange(V)] = 1
        ms = [0, GRID - 1] + [rng.randrange(GRID) for _ in range(30)]
        vec = inverse_cdf_pick(w, np.array(ms, dtype=np.int64))
        for m, got in zip(ms, vec):
            assert got == _brute_pick(w, m) == inverse_cdf_pick(w, m)


def test_fixed_point_weight_is_exact():
    x = np.array([0.5, 1.0, 0.0, 2.0 ** -61, 3 * 2.0 ** -60, 1.5, -0.25, float("nan")],
                 dtype=np.float32)
    got = fixed_point_weight(x).tolist()
    assert got == [2 ** 59, 2 ** 60, 0, 0, 3, 2 ** 60, 0, 0]
    f = np.float32(0.1)
    assert fixed_point_weight(f) == math.floor(float(f) * 2 ** 60)


def test_sample_consensus_composes_the_steps():
    w = Workload("s", 1, 4, 1, 1, 1, 1, 6, 40, 3.0, 21)
    for noise in (None, 0.3):
        p, q, cand, u = sample_inputs(w, draft_noise=noise)
        acc, corr = oracle.sample_consensus(p, q, cand, u)
        for b in range(4):
            pc = [p[b, i, cand[b, i]].item() for i in range(6)]
            qc = [q[b, i, cand[b, i]].item() for i in range(6)]
            a = accept_prefix(pc, qc, u[b, :6])
            assert acc[b] == a
            if a == 6:
                assert corr[b] == -1
            else:
                wts = residual_weights(p[b, a], q[b, a])
                assert corr[b] == _brute_pick(wts.tolist(), int(uniform_to_grid_int(u[b, 6])))
                assert wts[corr[b]] > 0
        assert oracle.tokens_committed(acc, 6).min() >= 1


@pytest.mark.parametrize("bad", [-1, -7, 37, 1 << 30])
def test_out_of_vocabulary_candidate_is_a_zero_probability_token(bad):
    """R28: a candidate outside [0, V) behaves exactly like an extra vocabulary
    entry V that the target gives probability 0 (and the draft 0 too, so no
    residual weight lands on it): the same accepted length and correction."""
    w = Workload("oov", 1, 4, 1, 1, 1, 1, 6, 37, 1.5, 61)
    p, q, cand, u = sample_inputs(w, draft_noise=0.3)
    B, K, V = p.shape
    for i in (0, 2, K - 1):
        c = cand.clone()
        c[:, i] = bad
        acc, corr = oracle.sample_consensus(p, q, c, u)
        pe = torch.cat([p, torch.zeros(B, K, 1)], dim=-1)
        qe = torch.cat([q, torch.zeros(B, K, 1)], dim=-1)
        ce = cand.clone()
        ce[:, i] = V
        racc, rcorr = oracle.sample_consensus(pe, qe, ce, u)
        assert np.array_equal(acc, racc) and np.array_equal(corr, rcorr), (i, acc, racc, corr, rcorr)
        assert (acc <= i).all()
