"""GPU parity of greedy and rejection-sampling consensus: bit-exact against the
oracle (accept_len, row_argmax, correction) on the same inputs."""
import numpy as np
import pytest
import torch

import dual_view_block_amd as dvb
import oracle
from synth import WORKLOADS, Workload, greedy_inputs, sample_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _greedy_gpu(logits, cand):
    acc, am, corr = dvb.orthrus_consensus_greedy(logits.to(DEV), cand.to(DEV))
    torch.cuda.synchronize()
    return acc.cpu().numpy(), am.cpu().numpy(), corr.cpu().numpy()


def _check_greedy(logits, cand, what):
    acc, am, corr = _greedy_gpu(logits, cand)
    racc, ram, rcorr = oracle.greedy_consensus(logits, cand)
    assert np.array_equal(am, ram), f"{what}: row_argmax differs"
    assert np.array_equal(acc, racc), f"{what}: accept_len {acc} vs {racc}"
    assert np.array_equal(corr, rcorr), f"{what}: correction {corr} vs {rcorr}"
    tokens = oracle.tokens_committed(acc, logits.shape[1])
    assert tokens.min() >= 1 and tokens.max() <= logits.shape[1]
    print(f"{what}: accept_len={acc.tolist()} correction={corr.tolist()}", flush=True)


@pytest.mark.parametrize("j", [0, 1, 2, 3, 4])
def test_greedy_tiny_every_first_mismatch(j):
    """Vocab 1000, K = 4, logits sigma 4, planted first mismatch j (4 = all match)."""
    logits, cand, _ = greedy_inputs(WORKLOADS["tiny"], first_mismatch=j)
    _check_greedy(logits, cand, f"tiny j={j}")


@pytest.mark.parametrize("j", [0, 1, 16, 31, 32])
@pytest.mark.parametrize("ties", [False, True])
def test_greedy_qwen_vocab(j, ties):
    """[1, 32, 151936] logits, sigma 3, with and without planted ties."""
    logits, cand, _ = greedy_inputs(WORKLOADS["qwen3_1p7b_layer"], first_mismatch=j, ties=ties)
    _check_greedy(logits, cand, f"qwen j={j} ties={ties}")


def test_greedy_batch_seeded_mismatch():
    w = WORKLOADS["ragged_b16"]
    logits, cand, _ = greedy_inputs(w)
    _check_greedy(logits, cand, "batch16")


@pytest.mark.parametrize("V", [3, 1001, 4099])
def test_greedy_odd_vocab(V):
    w = Workload("odd", 1, 3, 1, 1, 1, 1, 5, V, 2.0, 33)
    logits, cand, _ = greedy_inputs(w)
    _check_greedy(logits, cand, f"V={V}")


def test_greedy_nan_signed_zero_and_infinities():
    V, K = 5000, 4
    logits = torch.randn(1, K, V) * 3
    logits[0, 0, 17] = float("nan")
    logits[0, 0, 4000] = float("nan")
    logits[0, 1] = 0.0
    logits[0, 1, :10] = -0.0
    logits[0, 2, 99] = float("inf")
    logits[0, 2, 3000] = float("inf")
    logits[0, 3] = float("-inf")
    cand = torch.tensor([[17, 0, 99, 0]], dtype=torch.int32)
    _check_greedy(logits, cand, "special values")
    acc, am, _ = _greedy_gpu(logits, cand)
    assert am[0].tolist() == [17, 0, 99, 0] and acc[0] == 4


def _check_sample(p, q, cand, u, what):
    acc, corr = dvb.orthrus_consensus_sample(p.to(DEV), q.to(DEV), cand.to(DEV), u.to(DEV))
    torch.cuda.synchronize()
    acc, corr = acc.cpu().numpy(), corr.cpu().numpy()
    racc, rcorr = oracle.sample_consensus(p, q, cand, u)
    assert np.array_equal(acc, racc), f"{what}: accept_len {acc} vs {racc}"
    assert np.array_equal(corr, rcorr), f"{what}: correction {corr} vs {rcorr}"
    print(f"{what}: accept_len={acc.tolist()} correction={corr.tolist()}", flush=True)
    return acc, corr


@pytest.mark.parametrize("noise", [None, 0.5])
def test_sample_ragged_b16_qwen_vocab(noise):
    """B=16, K=32, V=151936; independent draft (rejects early) or a close one."""
    p, q, cand, u = sample_inputs(WORKLOADS["ragged_b16"], draft_noise=noise)
    _check_sample(p, q, cand, u, f"b16 noise={noise}")


@pytest.mark.parametrize("seed", range(4))
def test_sample_small_vocab(seed):
    w = Workload("s", 1, 8, 1, 1, 1, 1, 6, 37, 1.5, 40 + seed)
    p, q, cand, u = sample_inputs(w, draft_noise=0.7 if seed % 2 else None)
    _check_sample(p, q, cand, u, f"small seed={seed}")


@pytest.mark.parametrize("seed,noise", [(77, None), (79, 1.0), (87, 1.0)])
def test_sample_vocab_past_a_million(seed, noise):
    """V = 1,200,000: the residual splits the row into 256 chunks of 4688
    entries, longer than one pass of the chunk-sum and select loops (4096 per
    pass), so both loops take a second pass.  The cases reject at row 0, at
    row 1 or not at all."""
    w = Workload("big_vocab", 1, 2, 1, 1, 1, 1, 2, 1_200_000, 3.0, seed)
    p, q, cand, u = sample_inputs(w, draft_noise=noise)
    _check_sample(p, q, cand, u, f"V=1.2M seed={seed} noise={noise}")


def test_sample_degenerate_cases():
    B, K, V = 3, 4, 64
    g = torch.Generator().manual_seed(3)
    p = torch.softmax(torch.randn(B, K, V, generator=g, dtype=torch.float64), -1).float()
    q = p.clone()
    cand = torch.randint(0, V, (B, K), generator=g, dtype=torch.int32)
    u = torch.tensor([[0.0, 0.5, 1 - 2 ** -24, 0.25, 0.75]] * B, dtype=torch.float32)
    acc, corr = _check_sample(p, q, cand, u, "q == p")
    assert (acc == K).all() and (corr == -1).all()
    # target gives the candidate probability 0 at row 1 -> rejected there even for u = 0
    p2 = p.clone()
    p2[:, 1, :] = 0.0
    p2[:, 1, 7] = 1.0
    cand2 = cand.clone()
    cand2[:, 1] = 8
    u2 = torch.zeros(B, K + 1)
    acc, corr = _check_sample(p2, q, cand2, u2, "p(cand)=0")
    assert (acc == 1).all() and (corr == 7).all()
    # residual identically zero (p == q) at the rejected row -> falls back to p
    p3, q3 = p.clone(), p.clone()
    cand3 = cand.clone()
    cand3[:, 0] = 5
    p3[:, 0, 5] = 0.0
    q3[:, 0, 5] = 0.0
    _check_sample(p3, q3, cand3, u2, "zero residual")


@pytest.mark.parametrize("bad", [-1, -100000, 151936, 1 << 30])
def test_sample_out_of_vocabulary_candidates(bad):
    """A candidate outside [0, V) is rejected (the header's rule, R28 in the
    oracle): rejection at rows 0, 5 and 31 of different sequences of a
    [4, 32, 151936] problem with a draft close to its target."""
    w = WORKLOADS["ragged_b16"].replace(batch=4)
    p, q, cand, u = sample_inputs(w, draft_noise=0.5)
    cand = cand.clone()
    for b, i in ((0, 0), (1, 5), (2, 31)):
        cand[b, i] = bad
    acc, _ = _check_sample(p, q, cand, u, f"oov {bad}")
    assert acc[0] == 0 and acc[1] <= 5 and acc[2] <= 31


def _unplanted_greedy(B, seed, j_star):
    """N(0, 3) logits with no planted top (the configurations' own value law);
    candidates follow the oracle's row argmax up to j* and differ there."""
    V, K = 151936, 32
    g = torch.Generator().manual_seed(seed)
    logits = torch.randn((B, K, V), generator=g) * 3.0
    _, am, _ = oracle.greedy_consensus(logits, torch.zeros((B, K), dtype=torch.int32))
    am = torch.as_tensor(am, dtype=torch.int64)
    cand = am.clone()
    for b in range(B):
        j = int(j_star[b])
        if j < K:
            cand[b, j] = (am[b, j] + 1 + b) % V
            cand[b, j + 1:] = torch.randint(0, V, (K - j - 1,), generator=g)
    return logits, cand.to(torch.int32)


@pytest.mark.parametrize("B", [1, 16])
def test_greedy_unplanted_normal_logits(B):
    """Greedy parity on unplanted N(0, 3) logits at [B, 32, 151936]: every row's
    top is an ordinary draw, with no margin planted above the runner-up."""
    j_star = [(7 * b + 3) % 33 for b in range(B)] if B > 1 else [13]
    logits, cand = _unplanted_greedy(B, 1234 + B, j_star)
    _check_greedy(logits, cand, f"unplanted B={B}")
    acc, _, _ = _greedy_gpu(logits, cand)
    assert acc.tolist() == j_star
