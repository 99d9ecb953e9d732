"""Checks of the seeded input generators (no method arithmetic lives there)."""
import numpy as np
import torch

from synth import WORKLOADS, philox4x32, philox_uniforms, sample_inputs


def test_philox4x32_10_known_answers():
    """The known-answer vectors published with the Random123 library for
    Philox4x32 with 10 rounds: zero counter and key, all-ones, and the
    digits of pi."""
    cases = [
        ([0, 0, 0, 0], (0, 0), [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
        ([0xFFFFFFFF] * 4, (0xFFFFFFFF, 0xFFFFFFFF), [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
        ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], (0xA4093822, 0x299F31D0),
         [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
    ]
    for ctr, key, want in cases:
        got = philox4x32(np.array([ctr], dtype=np.uint64), key)[0]
        assert [int(x) for x in got] == want


def test_philox_uniforms_grid_and_spread():
    u = philox_uniforms(100003, seed=5)
    assert u.shape == (100003,)
    assert (u >= 0).all() and (u < 1).all()
    assert torch.equal(torch.floor(u * 2 ** 24), u * 2 ** 24)
    assert abs(float(u.mean()) - 0.5) < 0.01 and abs(float(u.var()) - 1 / 12) < 0.005
    assert torch.equal(philox_uniforms(10, seed=5), u[:10])


def test_sample_inputs_candidates_follow_the_draft():
    """cand[b, i] lies in the support of q[b, i] and the uniforms are on the grid."""
    w = WORKLOADS["ragged_b16"].replace(batch=2, vocab=50)
    p, q, cand, u = sample_inputs(w, draft_noise=0.5)
    assert cand.dtype == torch.int32 and u.shape == (2, 33)
    qc = torch.gather(q, 2, cand.long().unsqueeze(-1))
    assert (qc > 0).all()
    assert torch.equal(torch.floor(u.double() * 2 ** 24), u.double() * 2 ** 24)
