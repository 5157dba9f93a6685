"""rv_schedule against the oracle: windows, K* and E* bit for bit, at the
sizes where the kernel changes shape (one, four and eight waves: 512, 2048
and 4096 candidates), every block length class, and confidences full of
exact ties, so that K* falls inside a run of equal survivals and the windows
depend on the (request, position) order of equal ranks."""

import numpy as np
import pytest
import torch

import oracle
import parity_util as pu

pytestmark = pytest.mark.gpu

# (B, gamma): candidates B * (gamma - 1) around 64 (one lane per candidate
# up to there), 512, 2048 and 4096
SHAPES = [(1, 2), (1, 8), (3, 16), (9, 8), (32, 3), (64, 2), (13, 6), (73, 8), (74, 8), (256, 8), (292, 8),
          (293, 8), (585, 8), (273, 16), (4096, 2), (512, 9)]


def _conf(kind, B, g1, rng):
    if kind == "beta":
        return rng.beta(3.0, 1.2, size=(B, g1))
    if kind == "ties":
        return rng.choice([0.0, 0.25, 0.5, 0.75, 1.0], size=(B, g1), p=[0.1, 0.15, 0.25, 0.25, 0.25])
    if kind == "ones":
        return np.ones((B, g1))
    if kind == "zeros":
        return np.zeros((B, g1))
    if kind == "tiny":   # survivals far below 2^-40: distinct values, equal fixed-point sums
        return rng.uniform(1e-4, 2e-3, size=(B, g1))
    raise ValueError(kind)


def _tables(B, gamma, rng, kind):
    M = np.arange(B * gamma + 1, dtype=np.float64)
    b = np.arange(B + 1, dtype=np.float64)
    if kind == "linear":
        return 0.3, 0.001 * b, 0.0005 * M
    if kind == "steps":
        return 0.5, 0.001 * b, 0.01 * np.floor(M / 37.0)
    return 1.0, 0.001 * b, rng.uniform(0.0, 2.0, M.size)


def _run(conf, gamma, mode, bias, alpha, theta):
    from ragged_verification_amd import rv
    B = conf.shape[0]
    dev = "cuda"
    i32 = dict(dtype=torch.int32, device=dev)
    wc, wv, ks = torch.zeros(B, **i32), torch.zeros(B, **i32), torch.zeros(1, **i32)
    es = torch.zeros(1, dtype=torch.float64, device=dev)
    ws = torch.zeros(rv.rv_workspace_size(B, gamma), dtype=torch.uint8, device=dev)
    rv.rv_schedule(torch.tensor(conf, dtype=torch.float32, device=dev), gamma, mode, bias,
                   torch.tensor(alpha, dtype=torch.float64, device=dev),
                   torch.tensor(theta, dtype=torch.float64, device=dev), wc, wv, ks, es, ws)
    torch.cuda.synchronize()
    assert rv.rv_device_status(ws) == 0
    return pu.npi(wc), pu.npi(wv), int(ks.item()), float(es.item())


def _inside_tie(conf32, gamma, k_star):
    """K* splits a run of equal survivals (the tie order decides windows)."""
    S = oracle.survival(np.asarray(conf32, dtype=np.float32).astype(np.float64))[:, 1:].ravel()
    if k_star == 0 or k_star == S.size:
        return False
    s = np.sort(S)[::-1]
    return s[k_star - 1] == s[k_star]


@pytest.mark.parametrize("B,gamma", SHAPES)
def test_schedule_sizes_and_ties(B, gamma):
    rng = np.random.default_rng(1000 * B + gamma)
    split = 0
    for kind in ("beta", "ties", "ones", "zeros", "tiny"):
        conf = _conf(kind, B, gamma - 1, rng).astype(np.float32)
        for tk in ("linear", "steps", "random"):
            bias, alpha, theta = _tables(B, gamma, rng, tk)
            for mode in ("compact", "cap_accept"):
                got = _run(conf, gamma, mode, bias, alpha, theta)
                want = oracle.schedule(conf.astype(np.float64), gamma, pu.MODE_CODES[mode], bias, alpha, theta)
                assert np.array_equal(got[0], want[0]), (kind, tk, mode)
                assert np.array_equal(got[1], want[1]), (kind, tk, mode)
                assert got[2] == want[2], (kind, tk, mode)
                assert got[3] == want[3], (kind, tk, mode)
                split += _inside_tie(conf, gamma, want[2])
    pu.log(f"B={B} gamma={gamma}: 30 cases, K* inside a tie run in {split}")
    if B * (gamma - 1) >= 64:
        assert split >= 1


@pytest.mark.parametrize("B,gamma", [(1024, 8), (512, 16)])
def test_schedule_full_block_modes_beyond_ranked_limit(B, gamma):
    """static and no-trim are not ranked: any B * (gamma - 1) the row limit
    allows, E* as the oracle's full-block sum."""
    rng = np.random.default_rng(B)
    conf = rng.beta(2.0, 1.0, size=(B, gamma - 1)).astype(np.float32)
    bias, alpha, theta = _tables(B, gamma, rng, "linear")
    for mode in ("static", "no_trim"):
        got = _run(conf, gamma, mode, bias, alpha, theta)
        want = oracle.schedule(conf.astype(np.float64), gamma, pu.MODE_CODES[mode], bias, alpha, theta)
        assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
        assert got[2] == want[2] and got[3] == want[3], mode
