"""Pins of the float64 C oracle of the whole pass (collapsed form, oracle/collapsed_pass.c) against the NumPy
oracle's plain definition: scores to 1e-12 of the term magnitudes, the selection exactly as the NumPy selection
on the C scores and as on the definition's scores outside the boundary set, rows gathered bit for bit, and the
same results with one thread and with several."""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import cpass

RNG = np.random.default_rng(2024)


def _units(n, d, G, rope, theta, lens):
    """n random units of bf16 keys clustered around a centre, rotated to ascending positions."""
    out = []
    for i in range(n):
        L = lens[i]
        pos = np.sort(RNG.choice(5 * max(L, 1), size=L, replace=False)).astype(np.int32)
        k_pre = RNG.normal(size=(L, d)) * 0.3 + RNG.normal(size=d)
        K = torch.from_numpy(O.rotate(k_pre, pos, theta, rope)).to(torch.bfloat16)
        V = torch.from_numpy(RNG.normal(size=(L, d))).to(torch.bfloat16)
        qbar, c = RNG.normal(size=(G, d)), np.abs(RNG.normal(size=(G, d // 2)))
        t = int(pos[-1]) + 1 if L else 0
        out.append(dict(K=K.view(torch.int16).numpy().view(np.uint16), K64=K.double().numpy(),
                        V=V.view(torch.int16).numpy().view(np.uint16), pos=pos, qbar=qbar, c=c, t=t))
    return out


@pytest.mark.parametrize("rope", ["half", "interleaved"])
@pytest.mark.parametrize("budget,recent", [(40, 8), (40, 0), (40, 40), (1, 0), (500, 10)])
def test_collapsed_pass_against_the_definition(rope, budget, recent):
    d, G, theta, offs = 64, 4, 1e4, (1, 2, 4, 8, 64)
    lens = [0, 1, 39, 40, 41, 300, 257]
    units = _units(len(lens), d, G, rope, theta, lens)
    u = np.stack([O.centre_vector(x["qbar"], theta, offs, rope) for x in units])
    chat = np.stack([x["c"].mean(0) for x in units])
    cat = lambda key: np.concatenate([x[key] for x in units]) if sum(lens) else np.zeros((0, d))
    out = cpass.pass_units(cat("K").reshape(-1, d), cat("V").reshape(-1, d), cat("pos"), lens, u, chat,
                           [x["t"] for x in units], theta, budget, recent, rope, threads=3)
    r0 = np.concatenate([[0], np.cumsum(lens)[:-1]])
    for i, x in enumerate(units):
        L = lens[i]
        s_c = out["scores"][r0[i]:r0[i] + L]
        ref = O.score(x["K64"], x["qbar"], x["c"], theta, offs, x["t"], rope)
        A = O.abs_terms(x["K64"], x["qbar"], x["c"], theta, offs, x["t"], rope)
        assert np.all(np.abs(s_c - ref) <= 1e-12 * A), i
        keep = out["keep"][i, :min(L, budget)]
        assert int(out["new_len"][i]) == min(L, budget)
        assert keep.tolist() == O.select(s_c, x["pos"], budget, recent).tolist()
        bset = set(O.boundary_set(ref, A, budget, recent, 1e-12).tolist())
        assert set(keep.tolist()) - bset == set(O.select(ref, x["pos"], budget, recent).tolist()) - bset
        assert np.array_equal(out["k"][i, :len(keep)], x["K"][keep])
        assert np.array_equal(out["v"][i, :len(keep)], x["V"][keep])
        assert np.array_equal(out["pos"][i, :len(keep)], x["pos"][keep])


def test_thread_count_does_not_change_results():
    d, G, theta, offs = 128, 2, 1e6, (1, 16, 4096)
    lens = [700, 1000, 64, 3000, 1]
    units = _units(len(lens), d, G, "half", theta, lens)
    u = np.stack([O.centre_vector(x["qbar"], theta, offs) for x in units])
    chat = np.stack([x["c"].mean(0) for x in units])
    args = (np.concatenate([x["K"] for x in units]), np.concatenate([x["V"] for x in units]),
            np.concatenate([x["pos"] for x in units]), lens, u, chat, [x["t"] for x in units], theta, 256, 32)
    a, b = cpass.pass_units(*args, threads=1), cpass.pass_units(*args, threads=4)
    for key in a:
        assert np.array_equal(a[key], b[key], equal_nan=True), key


def test_exact_ties_keep_the_lower_position():
    d, theta = 64, 1e4
    x = _units(1, d, 1, "half", theta, [50])[0]
    K = x["K"].copy()
    K[30] = K[10]                                   # identical rows score bitwise equal
    u = O.centre_vector(x["qbar"], theta, (1, 2))[None]
    out = cpass.pass_units(K, x["V"], x["pos"], [50], u, x["c"].mean(0)[None], [x["t"]], theta, 49, 0)
    s = out["scores"]
    assert s[30] == s[10]
    rank = np.lexsort((x["pos"], -s))
    r10 = int(np.nonzero(rank == 10)[0][0])
    out = cpass.pass_units(K, x["V"], x["pos"], [50], u, x["c"].mean(0)[None], [x["t"]], theta, r10 + 1, 0)
    keep = out["keep"][0].tolist()
    assert 10 in keep and 30 not in keep


def test_bad_arguments_rejected():
    with pytest.raises(ValueError):
        cpass.pass_units(np.zeros((4, 8), np.uint16), np.zeros((4, 8), np.uint16), np.arange(4), [4],
                         np.zeros((1, 8)), np.zeros((1, 4)), [4], 1e4, 2, 3)
