"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each pin is chosen so that a plausible slip in the oracle (a dropped term, a sign, the wrong
rotary pairing, a transposed operand, a wrong frequency exponent, a wrong tie order) fails at
least one test: hand-derived closed forms, a textbook rotary routine, identities between
independently written forms, invariances the method relies on, and brute force.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


# ----------------------------------------------------------------------------- closed forms

def test_worked_example_by_hand():
    ex = json.load(open(os.path.join(GOLD, "worked_example.json")))
    expected = ((math.sin(4) + math.sin(5)) / 2 + 0.5 * (math.cos(0.04) + math.cos(0.05)) / 2) + 0.75
    # stored key = pre-rotation key rotated to its position, written with explicit 2x2 rotations
    k_pre = np.array(ex["k_pre"])
    p, theta = ex["p"], ex["theta"]
    om = [1.0, 0.01]
    K = np.zeros(4)
    for i in range(2):
        a, b = k_pre[i], k_pre[i + 2]
        K[i] = a * math.cos(p * om[i]) - b * math.sin(p * om[i])
        K[i + 2] = a * math.sin(p * om[i]) + b * math.cos(p * om[i])
    q = np.array([ex["qbar"]])
    c = np.array([ex["c"]])
    for fn in (lambda: O.score(K[None], q, c, theta, ex["offsets"], ex["t"]),
               lambda: O.score_collapsed(K[None], q, c, theta, ex["offsets"], ex["t"]),
               lambda: O.score_trig_series(K[None], [p], q, c, theta, ex["offsets"], ex["t"])):
        assert abs(fn()[0] - expected) < 1e-13
    assert abs(expected - 0.3916242067784527) < 1e-15


@pytest.mark.parametrize("theta", [10.0, 1e4, 1e6])
def test_d2_closed_form(theta):
    # d = 2: one pair with omega_0 = 1 for every theta.  s = |q||k| mean_D cos(t + D - p + arg q - arg k) + c |k|
    for _ in range(20):
        q = RNG.normal(size=2)
        k_pre = RNG.normal(size=2)
        p = int(RNG.integers(0, 50))
        t = p + int(RNG.integers(0, 30))
        offs = list(RNG.choice(np.arange(0, 40), size=3, replace=False))
        c = RNG.normal()
        K = np.array([k_pre[0] * math.cos(p) - k_pre[1] * math.sin(p),
                      k_pre[0] * math.sin(p) + k_pre[1] * math.cos(p)])
        aq, ak = math.atan2(q[1], q[0]), math.atan2(k_pre[1], k_pre[0])
        nq, nk = math.hypot(*q), math.hypot(*k_pre)
        want = np.mean([nq * nk * math.cos(t + dl - p + aq - ak) for dl in offs]) + c * nk
        got = O.score(K[None], q[None], np.array([[c]]), theta, offs, t)[0]
        assert abs(got - want) < 1e-12 * (nq * nk + abs(c) * nk)
    # the simplest instance: q = k = (1, 0), one offset, t = p  ->  cos(1)
    K = np.array([[math.cos(5.0), math.sin(5.0)]])
    assert abs(O.score(K, np.array([[1.0, 0.0]]), np.zeros((1, 1)), 1e4, [1], 5)[0] - math.cos(1.0)) < 1e-14


def _textbook_rope(x, n, theta):
    """Rotary embedding in the common 'rotate_half' formulation: x*cos + rotate_half(x)*sin with
    inv_freq = 1 / theta^(arange(0, d, 2)/d) duplicated over both halves."""
    d = x.shape[-1]
    inv_freq = 1.0 / (theta ** (np.arange(0, d, 2, dtype=np.float64) / d))
    ang = np.concatenate([n * inv_freq, n * inv_freq])
    x1, x2 = x[: d // 2], x[d // 2:]
    rot_half = np.concatenate([-x2, x1])
    return x * np.cos(ang) + rot_half * np.sin(ang)


@pytest.mark.parametrize("d", [4, 64, 128])
def test_textbook_rotary_logit(d):
    # offsets {0}, one head, c = 0: the score is the plain rotary logit q(t) . k(p)
    theta = 1e6 if d == 128 else 1e4
    q, k_pre = RNG.normal(size=d), RNG.normal(size=(5, d))
    ps = np.array([0, 3, 100, 4000, 32767])
    K = np.stack([_textbook_rope(k_pre[j], ps[j], theta) for j in range(5)])
    t = 40000
    want = K @ _textbook_rope(q, t, theta)
    got = O.score(K, q[None], np.zeros((1, d // 2)), theta, [0], t)
    assert np.allclose(got, want, rtol=0, atol=1e-10 * np.abs(K).sum(1).max() * np.abs(q).sum())
    # and the oracle's own rotation agrees with the textbook one
    assert np.allclose(O.rotate(k_pre[1], 3, theta), _textbook_rope(k_pre[1], 3, theta), atol=1e-13)


def test_frequencies_structure():
    for d, theta in [(2, 7.0), (64, 1e4), (128, 1e6)]:
        w = O.frequencies(d, theta)
        assert w.shape == (d // 2,) and w[0] == 1.0
        # geometric with ratio theta^(-2/d); the would-be next term is 1/theta
        assert np.allclose(w[1:] / w[:-1], theta ** (-2.0 / d), rtol=1e-13)
        assert abs(w[-1] * theta ** (-2.0 / d) - 1.0 / theta) < 1e-12 / theta


# ----------------------------------------------------------------------------- identities between forms

def _random_unit(d, G, L, theta, rope, n_off=5, tmax=50000):
    k_pre = RNG.normal(size=(L, d)) + RNG.normal(size=d) * 2
    pos = np.sort(RNG.choice(tmax // 2, size=L, replace=False))
    K = O.rotate(k_pre, pos, theta, rope)
    q = RNG.normal(size=(G, d))
    c = RNG.normal(size=(G, d // 2))
    offs = sorted(RNG.choice(4097, size=n_off, replace=False).tolist())
    t = int(pos.max()) + int(RNG.integers(1, 1000))
    return K, pos, q, c, offs, t


@pytest.mark.parametrize("rope", ["half", "interleaved"])
@pytest.mark.parametrize("d,G", [(2, 1), (4, 2), (64, 2), (128, 4), (128, 8)])
def test_trig_series_equals_definition_equals_collapsed(d, G, rope):
    theta = 1e6 if d == 128 else 1e4
    K, pos, q, c, offs, t = _random_unit(d, G, 40, theta, rope)
    A = O.abs_terms(K, q, c, theta, offs, t, rope)
    sB = O.score(K, q, c, theta, offs, t, rope)
    sA = O.score_trig_series(K, pos, q, c, theta, offs, t, rope)
    sC = O.score_collapsed(K, q, c, theta, offs, t, rope)
    assert np.all(np.abs(sA - sB) <= 1e-12 * A)
    assert np.all(np.abs(sC - sB) <= 1e-12 * A)
    assert np.all(np.abs(sB) <= A * (1 + 1e-12))


def test_pairing_conventions_differ():
    # the two conventions are genuinely different operations (guards against one silently aliasing the other)
    K, pos, q, c, offs, t = _random_unit(8, 1, 10, 1e4, "half")
    assert not np.allclose(O.score(K, q, c, 1e4, offs, t, "half"), O.score(K, q, c, 1e4, offs, t, "interleaved"))


def test_gqa_is_mean_of_heads():
    K, pos, q, c, offs, t = _random_unit(64, 4, 30, 1e4, "half")
    full = O.score(K, q, c, 1e4, offs, t)
    per = np.mean([O.score(K, q[g:g + 1], c[g:g + 1], 1e4, offs, t) for g in range(4)], axis=0)
    assert np.allclose(full, per, rtol=0, atol=1e-12 * O.abs_terms(K, q, c, 1e4, offs, t).max())


def test_offsets_are_averaged():
    K, pos, q, c, offs, t = _random_unit(64, 2, 30, 1e4, "half")
    both = O.score(K, q, np.zeros_like(c), 1e4, [3, 200], t)
    sep = 0.5 * (O.score(K, q, np.zeros_like(c), 1e4, [3], t) + O.score(K, q, np.zeros_like(c), 1e4, [200], t))
    assert np.allclose(both, sep, atol=1e-12 * np.abs(K).sum(1).max() * np.abs(q).sum())


def test_translation_invariance():
    # the centre-based score depends on the distance t - p only, never on absolute position
    d, theta = 128, 1e6
    k_pre = RNG.normal(size=(16, d))
    p = np.sort(RNG.choice(20000, size=16, replace=False))
    q, c = RNG.normal(size=(4, d)), RNG.normal(size=(4, d // 2))
    t = 20000
    s0 = O.score(O.rotate(k_pre, p, theta), q, c, theta, [1, 8, 4096], t)
    for m in (1, 777, 123456):
        s1 = O.score(O.rotate(k_pre, p + m, theta), q, c, theta, [1, 8, 4096], t + m)
        assert np.allclose(s0, s1, rtol=0, atol=1e-9 * np.abs(s0).max())


def test_norm_only_term():
    # zero query centres: the score is sum_i chat_i sqrt(x_i^2 + x_{i+d/2}^2), unchanged by any per-pair rotation
    d = 64
    K = RNG.normal(size=(12, d))
    c = RNG.normal(size=(2, d // 2))
    s = O.score(K, np.zeros((2, d)), c, 1e4, [1, 2], 99)
    want = np.sqrt(K[:, :d // 2] ** 2 + K[:, d // 2:] ** 2) @ c.mean(0)
    assert np.allclose(s, want, atol=1e-13)
    ang = RNG.uniform(0, 2 * np.pi, size=d // 2)
    z = (K[:, :d // 2] + 1j * K[:, d // 2:]) * np.exp(1j * ang)
    K2 = np.concatenate([z.real, z.imag], 1)
    assert np.allclose(O.score(K2, np.zeros((2, d)), c, 1e4, [1, 2], 99), s, atol=1e-12)


def test_distance_part_linear_in_key():
    K, pos, q, c, offs, t = _random_unit(64, 2, 5, 1e4, "half")
    z = np.zeros_like(c)
    a, b = 0.3, -1.7
    lhs = O.score(a * K[:1] + b * K[1:2], q, z, 1e4, offs, t)
    rhs = a * O.score(K[:1], q, z, 1e4, offs, t) + b * O.score(K[1:2], q, z, 1e4, offs, t)
    assert np.allclose(lhs, rhs, atol=1e-11)


# ----------------------------------------------------------------------------- selection

def _kept_by_counting(s, pos, B, R):
    """Independent characterisation: candidate p is kept iff fewer than B-R candidates beat it
    under (higher score, then lower position)."""
    s = np.where(np.isnan(s), -np.inf, s)
    L = len(s)
    if L <= B:
        return list(range(L))
    nc = L - R
    kept = []
    for p in range(nc):
        beat = sum(1 for q in range(nc) if (s[q] > s[p]) or (s[q] == s[p] and pos[q] < pos[p]))
        if beat < B - R:
            kept.append(p)
    return sorted(kept + list(range(nc, L)))


def test_selection_bruteforce_all_budgets():
    for L in (0, 1, 2, 5, 17, 40, 64):
        s = RNG.integers(0, 6, size=L).astype(np.float64)   # many exact ties
        pos = np.arange(L) * 3 + 1
        for B in range(1, L + 3):
            for R in range(0, B + 1):
                want = _kept_by_counting(s, pos, B, R)
                got = O.select(s, pos, B, R)
                assert got.tolist() == want, (L, B, R)
                assert O.select_bruteforce(s, pos, B, R).tolist() == want


def test_selection_invariants_random():
    for _ in range(50):
        L = int(RNG.integers(1, 300))
        B = int(RNG.integers(1, 200))
        R = int(RNG.integers(0, B + 1))
        s = RNG.normal(size=L)
        pos = np.arange(L)
        keep = O.select(s, pos, B, R)
        assert len(keep) == min(L, B)
        assert np.all(np.diff(keep) > 0)
        if L > B:
            assert set(range(L - R, L)) <= set(keep.tolist())
            cand_kept = [p for p in keep if p < L - R]
            cand_ev = sorted(set(range(L - R)) - set(keep.tolist()))
            if cand_kept and cand_ev:
                worst_kept = min((s[p], -p) for p in cand_kept)
                best_ev = max((s[p], -p) for p in cand_ev)
                assert worst_kept > best_ev


def test_exact_ties_keep_lower_position():
    d, theta = 64, 1e4
    K = RNG.normal(size=(20, d))
    K[15] = K[4]                      # identical stored rows score bitwise equal
    q, c = RNG.normal(size=(2, d)), RNG.normal(size=(2, d // 2))
    s = O.score(K, q, c, theta, [1, 2], 30)
    assert s[15] == s[4]
    rank = np.argsort(-s, kind="stable")
    r4 = int(np.nonzero(rank == 4)[0][0])   # place B-R exactly at the tie
    keep = O.select(s, np.arange(20), B := r4 + 1, 0)
    assert 4 in keep and 15 not in keep and len(keep) == B


def test_all_equal_scores():
    L, B, R = 50, 12, 4
    keep = O.select(np.zeros(L), np.arange(L), B, R)
    assert keep.tolist() == list(range(B - R)) + list(range(L - R, L))


def test_nan_and_signed_zero():
    s = np.array([np.nan, -0.0, 0.0, -1.0, np.nan, 2.0])
    # NaN ranks last; -0 and +0 tie, so the lower position wins
    assert O.select(s, np.arange(6), 2, 0).tolist() == [1, 5]
    assert O.select(s, np.arange(6), 3, 0).tolist() == [1, 2, 5]
    assert O.select(s, np.arange(6), 5, 0).tolist() == [0, 1, 2, 3, 5]


def test_bad_budget_rejected():
    with pytest.raises(ValueError):
        O.select(np.zeros(4), np.arange(4), 2, 3)
    with pytest.raises(ValueError):
        O.select(np.zeros(4), np.arange(4), 0, 0)


def test_boundary_set():
    s = np.array([5.0, 4.0, 3.0, 3.0 + 1e-9, 1.0, 0.0])
    b = O.boundary_set(s, np.ones(6), 3, 0, 1e-6)
    assert b.tolist() == [2, 3]
    assert O.boundary_set(s, np.ones(6), 6, 0, 1e-6).size == 0


# ----------------------------------------------------------------------------- compaction

def test_compaction_rows_bit_exact_and_ordered():
    import torch
    L, d = 100, 16
    K = torch.randn(L, d).to(torch.bfloat16)
    V = torch.randn(L, d).to(torch.bfloat16)
    pos = np.arange(L, dtype=np.int32) + 7
    keep = O.select(RNG.normal(size=L), pos, 30, 5)
    k2, v2, p2 = O.compact(K.view(torch.int16).numpy(), V.view(torch.int16).numpy(), pos, keep)
    for j, src in enumerate(keep):
        assert np.array_equal(k2[j], K[src].view(torch.int16).numpy())
        assert np.array_equal(v2[j], V[src].view(torch.int16).numpy())
        assert p2[j] == pos[src]
    assert np.all(np.diff(p2) > 0)


def test_pass_is_idempotent():
    d, theta = 64, 1e4
    K, pos, q, c, offs, t = _random_unit(d, 2, 300, theta, "half")
    V = RNG.normal(size=K.shape)
    first = O.evict_unit(K, V, pos, q, c, theta, offs, t, 64, 8)
    second = O.evict_unit(first["k"], first["v"], first["pos"], q, c, theta, offs, t, 64, 8)
    assert second["keep"].tolist() == list(range(64))
    assert np.array_equal(second["k"], first["k"]) and np.array_equal(second["pos"], first["pos"])


def test_paged_tables():
    row = RNG.permutation(np.arange(1, 41))
    for L in (1, 15, 16, 17, 300, 640):
        for B in (1, 16, 100, 2048):
            Ln = min(L, B)
            new, freed = O.paged_tables(row, L, Ln, 16)
            n_old = -(-L // 16)
            assert len(new) == -(-Ln // 16)
            assert new.tolist() + freed.tolist() == row[:n_old].tolist()
            assert len(set(new.tolist()) & set(freed.tolist())) == 0


def test_logical_view_matches_contiguous_generator():
    # the paged and contiguous generators draw identical per-sequence data; gathering through the
    # block table must give back the contiguous rows
    import synth
    base = synth.scaled(synth.CONFIGS["paged_8b"], layers=1, batch=3, max_len=96, len_lo=20, len_hi=96,
                        name="pagedview")
    paged = synth.make_cache(base)
    contig = synth.make_cache(synth.scaled(base, layout="contiguous"))
    for b in range(3):
        L = int(paged["lengths"][b])
        for h in (0, 5):
            kp = O.logical_unit(paged["k"][0].view(torch_int16()).numpy(), paged["block_table"][b].numpy(), L, h, 16)
            kc = contig["k"][0, b, h, :L].view(torch_int16()).numpy()
            assert np.array_equal(kp, kc)
            pp = O.logical_unit(paged["pos"][0].numpy(), paged["block_table"][b].numpy(), L, h, 16)
            assert pp.tolist() == list(range(L))


def torch_int16():
    import torch
    return torch.int16


# ----------------------------------------------------------------------------- generator sanity (inputs)

def test_generated_keys_are_rotated_centres():
    # derotating the stored keys by their positions recovers keys clustered around one centre
    import synth
    import torch
    cfg = synth.CONFIGS["tiny"]
    cache = synth.make_cache(cfg)
    K = cache["k"][0, 0, 0, :1024].double().numpy()
    k_pre = O.rotate(K, -np.arange(1024), cfg.theta)
    spread = k_pre.std(axis=0).mean()
    assert abs(spread - cfg.noise) < 0.05          # the noise scale, not the spread of rotated keys
    assert np.abs(K).std() > 0.5


def test_steady_state_cache_structure():
    # a cache as a recurring pass finds it: budget + steady slots per unit, ascending positions
    # ending in the protected window and the new tokens, keys rotated at the positions pos records
    import synth
    for layout in ("contiguous", "paged"):
        cfg = synth.scaled(synth.CONFIGS["paged_8b_steady"], layout=layout, layers=1, batch=2, max_len=700,
                           len_lo=400, len_hi=700, budget=200, recent=24, steady=40, name="steadygen")
        cache = synth.make_cache(cfg)
        t0 = synth.lengths_for(cfg).numpy()
        assert cache["lengths"].tolist() == [240, 240]
        assert cache["t"].tolist() == (t0 + 40).tolist()
        for b in range(2):
            for h in (0, 7):
                if layout == "paged":
                    table = cache["block_table"][b].numpy()
                    K = O.logical_unit(cache["k"][0].double().numpy(), table, 240, h, 16)
                    pos = O.logical_unit(cache["pos"][0].numpy(), table, 240, h, 16).astype(np.int64)
                else:
                    K = cache["k"][0, b, h, :240].double().numpy()
                    pos = cache["pos"][0, b, h, :240].numpy().astype(np.int64)
                assert np.all(np.diff(pos) > 0) and pos[0] >= 0
                assert pos[-64:].tolist() == list(range(t0[b] - 24, t0[b] + 40))
                assert pos[-65] < t0[b] - 24
                # derotating by the recorded positions gives keys clustered around one centre; on the
                # fast-turning pairs (i < 16) derotating by the slot index instead leaves them spread
                hi = np.r_[0:16, 64:80]
                right = O.rotate(K, -pos, cfg.theta)[:, hi].std(axis=0).mean()
                wrong = O.rotate(K, -np.arange(240), cfg.theta)[:, hi].std(axis=0).mean()
                assert right < 0.5 * wrong


# ----------------------------------------------------------------------------- calibration statistics

def test_calibration_closed_form():
    # one pair (d = 2): q1 = 3 + 4j, q2 = -3 + 4j -> centre 4j, mean |z| = 5, |z(centre)| = 4, c = 1
    qbar, c = O.calibration_stats(np.array([[3.0, 4.0], [-3.0, 4.0]]))
    assert np.allclose(qbar, [0.0, 4.0], atol=0, rtol=0) and np.allclose(c, [1.0], atol=1e-15)


def test_calibration_special_cases():
    v = RNG.normal(size=16)
    qbar, c = O.calibration_stats(np.tile(v, (7, 1)))           # identical queries: centre = v, nothing missed
    assert np.allclose(qbar, v, atol=1e-15) and np.allclose(c, 0.0, atol=1e-14)
    qbar, c = O.calibration_stats(np.stack([v, -v]))             # opposite queries: centre 0, c = |z(v)|
    assert np.allclose(qbar, 0.0, atol=0) and np.allclose(c, np.abs(O.to_pairs(v)), atol=1e-15)


@pytest.mark.parametrize("rope", ["half", "interleaved"])
def test_calibration_rotation_equivariant_and_nonnegative(rope):
    # rotating every query by the same rotary angles rotates the centre and leaves c unchanged; c >= 0
    Q = RNG.normal(size=(300, 64)) + RNG.normal(size=64)
    qbar, c = O.calibration_stats(Q, rope)
    Qr = O.rotate(Q, 1234, 1e4, rope)
    qbar_r, c_r = O.calibration_stats(Qr, rope)
    assert np.allclose(qbar_r, O.rotate(qbar, 1234, 1e4, rope), atol=1e-12)
    assert np.allclose(c_r, c, atol=1e-12)
    assert np.all(c >= -1e-15)
    other = O.calibration_stats(Q, "interleaved" if rope == "half" else "half")[1]
    assert not np.allclose(other, c)                             # the pairing matters


# ----------------------------------------------------------------------------- decode attention

def test_attention_two_keys_closed_form():
    # s = scale * q.k: with q = (1, 0), k0 = (2, 0), k1 = (0, 5), scale 0.5 -> s = (1, 0)
    out = O.decode_attention([[1.0, 0.0]], [[2.0, 0.0], [0.0, 5.0]], [[1.0, 3.0], [-1.0, 7.0]], 0.5)
    w0 = math.e / (math.e + 1.0)
    assert np.allclose(out, [[w0 * 1 + (1 - w0) * -1, w0 * 3 + (1 - w0) * 7]], atol=1e-15)


def test_attention_special_cases():
    K = RNG.normal(size=(50, 16))
    V = RNG.normal(size=(50, 16))
    assert np.allclose(O.decode_attention(np.zeros((3, 16)), K, V, 0.25), V.mean(axis=0), atol=1e-14)   # uniform
    assert np.allclose(O.decode_attention(RNG.normal(size=(2, 16)), K[:1], V[:1], 0.25), V[0], atol=1e-15)  # one key
    big = 1e4 * K[17]                                                         # one key dominates
    assert np.allclose(O.decode_attention(big[None], K, V, 1.0), V[17], atol=1e-12)


def test_attention_permutation_and_rows():
    # permuting the kept slots changes nothing; query rows are independent
    K, V, q = RNG.normal(size=(64, 32)), RNG.normal(size=(64, 32)), RNG.normal(size=(4, 32))
    perm = RNG.permutation(64)
    a = O.decode_attention(q, K, V, 0.125)
    assert np.allclose(a, O.decode_attention(q, K[perm], V[perm], 0.125), atol=1e-14)
    assert np.allclose(a[2], O.decode_attention(q[2:3], K, V, 0.125)[0], atol=1e-15)
    # brute force: explicit sums over keys
    s = 0.125 * np.array([[sum(q[g, e] * K[p, e] for e in range(32)) for p in range(64)] for g in range(4)])
    w = np.exp(s) / np.exp(s).sum(axis=1, keepdims=True)
    assert np.allclose(a, w @ V, atol=1e-13)


# ----------------------------------------------------------------------------- aggregation variants

@pytest.mark.parametrize("rope", ["half", "interleaved"])
def test_variant_mean_is_the_score(rope):
    K = RNG.normal(size=(40, 64))
    qbar, c = RNG.normal(size=(3, 64)), RNG.normal(size=(3, 32))
    ref = O.score(K, qbar, c, 1e4, (1, 4, 16), 77, rope)
    assert np.allclose(O.score_variant(K, qbar, c, 1e4, (1, 4, 16), 77, rope, "mean"), ref, atol=1e-12)


def test_variant_single_logit_and_order():
    # one head and one offset: max = head_max = mean; in general max >= head_max >= mean
    K = RNG.normal(size=(30, 32))
    q1, c1 = RNG.normal(size=(1, 32)), RNG.normal(size=(1, 16))
    a = [O.score_variant(K, q1, c1, 1e4, (5,), 100, "half", agg) for agg in ("mean", "max", "head_max")]
    assert np.allclose(a[0], a[1], atol=1e-13) and np.allclose(a[0], a[2], atol=1e-13)
    qg, cg = RNG.normal(size=(4, 32)), RNG.normal(size=(4, 16))
    m, mx, hm = [O.score_variant(K, qg, cg, 1e4, (1, 2, 4, 8), 100, "half", agg) for agg in ("mean", "max", "head_max")]
    assert np.all(mx >= hm - 1e-12) and np.all(hm >= m - 1e-12)


def test_variant_brute_force():
    # explicit loops: rotate each centre to each future position, dot with the key, aggregate
    K = RNG.normal(size=(6, 8))
    qbar, c = RNG.normal(size=(2, 8)), RNG.normal(size=(2, 4))
    offs, t, theta = (1, 3), 9, 100.0
    w = [theta ** (-2 * i / 8) for i in range(4)]
    def rot(x, n):   # half-split pairs (i, i + 4)
        out = list(x)
        for i in range(4):
            a, b = x[i], x[i + 4]
            out[i] = a * math.cos(n * w[i]) - b * math.sin(n * w[i])
            out[i + 4] = a * math.sin(n * w[i]) + b * math.cos(n * w[i])
        return out
    for agg in ("max", "head_max"):
        got = O.score_variant(K, qbar, c, theta, offs, t, "half", agg)
        for p in range(6):
            lg = [[sum(a * b for a, b in zip(rot(qbar[g], t + dl), K[p])) for dl in offs] for g in range(2)]
            dist = max(max(r) for r in lg) if agg == "max" else sum(max(r) for r in lg) / 2
            norm = sum(sum(c[g][i] * math.hypot(K[p][i], K[p][i + 4]) for i in range(4)) for g in range(2)) / 2
            assert abs(got[p] - (dist + norm)) < 1e-12


# ----------------------------------------------------------------------------- GQA mapping, pairings, error scales

def test_group_rows_is_the_contiguous_query_group():
    # query head hq belongs to KV head hq // G (the grouped-query mapping whose heads the score averages);
    # written here as an explicit loop over query heads
    for h_q, h_kv in ((4, 2), (8, 2), (32, 8), (64, 8), (6, 1)):
        G = h_q // h_kv
        x = RNG.normal(size=(h_q, 5))
        for h in range(h_kv):
            want = np.stack([x[hq] for hq in range(h_q) if hq // G == h])
            assert np.array_equal(O.group_rows(x, h, G), want), (h_q, h_kv, h)


def _textbook_logit(q, K, theta, offsets, t):
    """(1/|D|) sum over Delta of textbook-rotated q at t + Delta, dotted with each stored key (half-split)."""
    return np.mean([K @ _textbook_rope(q, t + dl, theta) for dl in offsets], axis=0)


def test_one_hot_query_head_moves_only_its_kv_head():
    # every query head, one at a time: a centre that is zero except on head hq changes only KV head hq // G,
    # whose score is 1/G of that one head's rotary logit averaged over the offsets (the other heads of the
    # group contribute zero)
    h_q, h_kv, d, theta = 8, 2, 16, 1e4
    G = h_q // h_kv
    K = RNG.normal(size=(7, d))
    offs, t = (1, 4, 64), 300
    v = RNG.normal(size=d)
    zc = np.zeros((G, d // 2))
    for hq in range(h_q):
        qbar = np.zeros((h_q, d))
        qbar[hq] = v
        for h in range(h_kv):
            u = O.centre_vector(O.group_rows(qbar, h, G), theta, offs)
            s = O.score(K, O.group_rows(qbar, h, G), zc, theta, offs, t)
            if h == hq // G:
                assert np.abs(u).max() > 0.1
                assert np.allclose(s, _textbook_logit(v, K, theta, offs, t) / G, rtol=0, atol=1e-12), (hq, h)
            else:
                assert np.abs(u).max() == 0.0 and np.abs(s).max() == 0.0, (hq, h)


def test_pair_layouts_by_hand():
    x = np.array([1.0, 2.0, 3.0, 4.0])
    assert O.to_pairs(x, "half").tolist() == [1 + 3j, 2 + 4j]           # (x[i], x[i + d/2])
    assert O.to_pairs(x, "interleaved").tolist() == [1 + 2j, 3 + 4j]    # (x[2i], x[2i + 1])
    for rope in ("half", "interleaved"):
        assert O.from_pairs(O.to_pairs(x, rope), rope).tolist() == x.tolist()


def _textbook_rope_interleaved(x, n, theta):
    """Rotary embedding in the 'rotate every two' form: dims (2i, 2i+1) turned by the angle n * theta^(-2i/d),
    written with explicit 2x2 rotations."""
    d = x.shape[-1]
    out = np.empty(d)
    for i in range(d // 2):
        ang = n * theta ** (-2.0 * i / d)
        a, b = x[2 * i], x[2 * i + 1]
        out[2 * i] = a * math.cos(ang) - b * math.sin(ang)
        out[2 * i + 1] = a * math.sin(ang) + b * math.cos(ang)
    return out


@pytest.mark.parametrize("d", [4, 64, 128])
def test_textbook_interleaved_rotary_logit(d):
    # the interleaved pairing against its textbook rotation: the rotation itself, the score with offsets {0},
    # one head and c = 0 (the plain rotary logit), and the norm term over (x[2i], x[2i+1]) pairs
    theta = 1e6 if d == 128 else 1e4
    q, k_pre = RNG.normal(size=d), RNG.normal(size=(5, d))
    ps = np.array([0, 3, 100, 4000, 32767])
    K = np.stack([_textbook_rope_interleaved(k_pre[j], ps[j], theta) for j in range(5)])
    for j in range(5):
        # one-ulp differences of the frequency grow with the angle: the tolerance scales with the position
        tol = 1e-15 * (1 + ps[j]) * np.abs(k_pre[j]).sum()
        assert np.allclose(O.rotate(k_pre[j], ps[j], theta, "interleaved"), K[j], rtol=0, atol=tol)
    t = 40000
    want = K @ _textbook_rope_interleaved(q, t, theta)
    got = O.score(K, q[None], np.zeros((1, d // 2)), theta, [0], t, "interleaved")
    assert np.allclose(got, want, rtol=0, atol=1e-10 * np.abs(K).sum(1).max() * np.abs(q).sum())
    c = RNG.normal(size=(1, d // 2))
    norm = [sum(c[0, i] * math.hypot(K[p, 2 * i], K[p, 2 * i + 1]) for i in range(d // 2)) for p in range(5)]
    got = O.score(K, np.zeros((1, d)), c, theta, [3], t, "interleaved")
    assert np.allclose(got, norm, rtol=0, atol=1e-12)


def test_abs_terms_worked_example_closed_form():
    # A(p) = sum_j |w_j K_j| + sum_i |chat_i| |z_i(K)| on the worked example, every factor written in closed
    # form: w = mean over Delta of RoPE(qbar, t + Delta) with qbar pairs (1, 0.5); the stored key's pairs are
    # i * e^{7i} and e^{0.07i}; |z_i(K)| = 1, c = (0.25, 0.5)
    ex = json.load(open(os.path.join(GOLD, "worked_example.json")))
    t, offs = ex["t"], ex["offsets"]
    w = np.array([np.mean([math.cos(t + dl) for dl in offs]),
                  0.5 * np.mean([math.cos(0.01 * (t + dl)) for dl in offs]),
                  np.mean([math.sin(t + dl) for dl in offs]),
                  0.5 * np.mean([math.sin(0.01 * (t + dl)) for dl in offs])])
    K = np.array([-math.sin(7.0), math.cos(0.07), math.cos(7.0), math.sin(0.07)])
    want = float(np.abs(w * K).sum()) + 0.25 + 0.5
    got = O.abs_terms(K[None], np.array([ex["qbar"]]), np.array([ex["c"]]), ex["theta"], offs, t)[0]
    assert abs(got - want) < 1e-14
    # the variant scale: the largest over offsets of sum_j |W_j K_j| with W = RoPE(qbar, t + Delta), + 0.75
    per = [abs(math.cos(t + dl) * K[0]) + abs(0.5 * math.cos(0.01 * (t + dl)) * K[1]) +
           abs(math.sin(t + dl) * K[2]) + abs(0.5 * math.sin(0.01 * (t + dl)) * K[3]) for dl in offs]
    got_v = O.abs_terms_variant(K[None], np.array([ex["qbar"]]), np.array([ex["c"]]), ex["theta"], offs, t)[0]
    assert abs(got_v - (max(per) + 0.75)) < 1e-14
    assert abs(per[0] - per[1]) > 1e-3          # the two offsets differ, so a mean would fail


@pytest.mark.parametrize("rope", ["half", "interleaved"])
def test_abs_terms_brute_force(rope):
    # explicit loops: rotate each head's centre to each future position (textbook rotations), average or take
    # each logit's own absolute sum, add the absolute norm term with the group-mean coefficients
    d, G, theta = 8, 3, 100.0
    rot = _textbook_rope if rope == "half" else _textbook_rope_interleaved
    K = RNG.normal(size=(5, d))
    qbar, c = RNG.normal(size=(G, d)), RNG.normal(size=(G, d // 2))
    offs, t = (1, 3, 10), 20
    pa = [i for i in range(d // 2)] if rope == "half" else [2 * i for i in range(d // 2)]
    pb = [i + d // 2 for i in range(d // 2)] if rope == "half" else [2 * i + 1 for i in range(d // 2)]
    W = [rot(qbar[g], t + dl, theta) for g in range(G) for dl in offs]
    w = np.sum(W, axis=0) / len(W)
    chat = [sum(c[g][i] for g in range(G)) / G for i in range(d // 2)]
    A = O.abs_terms(K, qbar, c, theta, offs, t, rope)
    Av = O.abs_terms_variant(K, qbar, c, theta, offs, t, rope)
    for p in range(5):
        norm_abs = sum(abs(chat[i]) * math.hypot(K[p][pa[i]], K[p][pb[i]]) for i in range(d // 2))
        want = sum(abs(w[j] * K[p][j]) for j in range(d)) + norm_abs
        want_v = max(sum(abs(Wr[j] * K[p][j]) for j in range(d)) for Wr in W) + norm_abs
        assert abs(A[p] - want) < 1e-12 * want
        assert abs(Av[p] - want_v) < 1e-12 * want_v
