"""GPU parity of the calibration statistics pass (tri_calibrate, through the C ABI) against the float64 oracle.

Tolerance (derived): the stored queries widen exactly; element sums run in float64 (relative error ~n * 2^-53),
pair norms in float32 (~1.5 ulp each), and the outputs round once to float32 (2^-24).  Both stay far below
    |qbar_gpu - qbar_ref|_j <= 1e-6 * mean_n |q_j|
    |c_gpu - c_ref|_i       <= 1e-6 * (mean_n |z_i(q)| + |z_i(qbar)|)
which the tests assert.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import token_eviction_scoring_amd as T
from gpu_util import say

pytestmark = pytest.mark.gpu
TOL = 1e-6


def check(q_host, rope, qbar, c, pairs=None):
    """q_host [layers, n, heads, d] (CPU); qbar, c GPU outputs; pairs: (layer, head) to check (default all)."""
    L, n, H, d = q_host.shape
    qbar, c = qbar.cpu().double().numpy(), c.cpu().double().numpy()
    worst = 0.0
    for (l, h) in pairs or [(l, h) for l in range(L) for h in range(H)]:
        Q = q_host[l, :, h].double().numpy()
        ref_q, ref_c = oracle.calibration_stats(Q, rope)
        aq = np.abs(Q).mean(axis=0)
        ac = np.abs(oracle.to_pairs(Q, rope)).mean(axis=0) + np.abs(oracle.to_pairs(ref_q, rope))
        eq, ec = np.abs(qbar[l, h] - ref_q), np.abs(c[l, h] - ref_c)
        assert np.all(eq <= TOL * aq), (l, h, float((eq / aq).max()))
        assert np.all(ec <= TOL * ac), (l, h, float((ec / ac).max()))
        worst = max(worst, float((eq / aq).max()), float((ec / ac).max()))
    return worst


CASES = {
    "bf16_d128_half": (synth.scaled(synth.CONFIGS["qwen3_8b"], layers=2, h_q=4, h_kv=1, name="cal1"), 3000, "half"),
    "f32_d64_interleaved": (synth.scaled(synth.CONFIGS["tiny"], layers=2, h_q=3, h_kv=1, rope="interleaved",
                                         name="cal2"), 1500, "interleaved"),
    "bf16_d64_one_chunk": (synth.scaled(synth.CONFIGS["qwen3_8b"], d=64, layers=1, h_q=8, h_kv=2, name="cal3"), 1024,
                           "half"),
    "f32_d128_few": (synth.scaled(synth.CONFIGS["tiny"], d=128, layers=1, h_q=2, h_kv=1, name="cal4"), 5, "half"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_calibration_every_head(name):
    cfg, n, rope = CASES[name]
    q = synth.calibration_queries(cfg, n)
    qbar, c = T.tri_calibrate(q.cuda(), rope)
    torch.cuda.synchronize()
    say(f"[{name}] worst error / bound scale = {check(q, rope, qbar, c):.3g}")


def test_single_query_has_no_missed_mass():
    cfg = synth.scaled(synth.CONFIGS["qwen3_8b"], layers=1, h_q=2, h_kv=1, name="cal5")
    q = synth.calibration_queries(cfg, 1).cuda()
    qbar, c = T.tri_calibrate(q)
    assert torch.equal(qbar, q[:, 0].float())
    assert bool((c.abs() <= 1e-6 * q[:, 0].float().abs().max()).all())


def test_strided_queries_and_determinism():
    # the same queries stored [n, layers, heads, d] (a strided view) give bitwise the same statistics
    cfg, n, rope = CASES["bf16_d128_half"]
    q = synth.calibration_queries(cfg, n).cuda()
    tm = q.permute(1, 0, 2, 3).contiguous().permute(1, 0, 2, 3)
    a = T.tri_calibrate(q, rope)
    b = T.tri_calibrate(tm, rope)
    c2 = T.tri_calibrate(q, rope)
    for x, y, z in zip(a, b, c2):
        assert torch.equal(x, y) and torch.equal(x, z)


def test_calibration_feeds_the_centres():
    # tri_calibrate -> tri_prepare_centres gives the u and c_hat of the oracle's statistics
    cfg, n, rope = CASES["bf16_d128_half"]
    cfg = synth.scaled(cfg, h_q=8, h_kv=2)
    q = synth.calibration_queries(cfg, n)
    qbar, c = T.tri_calibrate(q.cuda(), rope)
    u, c_hat = T.tri_prepare_centres(qbar, c, cfg.h_kv, cfg.theta, cfg.offsets, rope)
    u, c_hat = u.cpu().double().numpy(), c_hat.cpu().double().numpy()
    G = cfg.group
    for l in range(cfg.layers):
        stats = [oracle.calibration_stats(q[l, :, hq].double().numpy(), rope) for hq in range(cfg.h_q)]
        for h in range(cfg.h_kv):
            qg = np.stack([stats[hq][0] for hq in range(h * G, (h + 1) * G)])
            ref_u = oracle.centre_vector(qg, cfg.theta, cfg.offsets, rope)
            ref_c = np.mean([stats[hq][1] for hq in range(h * G, (h + 1) * G)], axis=0)
            assert np.allclose(u[l, h], ref_u, rtol=0, atol=2e-6 * np.abs(ref_u).max())
            assert np.allclose(c_hat[l, h], ref_c, rtol=0, atol=2e-6 * np.abs(ref_c).max())


def test_full_size_sampled():
    # Qwen3-8B shape: 36 layers x 32 query heads, 32768 calibration tokens (9.7 GB of bf16 queries)
    cfg = synth.CONFIGS["qwen3_8b"]
    n = 32768
    say("[calibration full size] generating on the GPU")
    q = synth.calibration_queries(cfg, n, device="cuda")
    qbar, c = T.tri_calibrate(q, cfg.rope)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    pairs = sorted({(0, 0), (cfg.layers - 1, cfg.h_q - 1)} |
                   {(int(rng.integers(cfg.layers)), int(rng.integers(cfg.h_q))) for _ in range(6)})
    host = {}
    for (l, h) in pairs:
        host[(l, h)] = q[l, :, h].cpu()
    del q
    torch.cuda.empty_cache()
    qb, cc = qbar.cpu().double().numpy(), c.cpu().double().numpy()
    worst = 0.0
    for (l, h) in pairs:
        Q = host[(l, h)].double().numpy()
        ref_q, ref_c = oracle.calibration_stats(Q, cfg.rope)
        aq = np.abs(Q).mean(axis=0)
        ac = np.abs(oracle.to_pairs(Q, cfg.rope)).mean(axis=0) + np.abs(oracle.to_pairs(ref_q, cfg.rope))
        assert np.all(np.abs(qb[l, h] - ref_q) <= TOL * aq), (l, h)
        assert np.all(np.abs(cc[l, h] - ref_c) <= TOL * ac), (l, h)
        worst = max(worst, float((np.abs(qb[l, h] - ref_q) / aq).max()), float((np.abs(cc[l, h] - ref_c) / ac).max()))
    say(f"[calibration full size] {len(pairs)} heads, worst error / bound scale = {worst:.3g}")


def test_full_size_every_head():
    # every (layer, query head) of the full-size pass against the definition evaluated in float64 on the GPU with
    # torch (no oracle): qbar = mean of the queries, c = mean |z_i(q)| - |z_i(qbar)|, to the same bounds
    cfg = synth.CONFIGS["qwen3_8b"]
    torch.cuda.empty_cache()
    say("[calibration full size, every head] generating on the GPU")
    q = synth.calibration_queries(cfg, 32768, device="cuda")
    qbar, c = T.tri_calibrate(q, cfg.rope)
    torch.cuda.synchronize()
    half = cfg.d // 2

    def pair_norm(x):   # [..., d] -> [..., d/2]
        a, b = (x[..., :half], x[..., half:]) if cfg.rope == "half" else (x[..., 0::2], x[..., 1::2])
        return torch.sqrt(a * a + b * b)

    worst = 0.0
    for l in range(cfg.layers):
        Q = q[l].double()                                   # [n, heads, d]
        ref_q = Q.mean(dim=0)
        ref_c = pair_norm(Q).mean(dim=0) - pair_norm(ref_q)
        aq = Q.abs().mean(dim=0)
        ac = pair_norm(Q).mean(dim=0) + pair_norm(ref_q)
        eq, ec = (qbar[l].double() - ref_q).abs(), (c[l].double() - ref_c).abs()
        assert bool((eq <= TOL * aq).all()), (l, float((eq / aq).max()))
        assert bool((ec <= TOL * ac).all()), (l, float((ec / ac).max()))
        worst = max(worst, float((eq / aq).max()), float((ec / ac).max()))
    say(f"[calibration full size, every head] {cfg.layers * cfg.h_q} heads, worst error / bound scale = {worst:.3g}")
