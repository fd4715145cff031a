"""GPU parity of decode attention over the kept cache (tri_decode_attention, through the C ABI) against the
float64 oracle.

Tolerance (derived): K, V and q are read exactly; a logit s = scale * q.K sums D float32 products, so its error
is at most gamma_D * scale * sum_j |q_j K_j| (gamma_D = D * 2^-24); exp and the running rescalings add a few
ulp.  A weight's relative error is then at most ds = max_p gamma_D * scale * sum_j |q_j K_pj| + 1e-6, and each
output element errs by at most 2 * ds * A_j with A_j = sum_p p_p |V_pj| (plus 1e-7 * max |V| for the final
float32 sums).  The tests assert exactly that bound.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import token_eviction_scoring_amd as T
from gpu_util import bits, params_for, say, tri_cache_of, unit_rows, unit_rows_after

pytestmark = pytest.mark.gpu
S = synth.scaled
C = synth.CONFIGS


def bound(qg, K, V, scale):
    """Per-element error bound of decode attention (see the module docstring); qg [G, d], K, V [L, d]."""
    d = K.shape[1]
    s = scale * (qg @ K.T)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    ds = (d * 2.0 ** -24) * scale * (np.abs(qg) @ np.abs(K).T).max(axis=1) + 1e-6     # [G]
    A = p @ np.abs(V)                                                                   # [G, d]
    return 2.0 * ds[:, None] * A + 1e-7 * np.abs(V).max()


def check_units(cfg, cache, q, out, lengths, units, scale, after=None):
    qh = q.cpu().double().numpy()
    oh = out.cpu().double().numpy()
    G = cfg.group
    worst = 0.0
    for (l, b, h) in units:
        L = int(lengths[b])
        rows = after(l, b, h, L) if after else unit_rows(cfg, cache, l, b, h, L)
        K, V = rows[0].double().numpy(), rows[1].double().numpy()
        got = oh[l, b, h * G:(h + 1) * G]
        if L == 0:
            assert np.all(got == 0.0)
            continue
        qg = qh[l, b, h * G:(h + 1) * G]
        ref = oracle.decode_attention(qg, K, V, scale)
        err = np.abs(got - ref)
        bd = bound(qg, K, V, scale)
        assert np.all(err <= bd), ((l, b, h), float((err / bd).max()))
        worst = max(worst, float((err / bd).max()))
    return worst


def run(cfg, lengths=None, max_length=None, units=None, gen_device="cpu"):
    cache = synth.make_cache(cfg, device=gen_device)
    cache = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in cache.items()}
    if lengths is not None:
        cache["lengths"] = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    lengths = cache["lengths"].cpu().numpy()
    q = synth.decode_queries(cfg, cache["t"]).cuda()
    tc = tri_cache_of(cfg, cache)
    scale = 1.0 / np.sqrt(cfg.d)
    out = T.tri_decode_attention(tc, cache["lengths"], q, scale, max_length=max_length)
    torch.cuda.synchronize()
    if units is None:
        units = [(l, b, h) for l in range(cfg.layers) for b in range(cfg.batch) for h in range(cfg.h_kv)]
    return check_units(cfg, cache, q, out, lengths, units, scale), cache, q, out


SPLITS = [0, 1, 2, 511, 512, 513, 1100, 2500]
CASES = {
    "bf16_g4": (S(C["qwen3_8b"], layers=2, batch=8, h_q=16, h_kv=4, max_len=2500, len_lo=2500, len_hi=2500,
                  name="dec1"), SPLITS),
    "f32_d64_g2": (S(C["tiny"], layers=1, batch=8, h_q=4, h_kv=2, max_len=2600, len_lo=2600, len_hi=2600, name="dec2"),
                   SPLITS),
    "bf16_g8": (S(C["qwen3_32b"], layers=1, batch=3, h_q=16, h_kv=2, max_len=1500, len_lo=1500, len_hi=1500,
                  outlier_frac=0.0, name="dec3"), [700, 1500, 3]),
    "bf16_g1": (S(C["qwen3_8b"], layers=1, batch=3, h_q=4, h_kv=4, max_len=1200, len_lo=1200, len_hi=1200,
                  name="dec4"), [1, 600, 1200]),
    "bf16_d64_g4": (S(C["qwen3_8b"], d=64, layers=1, batch=3, h_q=8, h_kv=2, max_len=1300, len_lo=1300, len_hi=1300,
                      name="dec5"), [13, 512, 1300]),
    "paged_kept": (S(C["paged_8b_kept"], layers=2, batch=4, max_len=4096, len_lo=1500, len_hi=4096, budget=1200,
                     recent=64, name="dec6"), None),
    "paged_g8": (S(C["paged_8b"], layers=1, batch=3, h_q=16, h_kv=2, max_len=2048, len_lo=300, len_hi=2048,
                   name="dec7"), None),
}


@pytest.mark.parametrize("name", list(CASES))
def test_decode_every_unit(name):
    cfg, lengths = CASES[name]
    worst, *_ = run(cfg, lengths)
    say(f"[{name}] worst error / bound = {worst:.3g}")


def test_decode_length_bound_and_determinism():
    cfg, lengths = CASES["bf16_g4"]
    w1, cache, q, out = run(cfg, lengths, max_length=2500)
    tc = tri_cache_of(cfg, cache)
    again = T.tri_decode_attention(tc, cache["lengths"], q, 1.0 / np.sqrt(cfg.d))
    assert np.array_equal(bits(out), bits(again))


def test_decode_after_the_pass():
    # evict on the GPU, then attend over the compacted paged cache through block_table_out and new_lengths;
    # the oracle evicts the same generated cache itself and attends over its own compacted rows
    cfg = S(C["paged_8b"], layers=2, batch=4, max_len=4096, len_lo=900, len_hi=4096, budget=700, recent=64,
            name="decpass")
    cache = synth.make_cache(cfg)
    host = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in cache.items()}
    cache = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in cache.items()}
    lengths = cache["lengths"].cpu().numpy()
    tc = tri_cache_of(cfg, cache)
    params, qbar, c = params_for(cfg, cache, "cuda")
    out = T.tri_evict_step(tc, params)
    torch.cuda.synchronize()
    kept = T.paged_cache(cache["k"], cache["v"], cache["pos"], out["block_table_out"], cfg.rope)
    q = synth.decode_queries(cfg, cache["t"]).cuda()
    scale = 1.0 / np.sqrt(cfg.d)
    att = T.tri_decode_attention(kept, out["new_lengths"], q, scale, max_length=cfg.budget)
    torch.cuda.synchronize()
    qh, ah = q.cpu().double().numpy(), att.cpu().double().numpy()
    G = cfg.group
    checked = 0
    for l in range(cfg.layers):
        for b in range(cfg.batch):
            for h in range(cfg.h_kv):
                K, V, P = unit_rows(cfg, host, l, b, h, int(lengths[b]))
                qg_c = oracle.group_rows(qbar[l].double().numpy(), h, G)
                cg = oracle.group_rows(c[l].double().numpy(), h, G)
                ev = oracle.evict_unit(K.double().numpy(), V.double().numpy(), P.numpy(), qg_c, cg, cfg.theta,
                                       cfg.offsets, int(host["t"][b]), cfg.budget, cfg.recent, cfg.rope)
                kg, vg, _ = unit_rows_after(cfg, cache, out, l, b, h, ev["new_len"])
                if not np.array_equal(kg.double().numpy(), ev["k"]):
                    continue   # a boundary key differs (allowed by the pass's tolerance): nothing to compare
                qg = qh[l, b, h * G:(h + 1) * G]
                ref = oracle.decode_attention(qg, ev["k"], ev["v"], scale)
                bd = bound(qg, ev["k"], ev["v"], scale)
                assert np.all(np.abs(ah[l, b, h * G:(h + 1) * G] - ref) <= bd), (l, b, h)
                checked += 1
    assert checked >= 0.95 * cfg.layers * cfg.batch * cfg.h_kv
    say(f"[decode after the pass] {checked} units checked")


def test_decode_full_size_sampled():
    # the Qwen3-8B-shape paged cache as the pass leaves it: 36 layers x 64 sequences x 8 KV heads x 2048 slots
    cfg = C["paged_8b_kept"]
    rng = np.random.default_rng(5)
    units = sorted({(0, 0, 0), (cfg.layers - 1, cfg.batch - 1, cfg.h_kv - 1)} |
                   {(int(rng.integers(cfg.layers)), int(rng.integers(cfg.batch)), int(rng.integers(cfg.h_kv)))
                    for _ in range(6)})
    say("[decode full size] generating on the GPU")
    worst, *_ = run(cfg, units=units, max_length=cfg.budget, gen_device="cuda")
    say(f"[decode full size] {len(units)} units, worst error / bound = {worst:.3g}")


def test_decode_full_size_every_unit():
    # Every (layer, sequence, KV head) and query head of the full-size paged cache, against the definition
    # evaluated in float64 on the GPU with torch (no oracle), to the same bound as the sampled test.
    cfg = C["paged_8b_kept"]
    torch.cuda.empty_cache()
    say("[decode full size, every unit] generating on the GPU")
    cache = synth.make_cache(cfg, device="cuda")
    q = synth.decode_queries(cfg, cache["t"]).cuda()
    tc = tri_cache_of(cfg, cache)
    scale = 1.0 / np.sqrt(cfg.d)
    out = T.tri_decode_attention(tc, cache["lengths"], q, scale, max_length=cfg.budget)
    torch.cuda.synchronize()
    G, H, bs = cfg.group, cfg.h_kv, cfg.block_size
    worst = 0.0
    for b, L in enumerate(cache["lengths"].cpu().tolist()):
        blocks = cache["block_table"][b, :(L + bs - 1) // bs].long()
        def rows(pool):   # [layers, blocks, bs, H, d] -> [layers, H, L, d], float64
            x = pool[:, blocks].reshape(cfg.layers, -1, H, cfg.d)[:, :L]
            return x.permute(0, 2, 1, 3).double().contiguous()
        K, V = rows(cache["k"]), rows(cache["v"])
        qb = q[:, b].double().reshape(cfg.layers, H, G, cfg.d)
        s = scale * torch.matmul(qb, K.transpose(-1, -2).contiguous())
        p = torch.softmax(s, dim=-1)
        ref = torch.matmul(p, V)
        ds = (cfg.d * 2.0 ** -24) * scale * torch.matmul(qb.abs(), K.abs().transpose(-1, -2).contiguous()).amax(-1) + 1e-6
        bnd = 2.0 * ds.unsqueeze(-1) * torch.matmul(p, V.abs()) + 1e-7 * V.abs().amax(dim=(-2, -1), keepdim=True)
        err = (out[:, b].double().reshape(cfg.layers, H, G, cfg.d) - ref).abs()
        assert bool((err <= bnd).all()), (b, float((err / bnd).max()))
        worst = max(worst, float((err / bnd).max()))
    say(f"[decode full size, every unit] {cfg.layers * cfg.batch * H} units, worst error / bound = {worst:.3g}")
