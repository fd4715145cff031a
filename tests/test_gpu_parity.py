"""GPU parity: the HIP pass (through the C ABI) against the float64 CPU oracle, unit by unit.

Small cases run every unit through the oracle and span several scoring tiles (1024 rows),
several compaction chunks (128 rows) and ragged tails; the full-size workloads check a
deterministic sample of units.  Comparison rules are in gpu_util.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import token_eviction_scoring_amd as T
from gpu_util import (bits, run_and_check, sampled_units, say, tri_cache_of, params_for, unit_rows)

pytestmark = pytest.mark.gpu
C = synth.CONFIGS
S = synth.scaled


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _report(name, stats):
    worst = max(s["worst_rel_A"] for s in stats)
    rel = max(s["worst_rel"] for s in stats)
    say(f"[{name}] units={len(stats)} worst |ds|/A={worst:.3g} worst |ds|/|s| (|s| >= 0.1 A)={rel:.3g} "
        f"boundary={sum(s['boundary'] for s in stats)}")


# ----------------------------------------------------------------------------- centre vectors

@pytest.mark.parametrize("name", ["tiny", "qwen3_8b", "qwen3_32b"])
@pytest.mark.parametrize("rope", ["half", "interleaved"])
def test_prepare_centres(name, rope):
    cfg = S(C[name], rope=rope, layers=min(C[name].layers, 3))
    qbar, c = synth.query_side(cfg)
    u, c_hat = T.tri_prepare_centres(qbar.cuda(), c.cuda(), cfg.h_kv, cfg.theta, cfg.offsets, rope)
    u, c_hat = u.cpu().double().numpy(), c_hat.cpu().double().numpy()
    for l in range(cfg.layers):
        for h in range(cfg.h_kv):
            qg = oracle.group_rows(qbar[l].double().numpy(), h, cfg.group)
            ref = oracle.centre_vector(qg, cfg.theta, cfg.offsets, rope)
            assert np.allclose(u[l, h], ref, rtol=0, atol=2e-7 * np.abs(ref).max())
            cref = oracle.group_rows(c[l].double().numpy(), h, cfg.group).mean(0)
            assert np.allclose(c_hat[l, h], cref, rtol=0, atol=2e-7 * np.abs(cref).max())


# ----------------------------------------------------------------------------- whole pass, small sizes, every unit

SMALL = {
    "tiny": C["tiny"],
    "tiny_interleaved": S(C["tiny"], rope="interleaved", name="tiny_il"),
    "tiny_f32_d128": S(C["tiny"], d=128, h_q=8, h_kv=2, max_len=2500, len_lo=2500, len_hi=2500, name="tiny128"),
    "bf16_d64": S(C["qwen3_8b"], d=64, layers=2, max_len=3000, len_lo=3000, len_hi=3000, budget=300, recent=40,
                  name="bf16d64"),
    "8b_small": S(C["qwen3_8b"], layers=2, batch=2, max_len=5000, len_lo=1500, len_hi=5000, budget=700, recent=64,
                  name="8bsmall"),
    "ragged_small": S(C["ragged_8b"], layers=2, batch=5, max_len=4100, len_lo=200, len_hi=4100, budget=512,
                      recent=128, name="raggedsmall"),
    "32b_small": S(C["qwen3_32b"], layers=2, batch=2, max_len=6000, len_lo=6000, len_hi=6000, budget=900, recent=256,
                   name="32bsmall"),
    "paged_small": S(C["paged_8b"], layers=2, batch=6, max_len=4096, len_lo=100, len_hi=4096, budget=700, recent=128,
                     name="pagedsmall"),
    "paged_interleaved": S(C["paged_8b"], layers=1, batch=3, max_len=2048, len_lo=500, len_hi=2048, budget=300,
                           recent=16, rope="interleaved", name="pagedil"),
    "paged_h4_d64": S(C["paged_8b"], layers=2, batch=3, h_q=16, h_kv=4, d=64, max_len=3000, len_lo=700, len_hi=3000,
                      budget=400, recent=32, name="pagedh4"),
    "paged_f32_h2": S(C["paged_8b"], dtype="f32", layers=1, batch=3, h_q=8, h_kv=2, max_len=2500, len_lo=900,
                      len_hi=2500, budget=300, recent=40, name="pagedf32h2"),
    "paged_f32_h8": S(C["paged_8b"], dtype="f32", layers=1, batch=2, max_len=2100, len_lo=1500, len_hi=2100,
                      budget=500, recent=64, name="pagedf32h8"),
    "paged_h1": S(C["paged_8b"], layers=1, batch=3, h_q=4, h_kv=1, max_len=3000, len_lo=1100, len_hi=3000,
                  budget=333, recent=3, name="pagedh1"),
    "paged_bs8": S(C["paged_8b"], block_size=8, layers=1, batch=3, max_len=2000, len_lo=500, len_hi=2000, budget=400,
                   recent=24, name="pagedbs8"),
    "paged_bs32": S(C["paged_8b"], block_size=32, layers=1, batch=3, max_len=3000, len_lo=900, len_hi=3000,
                    budget=333, recent=40, name="pagedbs32"),
    "paged_bs12": S(C["paged_8b"], block_size=12, layers=1, batch=3, max_len=2400, len_lo=700, len_hi=2400,
                    budget=300, recent=7, name="pagedbs12"),
    "paged_steady": S(C["paged_8b_steady"], layers=2, batch=4, max_len=8192, len_lo=2000, len_hi=8192, budget=1100,
                      recent=64, steady=96, name="pagedsteady"),
    # >= 1024 units: the unfused pass selects and compacts each unit in one workgroup; 135 (layer, sequence) pairs,
    # not a multiple of the 8 XCDs the paged moves group heads by, so that mapping's padding workgroups run too
    "paged_many_units": S(C["paged_8b"], layers=9, batch=15, max_len=1200, len_lo=300, len_hi=1200, budget=256,
                          recent=32, name="pagedmany"),
    "contiguous_steady": S(C["qwen3_8b_steady"], layers=2, batch=3, max_len=4096, len_lo=1700, len_hi=4096,
                           budget=1500, recent=128, steady=128, name="contigsteady"),
}


# caches of at most T.FUSED_MAX_LEN slots can run the fused single-kernel pass; the small cases have too few
# units for it to be the default, so both paths are forced
PATHS = {"fused": T.PASS_FUSED, "unfused": T.PASS_UNFUSED}


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("name", list(SMALL))
def test_pass_every_unit(name, path):
    cfg = SMALL[name]
    _, _, stats = run_and_check(cfg, flags=PATHS[path])
    _report(f"{name}/{path}", stats)


def _random_shape(i):
    """Seeded random small shape i: layout, storage type, head size, pairing, query heads per KV head, block size,
    lengths, budget, recent window and offset count all drawn, so that combinations no hand-picked case names are
    checked too."""
    rng = np.random.default_rng(1000 + i)
    layout = "paged" if i % 2 else "contiguous"
    h_kv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4]))
    max_len = int(rng.integers(200, 4500))
    len_lo = int(rng.integers(0, max_len + 1))
    budget = int(rng.integers(1, max_len + 200))
    recent = int(rng.integers(0, budget + 1)) if rng.random() < 0.8 else budget
    return S(C["paged_8b" if layout == "paged" else "ragged_8b"], name=f"rand{i}", seed=500 + i,
             layers=int(rng.integers(1, 4)), batch=int(rng.integers(1, 6)), h_q=h_kv * g, h_kv=h_kv,
             d=int(rng.choice([64, 128])), dtype=str(rng.choice(["bf16", "f32"])),
             rope=str(rng.choice(["half", "interleaved"])), block_size=int(rng.choice([8, 12, 16, 32])),
             max_len=max_len, len_lo=len_lo, len_hi=max_len, budget=budget, recent=recent,
             offsets=tuple(2 ** k for k in range(int(rng.integers(1, 14)))),
             centre=str(rng.choice(["normal", "lognormal"])), noise=float(rng.uniform(0.1, 0.6)))


@pytest.mark.parametrize("i", range(16))
def test_random_shapes_every_unit(i):
    # every unit of a seeded random shape through the oracle, on the fused path (when the cache fits it) and the
    # three-kernel path
    cfg = _random_shape(i)
    paths = ("unfused", "fused") if cfg.max_len <= T.FUSED_MAX_LEN else ("unfused",)
    for path in paths:
        _, _, stats = run_and_check(cfg, flags=PATHS[path])
        _report(f"{cfg.name}/{path} {cfg.layout} {cfg.dtype} d{cfg.d} {cfg.rope} G{cfg.group} H{cfg.h_kv} "
                f"B{cfg.budget} R{cfg.recent} bs{cfg.block_size} len{cfg.len_lo}-{cfg.len_hi}", stats)


@pytest.mark.parametrize("name", ["paged_small", "ragged_small", "paged_steady"])
def test_checked_pass_matches_unchecked(name):
    # tri_params.check on valid inputs: the word stays 0 and the pass is bitwise the unchecked one (scores, keep
    # lists, new lengths, compacted rows, paged tables); the composed calls check too.  Bad inputs are exercised on
    # the host only (tests/sanitize/checks_host.cpp): the GPU never sees a bad block id or length.
    cfg = SMALL[name]
    outs = []
    for checked in (False, True):
        for composed in (False, True):
            cache = synth.make_cache(cfg)
            cache = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in cache.items()}
            tc = tri_cache_of(cfg, cache)
            params, _, _ = params_for(cfg, cache, "cuda", flags=T.PASS_UNFUSED)
            word = torch.full((1,), -1, dtype=torch.int32, device="cuda")
            if checked:
                params.check = word
            stride = T.tri_score_stride(tc)
            scores = torch.zeros(cfg.layers, cfg.batch, cfg.h_kv, stride, device="cuda")
            keep = torch.zeros(cfg.layers, cfg.batch, cfg.h_kv, cfg.budget, dtype=torch.int32, device="cuda")
            if composed:
                T.tri_score(tc, params, scores)
                _, new_lengths = T.tri_topk(tc, params, scores, keep)
                out = T.tri_compact(tc, params, keep)
                out["new_lengths"] = new_lengths
            else:
                out = T.tri_evict_step(tc, params, scores=scores, keep=keep)
            torch.cuda.synchronize()
            if checked:
                assert int(word.cpu()[0]) == 0, (name, composed, int(word.cpu()[0]))
            lengths = cache["lengths"].cpu().tolist()
            got = [out["new_lengths"].cpu().numpy(), bits(cache["k"]), bits(cache["v"]), cache["pos"].cpu().numpy()]
            for b, L in enumerate(lengths):
                got += [bits(scores[:, b, :, :L]), keep[:, b, :, :min(L, cfg.budget)].cpu().numpy()]
            if cfg.layout == "paged":
                nf = int(out["n_freed"].cpu()[0])
                bto = out["block_table_out"].cpu().numpy()
                got += [np.array([nf]), out["freed"][:nf].cpu().numpy()]
                got += [bto[b, :-(-min(L, cfg.budget) // cfg.block_size)] for b, L in enumerate(lengths)]
            outs.append(got)
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            assert np.array_equal(a, b), name


def test_composed_calls_equal_evict_step():
    cfg = SMALL["paged_small"]
    ca, oa, _ = run_and_check(cfg)
    cb, ob, _ = run_and_check(cfg, composed=True)
    assert torch.equal(ca["k"].view(torch.int16), cb["k"].view(torch.int16))
    assert torch.equal(ca["v"].view(torch.int16), cb["v"].view(torch.int16))
    assert torch.equal(ca["pos"], cb["pos"])
    for key in ("block_table_out", "freed", "n_freed", "new_lengths"):
        assert torch.equal(oa[key], ob[key]), key


# ----------------------------------------------------------------------------- edge cases

@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("budget,recent", [(1, 0), (1, 1), (64, 0), (64, 64), (257, 129), (5000, 10)])
def test_budget_edges(budget, recent, path):
    cfg = S(C["qwen3_8b"], layers=1, batch=3, max_len=3000, len_lo=600, len_hi=3000, budget=budget, recent=recent,
            name="edges")
    _, _, stats = run_and_check(cfg, flags=PATHS[path])
    _report(f"budget{budget}/recent{recent}", stats)


def test_budget_beyond_the_in_lds_keep_list():
    # budgets above 8192 slots: the selection kernel no longer holds the keep list in LDS, so the pass selects and
    # compacts in separate kernels; every unit against the oracle, contiguous and paged
    for base, name in ((C["qwen3_8b"], "bigbudget"), (C["paged_8b"], "bigbudgetpaged")):
        cfg = S(base, layers=1, batch=2, h_q=8, h_kv=2, max_len=12000, len_lo=9000, len_hi=12000, budget=8500,
                recent=300, name=name)
        _, _, stats = run_and_check(cfg)
        _report(name, stats)


@pytest.mark.parametrize("path", list(PATHS))
def test_empty_and_tiny_lengths(path):
    cfg = S(C["ragged_8b"], layers=2, batch=6, h_kv=2, h_q=8, max_len=2100, len_lo=2100, len_hi=2100, budget=100,
            recent=20, name="emptylens")
    run_and_check(cfg, lengths_override=[0, 1, 99, 100, 101, 2100], flags=PATHS[path])
    pcfg = S(C["paged_8b"], layers=1, batch=5, max_len=1024, len_lo=1024, len_hi=1024, budget=100, recent=20,
             name="emptypaged")
    run_and_check(pcfg, lengths_override=[0, 15, 16, 17, 1000], flags=PATHS[path])


@pytest.mark.parametrize("path", list(PATHS))
def test_exact_ties_keep_lower_slot(path):
    cfg = S(C["qwen3_8b"], layers=1, batch=1, h_kv=2, h_q=8, max_len=4000, len_lo=4000, len_hi=4000, budget=500,
            recent=32, name="ties")

    def dup(cache):
        k = cache["k"]
        src = torch.arange(0, 1500, 3, device=k.device)
        k[:, :, :, src + 2000] = k[:, :, :, src]          # identical rows score bitwise equal
        k[:, :, :, 3000:3100] = k[:, :, :, 100:101]       # a block of 100 equal rows
    _, _, stats = run_and_check(cfg, mutate=dup, flags=PATHS[path])
    _report(f"ties/{path}", stats)


@pytest.mark.parametrize("path", list(PATHS))
def test_all_equal_scores(path):
    # zero query centres and zero norm weights: every score is 0, so the first budget-recent slots win
    cfg = S(C["qwen3_8b"], layers=1, batch=2, max_len=3000, len_lo=3000, len_hi=3000, budget=300, recent=30, name="eq")
    cache = synth.make_cache(cfg, device="cuda")
    tc = tri_cache_of(cfg, cache)
    params, _, _ = params_for(cfg, cache, "cuda", flags=PATHS[path])
    params.u.zero_()
    params.c_hat.zero_()
    out = T.tri_evict_step(tc, params, keep=torch.empty(1, 2, 8, 300, dtype=torch.int32, device="cuda"))
    keep = out["keep"].cpu().numpy()
    want = list(range(270)) + list(range(2970, 3000))
    assert all(keep[0, b, h].tolist() == want for b in range(2) for h in range(8))


def test_token_major_strides():
    # the same cache stored [layers, batch, slot, head, d]: results must match the head-major run
    cfg = S(C["qwen3_8b"], layers=2, batch=2, max_len=2500, len_lo=1000, len_hi=2500, budget=400, recent=50,
            name="tokenmajor")
    hm = synth.make_cache(cfg, device="cuda")
    tm = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in hm.items()}
    tm["k"] = hm["k"].permute(0, 1, 3, 2, 4).contiguous().permute(0, 1, 3, 2, 4)
    tm["v"] = hm["v"].permute(0, 1, 3, 2, 4).contiguous().permute(0, 1, 3, 2, 4)
    tm["pos"] = hm["pos"].clone()
    outs = []
    for cache in (hm, tm):
        tc = tri_cache_of(cfg, cache)
        params, _, _ = params_for(cfg, cache, "cuda")
        outs.append(T.tri_evict_step(tc, params, scores=torch.empty(2, 2, 8, T.tri_score_stride(tc), device="cuda"),
                                     keep=torch.empty(2, 2, 8, 400, dtype=torch.int32, device="cuda")))
    torch.cuda.synchronize()
    L = hm["lengths"].cpu()
    for b in range(2):
        assert torch.equal(outs[0]["scores"][:, b, :, :L[b]], outs[1]["scores"][:, b, :, :L[b]])
        assert torch.equal(outs[0]["keep"][:, b], outs[1]["keep"][:, b])
        n = min(int(L[b]), 400)
        assert torch.equal(hm["k"][:, b, :, :n].view(torch.int16), tm["k"][:, b, :, :n].view(torch.int16))
        assert torch.equal(hm["v"][:, b, :, :n].view(torch.int16), tm["v"][:, b, :, :n].view(torch.int16))


def test_deterministic_and_idempotent():
    cfg = S(C["ragged_8b"], layers=2, batch=3, max_len=3000, len_lo=1000, len_hi=3000, budget=300, recent=30,
            name="determinism")
    cache = synth.make_cache(cfg, device="cuda")
    tc = tri_cache_of(cfg, cache)
    params, _, _ = params_for(cfg, cache, "cuda")
    s1 = T.tri_score(tc, params)
    s2 = T.tri_score(tc, params)
    L = cache["lengths"].cpu()
    for b in range(3):
        assert torch.equal(s1[:, b, :, :L[b]].view(torch.int32), s2[:, b, :, :L[b]].view(torch.int32))
    out = T.tri_evict_step(tc, params)
    torch.cuda.synchronize()
    k_after = cache["k"].clone()
    # second pass at the same decode positions over the compacted cache keeps everything in place
    params2 = T.Params(params.u, params.c_hat, params.theta, out["new_lengths"], params.t, params.budget, params.recent)
    out2 = T.tri_evict_step(tc, params2, keep=torch.empty(2, 3, 8, 300, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(out2["new_lengths"], out["new_lengths"])
    for b in range(3):
        n = int(out["new_lengths"][b])
        assert out2["keep"][:, b, :, :n].cpu().eq(torch.arange(n, dtype=torch.int32)).all()
        assert torch.equal(cache["k"][:, b, :, :n].view(torch.int16), k_after[:, b, :, :n].view(torch.int16))


@pytest.mark.parametrize("pattern", ["first", "last", "every3", "random", "runs"])
@pytest.mark.parametrize("layout", ["contiguous", "paged"])
def test_compaction_adversarial_keep_lists(pattern, layout):
    # tri_compact with hand-made ascending keep lists: in-place moves must equal an out-of-place gather
    base = C["paged_8b"] if layout == "paged" else C["qwen3_8b"]
    cfg = S(base, layers=2, batch=2, max_len=6000, len_lo=6000, len_hi=6000, budget=2000, recent=0, name="adv" + layout)
    cache = synth.make_cache(cfg, device="cuda")
    L, B = 6000, 2000
    rng = np.random.default_rng(7)
    keep = np.zeros((cfg.layers, cfg.batch, cfg.h_kv, B), dtype=np.int32)
    for idx in np.ndindex(cfg.layers, cfg.batch, cfg.h_kv):
        if pattern == "first":
            k = np.arange(B)
        elif pattern == "last":
            k = np.arange(L - B, L)
        elif pattern == "every3":
            k = np.sort(np.concatenate([np.arange(0, L - 100, 3)[:B - 100], np.arange(L - 100, L)]))
        elif pattern == "random":
            k = np.sort(rng.choice(L, size=B, replace=False))
        else:
            starts = np.sort(rng.choice(L // 50, size=B // 50, replace=False)) * 50
            k = (starts[:, None] + np.arange(50)).ravel()
        keep[idx] = k
    units = [(l, b, h) for l in range(cfg.layers) for b in range(cfg.batch) for h in range(cfg.h_kv)]
    inputs = {u: unit_rows(cfg, cache, *u, L) for u in units}
    tc = tri_cache_of(cfg, cache)
    params, _, _ = params_for(cfg, cache, "cuda")
    out = T.tri_compact(tc, params, torch.from_numpy(keep).cuda())
    torch.cuda.synchronize()
    from gpu_util import unit_rows_after
    for u in units:
        k_in, v_in, p_in = inputs[u]
        k_out, v_out, p_out = unit_rows_after(cfg, cache, out, *u, B)
        kk = keep[u]
        assert np.array_equal(bits(k_out), bits(k_in)[kk]), u
        assert np.array_equal(bits(v_out), bits(v_in)[kk]), u
        assert np.array_equal(p_out.numpy(), p_in.numpy()[kk]), u


# ----------------------------------------------------------------------------- aggregation variants (matrix cores)

VARIANTS = {
    "max_8b": S(C["qwen3_8b_max"], layers=2, batch=2, max_len=3000, len_lo=1500, len_hi=3000, budget=500, recent=32,
                name="varmax"),
    "headmax_8b": S(C["qwen3_8b_headmax"], layers=2, batch=2, max_len=3000, len_lo=1500, len_hi=3000, budget=500,
                    recent=32, name="varhm"),
    "headmax_paged": S(C["paged_8b"], aggregation="head_max", layers=1, batch=4, max_len=2048, len_lo=300,
                       len_hi=2048, budget=400, recent=16, name="varpaged"),
    "max_interleaved_d64_g2": S(C["qwen3_8b"], aggregation="max", rope="interleaved", d=64, h_q=8, h_kv=4,
                                offsets=(1, 2, 4, 8, 16, 32, 64, 128, 256), layers=1, batch=3, max_len=2100,
                                len_lo=900, len_hi=2100, budget=300, recent=20, name="varil"),
    "headmax_g1": S(C["qwen3_8b"], aggregation="head_max", h_q=8, h_kv=8, layers=1, batch=2, max_len=1500,
                    len_lo=1500, len_hi=1500, budget=200, recent=10, name="varg1"),
    # more score tiles than one workgroup walks (20 of 1024 rows, so a unit is spread over several workgroups, each
    # taking every few-th tile) with ragged lengths: workgroups of one unit walk different numbers of tiles
    # paged pools: blocks of 12 (not a multiple of 16: 16-byte fragments per key) and of 32 (whole-row loads)
    "max_paged_bs12": S(C["paged_8b"], aggregation="max", h_q=8, h_kv=2, layers=1, batch=3, max_len=2400,
                        len_lo=700, len_hi=2400, budget=400, recent=16, block_size=12, name="varpg12"),
    "headmax_paged_bs32": S(C["paged_8b"], aggregation="head_max", h_q=8, h_kv=2, layers=2, batch=3, max_len=3200,
                            len_lo=900, len_hi=3200, budget=500, recent=16, block_size=32, name="varpg32"),
    "max_ragged_many_tiles": S(C["qwen3_8b_max"], h_q=8, h_kv=2, layers=1, batch=3, max_len=20000, len_lo=4100,
                               len_hi=20000, budget=700, recent=64, name="varmany"),
    # eight query heads per KV head (the Qwen3-32B shape): 128 columns, the last 64 from LDS
    "max_g8": S(C["qwen3_32b"], aggregation="max", layers=2, batch=2, max_len=3000, len_lo=1500, len_hi=3000,
                budget=500, recent=32, name="varg8"),
    "headmax_g8_paged": S(C["paged_8b"], aggregation="head_max", h_q=64, layers=1, batch=3, max_len=2500, len_lo=600,
                          len_hi=2500, budget=400, recent=16, name="varg8paged"),
    "headmax_g8_interleaved_d64": S(C["qwen3_32b"], aggregation="head_max", rope="interleaved", d=64, h_q=16, h_kv=2,
                                    layers=1, batch=2, max_len=2200, len_lo=1000, len_hi=2200, budget=300, recent=20,
                                    name="varg8il"),
    # more than 16 offsets: blocks of 32 columns per query head (4 heads x 32 = 128 columns; 2 heads x 32 = 64)
    "headmax_32_offsets_g4": S(C["qwen3_8b"], aggregation="head_max", h_q=16, h_kv=4, layers=1, batch=2,
                               offsets=tuple(range(1, 25)) + tuple(2 ** k for k in range(5, 13)), max_len=2100,
                               len_lo=900, len_hi=2100, budget=300, recent=16, name="var32off"),
    "max_20_offsets_g2_paged": S(C["paged_8b"], aggregation="max", h_q=8, h_kv=4, layers=1, batch=3,
                                 offsets=tuple(range(0, 40, 2)), max_len=2000, len_lo=500, len_hi=2000, budget=250,
                                 recent=8, name="var20off"),
}


@pytest.mark.parametrize("name", list(VARIANTS))
def test_variant_every_unit(name):
    _, _, stats = run_and_check(VARIANTS[name])
    _report(name, stats)


def test_variant_empty_and_tiny_lengths():
    # lengths of 0, below one 16-key step, one step, one step + 1 and ragged multi-tile lengths: steps past the end
    # re-read the last key and must leave only that key's own score behind
    cfg = S(C["qwen3_8b_max"], layers=1, batch=7, h_kv=2, h_q=8, max_len=2100, len_lo=2100, len_hi=2100, budget=12,
            recent=4, name="varempty")
    run_and_check(cfg, lengths_override=[0, 1, 5, 16, 17, 1025, 2100])
    pcfg = S(C["paged_8b"], aggregation="head_max", layers=1, batch=5, h_kv=2, h_q=8, max_len=1100, len_lo=1100,
             len_hi=1100, budget=12, recent=4, name="varemptypaged")
    run_and_check(pcfg, lengths_override=[0, 1, 15, 33, 1100])


# ----------------------------------------------------------------------------- full-size workloads, sampled units

FULL = ["qwen3_8b", "ragged_8b", "qwen3_32b", "paged_8b", "paged_8b_steady", "qwen3_8b_steady", "qwen3_8b_max",
        "qwen3_8b_headmax", "qwen3_32b_max"]
# 1024 units with budgets of 6000 slots: the select-and-move kernel with keep lists between 4096 and 8192 in LDS
BIG_BUDGET = {
    "paged_budget6k": S(C["paged_8b"], layers=4, batch=32, max_len=9000, len_lo=6500, len_hi=9000, budget=6000,
                        recent=256, name="pagedb6k"),
    "contig_budget6k": S(C["ragged_8b"], layers=8, batch=16, max_len=9000, len_lo=6500, len_hi=9000, budget=6000,
                         recent=256, name="contigb6k"),
}


def _full_cfg(name):
    return BIG_BUDGET[name] if name in BIG_BUDGET else C[name]


@pytest.mark.parametrize("name", ["paged_steady", "contiguous_steady", "ragged_small", "paged_small"])
def test_length_bound(name):
    # launches sized by the host bound on lengths instead of the capacity; every unit still checked
    _, _, stats = run_and_check(SMALL[name], max_length=-1)
    _report(name + "+bound", stats)


@pytest.mark.parametrize("name", ["paged_steady", "contiguous_steady", "tiny", "tiny_f32_d128", "bf16_d64",
                                  "paged_interleaved", "ragged_small", "paged_many_units"])
def test_paths_bitwise_equal(name):
    # the fused pass, the three-kernel pass, with and without the length bound: scores, keep lists, new
    # lengths, the compacted cache and the paged tables are bitwise the same
    cfg = SMALL[name]
    outs = []
    for ml, flags in ((0, T.PASS_UNFUSED), (-1, T.PASS_UNFUSED), (0, T.PASS_FUSED), (-1, T.PASS_FUSED), (-1, 0)):
        cache = synth.make_cache(cfg)
        cache = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in cache.items()}
        lengths = cache["lengths"].cpu()
        tc = tri_cache_of(cfg, cache)
        params, _, _ = params_for(cfg, cache, "cuda", int(lengths.max()) if ml < 0 else 0, flags)
        stride = T.tri_score_stride(tc)
        scores = torch.zeros(cfg.layers, cfg.batch, cfg.h_kv, stride, device="cuda")
        keep = torch.zeros(cfg.layers, cfg.batch, cfg.h_kv, cfg.budget, dtype=torch.int32, device="cuda")
        out = T.tri_evict_step(tc, params, scores=scores, keep=keep)
        torch.cuda.synchronize()
        got = [out["new_lengths"].cpu().numpy(), bits(cache["k"]), bits(cache["v"])]
        for b, L in enumerate(lengths.tolist()):
            n = min(L, cfg.budget)
            got += [bits(scores[:, b, :, :L]), keep[:, b, :, :n].cpu().numpy()]
            if cfg.layout == "contiguous":    # slots past the new length are unspecified
                got += [bits(cache["k"][:, b, :, :n]), bits(cache["v"][:, b, :, :n]), cache["pos"][:, b, :, :n].cpu().numpy()]
        if cfg.layout == "paged":
            got += [out["block_table_out"].cpu().numpy(), out["freed"].cpu().numpy(), out["n_freed"].cpu().numpy()]
        outs.append(got)
    for other in outs[1:]:
        assert len(other) == len(outs[0])
        for a, b in zip(outs[0], other):
            assert np.array_equal(a, b)


@pytest.mark.parametrize("name", FULL + list(BIG_BUDGET))
def test_full_size_sampled(name):
    cfg = _full_cfg(name)
    say(f"[{name}] generating on the GPU")
    lengths = synth.lengths_for(cfg).numpy()
    units = sampled_units(cfg, lengths, 6)
    # a serving engine knows its lengths on the host: give the library the bound, as the bench does
    _, _, stats = run_and_check(cfg, units=units, gen_device="cuda", max_length=-1)
    _report(name, stats)


@pytest.mark.parametrize("name", FULL + list(BIG_BUDGET))
def test_full_size_every_unit(name):
    # Every unit of the full-size workload, against properties that need no oracle: the keep list is the recent
    # window plus exactly the best budget-recent candidates of the GPU's own scores under (score descending, slot
    # ascending), and the compacted K, V and positions are a bitwise gather of the originals (paged caches: the
    # expected rows are gathered through the old block table from a separate scoring and selection, which leave
    # the cache untouched; the pass's rows are read through the new table).
    cfg = _full_cfg(name)
    torch.cuda.empty_cache()   # the full-size caches of earlier tests are large
    say(f"[{name}] generating on the GPU")
    cache = synth.make_cache(cfg, device="cuda")
    lengths = cache["lengths"].cpu().tolist()
    contiguous = cfg.layout == "contiguous"
    B, R, bs = cfg.budget, cfg.recent, cfg.block_size
    tc = tri_cache_of(cfg, cache)
    params, _, _ = params_for(cfg, cache, "cuda", max(lengths))
    lidx = torch.arange(cfg.layers, device="cuda").view(-1, 1, 1)
    hidx = torch.arange(cfg.h_kv, device="cuda").view(1, -1, 1)
    if contiguous:
        k0, v0, p0 = cache["k"].clone(), cache["v"].clone(), cache["pos"].clone()
    else:
        # expected rows of every unit: the slots a separate selection keeps, gathered through the old table
        s_ref = T.tri_score(tc, params)
        keep_ref, _ = T.tri_topk(tc, params, s_ref)
        expect = []
        for b, L in enumerate(lengths):
            kb = keep_ref[:, b, :, :min(L, B)].long()
            blk, off = cache["block_table"][b].long()[kb // bs], kb % bs
            expect.append((cache["k"][lidx, blk, off, hidx].clone(), cache["v"][lidx, blk, off, hidx].clone(),
                           cache["pos"][lidx, blk, off, hidx].clone()))
        torch.cuda.synchronize()
    scores = torch.empty(cfg.layers, cfg.batch, cfg.h_kv, T.tri_score_stride(tc), device="cuda")
    keep = torch.empty(cfg.layers, cfg.batch, cfg.h_kv, cfg.budget, dtype=torch.int32, device="cuda")
    out = T.tri_evict_step(tc, params, scores=scores, keep=keep)
    torch.cuda.synchronize()
    assert out["new_lengths"].cpu().tolist() == [min(L, B) for L in lengths]
    ibits = torch.int16 if cache["k"].element_size() == 2 else torch.int32
    for b, L in enumerate(lengths):
        Ln = min(L, B)
        kb = keep[:, b, :, :Ln].long()
        s = scores[:, b, :, :L]
        assert torch.isfinite(s).all(), (name, b)
        if L <= B:
            assert torch.equal(kb, torch.arange(L, device="cuda").expand_as(kb))
        else:
            n = L - R
            assert torch.equal(kb[..., B - R:], torch.arange(n, L, device="cuda").expand(cfg.layers, cfg.h_kv, R))
            # + 0.0 makes -0 and +0 one key; the stable sort keeps equal scores in slot order
            best = torch.sort(s[..., :n] + 0.0, dim=-1, descending=True, stable=True).indices[..., :B - R]
            assert torch.equal(kb[..., :B - R], torch.sort(best, dim=-1).values), (name, b)
        if contiguous:
            idx = kb.unsqueeze(-1).expand(-1, -1, -1, cfg.d)
            for now, before in ((cache["k"], k0), (cache["v"], v0)):
                assert torch.equal(now[:, b, :, :Ln].view(ibits), torch.gather(before[:, b], 2, idx).view(ibits))
            assert torch.equal(cache["pos"][:, b, :, :Ln], torch.gather(p0[:, b], 2, kb.int().long()))
        else:
            assert torch.equal(s.view(torch.int32), s_ref[:, b, :, :L].view(torch.int32)), (name, b)
            assert torch.equal(keep[:, b, :, :Ln], keep_ref[:, b, :, :Ln]), (name, b)
            sl = torch.arange(Ln, device="cuda").view(1, 1, -1)
            blk, off = out["block_table_out"][b].long()[sl // bs], sl % bs
            ek, ev, ep = expect[b]
            assert torch.equal(cache["k"][lidx, blk, off, hidx].view(ibits), ek.view(ibits)), (name, b)
            assert torch.equal(cache["v"][lidx, blk, off, hidx].view(ibits), ev.view(ibits)), (name, b)
            assert torch.equal(cache["pos"][lidx, blk, off, hidx], ep), (name, b)
    say(f"[{name}] {cfg.layers * cfg.batch * cfg.h_kv} units checked")


def _key_rows(cfg, cache, l, b, L):
    """K rows of layer l, sequence b, every KV head: float64 [heads, L, d] (paged pools through the block table)."""
    if cfg.layout == "paged":
        bs = cfg.block_size
        blocks = cache["block_table"][b, :(L + bs - 1) // bs].long()
        x = cache["k"][l, blocks].reshape(-1, cfg.h_kv, cfg.d)[:L]
        return x.permute(1, 0, 2).double()
    return cache["k"][l, b, :, :L].double()


@pytest.mark.parametrize("name", FULL)
def test_full_size_every_score(name):
    # Every key of every unit of the full-size workload: the GPU's scores against the definition evaluated in
    # float64 on the GPU with torch -- the centres are averaged and rotated here from qbar (pair form, RoPE(x, n)
    # multiplies z_i(x) by e^{j n w_i}), not taken from the library -- within SCORE_TOL * A(p) as in the sampled
    # oracle comparison.
    from gpu_util import SCORE_BUDGET, SCORE_TOL
    cfg = C[name]
    torch.cuda.empty_cache()
    say(f"[{name}] generating on the GPU")
    cache = synth.make_cache(cfg, device="cuda")
    lengths = cache["lengths"].cpu().tolist()
    tc = tri_cache_of(cfg, cache)
    params, _, _ = params_for(cfg, cache, "cuda", max(lengths))
    scores = T.tri_score(tc, params)
    torch.cuda.synchronize()
    d, H, G, half = cfg.d, cfg.h_kv, cfg.group, cfg.d // 2
    i = torch.arange(half, device="cuda")
    ia, ib = (i, i + half) if cfg.rope == "half" else (2 * i, 2 * i + 1)
    om = cfg.theta ** (-2.0 * torch.arange(half, dtype=torch.float64, device="cuda") / d)
    offs = torch.tensor(cfg.offsets, dtype=torch.float64, device="cuda")
    qbar, c = synth.query_side(cfg)
    qbar = qbar.double().cuda()
    qz = torch.complex(qbar[..., ia], qbar[..., ib]).reshape(cfg.layers, H, G, half)
    chat = c.double().cuda().reshape(cfg.layers, H, G, half).mean(2)            # [layers, H, d/2]

    def to_dims(z):   # pair form [..., d/2] -> dims [..., d]
        w = torch.empty(*z.shape[:-1], d, dtype=torch.float64, device="cuda")
        w[..., ia], w[..., ib] = z.real, z.imag
        return w

    worst = worst_rel = 0.0
    for b, L in enumerate(lengths):
        if L == 0:
            continue
        t = float(cache["t"][b])
        rot = torch.exp(1j * torch.outer(t + offs, om))                        # [|D|, d/2]
        for l in range(cfg.layers):
            K = _key_rows(cfg, cache, l, b, L)                                 # [H, L, d]
            kz = torch.sqrt(K[..., ia] ** 2 + K[..., ib] ** 2)                 # [H, L, d/2]
            norm = (kz * chat[l].unsqueeze(1)).sum(-1)
            norm_abs = (kz * chat[l].abs().unsqueeze(1)).sum(-1)
            if cfg.aggregation == "mean":
                w = to_dims(qz[l].mean(1) * rot.mean(0))                       # [H, d]
                dist = (K * w.unsqueeze(1)).sum(-1)
                A = (K.abs() * w.abs().unsqueeze(1)).sum(-1) + norm_abs
            else:
                W = to_dims(qz[l].unsqueeze(2) * rot).reshape(H, G * len(cfg.offsets), d)
                lg = torch.matmul(K, W.transpose(-1, -2).contiguous()).reshape(H, L, G, len(cfg.offsets))
                dist = lg.amax(dim=(-2, -1)) if cfg.aggregation == "max" else lg.amax(-1).mean(-1)
                A = torch.matmul(K.abs(), W.abs().transpose(-1, -2).contiguous()).amax(-1) + norm_abs
            ref = dist + norm
            err = (scores[l, b, :, :L].double() - ref).abs()
            assert bool((err <= SCORE_TOL * A).all()), (name, l, b, float((err / A).max()))
            assert bool((err <= SCORE_BUDGET[cfg.dtype] * A).all()), (name, l, b, float((err / A).max()))
            big = ref.abs() >= 0.2 * A
            assert bool((err[big] <= SCORE_TOL * ref.abs()[big]).all()), (name, l, b)
            sel = ref.abs() >= 0.1 * A
            worst = max(worst, float((err / A).max()))
            if bool(sel.any()):
                worst_rel = max(worst_rel, float((err[sel] / ref.abs()[sel]).max()))
    say(f"[{name}] every key of {cfg.layers * cfg.batch * H} units, worst |ds|/A = {worst:.3g}, "
        f"worst |ds|/|s| over |s| >= 0.1 A = {worst_rel:.3g}")
