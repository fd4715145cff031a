"""tri_evict_step_noalloc (control words in the library's own device array) against tri_evict_step (caller's
workspace): the same outputs bit for bit, on calls in a row of decreasing size -- so later calls find the array
holding an earlier call's words -- on both the path that selects and compacts in one kernel and the path with
separate selection and compaction (budgets above 8192, whose tickets and flags must be cleared per call)."""
import ctypes

import numpy as np
import pytest
import torch

import synth
import token_eviction_scoring_amd as T
from gpu_util import bits, params_for, say, tri_cache_of

C = synth.CONFIGS
S = synth.scaled


def _outputs(cfg, cache, out, scores, keep):
    """Everything the pass defines: new lengths, each unit's scores and keep list, the compacted rows (paged:
    through the new table), the paged tables and freed list."""
    lengths = cache["lengths"].cpu().tolist()
    got = [out["new_lengths"].cpu().numpy()]
    for b, L in enumerate(lengths):
        n = min(L, cfg.budget)
        got += [bits(scores[:, b, :, :L]), keep[:, b, :, :n].cpu().numpy()]
        if cfg.layout == "contiguous":
            got += [bits(cache["k"][:, b, :, :n]), bits(cache["v"][:, b, :, :n]), cache["pos"][:, b, :, :n].cpu().numpy()]
        else:
            bs = cfg.block_size
            s = torch.arange(n, device="cuda")
            blk = out["block_table_out"][b].long()[s // bs]
            got += [bits(cache["k"][:, blk, s % bs]), bits(cache["v"][:, blk, s % bs]),
                    cache["pos"][:, blk, s % bs].cpu().numpy()]
    if cfg.layout == "paged":
        nf = int(out["n_freed"].cpu()[0])
        got += [out["block_table_out"].cpu().numpy(), out["freed"][:nf].cpu().numpy(), np.array([nf])]
    return got


def _run(cfg, noalloc):
    cache = synth.make_cache(cfg, device="cuda")
    tc = tri_cache_of(cfg, cache)
    params, _, _ = params_for(cfg, cache, "cuda", flags=T.PASS_UNFUSED)
    scores = torch.full((cfg.layers, cfg.batch, cfg.h_kv, T.tri_score_stride(tc)), float("nan"), device="cuda")
    keep = torch.full((cfg.layers, cfg.batch, cfg.h_kv, cfg.budget), -1, dtype=torch.int32, device="cuda")
    if noalloc:
        out = T.tri_evict_step_noalloc(tc, params, scores, keep)
    else:
        out = T.tri_evict_step(tc, params, scores=scores, keep=keep)
    torch.cuda.synchronize()
    return _outputs(cfg, cache, out, scores, keep)


CASES = [
    S(C["paged_8b"], layers=2, batch=6, max_len=4096, len_lo=100, len_hi=4096, budget=700, recent=128,
      name="noalloc_paged_big"),
    S(C["qwen3_8b"], layers=1, batch=3, h_q=8, h_kv=2, max_len=12000, len_lo=9000, len_hi=12000, budget=8500,
      recent=300, name="noalloc_separate_kernels"),
    S(C["paged_8b"], layers=1, batch=3, h_q=8, h_kv=2, max_len=10000, len_lo=8700, len_hi=10000, budget=8600,
      recent=64, name="noalloc_paged_separate"),
    S(C["qwen3_8b"], layers=1, batch=2, h_q=8, h_kv=2, max_len=3000, len_lo=500, len_hi=3000, budget=300, recent=30,
      name="noalloc_small"),
]


@pytest.mark.gpu
def test_noalloc_matches_evict_step_on_calls_of_decreasing_size():
    assert torch.cuda.is_available()
    for cfg in CASES:
        say(f"[noalloc] {cfg.name}")
        want = _run(cfg, noalloc=False)
        got = _run(cfg, noalloc=True)
        assert len(got) == len(want)
        for a, b in zip(want, got):
            assert np.array_equal(a, b), cfg.name
    torch.cuda.empty_cache()


def test_noalloc_rejects_shapes_beyond_its_array():
    # checked on the host before anything touches a device: 262144 units of 32768 slots need more control words
    # than the library's array holds
    from token_eviction_scoring_amd import build
    build.ensure_built()
    lib = T.lib()
    s = T.CacheStruct()
    s.layout, s.dtype, s.rope = 1, 0, 0
    s.num_layers, s.batch, s.num_kv_heads, s.head_dim = 64, 512, 8, 128
    s.k, s.v, s.pos, s.block_table = 1 << 20, 1 << 21, 1 << 22, 1 << 23
    s.layer_stride, s.pos_layer_stride = 1 << 30, 1 << 24
    s.block_size, s.num_blocks, s.max_blocks_per_seq = 16, 1 << 20, 2048
    p = T.ParamsStruct()
    p.u, p.c_hat, p.lengths, p.t = 1 << 24, 1 << 25, 1 << 26, 1 << 27
    p.rope_theta, p.budget, p.recent = 1e6, 2048, 128
    fake = ctypes.c_void_p(1 << 28)
    st = lib.tri_evict_step_noalloc(ctypes.byref(s), ctypes.byref(p), fake, fake, ctypes.c_void_p(1 << 29),
                                    ctypes.c_void_p(1 << 31), ctypes.c_void_p(1 << 32), ctypes.c_void_p(1 << 33), None)
    assert st == T.TRI_ERR_UNSUPPORTED
    assert b"control words" in lib.tri_last_error()
    # outputs the caller must pass
    st = lib.tri_evict_step_noalloc(ctypes.byref(s), ctypes.byref(p), None, fake, ctypes.c_void_p(1 << 29),
                                    ctypes.c_void_p(1 << 31), ctypes.c_void_p(1 << 32), ctypes.c_void_p(1 << 33), None)
    assert st == T.TRI_ERR_INVALID_ARG
