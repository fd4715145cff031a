"""Helpers shared by the GPU parity tests: build a cache on the device from the seeded generator,
run the HIP pass through the C ABI, and check units against the CPU oracle.

Comparison rules (float scores, integer selection, bit-exact moves):
  * scores: |s_gpu(p) - s_ref(p)| <= SCORE_TOL * A(p), A(p) the sum of the magnitudes of the terms
    a float32 evaluation adds (oracle.abs_terms) -- the acceptance bound -- and also within the error
    budget derived from the kernels' arithmetic (SCORE_BUDGET, below), which is several times tighter;
    where |s_ref| >= 0.2 A(p) the plain relative error |ds| / |s_ref| is within SCORE_TOL too (the budget
    guarantees it there), and its maximum over |s_ref| >= 0.1 A(p) is reported;
  * selection: running the oracle's selection on the GPU's own float32 scores must give the GPU's
    keep list exactly; against the float64 reference, the kept sets must agree outside the boundary
    set (candidates within SCORE_BUDGET * (A(p) + max A) of the threshold score), with equal sizes;
  * compaction: every moved K/V row and position id equals its source bit for bit.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth
import token_eviction_scoring_amd as T

SCORE_TOL = 1e-4

# Error budget of the kernels' float32 arithmetic, as a multiple of A(p) (u = 2^-24, the float32 unit roundoff):
#   * u and w = RoPE(u, t) are each rounded once to float32 from float64: 2u per element of w;
#   * bf16 keys: w enters v_dot2_f32_bf16 (exact bf16 products) split into a bf16 high part and a bf16 residual;
#     each rounding to bf16's 8-bit significand errs by at most 2^-8 of its argument, so the split misses at most
#     2^-8 * 2^-8 = 2^-16 of |w_j| (matrix-core logits of the variants use the same split);
#   * float32 accumulation: at most 24 roundings along any term's path (16 dot2 or fma steps in a lane, the
#     butterfly over up to 8 lanes, the norm term's fma chain), each <= u of the running sum's terms;
#   * norm term: chat rounded once (u), |z|^2 rounded once (u/2 after the square root), the square root <= 2u.
# Total: bf16 keys (2^-16 + 30u) A, float32 keys 30u A.
SCORE_BUDGET = {"bf16": 2.0 ** -16 + 30 * 2.0 ** -24, "f32": 30 * 2.0 ** -24}


def say(*a):
    print(*a, flush=True)


AGG = {"max": T.AGG_MAX, "head_max": T.AGG_HEAD_MAX}


def params_for(cfg, cache, device, max_length=0, flags=0):
    qbar, c = synth.query_side(cfg)
    u, c_hat = T.tri_prepare_centres(qbar.to(device), c.to(device), cfg.h_kv, cfg.theta, cfg.offsets, cfg.rope)
    variant = None
    if cfg.aggregation != "mean":
        centres = T.tri_prepare_variant_centres(qbar.to(device), cfg.h_kv, cfg.theta, cfg.offsets, cfg.rope)
        variant = T.Variant(centres, AGG[cfg.aggregation], cfg.group, len(cfg.offsets))
    p = T.Params(u=u, c_hat=c_hat, theta=cfg.theta, lengths=cache["lengths"].to(device).int(),
                 t=cache["t"].to(device).int(), budget=cfg.budget, recent=cfg.recent, max_length=max_length,
                 flags=flags, variant=variant)
    return p, qbar, c


def tri_cache_of(cfg, cache):
    if cfg.layout == "paged":
        return T.paged_cache(cache["k"], cache["v"], cache["pos"], cache["block_table"], cfg.rope)
    return T.contiguous_cache(cache["k"], cache["v"], cache["pos"], cfg.rope)


def bits(x: torch.Tensor) -> np.ndarray:
    """Raw storage bits of a bf16/f32 tensor as an integer array."""
    return (x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)).cpu().numpy()


def unit_rows(cfg, cache, l, b, h, L):
    """(K, V, pos) of one unit's logical slots 0..L-1 (host copies of the stored values)."""
    if cfg.layout == "paged":
        bs = cfg.block_size
        s = torch.arange(L, device=cache["k"].device)
        blk = cache["block_table"][b].long()[s // bs]
        k = cache["k"][l, blk, s % bs, h]
        v = cache["v"][l, blk, s % bs, h]
        p = cache["pos"][l, blk, s % bs, h]
    else:
        k, v, p = cache["k"][l, b, h, :L], cache["v"][l, b, h, :L], cache["pos"][l, b, h, :L]
    return k.cpu(), v.cpu(), p.cpu()


def unit_rows_after(cfg, cache, out, l, b, h, Ln):
    """Compacted rows 0..Ln-1 of a unit after the pass (paged: through the new block table)."""
    if cfg.layout == "paged":
        bs = cfg.block_size
        s = torch.arange(Ln, device=cache["k"].device)
        table = out["block_table_out"][b].long()
        blk = table[s // bs]
        return (cache["k"][l, blk, s % bs, h].cpu(), cache["v"][l, blk, s % bs, h].cpu(),
                cache["pos"][l, blk, s % bs, h].cpu())
    return (cache["k"][l, b, h, :Ln].cpu(), cache["v"][l, b, h, :Ln].cpu(), cache["pos"][l, b, h, :Ln].cpu())


def check_unit(cfg, qbar, c, l, h, t, k_in, v_in, p_in, scores_gpu, keep_gpu, k_out, v_out, p_out):
    """All parity checks for unit (layer l, KV head h) of some sequence; returns error statistics."""
    G = cfg.group
    tag = (cfg.name, l, h)
    K64 = k_in.double().numpy()
    L = K64.shape[0]
    qg = oracle.group_rows(qbar[l].double().numpy(), h, G)
    cg = oracle.group_rows(c[l].double().numpy(), h, G)
    pos = p_in.numpy().astype(np.int64)
    if cfg.aggregation == "mean":
        ref = oracle.score(K64, qg, cg, cfg.theta, cfg.offsets, t, cfg.rope)
        A = oracle.abs_terms(K64, qg, cg, cfg.theta, cfg.offsets, t, cfg.rope)
    else:
        ref = oracle.score_variant(K64, qg, cg, cfg.theta, cfg.offsets, t, cfg.rope, cfg.aggregation)
        A = oracle.abs_terms_variant(K64, qg, cg, cfg.theta, cfg.offsets, t, cfg.rope)
    sg = scores_gpu.astype(np.float64)
    err = np.abs(sg - ref)
    worst = float((err / A).max()) if L else 0.0
    assert np.all(err <= SCORE_TOL * A), f"{tag}: score error {worst:.3g} x A exceeds {SCORE_TOL}"
    budget = SCORE_BUDGET[cfg.dtype]
    assert np.all(err <= budget * A), f"{tag}: score error {worst:.3g} x A exceeds the derived budget {budget:.3g}"
    big = np.abs(ref) >= 0.2 * A
    assert np.all(err[big] <= SCORE_TOL * np.abs(ref[big])), f"{tag}: relative score error exceeds {SCORE_TOL}"
    sel = np.abs(ref) >= 0.1 * A
    worst_rel = float((err[sel] / np.abs(ref[sel])).max()) if sel.any() else 0.0
    keep_ref = oracle.select(ref, pos, cfg.budget, cfg.recent)
    keep_self = oracle.select(sg, pos, cfg.budget, cfg.recent)
    assert np.array_equal(keep_gpu, keep_self), f"{tag}: GPU selection differs from the oracle's on GPU scores"
    # Keys whose membership may differ from the float64 reference's: if p is kept by one and q by the other,
    # s_ref(p) - s_ref(q) <= e_p + e_q <= budget * (A(p) + A(q)), and the threshold lies between them, so both are
    # within budget * (A(own) + max A) of it.  (The derived budget, not the looser acceptance bound.)
    cand = A[:max(L - cfg.recent, 0)]
    amax = float(cand.max()) if cand.size else 0.0
    bset = set(oracle.boundary_set(ref, A + amax, cfg.budget, cfg.recent, budget).tolist())
    assert len(keep_gpu) == len(keep_ref) == min(L, cfg.budget)
    assert set(keep_gpu.tolist()) - bset == set(keep_ref.tolist()) - bset, f"{tag}: kept set differs outside boundary"
    kb, vb = bits(k_in), bits(v_in)
    assert np.array_equal(bits(k_out), kb[keep_gpu]), f"{tag}: compacted K differs"
    assert np.array_equal(bits(v_out), vb[keep_gpu]), f"{tag}: compacted V differs"
    assert np.array_equal(p_out.numpy(), p_in.numpy()[keep_gpu]), f"{tag}: compacted pos differs"
    return {"worst_rel_A": worst, "worst_rel": worst_rel, "boundary": len(bset), "L": L}


def sampled_units(cfg, lengths, n, seed=0):
    """A deterministic sample of (layer, seq, head) including the first and last unit and the longest sequence."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lengths)
    picks = {(0, 0, 0), (cfg.layers - 1, cfg.batch - 1, cfg.h_kv - 1), (cfg.layers // 2, int(lens.argmax()), 1 % cfg.h_kv)}
    while len(picks) < n:
        picks.add((int(rng.integers(cfg.layers)), int(rng.integers(cfg.batch)), int(rng.integers(cfg.h_kv))))
    return sorted(picks)


def run_and_check(cfg, device="cuda", units=None, gen_device="cpu", composed=False, lengths_override=None,
                  mutate=None, max_length=0, flags=0):
    """Generate `cfg`, run the whole pass on the GPU and check `units` (default: all) against the oracle.

    lengths_override: shorter lengths to use instead of the generated ones (t follows them);
    mutate(cache): edits the generated cache in place before the pass (e.g. duplicate rows);
    max_length: the host bound on lengths given to the library (-1: the longest length);
    flags: tri_params.flags (T.PASS_UNFUSED keeps short caches on the three-kernel path)."""
    cache = synth.make_cache(cfg, device=gen_device)
    if gen_device != device:
        cache = {k: (v.to(device) if torch.is_tensor(v) else v) for k, v in cache.items()}
    if lengths_override is not None:
        lo = torch.tensor(lengths_override, dtype=torch.int32, device=device)
        assert bool((lo <= cache["lengths"]).all())
        cache["lengths"], cache["t"] = lo, lo.clone()
    if mutate is not None:
        mutate(cache)
    lengths = cache["lengths"].cpu().numpy()
    if units is None:
        units = [(l, b, h) for l in range(cfg.layers) for b in range(cfg.batch) for h in range(cfg.h_kv)]
    inputs = {u: unit_rows(cfg, cache, u[0], u[1], u[2], int(lengths[u[1]])) for u in units}
    tc = tri_cache_of(cfg, cache)
    if max_length == -1:
        max_length = int(lengths.max())
    params, qbar, c = params_for(cfg, cache, device, max_length, flags)
    stride = T.tri_score_stride(tc)
    scores = torch.full((cfg.layers, cfg.batch, cfg.h_kv, stride), float("nan"), device=device)
    keep = torch.full((cfg.layers, cfg.batch, cfg.h_kv, cfg.budget), -1, dtype=torch.int32, device=device)
    if composed:
        T.tri_score(tc, params, scores)
        _, new_lengths = T.tri_topk(tc, params, scores, keep)
        out = T.tri_compact(tc, params, keep)
        out["new_lengths"] = new_lengths
    else:
        out = T.tri_evict_step(tc, params, scores=scores, keep=keep)
    torch.cuda.synchronize()
    stats = []
    sc_host = scores.cpu().numpy()
    keep_host = keep.cpu().numpy()
    nl = out["new_lengths"].cpu().numpy()
    assert nl.tolist() == [min(int(L), cfg.budget) for L in lengths]
    for (l, b, h) in units:
        L = int(lengths[b])
        Ln = min(L, cfg.budget)
        k_in, v_in, p_in = inputs[(l, b, h)]
        k_out, v_out, p_out = unit_rows_after(cfg, cache, out, l, b, h, Ln)
        st = check_unit(cfg, qbar, c, l, h, int(cache["t"][b]), k_in, v_in, p_in, sc_host[l, b, h, :L],
                        keep_host[l, b, h, :Ln], k_out, v_out, p_out)
        # the score row of a unit is written for slots below its length only (the buffer started as NaN)
        assert np.isnan(sc_host[l, b, h, L:]).all(), (l, b, h, L)
        stats.append(st)
    if cfg.layout == "paged":
        check_tables(cfg, cache, out, lengths)
    return cache, out, stats


def check_tables(cfg, cache, out, lengths):
    bs = cfg.block_size
    table = cache["block_table"].cpu().numpy()
    bto = out["block_table_out"].cpu().numpy()
    freed = out["freed"].cpu().numpy()
    n_freed = int(out["n_freed"].cpu()[0])
    want_freed = []
    for b, L in enumerate(lengths):
        new, fr = oracle.paged_tables(table[b], int(L), min(int(L), cfg.budget), bs)
        assert bto[b, :len(new)].tolist() == new.tolist()
        want_freed += fr.tolist()
    assert n_freed == len(want_freed)
    assert freed[:n_freed].tolist() == want_freed


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch loaded (for tri_evict_step_profiled)."""

    def __init__(self, n):
        import ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(h)) == 0
            self.ev.append(h.value)
