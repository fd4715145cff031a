"""Seeded synthetic inputs for the KV-cache eviction pass.

This module only *makes inputs*: per-head key centres, noisy keys rotated to
their true positions (the cache a rotary-embedding model would have written),
values, query centres with their calibration norm statistics, ragged lengths
and paged block tables.  It holds none of the eviction method's arithmetic
(no scoring, no selection, no compaction) and is shared, as a producer of
inputs only, by the CPU oracle's tests and by the GPU path's tests and bench.

Workload shapes follow the model shapes the TriAttention pages evaluate on
("TriAttention：基于三角函数 KV 压缩的高效长推理", 实验结果: Qwen3-8B long
reasoning at 32K generated tokens; the news page on the single-RTX-4090 demo:
Qwen3-32B agent run).  Value structure follows the pages' observation that
pre-rotation keys cluster around a fixed per-head centre that is stable across
positions (same page, 核心洞见：Q/K 集中性).

Everything is generated with torch so that the same code can produce small
cases on the CPU and full-size caches directly in device memory.  Random
streams are seeded per (config seed, layer, tag) so any layer can be rebuilt
alone.  Generation on "cpu" and on "cuda" gives different (but each
deterministic) draws; a test always compares both sides on one draw, copied.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Optional

import torch

__all__ = ["Config", "CONFIGS", "scaled", "query_side", "lengths_for",
           "make_cache", "rotate_keys", "frequencies_f64", "steady_positions", "calibration_queries",
           "decode_queries"]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    layers: int
    h_q: int
    h_kv: int
    d: int
    theta: float
    batch: int
    dtype: str                    # "f32" or "bf16": storage type of K and V
    layout: str                   # "contiguous" or "paged"
    max_len: int                  # contiguous: slots per (layer, seq, head)
    len_lo: int                   # cache length drawn uniformly in [len_lo, len_hi]
    len_hi: int
    offsets: tuple                # future offsets Delta
    budget: int
    recent: int
    centre: str                   # "normal": mu ~ N(0,1)^d; "lognormal": pair magnitude ~ LogNormal(0, .5)
    noise: float                  # noise scale (absolute for "normal", times RMS(mu) for "lognormal")
    outlier_frac: float = 0.0     # fraction of tokens whose pre-rotation key is scaled
    outlier_scale: float = 1.0
    block_size: int = 16          # paged only
    seed: int = 0
    n_cal: int = 256              # calibration queries per query head
    cal_noise: float = 0.5        # calibration query spread around the centre
    rope: str = "half"            # "half" (pairs i, i+d/2) or "interleaved" (pairs 2i, 2i+1)
    steady: int = 0               # > 0: the cache as a later pass finds it (see make_cache)
    kept_only: bool = False       # the cache right after a pass: budget slots of earlier positions (see make_cache)
    aggregation: str = "mean"     # score variant: "mean" (collapsed), "max", "head_max"

    @property
    def group(self) -> int:
        return self.h_q // self.h_kv

    @property
    def units(self) -> int:
        return self.layers * self.batch * self.h_kv


def _pow2(n: int) -> tuple:
    return tuple(2 ** i for i in range(n + 1))


# The five workloads.  Lengths: fixed when len_lo == len_hi.
CONFIGS = {
    "tiny": Config("tiny", layers=1, h_q=4, h_kv=2, d=64, theta=1e4, batch=1, dtype="f32",
                   layout="contiguous", max_len=1024, len_lo=1024, len_hi=1024,
                   offsets=_pow2(8), budget=128, recent=32, centre="normal", noise=0.5, seed=1),
    "qwen3_8b": Config("qwen3_8b", layers=36, h_q=32, h_kv=8, d=128, theta=1e6, batch=1, dtype="bf16",
                       layout="contiguous", max_len=32768, len_lo=32768, len_hi=32768,
                       offsets=_pow2(12), budget=2048, recent=128, centre="lognormal", noise=0.3, seed=2),
    "ragged_8b": Config("ragged_8b", layers=36, h_q=32, h_kv=8, d=128, theta=1e6, batch=16, dtype="bf16",
                        layout="contiguous", max_len=32768, len_lo=8192, len_hi=32768,
                        offsets=_pow2(12), budget=2048, recent=128, centre="lognormal", noise=0.3, seed=3),
    "qwen3_32b": Config("qwen3_32b", layers=64, h_q=64, h_kv=8, d=128, theta=1e6, batch=4, dtype="bf16",
                        layout="contiguous", max_len=49152, len_lo=49152, len_hi=49152,
                        offsets=_pow2(12), budget=4096, recent=256, centre="lognormal", noise=0.15,
                        outlier_frac=0.05, outlier_scale=8.0, seed=4),
    "paged_8b": Config("paged_8b", layers=36, h_q=32, h_kv=8, d=128, theta=1e6, batch=64, dtype="bf16",
                       layout="paged", max_len=32768, len_lo=2048, len_hi=32768,
                       offsets=_pow2(12), budget=2048, recent=128, centre="lognormal", noise=0.3,
                       block_size=16, seed=5),
}
# The recurring pass: every `steady` decode steps a cache that was cut to `budget` slots has grown by
# `steady` tokens.  Same shapes and centres as the first-pass workloads.
CONFIGS["paged_8b_steady"] = dataclasses.replace(CONFIGS["paged_8b"], name="paged_8b_steady", steady=128)
CONFIGS["qwen3_8b_steady"] = dataclasses.replace(CONFIGS["qwen3_8b"], name="qwen3_8b_steady", steady=128)
# Non-collapsible aggregation variants of the score on the Qwen3-8B shape.
CONFIGS["qwen3_8b_max"] = dataclasses.replace(CONFIGS["qwen3_8b"], name="qwen3_8b_max", aggregation="max")
CONFIGS["qwen3_8b_headmax"] = dataclasses.replace(CONFIGS["qwen3_8b"], name="qwen3_8b_headmax",
                                                  aggregation="head_max")
CONFIGS["paged_8b_max"] = dataclasses.replace(CONFIGS["paged_8b"], name="paged_8b_max", aggregation="max")
# ... and on the Qwen3-32B shape (eight query heads per KV head)
CONFIGS["qwen3_32b_max"] = dataclasses.replace(CONFIGS["qwen3_32b"], name="qwen3_32b_max", aggregation="max")
# What decode attention reads between passes: every sequence holds the budget's kept slots.
CONFIGS["paged_8b_kept"] = dataclasses.replace(CONFIGS["paged_8b"], name="paged_8b_kept", kept_only=True)


def scaled(cfg: Config, **kw) -> Config:
    """A copy of `cfg` with some fields replaced (used for small test cases)."""
    return dataclasses.replace(cfg, **kw)


def _seed(cfg: Config, *tags) -> int:
    h = hashlib.sha256(repr((cfg.seed, cfg.name) + tags).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(cfg: Config, device, *tags) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(cfg, *tags))
    return g


def frequencies_f64(d: int, theta: float, device="cpu") -> torch.Tensor:
    """Rotary frequencies theta^(-2i/d), i < d/2, in float64."""
    i = torch.arange(d // 2, dtype=torch.float64, device=device)
    return torch.pow(torch.tensor(theta, dtype=torch.float64, device=device), -2.0 * i / d)


def _pair_split(x: torch.Tensor, rope: str):
    h = x.shape[-1] // 2
    if rope == "half":
        return x[..., :h], x[..., h:]
    return x[..., 0::2], x[..., 1::2]


def _pair_join(a: torch.Tensor, b: torch.Tensor, rope: str) -> torch.Tensor:
    if rope == "half":
        return torch.cat([a, b], dim=-1)
    return torch.stack([a, b], dim=-1).flatten(-2)


def rotate_keys(k_pre: torch.Tensor, positions: torch.Tensor, theta: float, rope: str) -> torch.Tensor:
    """Apply the rotary embedding to pre-rotation keys at their positions (float64 in, float64 out).

    k_pre [..., L, d]; positions [L] or broadcastable to [..., L].  This is how the model writes its
    cache, so it is input generation, not the scoring method.
    """
    d = k_pre.shape[-1]
    w = frequencies_f64(d, theta, k_pre.device)
    ang = positions.to(torch.float64).unsqueeze(-1) * w          # [..., L, d/2]
    cs, sn = torch.cos(ang), torch.sin(ang)
    a, b = _pair_split(k_pre, rope)
    return _pair_join(a * cs - b * sn, a * sn + b * cs, rope)


def _store(x: torch.Tensor, dtype: str) -> torch.Tensor:
    # round-to-nearest-even to the storage type
    return x.to(torch.bfloat16) if dtype == "bf16" else x.to(torch.float32)


def query_side(cfg: Config):
    """Query centres qbar [layers, h_q, d] and norm statistics c [layers, h_q, d/2], both float32.

    qbar ~ N(0,1)^d per (layer, query head).  Calibration queries q_n = qbar + cal_noise * N(0,1)^d,
    n < n_cal; c_i = mean_n |pair_i(q_n)| - |pair_i(qbar)|, the pair-norm mass that the centre
    does not carry (mostly positive; it can dip slightly below zero because qbar is the drawn
    centre, not the sample mean).  Always drawn on the CPU so that every device sees the same
    centres.
    """
    g = _gen(cfg, "cpu", "query")
    qbar = torch.randn(cfg.layers, cfg.h_q, cfg.d, generator=g, dtype=torch.float64)
    qbar = qbar.to(torch.float32).to(torch.float64)
    cal = qbar.unsqueeze(2) + cfg.cal_noise * torch.randn(cfg.layers, cfg.h_q, cfg.n_cal, cfg.d,
                                                          generator=g, dtype=torch.float64)
    a, b = _pair_split(cal, cfg.rope)
    mean_norm = torch.sqrt(a * a + b * b).mean(dim=2)
    qa, qb = _pair_split(qbar, cfg.rope)
    c = mean_norm - torch.sqrt(qa * qa + qb * qb)
    return qbar.to(torch.float32), c.to(torch.float32)


def decode_queries(cfg: Config, t: torch.Tensor, device="cpu") -> torch.Tensor:
    """Post-rotation decode queries [layers, batch, h_q, d] in the storage type: per (layer, sequence, query
    head) the query centre plus cal_noise * N(0,1)^d noise, rotated to the sequence's decode position t[b]."""
    qbar, _ = query_side(cfg)
    g = _gen(cfg, "cpu", "decode_q")
    pre = qbar.double().view(cfg.layers, 1, cfg.h_q, cfg.d) + cfg.cal_noise * torch.randn(
        cfg.layers, cfg.batch, cfg.h_q, cfg.d, generator=g, dtype=torch.float64)
    pos = t.to("cpu", torch.float64).view(1, cfg.batch, 1)
    q = rotate_keys(pre.unsqueeze(-2), pos.unsqueeze(-1), cfg.theta, cfg.rope).squeeze(-2)
    return _store(q, cfg.dtype).to(device)


def calibration_queries(cfg: Config, n: int, device="cpu") -> torch.Tensor:
    """n pre-rotation calibration queries per (layer, query head), [layers, n, h_q, d] in the storage type:
    q = qbar + cal_noise * N(0,1)^d around the query centres of `query_side` (token-major, as a model
    would emit them layer by layer)."""
    qbar, _ = query_side(cfg)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    out = torch.empty(cfg.layers, n, cfg.h_q, cfg.d, dtype=dt, device=device)
    for layer in range(cfg.layers):
        g = _gen(cfg, device, "calibration", layer)
        noise = torch.randn(n, cfg.h_q, cfg.d, generator=g, dtype=torch.float32, device=device)
        out[layer] = (qbar[layer].to(device).view(1, cfg.h_q, cfg.d) + cfg.cal_noise * noise).to(dt)
    return out


def lengths_for(cfg: Config) -> torch.Tensor:
    """Per-sequence cache lengths, int32 [batch], uniform in [len_lo, len_hi] (CPU)."""
    if cfg.len_lo == cfg.len_hi:
        return torch.full((cfg.batch,), cfg.len_lo, dtype=torch.int32)
    g = _gen(cfg, "cpu", "lengths")
    return torch.randint(cfg.len_lo, cfg.len_hi + 1, (cfg.batch,), generator=g, dtype=torch.int64).to(torch.int32)


def _key_centres(cfg: Config, layer: int, device) -> torch.Tensor:
    """Pre-rotation key centre per KV head, float64 [h_kv, d], and the noise scale per head [h_kv]."""
    g = _gen(cfg, device, "centre", layer)
    if cfg.centre == "normal":
        mu = torch.randn(cfg.h_kv, cfg.d, generator=g, dtype=torch.float64, device=device)
        scale = torch.full((cfg.h_kv,), cfg.noise, dtype=torch.float64, device=device)
        return mu, scale
    mag = torch.exp(0.5 * torch.randn(cfg.h_kv, cfg.d // 2, generator=g, dtype=torch.float64, device=device))
    ph = 2.0 * math.pi * torch.rand(cfg.h_kv, cfg.d // 2, generator=g, dtype=torch.float64, device=device)
    mu = _pair_join(mag * torch.cos(ph), mag * torch.sin(ph), cfg.rope)
    rms = torch.sqrt((mu * mu).mean(dim=-1))
    return mu, cfg.noise * rms


def steady_positions(cfg: Config, layer: int, b: int, t0: int, device) -> torch.Tensor:
    """Positions held by the slots of a cache that an earlier pass at decode position t0 cut to
    `budget` slots and that has since grown by `steady` tokens: int64 [h_kv, budget + steady].

    Per KV head: the `recent` positions just before t0, `budget - recent` distinct positions drawn
    uniformly from [0, t0 - recent), then the new positions t0 .. t0 + steady - 1; ascending.
    The draw is uniform (it does not imitate which keys a score would have kept)."""
    B, R = cfg.budget, cfg.recent
    g = _gen(cfg, device, "steady_pos", layer, b)
    n_old = t0 - R
    pick = torch.rand(cfg.h_kv, n_old, generator=g, device=device).argsort(dim=-1)[:, :B - R]
    old = torch.sort(pick, dim=-1).values
    tail = torch.arange(n_old, t0 + cfg.steady, device=device).expand(cfg.h_kv, -1)
    return torch.cat([old, tail], dim=-1)


def _seq_kv(cfg: Config, layer: int, b: int, L: int, device, mu=None, scale=None, positions=None):
    """Keys (post-rotation, stored dtype) and values of one (layer, sequence), [h_kv, L, d] each.

    positions: int64 [h_kv, L] (per head) or None for 0 .. L-1."""
    if mu is None:
        mu, scale = _key_centres(cfg, layer, device)
    g = _gen(cfg, device, "kv", layer, b)
    k_pre = torch.randn(cfg.h_kv, L, cfg.d, generator=g, dtype=torch.float32, device=device)
    k_pre = k_pre.to(torch.float64) * scale.view(-1, 1, 1) + mu.view(cfg.h_kv, 1, cfg.d)
    if cfg.outlier_frac > 0:
        # outlier tokens are per (layer, sequence, token) and shared by every KV head
        hit = torch.rand(1, L, 1, generator=g, device=device) < cfg.outlier_frac
        k_pre = torch.where(hit, k_pre * cfg.outlier_scale, k_pre)
    pos = torch.arange(L, device=device) if positions is None else positions
    k = _store(rotate_keys(k_pre, pos, cfg.theta, cfg.rope), cfg.dtype)
    del k_pre
    v = _store(torch.randn(cfg.h_kv, L, cfg.d, generator=g, dtype=torch.float32, device=device), cfg.dtype)
    return k, v


def block_tables(cfg: Config, lengths: torch.Tensor):
    """Paged layout: a random permutation of pool blocks 1..N-1 split into per-sequence tables.

    Returns (table int32 [batch, max_blocks] padded with -1, num_blocks).  Block 0 is never used.
    """
    bs = cfg.block_size
    nblk = [(int(l) + bs - 1) // bs for l in lengths]
    total = sum(nblk)
    g = _gen(cfg, "cpu", "blocks")
    perm = torch.randperm(total, generator=g) + 1
    max_blocks = (cfg.max_len + bs - 1) // bs
    table = torch.full((cfg.batch, max_blocks), -1, dtype=torch.int32)
    off = 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[off:off + n].to(torch.int32)
        off += n
    return table, total + 1


def make_cache(cfg: Config, device="cpu", layers: Optional[range] = None):
    """Build the whole cache for `cfg` on `device`.

    Contiguous: k, v [layers, batch, h_kv, max_len, d]; pos int32 [layers, batch, h_kv, max_len]
    holding the slot index (a fresh cache).  Slots at or past a sequence's length hold zeros.
    Paged: k, v [layers, num_blocks, block_size, h_kv, d]; pos int32 [layers, num_blocks, block_size, h_kv];
    block_table int32 [batch, max_blocks].  In both, lengths int32 [batch] and t = lengths (the
    current decode position of a fresh cache).

    With cfg.steady > 0 the cache is the one a recurring pass finds: every sequence holds
    budget + steady slots whose positions come from `steady_positions` (per head, ascending),
    t = t0 + steady with t0 the length drawn as above, and pos holds those positions.  With
    cfg.kept_only the same holds with no new tokens: the cache right after a pass at t0.
    """
    layers = range(cfg.layers) if layers is None else layers
    t0 = lengths_for(cfg)
    if cfg.steady or cfg.kept_only:
        assert cfg.len_lo >= cfg.budget and cfg.budget + cfg.steady <= cfg.max_len
        lengths = torch.full_like(t0, cfg.budget + cfg.steady)
        t = t0 + cfg.steady
    else:
        lengths, t = t0, t0.clone()
    out = {"lengths": lengths.to(device), "t": t.to(device)}
    steady = ((lambda layer, b: steady_positions(cfg, layer, b, int(t0[b]), device))
              if cfg.steady or cfg.kept_only else None)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    nl = len(layers)
    if cfg.layout == "contiguous":
        k = torch.zeros(nl, cfg.batch, cfg.h_kv, cfg.max_len, cfg.d, dtype=dt, device=device)
        v = torch.zeros_like(k)
        pos = torch.arange(cfg.max_len, dtype=torch.int32, device=device).view(1, 1, 1, -1)
        pos = pos.expand(nl, cfg.batch, cfg.h_kv, cfg.max_len).contiguous()
        for i, layer in enumerate(layers):
            mu, scale = _key_centres(cfg, layer, device)
            for b in range(cfg.batch):
                L = int(lengths[b])
                ps = steady(layer, b) if steady else None
                k[i, b, :, :L], v[i, b, :, :L] = _seq_kv(cfg, layer, b, L, device, mu, scale, ps)
                if steady:
                    pos[i, b, :, :L] = ps.to(torch.int32)
        out.update(k=k, v=v, pos=pos)
        return out
    bs = cfg.block_size
    table, nblocks = block_tables(cfg, lengths)
    k = torch.zeros(nl, nblocks, bs, cfg.h_kv, cfg.d, dtype=dt, device=device)
    v = torch.zeros_like(k)
    pos = torch.zeros(nl, nblocks, bs, cfg.h_kv, dtype=torch.int32, device=device)
    # logical slot s of sequence b lives in block table[b, s // bs] at offset s % bs
    phys, slot = [], []
    for b in range(cfg.batch):
        L = int(lengths[b])
        s = torch.arange(L)
        phys.append(table[b, s // bs].to(torch.int64) * bs + s % bs)
        slot.append(s)
    for i, layer in enumerate(layers):
        mu, scale = _key_centres(cfg, layer, device)
        kf, vf = k[i].view(-1, cfg.h_kv, cfg.d), v[i].view(-1, cfg.h_kv, cfg.d)
        pf = pos[i].view(-1, cfg.h_kv)
        for b in range(cfg.batch):
            L = int(lengths[b])
            ps = steady(layer, b) if steady else None
            kl, vl = _seq_kv(cfg, layer, b, L, device, mu, scale, ps)
            idx = phys[b].to(device)
            kf[idx] = kl.transpose(0, 1)
            vf[idx] = vl.transpose(0, 1)
            if steady:
                pf[idx] = ps.transpose(0, 1).to(torch.int32)
            else:
                pf[idx] = slot[b].to(device=device, dtype=torch.int32).view(-1, 1).expand(L, cfg.h_kv)
            del kl, vl
    out.update(k=k, v=v, pos=pos, block_table=table.to(device), num_blocks=nblocks)
    return out
