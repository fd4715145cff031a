"""Benchmark of the TriAttention KV-cache eviction pass on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload paged_8b] [--no-cpu-baseline]

The default workload is the largest single-GPU one: the paged serving-style cache on the Qwen3-8B shape (64
sequences of 2048..32768 tokens, 16-token blocks, 36 layers), first pass.  Other workloads: qwen3_8b, ragged_8b,
qwen3_32b, the steady-state and variant workloads of synth.CONFIGS, decode_paged_8b_kept, calib_qwen3_8b, and the
attainable-bandwidth probes hbm_read / hbm_copy.

One step = one whole pass (score every cached key, select the kept slots, compact K/V/pos in
place) over all layers of one synthetic cache resident in HBM.  Because compaction rewrites the
cache, every step starts from an untimed device-to-device restore of exactly the slots a pass
overwrites (the first `budget` slots of each unit), so each timed step is the first pass over the
same generated cache.  The restore is followed by an untimed read of a 1 GiB buffer, which writes
back the restored data and leaves the 256 MB Infinity Cache holding unrelated clean lines, so each
timed pass starts from cold caches.  The pass is timed with HIP events recorded by the library on the stream its
kernels run on: the whole pass (tri_evict_step) and, in separate passes of the same launch sequence
(tri_evict_step_profiled, which records events between its kernels), the scoring kernel and the selection and
compaction after it.

Prints one JSON line.  value = KV tokens (key vectors of all layers and heads) scored+compacted per
second; roofline = the scoring kernel (the dominant byte stream) against the 8 TB/s HBM peak.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "KV tokens scored+compacted/s (bf16, d=128); achieved HBM GB/s vs peak"
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SRC = os.path.join(ROOT, "token_eviction_scoring_amd", "csrc", "kernels.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="paged_8b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample (calibration and decode workloads)")
    ap.add_argument("--cpu-keys", type=int, default=24_000_000,
                    help="key vectors in the CPU oracle's all-core sample (the pass workloads)")
    ap.add_argument("--unfused", action="store_true",
                    help="run short caches as three kernels instead of the fused pass (for comparison)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB elementwise copy (for scaling HBM byte counters)")
    return ap.parse_args()


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch loaded (same library the kernels use)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(h)) == 0
            self.ev.append(h.value)

    def record(self, i, stream):
        assert self.hip.hipEventRecord(self.ev[i], stream) == 0

    def ms(self, a, b):
        self.hip.hipEventSynchronize(b)
        f = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(f), a, b) == 0
        return f.value


def source_hash():
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def read_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary, if it was taken on
    the current kernel source; else None."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != source_hash():
        return None
    try:
        return float(kv.get("hbm_bytes_per_launch", kv.get("score_hbm_bytes_per_launch")))
    except (KeyError, ValueError, TypeError):
        return None


def restore_fn(cfg, cache, torch):
    """Copy of the slots a pass overwrites, and a function that writes them back."""
    B = cfg.budget
    if cfg.layout == "contiguous":
        n = min(B, cfg.max_len)
        saved = [cache[x][..., :n, :].clone() for x in ("k", "v")] + [cache["pos"][..., :n].clone()]

        def restore():
            cache["k"][..., :n, :].copy_(saved[0])
            cache["v"][..., :n, :].copy_(saved[1])
            cache["pos"][..., :n].copy_(saved[2])
        return restore
    bs = cfg.block_size
    lengths = cache["lengths"].cpu().tolist()
    table = cache["block_table"].cpu()
    idx = torch.cat([table[b, :-(-min(L, B) // bs)] for b, L in enumerate(lengths) if L > B]).long().cuda()
    saved = [cache[x].index_select(1, idx) for x in ("k", "v", "pos")]

    def restore():
        for x, s in zip(("k", "v", "pos"), saved):
            cache[x].index_copy_(1, idx, s)
    return restore


def algorithmic_bytes(cfg, lengths):
    """Per pass: read every cached key (L*d*e per unit); read+write the kept K and V rows (4*B'*d*e)
    and positions (8*B'), B' = min(L, budget) where the unit is evicted (L > budget), else 0."""
    e = 2 if cfg.dtype == "bf16" else 4
    per_layer_head = 0
    k_read = 0
    for L in lengths:
        k_read += L * cfg.d * e
        Bp = min(L, cfg.budget) if L > cfg.budget else 0
        per_layer_head += 4 * Bp * cfg.d * e + 8 * Bp
    scale = cfg.layers * cfg.h_kv
    return k_read * scale, (k_read + per_layer_head) * scale


def unit_rows_host(cfg, cache, torch, l, b, L):
    """Host copies of the K, V rows (bf16 bits as uint16) and positions of every KV head of (layer l, sequence b):
    [H, L, d], [H, L, d], [H, L]; paged pools are gathered through the block table on the GPU."""
    if cfg.layout == "paged":
        bs = cfg.block_size
        blocks = cache["block_table"][b, :(L + bs - 1) // bs].long()
        k = cache["k"][l, blocks].reshape(-1, cfg.h_kv, cfg.d)[:L].transpose(0, 1)
        v = cache["v"][l, blocks].reshape(-1, cfg.h_kv, cfg.d)[:L].transpose(0, 1)
        p = cache["pos"][l, blocks].reshape(-1, cfg.h_kv)[:L].transpose(0, 1)
    else:
        k, v, p = cache["k"][l, b, :, :L], cache["v"][l, b, :, :L], cache["pos"][l, b, :, :L]
    as16 = lambda x: x.contiguous().view(torch.int16).cpu().numpy().view("uint16")
    return as16(k), as16(v), p.contiguous().cpu().numpy()


def cpu_baseline(cfg, cache, qbar, c, torch, target_keys):
    """The float64 C oracle of the pass (collapsed form: one dot product and the norm term per key, exact
    selection, gather of the kept K/V/pos rows; OpenMP over units) on a bounded sample of the same cache: the units
    of the first layers, about `target_keys` key vectors, with every host core; then the first eighth of those
    units with one thread.  Centre vectors come from the NumPy oracle (once per layer and head, untimed)."""
    import numpy as np
    import oracle
    from oracle import cpass
    cores = len(os.sched_getaffinity(0))
    lengths = cache["lengths"].cpu().tolist()
    t_seq = cache["t"].cpu().tolist()
    keys_per_layer = sum(lengths) * cfg.h_kv
    n_layers = max(1, min(cfg.layers, round(target_keys / max(keys_per_layer, 1))))
    K, V, P, lens, us, chats, ts = [], [], [], [], [], [], []
    for l in range(n_layers):
        q_l, c_l = qbar[l].double().numpy(), c[l].double().numpy()
        u_h = [oracle.centre_vector(oracle.group_rows(q_l, h, cfg.group), cfg.theta, cfg.offsets, cfg.rope)
               for h in range(cfg.h_kv)]
        c_h = [oracle.group_rows(c_l, h, cfg.group).mean(axis=0) for h in range(cfg.h_kv)]
        for b, L in enumerate(lengths):
            k, v, p = unit_rows_host(cfg, cache, torch, l, b, L)
            for h in range(cfg.h_kv):
                K.append(k[h]), V.append(v[h]), P.append(p[h])
                lens.append(L), us.append(u_h[h]), chats.append(c_h[h]), ts.append(t_seq[b])
    K, V, P = np.concatenate(K), np.concatenate(V), np.concatenate(P)
    us, chats = np.stack(us), np.stack(chats)
    args = (cfg.theta, cfg.budget, cfg.recent, cfg.rope)

    def timed(n, threads):
        r = int(sum(lens[:n]))
        t0 = time.perf_counter()
        cpass.pass_units(K[:r], V[:r], P[:r], lens[:n], us[:n], chats[:n], ts[:n], *args, threads=threads)
        return r / (time.perf_counter() - t0), r

    n_all = len(lens)
    v_all, keys_all = timed(n_all, cores)
    n_one = max(1, n_all // 8)
    v_one, keys_one = timed(n_one, 1)
    return {"value": v_all, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "value_1_thread": v_one,
            "sample": f"float64 C oracle of the pass (collapsed form, exact selection, gather; OpenMP over units): "
                      f"{n_all} units of the first {n_layers} of {cfg.layers} layers ({keys_all} key vectors) on "
                      f"{cores} threads; the first {n_one} of them ({keys_one} key vectors) on 1 thread"}


# Attainable-bandwidth probes ("hbm_read", "hbm_copy"): the plain read and copy kernels of include/tri_probe.h over
# buffers far larger than the caches.  Not the eviction pass; reported in the same JSON form with their own metric.
PROBE_METRIC = "attainable HBM bandwidth of a plain {} kernel (16-byte non-temporal accesses)"


def bench_probe(args, torch, T):
    kind = args.workload[len("hbm_"):]
    n = 8 << 30 if kind == "read" else 4 << 30
    src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src) if kind == "copy" else None
    sink = torch.empty(T.lib().tri_probe_sink_words(), dtype=torch.int32, device="cuda")
    ev = HipEvents(2)
    stream = torch.cuda.current_stream().cuda_stream

    def step():
        ev.record(0, stream)
        if kind == "read":
            T.tri_probe_read(src, sink)
        else:
            T.tri_probe_copy(dst, src)
        ev.record(1, stream)
        return ev.ms(ev.ev[0], ev.ev[1])

    for _ in range(args.warmup):
        step()
    times = [step() for _ in range(args.steps)]
    torch.cuda.synchronize()
    if kind == "copy":
        assert torch.equal(dst[:1 << 20], src[:1 << 20])
    ms = statistics.mean(times)
    moved = n if kind == "read" else 2 * n
    gbs = moved / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": PROBE_METRIC.format(kind), "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u8", "data": "synthetic",
        "config": {"workload": args.workload, "bytes_moved_per_launch": moved},
        "roofline": {"bound": "hbm", "kernel": f"k_probe_{kind}", "achieved": gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes_per_launch": moved, "avg_launch_ms": ms},
        "pass": {"ms_mean": ms, "ms_median": statistics.median(times), "ms_min": min(times)},
        "cpu_baseline": None}), flush=True)


# Calibration workloads: the statistics pass over n calibration tokens of a model shape (workload name
# "calib_<shape>").  Not the eviction pass; reported in the same JSON form with its own metric.
CALIB_TOKENS = 32768
CALIB_METRIC = "calibration queries reduced/s (bf16, d=128); achieved HBM GB/s vs peak"


def bench_calibration(args, torch, synth, T):
    import numpy as np
    cfg = synth.CONFIGS[args.workload[len("calib_"):]]
    n = CALIB_TOKENS
    print(f"[bench] generating {n} calibration queries of {cfg.name}", file=sys.stderr, flush=True)
    q = synth.calibration_queries(cfg, n, device="cuda")
    s = T.queries_struct(q, cfg.rope)
    qbar = torch.empty(cfg.layers, cfg.h_q, cfg.d, dtype=torch.float32, device="cuda")
    c = torch.empty(cfg.layers, cfg.h_q, cfg.d // 2, dtype=torch.float32, device="cuda")
    ws = torch.empty(T.lib().tri_calibrate_workspace_bytes(ctypes.byref(s)), dtype=torch.uint8, device="cuda")
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    ev = HipEvents(2)
    stream = torch.cuda.current_stream().cuda_stream

    def step():
        flush_buf.sum()
        ev.record(0, stream)
        T.tri_calibrate(q, cfg.rope, qbar, c, ws)
        ev.record(1, stream)
        return ev.ms(ev.ev[0], ev.ev[1])

    for _ in range(args.warmup):
        step()
    times = [step() for _ in range(args.steps)]
    torch.cuda.synchronize()
    ms = statistics.mean(times)
    vectors = cfg.layers * n * cfg.h_q
    bytes_read = q.numel() * q.element_size()
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        rng = np.random.default_rng(0)
        spent, done = 0.0, 0
        while spent < args.cpu_seconds and done < cfg.layers * cfg.h_q:
            l, h = int(rng.integers(cfg.layers)), int(rng.integers(cfg.h_q))
            Q = q[l, :, h].double().cpu().numpy()
            t0 = time.perf_counter()
            oracle.calibration_stats(Q, cfg.rope)
            spent += time.perf_counter() - t0
            done += 1
        cpu = {"value": done * n / spent, "unit": "queries/s", "cores": os.cpu_count(), "kind": "oracle",
               "sample": f"{done} (layer, head) pairs x {n} queries, float64 NumPy oracle, {spent:.1f} s"}
    gbs = bytes_read / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": CALIB_METRIC, "value": vectors / (ms * 1e-3), "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "config": {"workload": args.workload, "layers": cfg.layers, "query_heads": cfg.h_q, "head_dim": cfg.d,
                   "calibration_tokens": n, "q_dtype": cfg.dtype},
        "roofline": {"bound": "hbm", "kernel": "k_calib_partial + k_calib_finish", "achieved": gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": read_traffic("k_calib_partial", args.workload),
                     "algorithmic_bytes_per_launch": bytes_read, "avg_launch_ms": ms},
        "pass": {"ms_mean": ms, "ms_median": statistics.median(times), "ms_min": min(times)},
        "cpu_baseline": cpu}), flush=True)


# Decode-attention workloads ("decode_<cache>"): one decode step of attention over every layer of a cache as the
# pass leaves it.  Not the eviction pass; reported in the same JSON form with its own metric.
DECODE_METRIC = "decode attention: kept KV tokens attended/s (bf16, d=128); achieved HBM GB/s vs peak"


def bench_decode(args, torch, synth, T):
    import numpy as np
    cfg = synth.CONFIGS[args.workload[len("decode_"):]]
    print(f"[bench] generating {cfg.name} on the GPU", file=sys.stderr, flush=True)
    cache = synth.make_cache(cfg, device="cuda")
    q = synth.decode_queries(cfg, cache["t"], device="cuda")
    tc = (T.paged_cache(cache["k"], cache["v"], cache["pos"], cache["block_table"], cfg.rope)
          if cfg.layout == "paged" else T.contiguous_cache(cache["k"], cache["v"], cache["pos"], cfg.rope))
    lengths = cache["lengths"].cpu().tolist()
    max_length = max(lengths)
    scale = 1.0 / np.sqrt(cfg.d)
    out = torch.empty(cfg.layers, cfg.batch, cfg.h_q, cfg.d, dtype=torch.float32, device="cuda")
    ws = torch.empty(T.lib().tri_decode_workspace_bytes(ctypes.byref(tc.struct), cfg.h_q, max_length),
                     dtype=torch.uint8, device="cuda")
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    ev = HipEvents(2)
    stream = torch.cuda.current_stream().cuda_stream

    def step():
        flush_buf.sum()
        ev.record(0, stream)
        T.tri_decode_attention(tc, cache["lengths"], q, scale, max_length, out, ws)
        ev.record(1, stream)
        return ev.ms(ev.ev[0], ev.ev[1])

    for _ in range(args.warmup):
        step()
    times = [step() for _ in range(args.steps)]
    torch.cuda.synchronize()
    ms = statistics.mean(times)
    e = 2 if cfg.dtype == "bf16" else 4
    tokens = sum(lengths) * cfg.layers * cfg.h_kv
    alg = tokens * 2 * cfg.d * e + q.numel() * e + out.numel() * 4
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        rng = np.random.default_rng(0)
        spent, done, toks = 0.0, 0, 0
        G = cfg.group
        while spent < args.cpu_seconds and done < cfg.layers * cfg.batch * cfg.h_kv:
            l, b, h = int(rng.integers(cfg.layers)), int(rng.integers(cfg.batch)), int(rng.integers(cfg.h_kv))
            L = lengths[b]
            s_ = torch.arange(L, device="cuda")
            blk = cache["block_table"][b].long()[s_ // cfg.block_size] if cfg.layout == "paged" else None
            K = (cache["k"][l, blk, s_ % cfg.block_size, h] if blk is not None else cache["k"][l, b, h, :L]).double().cpu().numpy()
            V = (cache["v"][l, blk, s_ % cfg.block_size, h] if blk is not None else cache["v"][l, b, h, :L]).double().cpu().numpy()
            qg = q[l, b, h * G:(h + 1) * G].double().cpu().numpy()
            t0 = time.perf_counter()
            oracle.decode_attention(qg, K, V, scale)
            spent += time.perf_counter() - t0
            done += 1
            toks += L
        cpu = {"value": toks / spent, "unit": "tokens/s", "cores": os.cpu_count(), "kind": "oracle",
               "sample": f"{done} units ({toks} kept key/value rows), float64 NumPy oracle, {spent:.1f} s"}
    gbs = alg / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": DECODE_METRIC, "value": tokens / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": args.workload, "layers": cfg.layers, "batch": cfg.batch, "kv_heads": cfg.h_kv,
                   "query_heads": cfg.h_q, "head_dim": cfg.d, "kv_dtype": cfg.dtype, "layout": cfg.layout,
                   "kept_tokens_per_seq": max_length},
        "roofline": {"bound": "hbm", "kernel": "k_decode_partial + k_decode_combine", "achieved": gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": read_traffic("k_decode_partial", args.workload),
                     "algorithmic_bytes_per_launch": alg, "avg_launch_ms": ms},
        "pass": {"ms_mean": ms, "ms_median": statistics.median(times), "ms_min": min(times)},
        "cpu_baseline": cpu}), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the pass is measured on one GPU only (it has no cross-GPU step); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    import token_eviction_scoring_amd as T
    from token_eviction_scoring_amd import build
    build.ensure_built()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.workload.startswith("calib_"):
        return bench_calibration(args, torch, synth, T)
    if args.workload.startswith("decode_"):
        return bench_decode(args, torch, synth, T)
    if args.workload.startswith("hbm_"):
        return bench_probe(args, torch, T)
    cfg = synth.CONFIGS[args.workload]
    print(f"[bench] generating {cfg.name} on the GPU", file=sys.stderr, flush=True)
    cache = synth.make_cache(cfg, device="cuda")
    qbar, c = synth.query_side(cfg)
    u, c_hat = T.tri_prepare_centres(qbar.cuda(), c.cuda(), cfg.h_kv, cfg.theta, cfg.offsets, cfg.rope)
    # the serving engine knows its sequences' lengths on the host: pass the bound that sizes the launches
    max_length = int(cache["lengths"].max())
    variant = None
    if cfg.aggregation != "mean":   # a non-collapsible score: every logit on the matrix cores
        centres = T.tri_prepare_variant_centres(qbar.cuda(), cfg.h_kv, cfg.theta, cfg.offsets, cfg.rope)
        variant = T.Variant(centres, {"max": T.AGG_MAX, "head_max": T.AGG_HEAD_MAX}[cfg.aggregation], cfg.group,
                            len(cfg.offsets))
    params = T.Params(u, c_hat, cfg.theta, cache["lengths"], cache["t"], cfg.budget, cfg.recent, max_length,
                      T.PASS_UNFUSED if args.unfused else 0, variant)
    tc = (T.paged_cache(cache["k"], cache["v"], cache["pos"], cache["block_table"], cfg.rope)
          if cfg.layout == "paged" else T.contiguous_cache(cache["k"], cache["v"], cache["pos"], cfg.rope))
    ws = torch.empty(T.tri_workspace_bytes(tc, params), dtype=torch.uint8, device="cuda")
    new_lengths = torch.empty(cfg.batch, dtype=torch.int32, device="cuda")
    lengths = cache["lengths"].cpu().tolist()
    tokens = sum(lengths) * cfg.layers * cfg.h_kv
    k_bytes, alg_bytes = algorithmic_bytes(cfg, lengths)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg, cache, qbar, c, torch, args.cpu_keys)

    restore = restore_fn(cfg, cache, torch)
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    ev = HipEvents(4)
    outs = {}
    paged_out = {}
    if cfg.layout == "paged":
        bs = cfg.block_size
        paged_out = dict(block_table_out=torch.empty(cfg.batch, -(-cfg.budget // bs), dtype=torch.int32, device="cuda"),
                         freed=torch.empty(cfg.batch * cache["block_table"].shape[1], dtype=torch.int32, device="cuda"),
                         n_freed=torch.empty(1, dtype=torch.int32, device="cuda"))

    stream = torch.cuda.current_stream().cuda_stream

    def prepare():
        restore()
        flush_buf.sum()

    def step():
        """One timed pass: tri_evict_step bracketed by events recorded on the stream it runs on."""
        prepare()
        ev.record(0, stream)
        outs.update(T.tri_evict_step(tc, params, ws=ws, new_lengths=new_lengths, **paged_out))
        ev.record(3, stream)
        return ev.ms(ev.ev[0], ev.ev[3])

    def profiled_step():
        """One pass with an event between its kernels (for the per-kernel roofline)."""
        prepare()
        outs.update(T.tri_evict_step_profiled(tc, params, ev.ev, ws=ws, new_lengths=new_lengths, **paged_out))
        return [ev.ms(ev.ev[0], ev.ev[3]), ev.ms(ev.ev[0], ev.ev[1]), ev.ms(ev.ev[1], ev.ev[2]),
                ev.ms(ev.ev[2], ev.ev[3])]

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    pass_ms = []
    w0 = time.perf_counter()
    for _ in range(args.steps):
        pass_ms.append(step())
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    print("[bench] per-kernel profile", file=sys.stderr, flush=True)
    profiled_step()
    times = [profiled_step() for _ in range(max(3, min(args.steps, 10)))]
    serial_ms = [t[0] for t in times]
    score_ms = [t[1] for t in times]
    select_ms = [t[2] for t in times]
    compact_ms = [t[3] for t in times]
    ms = statistics.mean(pass_ms)
    t_score = statistics.mean(score_ms)

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1, out=dst)
        torch.cuda.synchronize()

    # Caches within the fused pass's limits run as one kernel (k_fused): its roofline covers the whole pass.
    bs = cfg.block_size
    units = cfg.layers * cfg.batch * cfg.h_kv
    fused = variant is None and not args.unfused and units >= T.FUSED_MIN_UNITS and max_length <= T.FUSED_MAX_LEN and (cfg.layout != "paged" or -(-max_length // bs) <= T.FUSED_MAX_BLOCKS)
    kernel, kernel_bytes = ("k_fused", alg_bytes) if fused else ("k_score_var" if variant else "k_score", k_bytes)
    # budgets up to 8192 slots: one kernel selects and compacts each unit; larger ones take two
    path = "fused" if fused else ("score, select+compact" if cfg.budget <= 8192 and units >= 1024
                                  else "score, select, compact")
    traffic = read_traffic(kernel, cfg.name)
    ach = kernel_bytes / (t_score * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": cfg.name,
            "layers": cfg.layers, "batch": cfg.batch, "kv_heads": cfg.h_kv, "query_heads": cfg.h_q,
            "head_dim": cfg.d, "kv_dtype": cfg.dtype, "layout": cfg.layout, "cache_tokens_per_seq": lengths,
            "budget": cfg.budget, "recent": cfg.recent, "rope_theta": cfg.theta, "n_offsets": len(cfg.offsets),
            "key_vectors_per_pass": tokens, "max_length_bound": max_length,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "achieved": ach,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": ach / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": kernel_bytes,
            "avg_launch_ms": t_score,
        },
        "pass": {
            "algorithmic_bytes": alg_bytes,
            "gbps": alg_bytes / (ms * 1e-3) / 1e9,
            "frac_of_peak": alg_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "ms_mean": ms, "ms_median": statistics.median(pass_ms), "ms_min": min(pass_ms),
            "profiled_pass_ms": statistics.mean(serial_ms),
            "path": path,
            "score_ms": t_score, "select_compact_ms": statistics.mean(select_ms) + statistics.mean(compact_ms),
            "wall_ms_per_step_incl_restore_and_flush": wall * 1e3 / args.steps,
        },
        "cpu_baseline": cpu,
    }
    if variant is not None:
        # matrix-core work of the variant scoring kernel: per key 2 (bf16 high part and residual) x 64 or 128
        # columns x d multiply-adds issued, of which G x |D| columns are real
        issued = 2 * T.tri_variant_columns(cfg.group, len(cfg.offsets)) * cfg.d * 2 * tokens
        useful = 2 * cfg.group * len(cfg.offsets) * cfg.d * 2 * tokens
        tf = issued / (t_score * 1e-3) / 1e12
        line["mfma"] = {"dtype": "bf16", "issued_tflops": tf, "peak_tflops": 2500.0, "frac": tf / 2500.0,
                        "useful_tflops": useful / (t_score * 1e-3) / 1e12, "aggregation": cfg.aggregation}
        line["config"]["aggregation"] = cfg.aggregation
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
