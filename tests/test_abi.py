"""Host-side checks of the C ABI: the library loads, exports every declared symbol, its structs
have the layout the binding assumes, and argument validation rejects bad input before anything
is enqueued.  No call here reaches the GPU (every call fails validation first)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tri.h")


@pytest.fixture(scope="module")
def T():
    from token_eviction_scoring_amd import build
    build.ensure_built()
    import token_eviction_scoring_amd as T
    return T


def declared_functions():
    """Every function any header under include/ declares."""
    names = set()
    for f in sorted(os.listdir(os.path.dirname(HEADER))):
        if f.endswith(".h"):
            text = open(os.path.join(os.path.dirname(HEADER), f)).read()
            names |= set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s+\**\s*(tri_[a-z_]+)\s*\(", text, re.M))
    return sorted(names)


def test_header_declares_the_pass():
    names = declared_functions()
    for n in ("tri_prepare_centres", "tri_score", "tri_topk", "tri_compact", "tri_evict_step",
              "tri_workspace_bytes", "tri_score_stride", "tri_status_string", "tri_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(T):
    lib = T.lib()
    for n in declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", T.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (tri_\w+)", out))
    # the C ABI is exactly what the headers declare
    assert set(declared_functions()) == exported, exported ^ set(declared_functions())


def test_probe_validation(T):
    lib = T.lib()
    lib.tri_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    lib.tri_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.tri_probe_sink_words.restype = ctypes.c_size_t
    assert lib.tri_probe_sink_words() >= 1
    g = 16384
    for args in ((None, g, 256, None), (256, g, None, None), (8, g, 256, None), (256, 100, 256, None),
                 (256, 0, 256, None)):
        assert lib.tri_probe_read(*args) == 1
        assert b"tri_probe_read" in T.lib().tri_last_error()
    for args in ((None, 256, g, None), (1 << 20, 1 << 20, g, None), (1 << 20, (1 << 20) + g // 2, g, None),
                 (1 << 20, 1 << 24, 100, None), (1 << 20 | 8, 1 << 24, g, None)):
        assert lib.tri_probe_copy(*args) == 1


def test_struct_layout_matches_c(T, tmp_path):
    src = tmp_path / "layout.c"
    fields_c = [f for f, _ in T.CacheStruct._fields_]
    fields_p = [f for f, _ in T.ParamsStruct._fields_]
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "tri.h"', "int main(void){",
             'printf("%zu %zu\\n", sizeof(tri_cache), sizeof(tri_params));']
    lines += [f'printf("%zu\\n", offsetof(tri_cache, {f}));' for f in fields_c]
    lines += [f'printf("%zu\\n", offsetof(tri_params, {f}));' for f in fields_p]
    lines += ["return 0;}"]
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    r = subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                        str(src), "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    vals = subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()
    vals = [int(v) for v in vals]
    assert vals[0] == ctypes.sizeof(T.CacheStruct) and vals[1] == ctypes.sizeof(T.ParamsStruct)
    offs = vals[2:]
    assert offs[:len(fields_c)] == [getattr(T.CacheStruct, f).offset for f in fields_c]
    assert offs[len(fields_c):] == [getattr(T.ParamsStruct, f).offset for f in fields_p]


FAKE = 0x10000  # a non-null, well-aligned address; never dereferenced because validation fails first


def good_cache(T, **kw):
    s = T.CacheStruct()
    s.layout, s.dtype, s.rope = 0, 0, 0
    s.num_layers, s.batch, s.num_kv_heads, s.head_dim, s.max_len = 2, 3, 4, 128, 1000
    s.k, s.v, s.pos = FAKE, FAKE * 2, FAKE * 3
    s.layer_stride, s.stride_b, s.stride_h, s.stride_s = 3 * 4 * 1000 * 128, 4 * 1000 * 128, 1000 * 128, 128
    s.pos_layer_stride, s.pos_stride_b, s.pos_stride_h = 3 * 4 * 1000, 4 * 1000, 1000
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def good_params(T, **kw):
    p = T.ParamsStruct()
    p.u, p.c_hat, p.lengths, p.t = FAKE * 4, FAKE * 5, FAKE * 6, FAKE * 7
    p.rope_theta, p.budget, p.recent = 1e6, 256, 32
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def call_score(T, c, p, scores=FAKE * 8):
    return T.lib().tri_score(ctypes.byref(c) if c is not None else None, ctypes.byref(p) if p is not None else None,
                             scores, None)


BAD_CACHES = [
    ({"layout": 5}, 1), ({"dtype": 7}, 1), ({"rope": 3}, 1), ({"num_layers": 0}, 1), ({"batch": 0}, 1),
    ({"num_kv_heads": 0}, 1), ({"head_dim": 96}, 2), ({"head_dim": 256}, 2), ({"k": 0}, 1), ({"v": 0}, 1),
    ({"pos": 0}, 1), ({"k": FAKE + 8}, 1), ({"pos": FAKE + 2}, 1), ({"stride_s": 100}, 1), ({"stride_s": 64}, 1),
    ({"stride_b": -8}, 1), ({"layer_stride": 3}, 1), ({"max_len": 0}, 1), ({"max_len": 70000}, 2),
]


@pytest.mark.parametrize("kw,code", BAD_CACHES)
def test_bad_cache_rejected(T, kw, code):
    assert call_score(T, good_cache(T, **kw), good_params(T)) == code
    assert T.lib().tri_last_error().decode()


BAD_PARAMS = [({"u": 0}, 1), ({"t": 0}, 1), ({"lengths": FAKE + 1}, 1), ({"budget": 0}, 1), ({"recent": -1}, 1),
              ({"recent": 257}, 1), ({"rope_theta": 0.0}, 1), ({"rope_theta": float("inf")}, 1),
              ({"max_length": -1}, 1), ({"max_length": 1001}, 1), ({"flags": 3}, 1), ({"flags": 4}, 1)]


@pytest.mark.parametrize("kw,code", BAD_PARAMS)
def test_bad_params_rejected(T, kw, code):
    assert call_score(T, good_cache(T), good_params(T, **kw)) == code


def test_null_structs_and_outputs(T):
    assert call_score(T, None, good_params(T)) == 1
    assert call_score(T, good_cache(T), None) == 1
    assert call_score(T, good_cache(T), good_params(T), scores=None) == 1
    assert call_score(T, good_cache(T), good_params(T), scores=FAKE + 4) == 1   # scores need 16-byte alignment


def test_paged_requirements(T):
    c = good_cache(T, layout=1, block_size=16, num_blocks=100, max_blocks_per_seq=10)
    assert call_score(T, c, good_params(T)) == 1            # no block table
    c.block_table = FAKE * 9
    c.max_blocks_per_seq = 5000                              # capacity 80000 > limit
    assert call_score(T, c, good_params(T)) == 2
    c.max_blocks_per_seq = 10
    lib = T.lib()
    p = good_params(T)
    ws = lib.tri_workspace_bytes(ctypes.byref(c), ctypes.byref(p))
    assert ws > 0
    # paged compaction needs the table outputs; contiguous compaction must not get them
    assert lib.tri_compact(ctypes.byref(c), ctypes.byref(p), FAKE, None, None, None, FAKE * 16, ws, None) == 1
    assert lib.tri_compact(ctypes.byref(c), ctypes.byref(p), FAKE, c.block_table, FAKE, FAKE, FAKE * 16, ws, None) == 1
    cc = good_cache(T)
    wsc = lib.tri_workspace_bytes(ctypes.byref(cc), ctypes.byref(p))
    assert lib.tri_compact(ctypes.byref(cc), ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE * 16, wsc, None) == 1


def test_workspace_checks(T):
    lib = T.lib()
    c, p = good_cache(T), good_params(T)
    ws = lib.tri_workspace_bytes(ctypes.byref(c), ctypes.byref(p))
    units = 2 * 3 * 4
    # at least scores (stride 1024 floats per unit), keep (budget ints per unit) and two flags per unit
    assert ws >= units * 1024 * 4 + units * 256 * 4 + units * 2 * 4
    assert ws % 256 == 0
    assert lib.tri_score_stride(ctypes.byref(c)) == 1024
    assert lib.tri_evict_step(ctypes.byref(c), ctypes.byref(p), None, None, FAKE, None, None, None, FAKE * 16, ws - 1, None) == 3
    assert lib.tri_evict_step(ctypes.byref(c), ctypes.byref(p), None, None, FAKE, None, None, None, FAKE * 16 + 64, ws, None) == 1
    assert lib.tri_evict_step(ctypes.byref(c), ctypes.byref(p), None, None, None, None, None, None, FAKE * 16, ws, None) == 1
    # new_lengths must not alias lengths
    assert lib.tri_evict_step(ctypes.byref(c), ctypes.byref(p), None, None, p.lengths, None, None, None, FAKE * 16, ws, None) == 1
    # bad inputs give a zero size
    assert lib.tri_workspace_bytes(ctypes.byref(good_cache(T, head_dim=80)), ctypes.byref(p)) == 0
    # the size grows with every shape parameter
    for field, val in (("num_layers", 4), ("batch", 5), ("num_kv_heads", 8), ("max_len", 3000)):
        c2 = good_cache(T, **{field: val})
        assert lib.tri_workspace_bytes(ctypes.byref(c2), ctypes.byref(p)) > ws
    assert lib.tri_workspace_bytes(ctypes.byref(c), ctypes.byref(good_params(T, budget=512))) > ws


def test_prepare_centres_validation(T):
    lib = T.lib()
    offs = (ctypes.c_int32 * 3)(1, 2, 4)
    po = ctypes.cast(offs, ctypes.c_void_p)
    args = [FAKE, FAKE * 2, 2, 8, 4, 128, 1e6, 0, po, 3, FAKE * 3, FAKE * 4, None]
    def with_(i, v):
        a = list(args)
        a[i] = v
        return lib.tri_prepare_centres(*a)
    assert with_(0, None) == 1
    assert with_(3, 6) == 1      # h_q not a multiple of h_kv
    assert with_(4, 0) == 1
    assert with_(5, 32) == 2
    assert with_(7, 9) == 1
    assert with_(9, 0) == 1
    assert with_(9, 65) == 1
    assert with_(6, -1.0) == 1


def test_status_strings(T):
    lib = T.lib()
    assert [lib.tri_status_string(i).decode() for i in range(5)] == [
        "TRI_OK", "TRI_ERR_INVALID_ARG", "TRI_ERR_UNSUPPORTED", "TRI_ERR_WORKSPACE", "TRI_ERR_HIP"]


def test_binding_refuses_cpu_tensors(T):
    import torch
    k = torch.zeros(1, 1, 1, 64, 64)
    with pytest.raises(T.TriError):
        T.contiguous_cache(k, k.clone(), torch.zeros(1, 1, 1, 64, dtype=torch.int32))


def test_queries_struct_layout_matches_c(T, tmp_path):
    src = tmp_path / "qlayout.c"
    fields = [f for f, _ in T.QueriesStruct._fields_]
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "tri.h"', "int main(void){",
             'printf("%zu\\n", sizeof(tri_queries));']
    lines += [f'printf("%zu\\n", offsetof(tri_queries, {f}));' for f in fields]
    lines += ["return 0;}"]
    src.write_text("\n".join(lines))
    exe = tmp_path / "qlayout"
    r = subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                        str(src), "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    vals = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(T.QueriesStruct)
    assert vals[1:] == [getattr(T.QueriesStruct, f).offset for f in fields]


def good_queries(T, **kw):
    q = T.QueriesStruct()
    q.dtype, q.rope, q.num_layers, q.num_heads, q.head_dim, q.n = 0, 0, 2, 4, 128, 3000
    q.q = FAKE
    q.stride_l, q.stride_n, q.stride_h = 3000 * 4 * 128, 4 * 128, 128
    for k, v in kw.items():
        setattr(q, k, v)
    return q


BAD_QUERIES = [({"dtype": 2}, 1), ({"rope": 2}, 1), ({"num_layers": 0}, 1), ({"num_heads": 0}, 1), ({"n": 0}, 1),
               ({"head_dim": 96}, 2), ({"reserved": 1}, 1), ({"q": 0}, 1), ({"q": FAKE + 8}, 1),
               ({"stride_n": 100}, 1), ({"stride_h": -128}, 1)]


@pytest.mark.parametrize("kw,code", BAD_QUERIES)
def test_bad_queries_rejected(T, kw, code):
    q = good_queries(T, **kw)
    assert T.lib().tri_calibrate_workspace_bytes(ctypes.byref(q)) == 0
    assert T.lib().tri_calibrate(ctypes.byref(q), FAKE * 2, FAKE * 3, FAKE * 4, 1 << 30, None) == code
    assert T.lib().tri_last_error().decode()


def test_calibrate_workspace_and_outputs(T):
    q = good_queries(T)
    need = T.lib().tri_calibrate_workspace_bytes(ctypes.byref(q))
    assert need >= 2 * 4 * 192 * 8 and need % 256 == 0      # float64 partial sums: 3d/2 per (layer, head, chunk)
    assert T.lib().tri_calibrate(ctypes.byref(q), FAKE * 2, FAKE * 3, FAKE * 4, need - 1, None) == 3
    assert T.lib().tri_calibrate(ctypes.byref(q), None, FAKE * 3, FAKE * 4, need, None) == 1
    assert T.lib().tri_calibrate(ctypes.byref(q), FAKE * 2, FAKE * 3, FAKE + 16, need, None) == 1


def test_decode_validation(T):
    c = good_cache(T)       # 4 KV heads, capacity 1000, d 128
    lib = T.lib()
    need = lib.tri_decode_workspace_bytes(ctypes.byref(c), 16, 1000)
    assert need > 0 and need % 256 == 0
    ok = (ctypes.byref(c), FAKE * 2, 1000, FAKE * 3, 16, ctypes.c_float(0.088), FAKE * 4, FAKE * 5, need, None)
    bad = [
        ((ok[0], None) + ok[2:], 1),                       # lengths NULL
        (ok[:2] + (0,) + ok[3:], 1),                       # max_length 0
        (ok[:2] + (1001,) + ok[4 - 1:], 1),                # max_length above capacity
        (ok[:3] + (FAKE + 8,) + ok[4:], 1),                # q misaligned
        (ok[:4] + (18,) + ok[5:], 1),                      # h_q not a multiple of the KV heads
        (ok[:4] + (12,) + ok[5:], 2),                      # 3 query heads per KV head
        (ok[:5] + (ctypes.c_float(float("nan")),) + ok[6:], 1),
        (ok[:6] + (None,) + ok[7:], 1),                    # out NULL
        (ok[:8] + (need - 1,) + ok[9:], 3),                # workspace too small
    ]
    for args, code in bad:
        assert lib.tri_decode_attention(*args) == code, (args, code)
        assert lib.tri_last_error().decode()
    assert lib.tri_decode_workspace_bytes(ctypes.byref(c), 16, 0) == 0
