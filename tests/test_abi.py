"""The C-ABI library loads, exports every entry point include/fp8kv.h
declares, and its host-only entry points behave as documented (CPU only: no
call here reaches the GPU)."""
import ctypes
import os
import re

import numpy as np

import decode_attention_paged_fp8kv_amd as fp8kv
from _helpers import tile_index

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8kv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8kv_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 18, names
    lib = ctypes.CDLL(fp8kv.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings():
    assert fp8kv.status_string(0) == "ok"
    assert fp8kv.status_string(-4) == "workspace too small"
    assert fp8kv.status_string(123) == "unknown status"


def test_cache_bytes_and_layout_formula():
    for dt, tb in ((fp8kv.E4M3, 2048), (fp8kv.BF16, 4096)):
        d = fp8kv.desc(10, 3, dt)
        assert fp8kv.cache_bytes(d) == 10 * 3 * tb
        eb = 1 if dt == fp8kv.E4M3 else 2
        for is_v in (0, 1):
            idx = tile_index(bool(is_v), eb)  # written independently from the header text
            for page, h in ((0, 0), (7, 2)):
                base = (page * 3 + h) * tb
                for slot in (0, 3, 4, 15):
                    for dim in (0, 7, 8, 31, 32, 77, 127):
                        off = fp8kv.cache_offset(d, is_v, page, h, slot, dim)
                        assert off == base + eb * idx[slot, dim], (dt, is_v, slot, dim)
    d = fp8kv.desc(4, 2)
    assert fp8kv.cache_offset(d, 0, 4, 0, 0, 0) == -1
    assert fp8kv.cache_offset(d, 0, 0, 0, 16, 0) == -1
    assert fp8kv.cache_offset(d, 1, 0, 0, 0, 128) == -1
    # every byte of a tile is addressed exactly once, for K and for V
    for dt in (fp8kv.E4M3, fp8kv.BF16):
        d = fp8kv.desc(1, 1, dt)
        for is_v in (0, 1):
            offs = {fp8kv.cache_offset(d, is_v, 0, 0, s, k) for s in range(16) for k in range(128)}
            assert len(offs) == 16 * 128


def _lib():
    return fp8kv.raw_library()


def test_argument_validation_before_any_device_call():
    lib = _lib()
    P = ctypes.c_void_p
    bad = fp8kv.CacheDesc(8, 32, 2, 128, 0)         # page_size 32 unsupported
    ok = fp8kv.desc(8, 2)
    fake = P(16)                                     # never dereferenced: calls fail first
    f = lib.fp8kv_decode_attention
    args_tail = [ctypes.c_int32(8), fake, ctypes.c_int32(4), fake, ctypes.c_int32(2),
                 ctypes.c_float(0.1), None, fake, ctypes.c_int32(0), ctypes.c_int32(0), fake,
                 ctypes.c_size_t(1 << 20), None]
    assert f(ctypes.byref(bad), fake, fake, fake, fake, fake, *args_tail) == -2
    # Hq not a multiple of Hkv
    t2 = list(args_tail)
    t2[0] = ctypes.c_int32(7)
    assert f(ctypes.byref(ok), fake, fake, fake, fake, fake, *t2) == -2
    # G > 32
    t3 = list(args_tail)
    t3[0] = ctypes.c_int32(66)
    assert f(ctypes.byref(ok), fake, fake, fake, fake, fake, *t3) == -2
    # null output
    t4 = list(args_tail)
    t4[7] = None
    assert f(ctypes.byref(ok), fake, fake, fake, fake, fake, *t4) == -1
    # empty batch is a no-op
    t5 = list(args_tail)
    t5[4] = ctypes.c_int32(0)
    assert f(ctypes.byref(ok), fake, fake, fake, fake, fake, *t5) == 0
    # bad output dtype
    t6 = list(args_tail)
    t6[8] = ctypes.c_int32(5)
    assert f(ctypes.byref(ok), fake, fake, fake, fake, fake, *t6) == -1
    # append: negative token count, missing scales for e4m3
    a = lib.fp8kv_append
    assert a(ctypes.byref(ok), fake, fake, fake, fake, fake, fake, ctypes.c_int32(-1), fake, fake,
             ctypes.c_int32(1), fake, ctypes.c_int32(4), None, None) == -1
    assert a(ctypes.byref(ok), fake, fake, None, fake, fake, fake, ctypes.c_int32(3), fake, fake,
             ctypes.c_int32(1), fake, ctypes.c_int32(4), None, None) == -1
    assert a(ctypes.byref(ok), fake, fake, fake, fake, fake, fake, ctypes.c_int32(0), fake, fake,
             ctypes.c_int32(1), fake, ctypes.c_int32(4), None, None) == 0
    # tag check: missing abort output
    v = lib.fp8kv_verify_tags
    assert v(fake, fake, ctypes.c_int32(4), fake, ctypes.c_int32(2), fake, ctypes.c_int32(8),
             ctypes.c_int32(16), None, None) == -1
    assert v(fake, fake, ctypes.c_int32(4), fake, ctypes.c_int32(0), fake, ctypes.c_int32(8),
             ctypes.c_int32(16), None, None) == 0
    # fused check + append: too many kv-heads for one workgroup
    va = lib.fp8kv_verify_append
    big = fp8kv.desc(8, 17)
    assert va(ctypes.byref(big), fake, fake, fake, fake, fake, fake, fake, fake, fake,
              ctypes.c_int32(4), fake, ctypes.c_int32(2), fake, fake, None) == -2


def test_workspace_size_grows_with_workers_and_batch():
    # explicit worker counts need no device query
    d = fp8kv.desc(100, 8)
    s1 = fp8kv.decode_workspace_size(d, 64, 64, 3072)
    s2 = fp8kv.decode_workspace_size(d, 64, 64, 6144)
    s3 = fp8kv.decode_workspace_size(d, 128, 64, 3072)
    assert 0 < s1 < s2 and s1 < s3
    # slots = workgroups + segments, each G heads x (128 + 2) floats, plus B+1 prefix ints
    G, slots = 8, 3072 // 4 + 64 * 8
    assert s1 >= slots * G * 130 * 4 + 65 * 4
    assert fp8kv.decode_num_workers(10) == 12
    assert fp8kv.decode_workspace_size(fp8kv.desc(100, 8), 4, 60, 64) == 0  # Hq % Hkv != 0


def test_multi_query_column_limit():
    # (Hq / Hkv) * q_len (query, head) pairs per kv-head: at most two 16-column tiles
    d = fp8kv.desc(100, 8)
    ws = fp8kv.decode_workspace_size_q
    one = ws(d, 4, 64, 1, 64)
    assert one == fp8kv.decode_workspace_size(d, 4, 64, 64)
    assert ws(d, 4, 64, 2, 64) > one                 # 16 columns
    assert ws(d, 4, 64, 4, 64) > ws(d, 4, 64, 3, 64)  # 32 > 24 columns
    assert ws(d, 4, 64, 5, 64) == 0                  # 40 columns
    assert ws(fp8kv.desc(100, 2), 4, 64, 1, 64) > 0   # G = 32
    assert ws(fp8kv.desc(100, 2), 4, 66, 1, 64) == 0  # G = 33
    assert ws(d, 4, 64, 0, 64) == 0                  # no query


def test_prepared_launch_checks_once_and_keeps_its_tensors():
    import torch
    # arguments are checked when the launch is prepared, before any device call
    cpu = torch.zeros(4, dtype=torch.int32)
    try:
        fp8kv.verify_tags(cpu.view(1, 4), cpu.view(1, 4), cpu[:1], cpu, prepare=True)
    except ValueError as e:
        assert "device tensor" in str(e)
    else:
        raise AssertionError("a host tensor was accepted")
    # a prepared launch holds the tensors its pointers refer to
    assert "_keep" in fp8kv.Launch.__slots__


def test_shared_prompt_workspace():
    # the shared-prompt call's workspace: the plain decode's plus the prompts'
    # partial states, the own-token rows and views; groups are checked
    d = fp8kv.desc(4096, 8)
    ws = fp8kv.decode_workspace_size_shared
    plain = fp8kv.decode_workspace_size(d, 64, 64, 3072)
    assert ws(d, 64, 64, 1100, [0, 64], [0], 3072) == plain
    assert ws(d, 64, 64, 1100, [0], [], 3072) == plain
    a, b = ws(d, 64, 64, 1100, [0, 64], [1024], 3072), ws(d, 64, 64, 1100, [0, 64], [16384], 3072)
    assert plain < a <= b
    assert a >= plain + 64 * 64 * (128 + 2) * 4 + 64 * 64 * (128 + 1) * 4 + 64 * 1100 * 4
    two = ws(d, 64, 64, 1100, [0, 30, 64], [1024, 2048], 3072)
    assert two > plain
    for gs, pl in (([0, 64], [8]), ([0, 64], [-16]), ([0, 64], [16 * 1101]), ([0, 70], [16]),
                   ([10, 5], [16]), ([-1, 5], [16]), ([0] * 34, [16] * 33)):
        assert ws(d, 64, 64, 1100, gs, pl, 3072) == 0, (gs, pl)
    assert ws(d, 64, 66, 1100, [0, 64], [1024], 3072) == 0          # Hq % Hkv != 0
