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
    # a table so wide that the work split's 32-bit page counts could overflow
    t7 = list(args_tail)
    t7[4] = ctypes.c_int32(4096)
    t7[2] = ctypes.c_int32((1 << 31) // 4096 - 16)
    assert f(ctypes.byref(ok), fake, fake, fake, fake, fake, *t7) == -2
    t7[2] = ctypes.c_int32((1 << 31) // 4096 - 17)   # the widest accepted: fails later (no GPU)
    assert f(ctypes.byref(ok), fake, fake, fake, fake, fake, *t7) != -2
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


def _cpu_args(B=3, P=4, Hkv=2, G=4, T=2, N=16, cache=0):
    """A well-shaped argument set on the host: any call with it fails only at
    the device check, so a perturbed argument must fail earlier, on its shape."""
    import torch
    d = fp8kv.desc(N, Hkv, cache)
    nb = fp8kv.cache_bytes(d)
    z = lambda *s, dt=torch.int32: torch.zeros(*s, dtype=dt)  # noqa: E731
    return d, dict(
        k_cache=z(nb, dt=torch.uint8), v_cache=z(nb, dt=torch.uint8),
        k_scale=z(Hkv, dt=torch.float32), v_scale=z(Hkv, dt=torch.float32),
        q=z(B, Hkv * G, 128, dt=torch.bfloat16), q_multi=z(B, T, Hkv * G, 128, dt=torch.bfloat16),
        page_table=z(B, P), expected_tags=z(B, P), ctx_lens=z(B), pool_tags=z(N),
        abort=z(B, dt=torch.uint8), k_new=z(B, Hkv, 128, dt=torch.bfloat16),
        v_new=z(B, Hkv, 128, dt=torch.bfloat16), k_new_q=z(B, T, Hkv, 128, dt=torch.bfloat16),
        v_new_q=z(B, T, Hkv, 128, dt=torch.bfloat16), new_pos=z(B), token_seq=z(B),
        out=z(B, Hkv * G, 128, dt=torch.bfloat16), out_q=z(B, T, Hkv * G, 128, dt=torch.bfloat16))


def _calls(d, a):
    """Every hot-path wrapper with the argument set a (keyword names as in a)."""
    return {
        "verify_tags": lambda: fp8kv.verify_tags(a["page_table"], a["expected_tags"], a["ctx_lens"],
                                                 a["pool_tags"], abort=a["abort"]),
        "append": lambda: fp8kv.append(d, a["k_cache"], a["v_cache"], a["k_scale"], a["v_scale"],
                                       a["k_new"], a["v_new"], a["token_seq"], a["new_pos"],
                                       a["page_table"], abort=a["abort"]),
        "verify_append": lambda: fp8kv.verify_append(
            d, a["k_cache"], a["v_cache"], a["k_scale"], a["v_scale"], a["k_new"], a["v_new"],
            a["new_pos"], a["page_table"], a["expected_tags"], a["ctx_lens"], a["pool_tags"],
            abort=a["abort"]),
        "verify_append_q": lambda: fp8kv.verify_append_q(
            d, a["k_cache"], a["v_cache"], a["k_scale"], a["v_scale"], a["k_new_q"], a["v_new_q"],
            a["new_pos"], a["page_table"], a["expected_tags"], a["ctx_lens"], a["pool_tags"],
            abort=a["abort"]),
        "decode_attention": lambda: fp8kv.decode_attention(
            d, a["k_cache"], a["v_cache"], a["k_scale"], a["v_scale"], a["q"], a["page_table"],
            a["ctx_lens"], abort=a["abort"], out=a["out"], workspace=a["k_cache"]),
        "decode_attention_q": lambda: fp8kv.decode_attention_q(
            d, a["k_cache"], a["v_cache"], a["k_scale"], a["v_scale"], a["q_multi"],
            a["page_table"], a["ctx_lens"], abort=a["abort"], out=a["out_q"],
            workspace=a["k_cache"]),
        "decode_attention_shared": lambda: fp8kv.decode_attention_shared(
            d, a["k_cache"], a["v_cache"], a["k_scale"], a["v_scale"], a["q"], a["page_table"],
            a["ctx_lens"], [0, 2], [16], abort=a["abort"], out=a["out"], workspace=a["k_cache"]),
    }


def _expect(fn, *words):
    try:
        fn()
    except ValueError as e:
        msg = str(e)
        assert all(w in msg for w in words), (msg, words)
        return msg
    raise AssertionError(f"accepted; expected an error naming {words}")


def test_wrappers_check_shapes_before_any_device_call():
    """Each hot-path wrapper rejects arguments whose shape or size would make a
    kernel read or write outside a buffer, before taking any pointer."""
    import torch
    d, good = _cpu_args()
    for name, fn in _calls(d, good).items():
        _expect(fn, "device tensor")          # well-shaped: fails only on the device check
    z = torch.zeros
    bad = {  # argument -> (replacement, wrappers that must reject it)
        "page_table": (z(2, 4, dtype=torch.int32), ["verify_tags", "verify_append",
                                                      "verify_append_q", "decode_attention",
                                                      "decode_attention_q",
                                                      "decode_attention_shared"]),
        "expected_tags": (z(3, 5, dtype=torch.int32), ["verify_tags", "verify_append",
                                                         "verify_append_q"]),
        "abort": (z(2, dtype=torch.uint8), list(_calls(d, good))),
        "pool_tags": (z(15, dtype=torch.int32), ["verify_append", "verify_append_q"]),
        "k_cache": (z(fp8kv.cache_bytes(d) - 1, dtype=torch.uint8),
                    ["append", "verify_append", "verify_append_q", "decode_attention",
                     "decode_attention_q", "decode_attention_shared"]),
        "v_scale": (z(1, dtype=torch.float32), ["append", "verify_append", "decode_attention"]),
        "k_new": (z(3, 2, 64, dtype=torch.bfloat16), ["append", "verify_append"]),
        "v_new_q": (z(3, 3, 2, 128, dtype=torch.bfloat16), ["verify_append_q"]),
        "new_pos": (z(4, dtype=torch.int32), ["verify_append", "verify_append_q"]),
        "token_seq": (z(4, dtype=torch.int32), ["append"]),
        "q": (z(3, 8, 64, dtype=torch.bfloat16), ["decode_attention", "decode_attention_shared"]),
        "out": (z(3, 8, 128, dtype=torch.float32), ["decode_attention",
                                                    "decode_attention_shared"]),
        "out_q": (z(3, 1, 8, 128, dtype=torch.bfloat16), ["decode_attention_q"]),
        "ctx_lens": (z(2, dtype=torch.int32), ["decode_attention", "decode_attention_q"]),
    }
    for arg, (value, names) in bad.items():
        a = dict(good)
        a[arg] = value
        calls = _calls(d, a)
        for name in names:
            msg = _expect(calls[name], "")
            assert "device tensor" not in msg, (arg, name, msg)
    # out of the wrong dtype for out_dtype (a bf16 buffer asked for f32 rows)
    _expect(lambda: fp8kv.decode_attention(d, good["k_cache"], good["v_cache"], good["k_scale"],
                                           good["v_scale"], good["q"], good["page_table"],
                                           good["ctx_lens"], out=good["out"],
                                           out_dtype=fp8kv.OUT_F32, workspace=good["k_cache"]),
            "out", "dtype")
    # a pool's device tag array must hold every page
    pool = fp8kv.Pool(16)
    _expect(lambda: pool.sync(z(15, dtype=torch.int32)), "d_tags", "16")
    pool.close()
