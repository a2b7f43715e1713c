"""Pins for the oracle's e4m3 decode table and encoder (CPU only).

The oracle is checked against things other than itself:
  * the format's spot values (tests/golden/e4m3_spot_values.txt);
  * torch's float8_e4m3fn conversion (a library routine) for the decode table
    and for in-range encoding;
  * an independently written bit-level encoder (below) over the inputs that
    matter: every binary32 within +-64 ulps of every code and every midpoint,
    and random inputs across the whole exponent range; the same method in C
    over all 2^32 binary32 inputs (tests/c/e4m3_every_binary32.c);
  * closed forms: round trip of all 256 codes, ties-to-even at all 126
    midpoints, saturation, sign-preserving underflow.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "e4m3_spot_values.txt")


def _gold():
    rows = []
    for line in open(GOLD):
        line = line.split("#")[0].strip()
        if not line:
            continue
        c, v = line.split()
        rows.append((int(c, 16), float(v)))
    return rows


def test_spot_values_from_golden():
    for code, val in _gold():
        got = oracle.e4m3_decode(code)
        if math.isnan(val):
            assert math.isnan(got), hex(code)
        else:
            assert got == val, (hex(code), got, val)
            assert math.copysign(1.0, got) == math.copysign(1.0, val), hex(code)


def test_table_matches_torch_float8_e4m3fn():
    tab = oracle.e4m3_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    nan_t = np.isnan(tab)
    assert (nan_t == np.isnan(ref)).all()
    assert (tab[~nan_t] == ref[~nan_t]).all()
    assert (np.signbit(tab[~nan_t]) == np.signbit(ref[~nan_t])).all()


def test_table_structure():
    tab = oracle.e4m3_table()
    assert np.isnan(tab).sum() == 2 and np.isnan(tab[0x7F]) and np.isnan(tab[0xFF])
    pos = tab[:0x7F]
    assert (np.diff(pos) > 0).all(), "codes 0x00..0x7E strictly increasing"
    assert (tab[0x80:0xFF] == -tab[:0x7F]).all()
    # every finite value is exact in binary32, bf16 and f16
    f = tab[~np.isnan(tab)]
    assert (f.astype(np.float32).astype(np.float64) == f).all()
    assert (torch.tensor(f).to(torch.bfloat16).double().numpy() == f).all()
    assert (torch.tensor(f).to(torch.float16).double().numpy() == f).all()


def test_round_trip_all_codes():
    tab = oracle.e4m3_table()
    for c in range(256):
        v = tab[c]
        e = oracle.e4m3_encode(v)
        if c in (0x7F, 0xFF):
            assert e == c, hex(c)
        else:
            assert e == c, (hex(c), v, hex(e))


def test_midpoints_tie_to_even_and_neighbours():
    tab = oracle.e4m3_table()
    for c in range(126):
        lo, hi = tab[c], tab[c + 1]
        mid = (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(mid) == even, (c, mid)
        assert oracle.e4m3_encode(-mid) == 0x80 | even
        m32 = np.float32(mid)
        assert float(m32) == mid  # midpoints are exact in binary32
        below = float(np.nextafter(m32, np.float32(-1)))
        above = float(np.nextafter(m32, np.float32(1e9)))
        assert oracle.e4m3_encode(below) == c
        assert oracle.e4m3_encode(above) == c + 1


def test_saturation_and_specials():
    assert oracle.e4m3_encode(432.0) == 0x7E       # 416/448 midpoint -> even 0x7E
    for v in (448.0, 464.0, 1e6, 3.0e38, math.inf):
        assert oracle.e4m3_encode(v) == 0x7E
        assert oracle.e4m3_encode(-v) == 0xFE
    assert oracle.e4m3_encode(math.nan) == 0x7F
    assert oracle.e4m3_encode(-math.nan) == 0xFF
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00   # tie between 0 and 2^-9 -> even 0
    assert oracle.e4m3_encode(-(2.0 ** -10)) == 0x80
    assert oracle.e4m3_encode(1.5 * 2.0 ** -10) == 0x01
    assert oracle.e4m3_encode(0.0) == 0x00
    assert oracle.e4m3_encode(-0.0) == 0x80
    assert oracle.e4m3_encode(-1e-30) == 0x80


# ---------------------------------------------------------------------------
# independent bit-level encoder (binary32 in, code out)
# ---------------------------------------------------------------------------
def bitlevel_encode(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, np.float32)
    u = x.view(np.uint32).astype(np.int64)
    sign = (u >> 24) & 0x80
    a = u & 0x7FFFFFFF
    is_nan = a > 0x7F800000
    sat = a >= 0x43E00000                     # |x| >= 448
    sub = a < 0x3C800000                      # |x| < 2^-6 (smallest e4m3 normal)
    # normal range: keep 3 mantissa bits, round half to even on the dropped 20
    r = a + 0x7FFFF + ((a >> 20) & 1)
    code_n = (r >> 20) - (120 << 3)
    # subnormal range: multiples of 2^-9; |x| * 512 is exact, rint is half-even
    ax = np.minimum(np.abs(x), np.float32(1.0)).astype(np.float32)  # only used below 2^-6
    code_s = np.rint(ax * np.float32(512.0)).astype(np.int64)
    code = np.where(sub, code_s, code_n)
    code = np.where(sat, 0x7E, code)
    code = np.where(is_nan, 0x7F, code)
    return (code | sign).astype(np.uint8)


def _edge_inputs():
    tab = oracle.e4m3_table()
    pts = list(tab[:0x7F]) + [(tab[c] + tab[c + 1]) / 2 for c in range(126)]
    pts += [448.0, 464.0, 480.0, 2.0 ** -10, 2.0 ** -11]
    base = np.array(pts, np.float32).view(np.uint32).astype(np.int64)
    offs = np.arange(-64, 65, dtype=np.int64)
    u = (base[:, None] + offs[None, :]).ravel()
    u = u[(u >= 0) & (u < 0x7F800000)]
    x = u.astype(np.uint32).view(np.float32)
    return np.concatenate([x, -x])


def test_bitlevel_encoder_agrees_on_edges():
    x = _edge_inputs()
    assert (oracle.e4m3_encode_f32(x) == bitlevel_encode(x)).all()


def test_bitlevel_encoder_agrees_on_every_binary32():
    """All 2^32 binary32 inputs, NaNs, infinities and subnormals included,
    through the oracle's encoder and the bit-level method in C (OpenMP; about
    10 s on 8 cores)."""
    import importlib.util
    import subprocess
    here = os.path.dirname(os.path.abspath(__file__))
    spec = importlib.util.spec_from_file_location("c_tests_build", os.path.join(here, "c", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    oracle.lib()                       # the oracle's library, built if missing
    binary = b.E4M3_BIN if os.path.exists(b.E4M3_BIN) else b.build_e4m3()
    r = subprocess.run([binary], capture_output=True, text=True, timeout=600)
    print(r.stdout.strip())
    assert r.returncode == 0 and " 0 mismatches" in r.stdout, r.stdout + r.stderr


def test_bitlevel_encoder_agrees_random():
    rng = np.random.default_rng(11)
    u = rng.integers(0, 2 ** 32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[~np.isnan(x)]
    assert (oracle.e4m3_encode_f32(x) == bitlevel_encode(x)).all()


def test_torch_agrees_in_range():
    # torch's conversion is round-to-nearest-even but does not saturate
    # (values past 464 become NaN), so compare inside the finite range.
    rng = np.random.default_rng(12)
    x = (rng.standard_normal(2_000_000) * rng.choice([1e-3, 1e-1, 1, 30, 150], 2_000_000))
    x = x.astype(np.float32)
    x = x[np.abs(x) < 448.0]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (oracle.e4m3_encode_f32(x) == ref).all()


def test_bf16_rne_pins():
    assert oracle.bf16_rne(1.0) == 0x3F80
    assert oracle.bf16_rne(-2.0) == 0xC000
    assert oracle.bf16_rne(1.0 + 2.0 ** -8) == 0x3F80            # tie -> even
    assert oracle.bf16_rne(1.0 + 3 * 2.0 ** -8) == 0x3F82        # tie -> even (up)
    assert oracle.bf16_rne(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81
    assert oracle.bf16_rne(0.0) == 0 and oracle.bf16_rne(-0.0) == 0x8000
    assert oracle.bf16_rne(3.4e38) == 0x7F80                      # overflow
    assert oracle.bf16_rne(2.0 ** -133) == 0x0001                 # smallest subnormal
    # agree with a direct nearest-neighbour search over bf16 values
    rng = np.random.default_rng(5)
    vals = rng.standard_normal(3000) * rng.choice([1e-3, 1, 100], 3000)
    allbits = np.arange(0, 0x7F80, dtype=np.uint32)
    allv = (allbits << np.uint32(16)).view(np.float32).astype(np.float64)
    for v in vals:
        got = oracle.bf16_rne(v) & 0x7FFF
        i = np.searchsorted(allv, abs(v))
        cands = [j for j in (i - 1, i) if 0 <= j < allv.size]
        best = min(cands, key=lambda j: (abs(allv[j] - abs(v)), j % 2))
        assert got == best, v
