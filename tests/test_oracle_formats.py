"""Pins of the oracle's element decoders and encoders (CPU only).

Decoders: every code against the printed OCP MX value tables (tests/golden)
and, for E4M3FN, against torch's float8_e4m3fn cast on all 254 finite codes.
Encoders: against brute-force nearest-value search with the even-code tie
rule, against torch's round-to-nearest-even cast, and round trips.
"""

import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                c, v = line.split()
                rows.append((int(c, 16), float(v)))
    return rows


def test_e2m1_decode_matches_spec_table():
    rows = _read_table("e2m1_values.txt")
    assert len(rows) == 16
    codes = np.array([c for c, _ in rows])
    got = oracle.e2m1_decode(codes)
    want = np.array([v for _, v in rows])
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))  # 0x8 is -0


def test_e4m3_decode_special_values():
    for code, val in _read_table("e4m3_special.txt"):
        got = float(oracle.e4m3_decode(np.array([code]))[0])
        if np.isnan(val):
            assert np.isnan(got), hex(code)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), hex(code)


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    finite = ~np.isnan(ref)
    assert finite.sum() == 254
    assert np.array_equal(got[finite], ref[finite])
    assert np.isnan(got[~finite]).all()
    assert set(np.nonzero(np.isnan(got))[0]) == {0x7F, 0xFF}


def test_e4m3_decode_monotone_positive():
    v = oracle.e4m3_decode(np.arange(0x7F))
    assert np.all(np.diff(v) > 0)
    assert v.max() == 448.0


def _brute_encode(values, table_codes, table_vals):
    """Nearest representable value; ties to the even code; beyond max -> max."""
    out = []
    for v in values:
        a = abs(v)
        d = np.abs(table_vals - a)
        best = np.flatnonzero(d == d.min())
        code = table_codes[best[0]] if len(best) == 1 else [c for c in table_codes[best] if c % 2 == 0][0]
        if a > table_vals.max():
            code = table_codes[np.argmax(table_vals)]
        out.append(code)
    return np.array(out)


def _probe_values(table_vals):
    pos = np.unique(table_vals)
    mids = (pos[1:] + pos[:-1]) / 2
    eps = np.concatenate([mids * (1 + 1e-9), mids * (1 - 1e-9)])
    extra = np.array([pos.max() * 1.01, pos.max() * 1.5, pos.max() * 100, 1e-30, 0.0])
    vals = np.concatenate([pos, mids, eps, extra])
    return np.concatenate([vals, -vals])


def test_e2m1_encode_against_brute_force():
    codes = np.arange(8)
    vals = oracle.e2m1_decode(codes)
    probe = _probe_values(vals)
    got = oracle.e2m1_encode(probe)
    want_mag = _brute_encode(probe, codes, vals)
    assert np.array_equal(got & 7, want_mag)
    assert np.array_equal((got >> 3) & 1, np.signbit(probe).astype(np.uint8))


def test_e2m1_encode_printed_midpoints():
    # Midpoints between neighbours go to the even code.
    pairs = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0, 7.0: 6.0, 1e9: 6.0}
    for v, want in pairs.items():
        assert oracle.e2m1_decode(oracle.e2m1_encode(np.array([v])))[0] == want, v


def test_e4m3_encode_against_brute_force():
    codes = np.arange(0x7F)
    vals = oracle.e4m3_decode(codes)
    probe = _probe_values(vals)
    got = oracle.e4m3_encode(probe)
    want_mag = _brute_encode(probe, codes, vals)
    assert np.array_equal(got & 0x7F, want_mag)
    assert np.array_equal(got >> 7, np.signbit(probe).astype(np.uint8))


def test_e4m3_encode_matches_torch_rne_below_saturation():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.uniform(-448, 448, 20000), np.exp(rng.uniform(-12, 6, 20000)),
                        oracle.e4m3_decode(np.arange(0x7F))])
    got = oracle.e4m3_decode(oracle.e4m3_encode(v))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(got, ref)


def test_e4m3_encode_saturates():
    got = oracle.e4m3_decode(oracle.e4m3_encode(np.array([449.0, 464.0, 465.0, 1e6, -1e6])))
    assert np.array_equal(got, [448, 448, 448, 448, -448])


def test_encode_decode_round_trip():
    e2 = oracle.e2m1_decode(np.arange(16))
    assert np.array_equal(oracle.e2m1_encode(e2), np.arange(16))
    c = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(c)), c)


def test_e4m3_encode_rejects_nan():
    with pytest.raises(ValueError):
        oracle.e4m3_encode(np.array([np.nan]))
