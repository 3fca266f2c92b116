"""Pins of the oracle's quantiser, word packing and packed cache (CPU only).

Hand-derived examples (``golden/quantize_examples.txt``) fix the scale rounding and the
half-to-even rule; properties that hold for any group (min -> 0, max -> 2^b - 1, error at most
half a step) and an independent bit-level unpacker check the rest.  The packed byte layout is
this library's own convention (parity unpinned); it is checked for self-consistency by a
decoder written here from its documented description.
"""

import os

import numpy as np
import pytest

import oracle
from workloads import make_inputs, bf16_bits_to_f32, f32_to_bf16_bits


def _expand(tokens):
    out = []
    for t in tokens:
        if "*" in t:
            v, n = t.split("*")
            out += [v] * int(n)
        else:
            out.append(t)
    return out


def _read_cases(path):
    cases, cur = [], None
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *rest = line.split()
            if key == "case":
                cur = {"name": rest[0]}
                cases.append(cur)
            else:
                cur[key] = _expand(rest)
    return cases


def _unpack(words, b, m):
    """Independent unpacker: concatenate the words into one little-endian integer."""
    big = 0
    for i, w in enumerate(int(x) for x in words):
        big |= w << (32 * i)
    return [(big >> (e * b)) & ((1 << b) - 1) for e in range(m)]


def test_hand_examples(golden_dir):
    for case in _read_cases(os.path.join(golden_dir, "quantize_examples.txt")):
        b = int(case["b"][0])
        x = np.array([float(v) for v in case["x"]])
        assert np.array_equal(bf16_bits_to_f32(f32_to_bf16_bits(x.astype(np.float32))), x)
        codes, s, z = oracle.quantize_group(x, b)
        assert int(s.view(np.uint32)[0]) == int(case["scale"][0], 16), case["name"]
        assert float(z[0]) == float(case["zero"][0]), case["name"]
        assert codes[0].tolist() == [int(c) for c in case["codes"]], case["name"]
        words = oracle.pack_group_words(codes, b)[0]
        assert _unpack(words, b, 32) == codes[0].tolist()
        if "words" in case:
            assert words.tolist() == [int(w) for w in case["words"]], case["name"]


@pytest.mark.parametrize("b", [2, 4, 8])
def test_group_properties(b):
    rng = np.random.default_rng(b)
    x = bf16_bits_to_f32(f32_to_bf16_bits(rng.standard_normal((500, 32)).astype(np.float32) * 3))
    x = x.astype(np.float64)
    codes, s, z = oracle.quantize_group(x, b)
    lo = x.argmin(axis=1)
    hi = x.argmax(axis=1)
    r = np.arange(500)
    assert (codes[r, lo] == 0).all()
    assert (codes[r, hi] == 2 ** b - 1).all()
    xh = z.astype(np.float64)[:, None] + s.astype(np.float64)[:, None] * codes
    assert (np.abs(xh - x) <= s.astype(np.float64)[:, None] / 2 * (1 + 1e-6)).all()
    assert ((codes >= 0) & (codes < 2 ** b)).all()
    for i in range(0, 500, 37):
        assert _unpack(oracle.pack_group_words(codes[i:i + 1], b)[0], b, 32) == codes[i].tolist()


def test_sixteen_bit_words_are_raw_bf16():
    rng = np.random.default_rng(3)
    raw = f32_to_bf16_bits(rng.standard_normal(32).astype(np.float32))
    words = oracle.pack_group_words(raw.astype(np.uint64)[None, :], 16)[0]
    assert _unpack(words, 16, 32) == raw.astype(int).tolist()
    assert words.tobytes() == raw.tobytes()           # little-endian: the raw bf16 stream


def _decode_cache(c, hkv, n, d):
    """Decoder written from the documented layout (see oracle.pack_cache's docstring)."""
    H = c["header"]
    widths = (2, 4, 8, 16)
    out = []
    for g in range(hkv):
        base = 16 + 24 * g
        R = int(H[base + 4])
        keep = c["k_keep"][H[base + 17]: H[base + 17] + R]
        vloc = c["k_vloc"][H[base + 17]: H[base + 17] + R]
        v_hat = np.zeros((R, d))
        for j in range(R):
            z, p = int(vloc[j]) >> 29, int(vloc[j]) & ((1 << 29) - 1)
            b = widths[z]
            assert c["v_idx"][H[base + 5 + z] + p] == keep[j]
            wbase = H[base + 9 + z] + p * (d // 32) * b
            for grp in range(d // 32):
                w = c["v_words"][wbase + grp * b: wbase + (grp + 1) * b]
                vals = _unpack(w, b, 32)
                if b == 16:
                    v_hat[j, 32 * grp:32 * grp + 32] = bf16_bits_to_f32(np.array(vals, dtype=np.uint16))
                else:
                    s, zz = c["v_par"][H[base + 13 + z] + p * (d // 32) + grp]
                    v_hat[j, 32 * grp:32 * grp + 32] = float(zz) + float(s) * np.array(vals)
        bk = c["k_width"][g]
        wk = int(H[base + 20])
        qk = int(H[base + 21])
        assert wk == int(bk.astype(int).sum()) and int(H[base + 22]) == (R + 31) // 32
        k_hat = np.zeros((R, d))
        for j in range(0, R, 32):
            grp = j // 32
            woff = H[base + 18] + grp * wk
            poff = H[base + 19] + grp * qk
            m = min(32, R - j)
            for c_ in range(d):
                b = int(bk[c_])
                if b == 0:
                    continue
                vals = _unpack(c["k_words"][woff: woff + b], b, 32)
                woff += b
                if b == 16:
                    k_hat[j:j + m, c_] = bf16_bits_to_f32(np.array(vals[:m], dtype=np.uint16))
                else:
                    s, zz = c["k_par"][poff]
                    poff += 1
                    k_hat[j:j + m, c_] = float(zz) + float(s) * np.array(vals[:m])
                    assert all(v == 0 for v in vals[m:])      # tail padding
        out.append((keep, k_hat, v_hat))
    return out


@pytest.mark.parametrize("seed,n", [(0, 70), (1, 96), (2, 33)])
def test_packed_cache_decodes_to_dequantized_units(seed, n):
    hkv, d = 2, 64
    x = make_inputs(2, hkv, d, n, n, seed=seed)
    rng = np.random.default_rng(100 + seed)
    bits_v = rng.choice(np.array([0, 2, 4, 8, 16], dtype=np.uint8), (hkv, n))
    bits_k = rng.choice(np.array([0, 2, 4, 8, 16], dtype=np.uint8), (hkv, d))
    c = oracle.pack_cache(x["k"], x["v"], bits_v, bits_k)
    dec = _decode_cache(c, hkv, n, d)
    for g in range(hkv):
        toks, k_hat, v_hat = oracle.dequantized_head(x["k"][g], x["v"][g], bits_v[g], bits_k[g])
        assert np.array_equal(dec[g][0], toks)
        np.testing.assert_array_equal(dec[g][1], k_hat)
        np.testing.assert_array_equal(dec[g][2], v_hat)
    H = c["header"]
    assert H[4] == c["v_idx"].size and H[5] == c["v_words"].size and H[6] == c["v_par"].shape[0]
    assert H[7] == c["k_keep"].size and H[8] == c["k_words"].size and H[9] == c["k_par"].shape[0]


def test_invalid_width_rejected():
    x = make_inputs(1, 1, 32, 8, 8, seed=0)
    with pytest.raises(ValueError):
        oracle.pack_cache(x["k"], x["v"], np.full((1, 8), 3, dtype=np.uint8), np.zeros((1, 32), np.uint8))
