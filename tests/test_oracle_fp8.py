"""Pins of the FP8 oracle (oracle/fp8.py) to the E4M3 format definition, to
hand-worked encodings and to closed forms (VC-Attention page, iitak.ru news on
MiniMax-H3, V-Smooth and ExpCast-FP8 paragraphs)."""

import os

import numpy as np
import pytest

from oracle import fp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_e4m3.txt")


def _golden(kind):
    out = []
    for line in open(GOLDEN):
        line = line.split("#")[0].split()
        if len(line) == 3 and line[0] == kind:
            out.append((float(line[1]), int(line[2], 16)))
    return out


def test_decode_matches_format_definition():
    v = fp8.e4m3_decode(np.arange(256))
    assert v[0x38] == 1.0 and v[0x40] == 2.0 and v[0xB8] == -1.0
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert v[0x08] == 2.0 ** -6  # smallest normal
    assert v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9  # subnormals
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and np.signbit(v[0x80])
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)  # codes 0x00..0x7E increase in value
    # within each binade the step is 2^(e-7)/8 (2^-9 for the subnormal range)
    for e in range(1, 15):
        seg = v[8 * e: 8 * e + 8]
        assert np.allclose(np.diff(seg), 2.0 ** (e - 7) / 8)


@pytest.mark.parametrize("value,code", _golden("encode"))
def test_encode_golden(value, code):
    assert int(fp8.e4m3_encode(np.array([value]))[0]) == code


def test_encode_round_trip_and_ties():
    v = fp8.e4m3_decode(np.arange(256))
    fin = ~np.isnan(v)
    assert np.array_equal(fp8.e4m3_encode(v[fin]), np.arange(256)[fin])
    pos = v[:0x7F]
    mid = (pos[:-1] + pos[1:]) / 2
    got = fp8.e4m3_encode(mid).astype(int)
    lo = np.arange(0x7E)
    assert np.array_equal(got, np.where(lo % 2 == 0, lo, lo + 1))  # ties -> even code
    up = fp8.e4m3_encode(np.nextafter(mid, np.inf)).astype(int)
    down = fp8.e4m3_encode(np.nextafter(mid, -np.inf)).astype(int)
    assert np.array_equal(up, lo + 1) and np.array_equal(down, lo)
    assert int(fp8.e4m3_encode(np.array([465.0]))[0]) == 0x7F  # no saturation


@pytest.mark.parametrize("y,code", _golden("expcast"))
def test_expcast_golden(y, code):
    assert int(fp8.expcast_codes(np.array([y]))[0]) == code


def test_expcast_is_exact_at_aligned_exponents_and_bounded_elsewhere():
    # 8*y + 126 a multiple of 8: the code is exactly 2^(y + 8.75)
    y = -0.75 - np.arange(0, 14)
    assert np.array_equal(fp8.e4m3_decode(fp8.expcast_codes(y)), 2.0 ** (y + 8.75))
    # elsewhere: linear interpolation of 2^f on [0, 1] (error below 6.2 %) after
    # rounding y to a multiple of 1/8 (a factor below 2^(1/16)), in the normal range
    y = np.linspace(-12.0, 0.0, 20001)
    ratio = fp8.e4m3_decode(fp8.expcast_codes(y)) / 2.0 ** (y + 8.75)
    bound = (1 + 0.0616) * 2 ** (1 / 16)
    assert np.all(ratio < bound) and np.all(ratio > 1 / bound)
    assert np.all(np.diff(fp8.expcast_codes(y).astype(int)) >= 0)  # monotone
    assert int(fp8.expcast_codes(np.array([-np.inf]))[0]) == 0


def test_quantize_block_maps_the_largest_magnitude_to_448():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal((16, 8)) * 3).astype(np.float32)
    codes, s = fp8.quantize_block(x)
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert codes[i] in (0x7E, 0xFE)
    assert s == np.float32(np.max(np.abs(x)) / np.float32(448.0))
    deq = s * fp8.e4m3_decode(codes)
    # half a step: 2^-4 of a normal value, 2^-10 * s absolute in the subnormal range
    err = np.abs(deq - x)
    assert np.all(err <= np.maximum(np.abs(x) * 2.0 ** -4, s * 2.0 ** -10) * 1.0001)
    z, sz = fp8.quantize_block(np.zeros((4, 4), np.float32))
    assert sz == 0.0 and not z.any()


def _bf16(a):
    return fp8.bf16_round(np.asarray(a, np.float32))


def test_prepare_v_smooth_reconstructs_values_and_means():
    rng = np.random.default_rng(1)
    B, H, N, d, bq, bk = 1, 2, 80, 16, 32, 16
    q, k = (_bf16(rng.standard_normal((B, H, N, d))) for _ in range(2))
    v = _bf16(rng.standard_normal((B, H, N, d)) + 20.0)  # a large common offset
    p = fp8.prepare(q, k, v, bq, bk)
    for j in range(N // bk):
        exact = v[0, 0, j * bk:(j + 1) * bk].astype(np.float64).mean(axis=0)
        assert np.all(np.abs(p["vmean"][0, 0, j] - exact) <= np.abs(exact) * 2.0 ** -8 + 1e-6)
    recon = np.repeat(p["vmean"], bk, axis=2)[:, :, :N] + p["vscale"][:, :, None, None] * fp8.e4m3_decode(p["vcode"])
    # the residual is quantised, not the offset: error bounded by half a step of the residual scale range
    assert np.max(np.abs(recon - v)) <= float(p["vscale"].max()) * 448 * 2.0 ** -4
    # quantising the residual beats quantising the values themselves (the point of V-Smooth)
    plain = np.zeros_like(recon)
    for h in range(H):
        c, sc = fp8.quantize_block(v[0, h])
        plain[0, h] = sc * fp8.e4m3_decode(c)
    assert np.mean(np.abs(recon - v)) < 0.5 * np.mean(np.abs(plain - v))


def _small_case(seed, N=100, d=16, bq=32, bk=16):
    rng = np.random.default_rng(seed)
    B, H = 1, 1
    q, k, v = (_bf16(rng.standard_normal((B, H, N, d))) for _ in range(3))
    nqb, nkb = -(-N // bq), -(-N // bk)
    idx = np.tile(np.arange(nkb, dtype=np.int32), (B, H, nqb, 1))
    w = np.ones((B, H, nqb, nkb), np.float32)
    cnt = np.full((B, H, nqb), nkb, np.int32)
    return q, k, v, idx, w, cnt, bq, bk


def test_attention_with_equal_logits_is_the_mean_of_the_reconstructed_values():
    q, k, v, idx, w, cnt, bq, bk = _small_case(2)
    q[:] = 0.0
    p = fp8.prepare(q, k, v, bq, bk)
    N = q.shape[2]
    recon = np.repeat(p["vmean"], bk, axis=2)[:, :, :N] + p["vscale"][:, :, None, None] * fp8.e4m3_decode(p["vcode"])
    res = fp8.attn_rows_fp8(p, idx, w, cnt, bq, bk, 0.25, [(0, 0, 0), (0, 0, 77)])
    for key, (o, lse) in res.items():
        assert np.allclose(o, recon[0, 0].mean(axis=0), rtol=1e-12, atol=1e-12)
        # every p is 448 = 2^(8.75 + log2(448) - 8.75): lse = ln(N) exactly when all logits are 0
        assert abs(lse - (np.log(N) + (np.log2(448.0) - 8.75) * np.log(2))) < 1e-12


def test_attention_of_one_kept_block_with_one_key():
    q, k, v, idx, w, cnt, bq, bk = _small_case(3, N=97, bk=16)
    # keep only the tail sub-block of query block 1: keys 96 (one real key)
    cnt[:] = 0
    cnt[0, 0, 1] = 1
    idx[0, 0, 1, 0] = 6
    p = fp8.prepare(q, k, v, bq, bk)
    res = fp8.attn_rows_fp8(p, idx, w, cnt, bq, bk, 0.25, [(0, 0, 40), (0, 0, 5)])
    recon = p["vmean"][0, 0, 6] + p["vscale"][0, 0] * fp8.e4m3_decode(p["vcode"][0, 0, 96])
    assert np.allclose(res[(0, 0, 40)][0], recon, atol=1e-12)
    assert np.all(res[(0, 0, 5)][0] == 0) and res[(0, 0, 5)][1] == -np.inf  # empty list


def test_attention_close_to_dense_attention():
    q, k, v, idx, w, cnt, bq, bk = _small_case(4, N=160, d=32)
    scale = 1 / np.sqrt(32)
    p = fp8.prepare(q, k, v, bq, bk)
    rows = [(0, 0, r) for r in (0, 31, 64, 100, 159)]
    res = fp8.attn_rows_fp8(p, idx, w, cnt, bq, bk, scale, rows)
    for (b, h, r) in rows:
        s = (k[0, 0].astype(np.float64) @ q[0, 0, r].astype(np.float64)) * scale
        e = np.exp(s - s.max())
        ref = e @ v[0, 0].astype(np.float64) / e.sum()
        o, lse = res[(b, h, r)]
        assert np.linalg.norm(o - ref) / np.linalg.norm(ref) < 0.08
        assert abs(lse - (s.max() + np.log(e.sum()))) < 0.1
