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
    y = np.linspace(-14.8, 0.0, 24001)  # the normal range: 8 y + 126 >= 7.5
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


# ---- the weighted FP8 attention against exact weighted attention -------------------
#
# Both FP8 references (attn_rows_fp8_plain, one reference per row; attn_rows_fp8, the
# kernel's tile walk) replace each exact probability a_k = 2^(y_k + 8.75), y_k = x_k - M
# (x_k the weighted logit in log2 units, M its row maximum), by an E4M3 value p_k. For a
# code in the normal range (8 y + 126 >= 7.5 against the row maximum; the tile walk's
# references lie at or below M, so such a key is normal there too) the ratio p_k / a_k
# lies within [1/F, F], F = 1.0616 * 2^(1/16) (pinned above); every other key has
# a_k < 2^-6.06 and p_k <= 7 * 2^-9, so |p_k - a_k| < 2^-6.06. With O the exact output
# and any constant c, O' - O = sum_k (p_k - c a_k)(v_k - O) / sum_k p_k, because
# sum_k a_k (v_k - O) = 0; c = (F + 1/F)/2 gives, per output element d,
#   |O'_d - O_d| <= [ (F - 1/F)/2 sum_normal a_k |v_kd - O_d|
#                    + c 2^-6.06 sum_other |v_kd - O_d| ] / (sum_normal a_k / F).
F_EXPCAST = 1.0616 * 2.0 ** (1 / 16)


def expcast_output_bound(logits, v_rows, o_exact, F=F_EXPCAST, small=2.0 ** -6.06):
    """The bound above for one query row. logits: exact weighted logits of its kept keys
    (natural units, the log of the weight included); v_rows: [keys, d] values; o_exact:
    the exact output [d]; small: the bound on |p_k - a_k| outside the normal range."""
    y = (logits - logits.max()) / np.log(2.0)
    a = 2.0 ** (y + fp8.EXPCAST_LOG2_TOP)
    normal = 8.0 * y + fp8.EXPCAST_TOP >= 7.5
    dev = np.abs(v_rows - o_exact[None, :])
    c = (F + 1.0 / F) / 2.0
    num = (F - 1.0 / F) / 2.0 * (a[normal] @ dev[normal]) + c * small * dev[~normal].sum(axis=0)
    return num / (a[normal].sum() / F) + 1e-12


def _weighted_case(seed, N=200, d=32, bq=64, bk=16, qmul=1.0):
    """Bf16-valued Q, K, V with a common direction in Q and K (so some sub-blocks carry
    most of a row's mass), random kept lists whose weights span 1..64."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(d)
    q = _bf16((qmul * (1.5 * u + rng.standard_normal((1, 1, N, d)))).astype(np.float32))
    k = _bf16((rng.standard_normal((1, 1, N, d)) + 0.8 * u * rng.random((1, 1, N, 1))).astype(np.float32))
    v = _bf16((rng.standard_normal((1, 1, N, d)) + 1.0).astype(np.float32))
    nqb, nkb = -(-N // bq), -(-N // bk)
    idx = np.zeros((1, 1, nqb, nkb), np.int32)
    w = np.zeros((1, 1, nqb, nkb), np.float32)
    cnt = np.zeros((1, 1, nqb), np.int32)
    for i in range(nqb):
        c = int(rng.integers(2, nkb))
        sel = np.sort(rng.choice(nkb, c, replace=False))
        idx[0, 0, i, :c] = sel
        w[0, 0, i, :c] = rng.choice(np.array([1.0, 2.5, 4.0, 16.0, 64.0], np.float32), c)
        cnt[0, 0, i] = c
    return q, k, v, idx, w, cnt, bq, bk


def _check_against_exact(fn, seed, expect_pass=True):
    from oracle import sparse_ht_attention

    q, k, v, idx, w, cnt, bq, bk = _weighted_case(seed)
    scale = 1.0 / np.sqrt(q.shape[3])
    p = fp8.prepare(q, k, v, bq, bk)
    qd, kd, vd = fp8.dequantize(p, bq, bk)
    N = q.shape[2]
    rows = [(0, 0, r) for r in range(0, N, 7)] + [(0, 0, N - 1)]
    res = fn(p, idx, w, cnt, bq, bk, scale, rows)
    worst = 0.0
    for (b, h, r) in rows:
        i = r // bq
        c = int(cnt[0, 0, i])
        sel, wt = idx[0, 0, i, :c], w[0, 0, i, :c]
        o_ex, lse_ex = sparse_ht_attention(qd[0, 0, r:r + 1], kd[0, 0], vd[0, 0], sel, wt, bk, scale)
        keys = np.concatenate([np.arange(j * bk, min(N, (j + 1) * bk)) for j in sel])
        lw = np.concatenate([np.full(min(N, (j + 1) * bk) - j * bk, np.log(float(x))) for j, x in zip(sel, wt)])
        logits = scale * (kd[0, 0, keys] @ qd[0, 0, r]) + lw
        bound = expcast_output_bound(logits, vd[0, 0, keys], o_ex[0])
        err = np.abs(res[(b, h, r)][0] - o_ex[0])
        worst = max(worst, float((err / bound).max()))
        if expect_pass:
            assert np.all(err <= bound), (r, float((err / bound).max()))
            # lse: the row sum moves by at most the factor F (plus the tiny keys)
            assert abs(res[(b, h, r)][1] - lse_ex[0]) <= np.log(F_EXPCAST) + 1e-3, r
    return worst


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_plain_fp8_attention_within_expcast_bound_of_exact_weighted_attention(seed):
    """Pins the plain FP8 reference, weights included, to sparse_ht_attention (the
    float64 weighted attention, pinned elsewhere) on the values the FP8 operands stand
    for: within the ExpCast bound element by element."""
    assert _check_against_exact(fp8.attn_rows_fp8_plain, seed) <= 1.0


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiled_fp8_attention_within_expcast_bound_of_exact_weighted_attention(seed):
    """The same pin for the kernel's tile walk (attn_rows_fp8), non-unit weights."""
    assert _check_against_exact(fp8.attn_rows_fp8, seed) <= 1.0


class _NumpyWith:
    """numpy with some functions replaced: plants a mistake in the oracle module."""

    def __init__(self, **override):
        self._override = override

    def __getattr__(self, name):
        return self._override.get(name, getattr(np, name))


@pytest.mark.parametrize("fn", ["attn_rows_fp8_plain", "attn_rows_fp8"])
@pytest.mark.parametrize("mistake", ["natural-log weight", "inverted weight"])
def test_weight_pin_has_power(monkeypatch, fn, mistake):
    """The pin above catches a wrong weight term: with the log2 of the weight replaced by
    its natural log, or negated, the same check fails by a wide margin."""
    log2 = np.log2
    bad = np.log if mistake == "natural-log weight" else (lambda x: -log2(x))
    ref = getattr(fp8, fn)

    def planted(p, idx, w, cnt, bq, bk, scale, rows, **kw):
        # the logit part of the row terms stays right: only the weight's log changes
        monkeypatch.setattr(fp8, "np", _NumpyWith(log2=bad))
        try:
            out = ref(p, idx, w, cnt, bq, bk, scale, rows, **kw)
        finally:
            monkeypatch.setattr(fp8, "np", np)
        return out

    assert _check_against_exact(planted, 0, expect_pass=False) > 3.0


def test_plain_power_of_two_weight_equals_repeated_sub_block():
    """Closed form of the weight term: a weight 2^k on a sub-block is the sub-block kept
    2^k times with weight 1. Exact in the plain reference when the row maximum lies in
    a weight-1 sub-block and every code is in the normal range (then ExpCast of x + k is
    the code of x plus 8k, whose value is 2^k times larger)."""
    rng = np.random.default_rng(9)
    N, d, bq, bk = 96, 32, 32, 16
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    # queries share the direction u; sub-block 0 leans along it, so it holds every row's
    # largest logit, and all logits of a row lie within a few units (normal codes only)
    q = _bf16((3.0 * u + 0.5 * rng.standard_normal((1, 1, N, d))).astype(np.float32))
    k = _bf16((0.5 * rng.standard_normal((1, 1, N, d))).astype(np.float32))
    k[0, 0, 0:bk] = _bf16((k[0, 0, 0:bk] + 6.0 * u).astype(np.float32))
    v = _bf16(rng.standard_normal((1, 1, N, d)).astype(np.float32))
    p = fp8.prepare(q, k, v, bq, bk)
    nqb, nkb = N // bq, N // bk
    scale = 1.0 / np.sqrt(d)
    # weighted lists: sub-block 0 (weight 1, holds each row's maximum), 2 (weight 4), 5 (weight 2)
    idx = np.zeros((1, 1, nqb, nkb), np.int32)
    w = np.zeros((1, 1, nqb, nkb), np.float32)
    cnt = np.full((1, 1, nqb), 3, np.int32)
    idx[..., :3] = [0, 2, 5]
    w[..., :3] = [1.0, 4.0, 2.0]
    # repeated lists: 0 once, 2 four times, 5 twice, all weight 1
    rep = [0, 2, 2, 2, 2, 5, 5]
    idx_r = np.zeros((1, 1, nqb, len(rep)), np.int32)
    idx_r[..., :] = rep
    w_r = np.ones((1, 1, nqb, len(rep)), np.float32)
    cnt_r = np.full((1, 1, nqb), len(rep), np.int32)
    rows = [(0, 0, r) for r in range(N)]
    a = fp8.attn_rows_fp8_plain(p, idx, w, cnt, bq, bk, scale, rows)
    b = fp8.attn_rows_fp8_plain(p, idx_r, w_r, cnt_r, bq, bk, scale, rows)
    checked = 0
    for key in rows:
        r = key[2]
        _, _, xw = fp8._row_terms(p, idx, w, cnt, bq, bk, scale, 0, 0, r)  # weighted logits
        _, _, xs = fp8._row_terms(p, idx_r, w_r, cnt_r, bq, bk, scale, 0, 0, r)
        if xw.argmax() >= bk or np.any(8 * (xs - xs.max()) + 126 < 7.5):
            continue  # outside the closed form's conditions
        checked += 1
        assert np.allclose(a[key][0], b[key][0], rtol=1e-12, atol=1e-12), r
        assert abs(a[key][1] - b[key][1]) < 1e-12, r
    assert checked >= N // 2
