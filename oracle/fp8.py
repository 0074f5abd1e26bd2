"""FP8 (OCP E4M3) arithmetic and the FP8 attention variant (oracle side; test infrastructure).

Only tests, the smoke check and the benchmark's CPU baseline use this module; the
product path never does.

VC-Attention page (iitak.ru news on MiniMax-H3), V-Smooth and ExpCast-FP8
paragraphs: the attention products run in 8-bit floating point; values are made
easier to quantise by subtracting a per-block mean and quantising only the
residual (V-Smooth); the FP8 byte of each softmax probability is produced
directly by one linear formula with rounding instead of an exponential followed
by a conversion (ExpCast-FP8). The format is the OCP 8-bit E4M3 ("fn") format:
1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, one NaN
pattern per sign (exponent and mantissa all ones), largest finite value 448.
"""

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN = 0x7F


def e4m3_decode(codes):
    """Exact value (float64) of E4M3 codes (uint8 array); NaN for 0x7F / 0xFF."""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = np.where((e == 15) & ((c & 7) == 7), np.nan, val)
    return s * val


# the 127 non-negative finite codes 0x00 .. 0x7E in increasing value order
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = e4m3_decode(_POS_CODES)


def e4m3_encode(x):
    """Round values to E4M3 codes: nearest representable value, ties to the even
    code (even mantissa); without saturation, so a magnitude above 464 (the
    midpoint between 448 and the next step, 480, which the format lacks) gives the
    NaN code, as does NaN. Input of any float dtype; the rounding is exact (float64)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    a_sat = np.minimum(a, E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS_VALUES, a_sat, side="left"), 0, 0x7E)  # first value >= a
    lo = np.clip(hi - 1, 0, 0x7E)
    d_hi = _POS_VALUES[hi] - a_sat
    d_lo = a_sat - _POS_VALUES[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & ((lo & 1) == 0))
    code = np.where(pick_lo, lo, hi)
    code = np.where(a_sat == _POS_VALUES[hi], hi, code)
    code = np.where(np.signbit(x), code | 0x80, code)
    code = np.where(np.isnan(x) | (a > 464.0), np.where(np.signbit(x), 0xFF, E4M3_NAN), code)
    return code.astype(np.uint8)


def bf16_round(x):
    """Round float32 values to bfloat16 (nearest, ties to even), returned as float32."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def quantize_block(x):
    """One block of values -> (E4M3 codes, fp32 scale), the block's largest magnitude
    mapping to 448: amax = max |x|; inv = fp32(448 / amax); codes = E4M3(fp32(x * inv));
    scale = fp32(amax / 448), so x ~ scale * decode(codes). An all-zero block gives
    codes 0 and scale 0. x: float32 array (any shape)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    if amax == 0.0:
        return np.zeros(x.shape, dtype=np.uint8), np.float32(0.0)
    inv = np.float32(np.float32(E4M3_MAX) / amax)
    codes = e4m3_encode((x * inv).astype(np.float32))
    return codes, np.float32(amax / np.float32(E4M3_MAX))


def prepare(q, k, v, q_block, k_block):
    """FP8 operands of one layer (VC-Attention page, V-Smooth paragraph; the QK side
    follows the page's remark that low-precision Q K^T is already handled well by
    per-block scaling).

    q, k, v: float32 [B, H, N, d] holding bfloat16 values. Returns a dict:
      qcode uint8 [B,H,N,d], qscale f32 [B,H,NQB]   (one scale per query block)
      kcode uint8 [B,H,N,d], kscale f32 [B,H,NKB]   (one scale per key sub-block)
      vmean f32 [B,H,NKB,d]  bfloat16-rounded mean of each key sub-block's values
                             (fp32 sum in ascending key order, one fp32 division)
      vcode uint8 [B,H,N,d], vscale f32 [B,H]       residual v - vmean of its
                             sub-block, one scale per head
    V-Smooth's block is the key sub-block itself: tokens are never permuted.
    """
    B, H, N, d = q.shape
    nqb = -(-N // q_block)
    nkb = -(-N // k_block)
    out = {
        "qcode": np.zeros((B, H, N, d), np.uint8), "qscale": np.zeros((B, H, nqb), np.float32),
        "kcode": np.zeros((B, H, N, d), np.uint8), "kscale": np.zeros((B, H, nkb), np.float32),
        "vcode": np.zeros((B, H, N, d), np.uint8), "vscale": np.zeros((B, H), np.float32),
        "vmean": np.zeros((B, H, nkb, d), np.float32),
    }
    for b in range(B):
        for h in range(H):
            for i in range(nqb):
                r0, r1 = i * q_block, min(N, (i + 1) * q_block)
                out["qcode"][b, h, r0:r1], out["qscale"][b, h, i] = quantize_block(q[b, h, r0:r1])
            res = np.zeros((N, d), np.float32)
            for j in range(nkb):
                r0, r1 = j * k_block, min(N, (j + 1) * k_block)
                out["kcode"][b, h, r0:r1], out["kscale"][b, h, j] = quantize_block(k[b, h, r0:r1])
                blk = np.asarray(v[b, h, r0:r1], dtype=np.float32)
                s = np.zeros(d, np.float32)
                for r in range(r1 - r0):  # ascending key order, fp32 adds
                    s = (s + blk[r]).astype(np.float32)
                mean = bf16_round((s / np.float32(r1 - r0)).astype(np.float32))
                out["vmean"][b, h, j] = mean
                res[r0:r1] = (blk - mean).astype(np.float32)
            out["vcode"][b, h], out["vscale"][b, h] = quantize_block(res)
    return out


EXPCAST_TOP = 126  # code of the row reference: 0x7E = 448, the largest finite E4M3 value


def expcast_codes(y):
    """ExpCast-FP8 (VC-Attention page, ExpCast-FP8 paragraph): the E4M3 code of a
    probability straight from its base-2 exponent y = x - m (x the weighted logit in
    log2 units, m the row reference, y <= 0) by one linear formula with rounding:
      code = clamp(round_half_even(8 * y + 126), 0, 126).
    An E4M3 code read as an integer is 8 * (exponent + 7) + mantissa, which grows
    linearly with log2 of the value between powers of two, so the code approximates
    448 * 2^y * 2^-0.05 (exactly 2^(y + 8.75) where 8 * y + 126 is a multiple of 8).
    Codes below 8 are subnormal values (tiny); y = -inf gives 0."""
    y = np.asarray(y, dtype=np.float64)
    t = 8.0 * y + EXPCAST_TOP
    return np.clip(np.rint(np.where(np.isfinite(t), t, -1.0)), 0, EXPCAST_TOP).astype(np.uint8)


EXPCAST_LOG2_TOP = 8.75  # 2^(y + 8.75) is what a code stands for: log2 of the row scale


def dequantize(prep, q_block, k_block):
    """The values the FP8 operands stand for, float64 [B,H,N,d] each: q = qscale of the
    row's query block x decode(qcode), k = kscale of the key's sub-block x
    decode(kcode), v = vmean of the key's sub-block + vscale x decode(vcode)
    (V-Smooth reconstruction)."""
    qc, kc, vc = prep["qcode"], prep["kcode"], prep["vcode"]
    N = qc.shape[2]
    rq = np.arange(N) // q_block
    rk = np.arange(N) // k_block
    q = prep["qscale"][:, :, rq, None].astype(np.float64) * e4m3_decode(qc)
    k = prep["kscale"][:, :, rk, None].astype(np.float64) * e4m3_decode(kc)
    v = prep["vmean"][:, :, rk, :].astype(np.float64) + prep["vscale"][:, :, None, None].astype(np.float64) * e4m3_decode(vc)
    return q, k, v


def _row_terms(prep, idx, weights, counts, q_block, k_block, scale, b, h, r):
    """Kept key rows of query row (b, h, r) in list order, each with its sub-block's
    position t in the list and its weighted logit in log2 units,
      x = (qscale * kscale_j * scale * log2(e)) * (qcode . kcode) + log2(w_t),
    computed exactly (float64)."""
    qc, kc = prep["qcode"], prep["kcode"]
    N = qc.shape[2]
    i = r // q_block
    cnt = int(counts[b, h, i])
    c2 = float(scale) * np.log2(np.e)
    qv = e4m3_decode(qc[b, h, r]).astype(np.float64)
    rows, pos, xs = [], [], []
    for t in range(cnt):
        j = int(idx[b, h, i, t])
        a = float(prep["qscale"][b, h, i]) * float(prep["kscale"][b, h, j]) * c2
        lw = float(np.log2(np.float64(weights[b, h, i, t])))
        for kk in range(k_block):
            row = j * k_block + kk
            if row >= N:
                continue
            rows.append(row)
            pos.append(t)
            xs.append(a * float(np.dot(qv, e4m3_decode(kc[b, h, row]).astype(np.float64))) + lw)
    return np.array(rows, dtype=np.int64), np.array(pos, dtype=np.int64), np.array(xs, dtype=np.float64)


def attn_rows_fp8_plain(prep, idx, weights, counts, q_block, k_block, scale, rows):
    """FP8 weighted block-sparse attention for query rows by its plain definition
    (VC-Attention page, ExpCast-FP8 paragraph; float64): one reference per row,
    M = the largest weighted logit x (log2 units) over all kept keys, and every
    probability is the E4M3 value of its ExpCast code against it,
      p_k = decode(ExpCast(x_k - M)),   l = sum_k p_k,
      O = (vscale * sum_k p_k decode(vcode_k) + sum_t (sum_{k in t} p_k) vmean_t) / l,
      lse = (M + log2 l - 8.75) * ln 2,
    with x_k as in _row_terms; O = 0 and lse = -inf for an empty list. No tiles: the
    order in which keys are visited does not enter.

    rows: iterable of (b, h, r). Returns {(b, h, r): (out float64 [d], lse float)}."""
    vc = prep["vcode"]
    d = vc.shape[3]
    res = {}
    for (b, h, r) in rows:
        i = r // q_block
        krows, pos, xs = _row_terms(prep, idx, weights, counts, q_block, k_block, scale, b, h, r)
        if krows.size == 0:
            res[(b, h, r)] = (np.zeros(d, np.float64), -np.inf)
            continue
        M = float(xs.max())
        p = e4m3_decode(expcast_codes(xs - M))
        l = float(p.sum())
        o = float(prep["vscale"][b, h]) * (p @ e4m3_decode(vc[b, h, krows]))
        for t in np.unique(pos):
            j = int(idx[b, h, i, t])
            o = o + float(p[pos == t].sum()) * prep["vmean"][b, h, j].astype(np.float64)
        res[(b, h, r)] = (o / l, (M + np.log2(l) - EXPCAST_LOG2_TOP) * np.log(2.0))
    return res


def attn_rows_fp8(prep, idx, weights, counts, q_block, k_block, scale, rows, tile=64):
    """FP8 weighted block-sparse attention for query rows, computed exactly (float64)
    from the FP8 operands, in the online form the kernel uses (a reading of how the
    codes are taken when the rows are walked in tiles; the plain definition, one
    reference for the whole row, is attn_rows_fp8_plain): the kept sub-blocks of query
    block (b, h, i) are laid end to end and walked in tiles of `tile` key slots; per
    tile, for each row
      x = (qscale * kscale_j * scale * log2(e)) * (qcode . kcode) + log2(w_j)  (log2 units)
      m <- max(m, max over the tile's real keys of x); O, l rescaled by 2^(m_old - m)
      p = decode(ExpCast(x - m))                      (E4M3 values; padding keys p = 0)
      l += sum p;  O += vscale * sum p * decode(vcode) + sum over the tile's
           sub-blocks t of (sum of p over t) * vmean_t         (V-Smooth add-back)
    out = O / l (0 for an empty list), lse = (m + log2 l - 8.75) * ln 2 (-inf if empty).

    rows: iterable of (b, h, r). Returns {(b, h, r): (out float64 [d], lse float)}.
    idx/weights/counts: the SIP outputs (int32/float32 [B,H,NQB,NKB], int32 [B,H,NQB]).
    """
    qc, kc, vc = prep["qcode"], prep["kcode"], prep["vcode"]
    N = qc.shape[2]
    c2 = float(scale) * np.log2(np.e)
    res = {}
    cache = {}
    for (b, h, r) in rows:
        i = r // q_block
        key = (b, h, i)
        if key not in cache:
            cnt = int(counts[b, h, i])
            js = [int(j) for j in idx[b, h, i, :cnt]]
            slots = []  # (key row or -1 for padding, sub-block position t in list order)
            for t, j in enumerate(js):
                for kk in range(k_block):
                    row = j * k_block + kk
                    slots.append((row if row < N else -1, t))
            cache[key] = (js, slots)
        js, slots = cache[key]
        qv = e4m3_decode(qc[b, h, r]).astype(np.float64)
        m = -np.inf
        l = 0.0
        o = np.zeros(qc.shape[3], np.float64)
        for t0 in range(0, len(slots), tile):
            part = slots[t0:t0 + tile]
            xs = []
            for (row, t) in part:
                if row < 0:
                    xs.append(-np.inf)
                    continue
                j = js[t]
                dot = float(np.dot(qv, e4m3_decode(kc[b, h, row]).astype(np.float64)))
                a = float(prep["qscale"][b, h, i]) * float(prep["kscale"][b, h, j]) * c2
                xs.append(a * dot + float(np.log2(np.float64(weights[b, h, i, t]))))
            xs = np.array(xs)
            mt = np.max(xs)
            if mt > m:
                alpha = 0.0 if m == -np.inf else 2.0 ** (m - mt)
                o *= alpha
                l *= alpha
                m = mt
            p = e4m3_decode(expcast_codes(xs - m))
            sub = {}
            for (row, t), pk in zip(part, p):
                if row < 0 or pk == 0.0:
                    continue
                o += float(prep["vscale"][b, h]) * pk * e4m3_decode(vc[b, h, row])
                sub[t] = sub.get(t, 0.0) + pk
                l += pk
            for t, s_t in sub.items():
                o += s_t * prep["vmean"][b, h, js[t]].astype(np.float64)
        if l > 0.0:
            res[(b, h, r)] = (o / l, (m + np.log2(l) - EXPCAST_LOG2_TOP) * np.log(2.0))
        else:
            res[(b, h, r)] = (np.zeros_like(o), -np.inf)
    return res
