"""GPU parity of the FP8 variant (VC-Attention page: 8-bit products, V-Smooth,
ExpCast-FP8) through the C ABI, against oracle/fp8.py.

ab_fp8_prepare: every output bit-exact (codes, scales, V-Smooth means and the
scaled-mean pairs): each is a fixed sequence of correctly rounded fp32 operations
and one E4M3 rounding, computed the same way on both sides.
"""

import functools

import numpy as np
import pytest
import torch

import block_sparse_attention_ibcs_amd as ab
import workloads
from oracle import fp8

pytestmark = pytest.mark.gpu


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _bf16_inputs(shape, seed, offset=0.0):
    g = torch.Generator().manual_seed(seed)
    t = [(torch.randn(shape, generator=g) * s + o).to(torch.bfloat16) for s, o in ((1.0, 0.0), (1.0, 0.0), (1.5, offset))]
    return t


def vcode_natural(vcode, N, bk):
    """[B,H,NKB,2,d,bk/2] operand layout -> [B,H,N,d] in key order."""
    B, H, nkb, _, d, _ = vcode.shape
    t = np.arange(bk)
    g = vcode[:, :, :, (t >> 2) & 1, :, (t >> 3) * 4 + (t & 3)]  # [bk, B, H, nkb, d] (advanced indices first)
    g = np.moveaxis(g, 0, 3)  # [B, H, nkb, bk, d]
    return g.reshape(B, H, nkb * bk, d)[:, :, :N]


def _check_prepare(q, k, v, bq, bk):
    dev = _gpu()
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    desc = ab.Desc.for_tensor(qd, bq, bk, 1)
    ops = ab.ab_fp8_prepare(desc, qd, kd, vd)
    torch.cuda.synchronize()
    ref = fp8.prepare(q.float().numpy(), k.float().numpy(), v.float().numpy(), bq, bk)
    N = q.shape[2]
    assert np.array_equal(ops.qcode.cpu().numpy(), ref["qcode"])
    assert np.array_equal(ops.qscale.cpu().numpy().view(np.uint32), ref["qscale"].view(np.uint32))
    assert np.array_equal(ops.kcode.cpu().numpy(), ref["kcode"])
    assert np.array_equal(ops.kscale.cpu().numpy().view(np.uint32), ref["kscale"].view(np.uint32))
    assert np.array_equal(ops.vmean.float().cpu().numpy(), ref["vmean"])
    assert np.array_equal(ops.vscale.cpu().numpy().view(np.uint32), ref["vscale"].view(np.uint32))
    got_v = ops.vcode.cpu().numpy()
    assert np.array_equal(vcode_natural(got_v, N, bk), ref["vcode"])
    # padding keys of the last sub-block hold code 0
    full = vcode_natural(got_v, desc.nkb * bk, bk) if desc.nkb * bk > N else None
    if full is not None:
        assert not full[:, :, N:].any()
    vs = np.where(ref["vscale"] > 0, ref["vscale"], np.float32(1.0))
    qv = (ref["vmean"] / vs[:, :, None, None]).astype(np.float32)
    hi = fp8.bf16_round(qv)
    lo = fp8.bf16_round((qv - hi).astype(np.float32))
    pairs = ops.vmean_scaled.cpu().numpy().view(np.uint32)
    assert np.array_equal((pairs & 0xFFFF).astype(np.uint32) << 16, hi.view(np.uint32))
    assert np.array_equal(pairs & 0xFFFF0000, lo.view(np.uint32))


@pytest.mark.parametrize("bk", [16, 32, 64, 128])
def test_prepare_small_ragged(bk):
    q, k, v = _bf16_inputs((1, 2, 300, 128), seed=bk, offset=3.0)
    _check_prepare(q, k, v, 128, bk)


def test_prepare_head_dim_64_and_zero_blocks():
    q, k, v = _bf16_inputs((2, 1, 200, 64), seed=5)
    q[:, :, :64] = 0  # an all-zero query block: scale 0, codes 0
    k[:, :, 32:64] = 0
    v[1] = 2.5  # constant values: residuals 0, vscale 0
    _check_prepare(q, k, v, 64, 32)


@functools.lru_cache(maxsize=2)
def _two_heads(name):
    """The workload's first and last head at full sequence length, as bf16 CPU tensors."""
    w = workloads.get(name)
    q, k, v = workloads.generate(w, seed=0)
    sel = [0, w.H - 1]
    return tuple(torch.from_numpy(np.ascontiguousarray(x[:, sel])).to(torch.bfloat16) for x in (q, k, v))


@pytest.mark.parametrize("name", ["wan1.3b", "hunyuan"])
def test_prepare_video_shape_two_heads(name):
    w = workloads.get(name)
    q, k, v = _two_heads(name)
    _check_prepare(q, k, v, w.q_block, w.k_block)


# ---- ab_attn_fwd_fp8 against oracle/fp8.attn_rows_fp8 ----
# The kernel forms x in fp32 (matrix-core sums, one fused multiply-add) where the
# oracle is exact, so a key whose exact code argument 8 (x - m) + 126 lies within
# the fp32 error of a rounding boundary may take the neighbouring ExpCast code (one
# E4M3 step: at most 1/8 of its probability). Outputs are compared within
#   |error| <= 2e-2 + 2^-7 |O| + F elementwise, relative L2 <= 1e-2 + |F| / |O| per
#   query block, |LSE error| <= 2e-3 max(1, |LSE|) + ln(1 + f),
# where F (per element) and f (per row) are what such steps can move (flip_bound);
# they are 0 for a row with no key in the band. A row that keeps one 64-key
# sub-block can move by more than 2e-2 on one step of a key holding 6 % of its mass.
TOL_ABS, TOL_REL, TOL_RL2, TOL_LSE = 2e-2, 2.0 ** -7, 1e-2, 2e-3
U32 = 2.0 ** -24


def flip_bound(prep, vdeq, idx, weights, counts, bq, bk, scale, b, h, r, o_ref, tile=64):
    """Largest change of row r's output (per element) and of its l (relative) that
    one-step code changes of the keys in the fp32 band of a rounding boundary can make.

    The band of a key: the kernel's logit x = a (q . k) + log2 w (a = qscale kscale
    scale log2 e, 128 exact FP8 products summed in fp32) is within
    e_x = 132 u a sum|q_c k_c| + 2u (|x| + |log2 w|) of the exact one (u = 2^-24), the
    running reference m within the largest e_x of its keys, and the argument
    8 (x - m) + 126 within 8 (e_x + e_m) + 2u (8 |x - m| + 126); a key whose exact
    argument is that close to a half-integer may round either way."""
    i = r // bq
    N = prep["qcode"].shape[2]
    c = int(counts[b, h, i])
    if c == 0:
        return np.zeros_like(o_ref), 0.0
    # the kept keys in list order, their list position and their slot in the tile walk
    pos = np.repeat(np.arange(c), bk)
    slot = np.arange(c * bk)
    krows = idx[b, h, i, pos].astype(np.int64) * bk + slot % bk
    real = krows < N
    pos, slot, krows = pos[real], slot[real], krows[real]
    js = idx[b, h, i, pos].astype(np.int64)
    t = slot // tile
    qv = fp8.e4m3_decode(prep["qcode"][b, h, r]).astype(np.float64)
    kv = fp8.e4m3_decode(prep["kcode"][b, h, krows]).astype(np.float64)
    a = prep["qscale"][b, h, i].astype(np.float64) * prep["kscale"][b, h, js].astype(np.float64) * scale * np.log2(np.e)
    lw = np.log2(weights[b, h, i, pos].astype(np.float64))
    xs = a * (kv @ qv) + lw  # in float64, where the FP8 products sum exactly
    ex = 132 * U32 * a * (np.abs(kv) @ np.abs(qv)) + 2 * U32 * (np.abs(xs) + np.abs(lw))
    nt = int(t.max()) + 1
    tmax = np.full(nt, -np.inf)
    temax = np.zeros(nt)
    np.maximum.at(tmax, t, xs)
    np.maximum.at(temax, t, ex)
    mrun, emrun = np.maximum.accumulate(tmax)[t], np.maximum.accumulate(temax)[t]
    arg = 8 * (xs - mrun) + 126
    band = np.abs(arg - np.floor(arg) - 0.5) <= 8 * (ex + emrun) + 2 * U32 * (8 * np.abs(xs - mrun) + 126)
    if not band.any():
        return np.zeros_like(o_ref), 0.0
    sc = 2.0 ** (mrun - xs.max())  # each tile's probabilities in the final reference
    p = fp8.e4m3_decode(fp8.expcast_codes(xs - mrun)).astype(np.float64) * sc
    dp = np.maximum(0.125 * fp8.e4m3_decode(fp8.expcast_codes(xs - mrun)).astype(np.float64), 2.0 ** -9) * sc
    l = p.sum()
    dl = dp[band].sum()
    F = (dp[band, None] * np.abs(vdeq[b, h, krows[band]] - o_ref[None, :])).sum(0) / (l - dl)
    return F, dl / (l - dl)


def _lists(B, H, nqb, nkb, density, seed, empty_row=None):
    """Seeded kept lists (ascending, unique, the tail sub-block kept in some rows) and weights."""
    rng = np.random.default_rng(seed)
    idx = np.zeros((B, H, nqb, nkb), np.int32)
    w = np.zeros((B, H, nqb, nkb), np.float32)
    cnt = np.zeros((B, H, nqb), np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(nqb):
                k = max(1, int(round(density * nkb)))
                sel = np.sort(rng.choice(nkb, k, replace=False))
                if rng.random() < 0.3 and nkb - 1 not in sel:
                    sel[-1] = nkb - 1
                    sel = np.sort(sel)
                idx[b, h, i, :k] = sel
                w[b, h, i, :k] = rng.uniform(1.0, 8.0, k).astype(np.float32)
                cnt[b, h, i] = k
    if empty_row is not None:
        cnt[empty_row] = 0
    return idx, w, cnt


def _check_attn(q, k, v, bk, density, seed, blocks=None, rows_per_block=None, empty_row=None, scale=0.0,
                every_row_written=False):
    dev = _gpu()
    bq = 128
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    desc = ab.Desc.for_tensor(qd, bq, bk, 1, scale=scale)
    B, H, N, d = q.shape
    idx, w, cnt = _lists(B, H, desc.nqb, desc.nkb, density, seed, empty_row)
    ops = ab.ab_fp8_prepare(desc, qd, kd, vd)
    out0 = lse0 = None
    if every_row_written:  # outputs start as NaN: every row must be overwritten
        out0 = torch.full((B, H, N, d), float("nan"), dtype=torch.bfloat16, device=dev)
        lse0 = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
    out, lse = ab.ab_attn_fwd_fp8(desc, ops, torch.from_numpy(idx).to(dev), torch.from_numpy(w).to(dev),
                                  torch.from_numpy(cnt).to(dev), out=out0, lse=lse0)
    torch.cuda.synchronize()
    if every_row_written:
        assert not torch.isnan(out).any() and not torch.isnan(lse).any()
    out = out.float().cpu().numpy()
    lse = lse.cpu().numpy()
    heads = [(b, h) for b in range(B) for h in range(H)] if blocks is None else sorted({(b, h) for (b, h, _) in blocks})
    rng = np.random.default_rng(seed + 1)
    sc = scale if scale > 0 else desc_scale(d)
    for (b, h) in heads:
        qs, ks, vs = (x[b:b + 1, h:h + 1].float().numpy() for x in (q, k, v))
        prep = fp8.prepare(qs, ks, vs, bq, bk)
        vdeq = fp8.dequantize(prep, bq, bk)[2]
        blist = range(desc.nqb) if blocks is None else [i for (bb, hh, i) in blocks if (bb, hh) == (b, h)]
        for i in blist:
            r0, r1 = i * bq, min(N, (i + 1) * bq)
            rows = list(range(r0, r1))
            if rows_per_block is not None:
                rows = sorted(set([r0, r1 - 1] + list(rng.choice(rows, min(rows_per_block, len(rows)), replace=False))))
            one = (idx[b:b + 1, h:h + 1], w[b:b + 1, h:h + 1], cnt[b:b + 1, h:h + 1])
            res = fp8.attn_rows_fp8(prep, *one, bq, bk, sc, [(0, 0, r) for r in rows])
            o_ref = np.stack([res[(0, 0, r)][0] for r in rows])
            l_ref = np.array([res[(0, 0, r)][1] for r in rows])
            fl = [flip_bound(prep, vdeq, *one, bq, bk, sc, 0, 0, r, o_ref[n]) for n, r in enumerate(rows)]
            F = np.stack([f[0] for f in fl])
            fr = np.array([f[1] for f in fl])
            got = out[b, h, rows]
            err = np.abs(got - o_ref)
            assert np.all(err <= TOL_ABS + TOL_REL * np.abs(o_ref) + F), (b, h, i, float(err.max()))
            nrm = np.linalg.norm(o_ref)
            if nrm > 0:
                assert np.linalg.norm(got - o_ref) / nrm <= TOL_RL2 + np.linalg.norm(F) / nrm, (b, h, i)
            else:
                assert not got.any()
            lg = lse[b, h, rows]
            fin = np.isfinite(l_ref)
            assert np.array_equal(np.isfinite(lg), fin)
            lim = TOL_LSE * np.maximum(1.0, np.abs(l_ref[fin])) + np.log1p(fr[fin])
            assert np.all(np.abs(lg[fin] - l_ref[fin]) <= lim), (b, h, i)


def desc_scale(d):
    return 1.0 / np.sqrt(d)


@pytest.mark.parametrize("bk", [16, 32, 64, 128])
def test_attn_fp8_small(bk):
    q, k, v = _bf16_inputs((1, 2, 300, 128), seed=10 + bk, offset=2.0)
    _check_attn(q, k, v, bk, 0.4, seed=bk, empty_row=(0, 1, 1))


def test_attn_fp8_dense_and_peaked():
    g = torch.Generator().manual_seed(3)
    q = (torch.randn((1, 1, 256, 128), generator=g) * 3).to(torch.bfloat16)  # peaked softmax
    k = torch.randn((1, 1, 256, 128), generator=g).to(torch.bfloat16)
    v = (torch.randn((1, 1, 256, 128), generator=g) + 4).to(torch.bfloat16)
    _check_attn(q, k, v, 32, 1.0, seed=7)


def test_attn_fp8_explicit_scale():
    """A caller-given softmax scale (0.2 instead of 1/sqrt(128)) in the FP8 kernel."""
    q, k, v = _bf16_inputs((1, 2, 300, 128), seed=77, offset=1.0)
    _check_attn(q, k, v, 32, 0.4, seed=77, scale=0.2)


def test_attn_fp8_two_batch_entries():
    """B = 2 (and a ragged N): every query block of both entries against the oracle,
    with an empty row in the second entry."""
    q, k, v = _bf16_inputs((2, 2, 260, 128), seed=31, offset=1.0)
    _check_attn(q, k, v, 32, 0.4, seed=31, empty_row=(1, 0, 1))


def test_attn_fp8_extreme_logits():
    """Query blocks whose logits reach +-200 in base-2 units, lie below -40 everywhere,
    or jump by more than 64 within a row's list (the inputs of the scorer's
    reference-path test), every block against the exact FP8 computation."""
    from test_gpu_parity import _reference_path_inputs

    q, k, v = (torch.from_numpy(x).to(torch.bfloat16) for x in _reference_path_inputs())
    _check_attn(q, k, v, 32, 0.5, seed=21)


def _random_fp8_configs(n, seed=88):
    rng = np.random.default_rng(seed)
    return [dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 3)), N=int(rng.integers(1, 1500)),
                 Bk=int(rng.choice([16, 32, 64, 128])), density=float(rng.choice([0.05, 0.2, 0.5, 1.0])),
                 scale=float(rng.choice([0.0, 0.0, 0.05, 0.15])), offset=float(rng.choice([0.0, 1.0, 4.0])),
                 seed=int(rng.integers(0, 2**31))) for _ in range(n)]


@pytest.mark.parametrize("cfg", _random_fp8_configs(12), ids=lambda c: "-".join(str(v) for v in c.values()))
def test_fp8_random_configurations(cfg):
    """Seeded random FP8 descriptors (batch, heads, length, every sub-block size, densities
    0.05-1, default or caller-given scale, V offsets that V-Smooth removes): the prepared
    operands bit-exact, then attention on every query block (its first and last row and
    16 seeded others) against the exact FP8 computation."""
    c = cfg
    q, k, v = _bf16_inputs((c["B"], c["H"], c["N"], 128), seed=c["seed"] % 100000, offset=c["offset"])
    _check_prepare(q, k, v, 128, c["Bk"])
    _check_attn(q, k, v, c["Bk"], c["density"], seed=c["seed"] % 1000, scale=c["scale"], rows_per_block=16)


@pytest.mark.parametrize("name", ["wan1.3b", "hunyuan"])
def test_attn_fp8_video_shape(name):
    """Full sequence length of the workload (its first and last head), sampled blocks
    and rows: the wan1.3b shape (k_block 32, 1024 sub-blocks a row) and the
    HunyuanVideo shape (k_block 16, 7425 sub-blocks a row, ragged tail; eight heads'
    FP8 operands exceed the Infinity Cache, so the kernel takes its query blocks
    head-major). Every row of the output is written (it starts as NaN)."""
    w = workloads.get(name)
    q, k, v = _two_heads(name)
    nqb = -(-w.N // w.q_block)
    blocks = [(0, 0, 0), (0, 0, nqb - 1), (0, 1, 77), (0, 1, nqb - 1)]
    _check_attn(q, k, v, w.k_block, w.density, seed=11, blocks=blocks, rows_per_block=6, every_row_written=True)


# ---- ab_attn_fwd_fp8 against the plain definition (one reference per row) -----------
# The kernel takes each tile's codes against a running reference (raised to the tile
# maximum when it grows); the plain definition takes every code against the row's
# overall maximum (oracle.fp8.attn_rows_fp8_plain). Both replace each exact probability
# a_k = 2^(y_k + 8.75) by an E4M3 value within the ExpCast factor F = 1.0616 * 2^(1/16)
# (pinned in tests/test_oracle_fp8.py); the kernel's fp32 logits move y by less than
# 2^-7, so its codes are within F_k = 1.0616 * 2^(1/16 + 1/128), and its keys outside
# the normal range within 2^-6 absolutely. expcast_output_bound turns these into a
# bound per output element around the exact weighted attention over the values the
# FP8 operands stand for (sparse_ht_attention on the dequantised operands), so
#   |O_kernel - O_exact| <= B(F_k) + 2^-8 |O| + 1e-4   (output rounding, fp32 sums)
#   |O_kernel - O_plain| <= B(F_k) + B(F) + 2^-8 |O| + 1e-4
#   |LSE_kernel - LSE_exact| <= ln F_k + 1e-3.
F_KERNEL = 1.0616 * 2.0 ** (1 / 16 + 1 / 128)


def _hot_first_lists(nqb, nkb, density, seed):
    """Kept lists that always start with sub-block 0 (made to hold every row's largest
    logit), then a seeded choice of the others; weights 1 on sub-block 0, 1..8 elsewhere."""
    rng = np.random.default_rng(seed)
    idx = np.zeros((1, 1, nqb, nkb), np.int32)
    w = np.zeros((1, 1, nqb, nkb), np.float32)
    cnt = np.zeros((1, 1, nqb), np.int32)
    for i in range(nqb):
        k = max(2, int(round(density * nkb)))
        sel = np.concatenate([[0], np.sort(rng.choice(np.arange(1, nkb), k - 1, replace=False))])
        idx[0, 0, i, :k] = sel
        w[0, 0, i, :k] = np.concatenate([[1.0], rng.uniform(1.0, 8.0, k - 1)]).astype(np.float32)
        cnt[0, 0, i] = k
    return idx, w, cnt


def _plain_case(q, k, v, bk, idx, w, cnt, rows_per_block, seed):
    from oracle import sparse_ht_attention
    from test_oracle_fp8 import F_EXPCAST, expcast_output_bound

    dev = _gpu()
    bq = 128
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    desc = ab.Desc.for_tensor(qd, bq, bk, 1)
    N, d = q.shape[2], q.shape[3]
    scale = desc_scale(d)
    ops = ab.ab_fp8_prepare(desc, qd, kd, vd)
    out, lse = ab.ab_attn_fwd_fp8(desc, ops, torch.from_numpy(idx).to(dev), torch.from_numpy(w).to(dev),
                                  torch.from_numpy(cnt).to(dev))
    torch.cuda.synchronize()
    out, lse = out.float().cpu().numpy(), lse.cpu().numpy()
    prep = fp8.prepare(q.float().numpy(), k.float().numpy(), v.float().numpy(), bq, bk)
    qx, kx, vx = fp8.dequantize(prep, bq, bk)
    rng = np.random.default_rng(seed)
    rows = []
    for i in range(desc.nqb):
        r0, r1 = i * bq, min(N, (i + 1) * bq)
        rows += sorted(set([r0, r1 - 1] + rng.choice(np.arange(r0, r1), min(rows_per_block, r1 - r0), replace=False).tolist()))
    plain = fp8.attn_rows_fp8_plain(prep, idx, w, cnt, bq, bk, scale, [(0, 0, r) for r in rows])
    stats = {"exact": 0.0, "plain": 0.0, "plain_abs": 0.0}
    for r in rows:
        i = r // bq
        c = int(cnt[0, 0, i])
        sel, wt = idx[0, 0, i, :c], w[0, 0, i, :c]
        o_ex, lse_ex = sparse_ht_attention(qx[0, 0, r:r + 1], kx[0, 0], vx[0, 0], sel, wt, bk, scale)
        keys = np.concatenate([np.arange(j * bk, min(N, (j + 1) * bk)) for j in sel])
        lw = np.concatenate([np.full(min(N, (j + 1) * bk) - j * bk, np.log(float(x))) for j, x in zip(sel, wt)])
        logits = scale * (kx[0, 0, keys] @ qx[0, 0, r]) + lw
        b_k = expcast_output_bound(logits, vx[0, 0, keys], o_ex[0], F=F_KERNEL, small=2.0 ** -6)
        b_p = expcast_output_bound(logits, vx[0, 0, keys], o_ex[0], F=F_EXPCAST)
        got = out[0, 0, r]
        slack = 2.0 ** -8 * np.abs(o_ex[0]) + 1e-4
        e_ex = np.abs(got - o_ex[0])
        e_pl = np.abs(got - plain[(0, 0, r)][0])
        assert np.all(e_ex <= b_k + slack), (r, float((e_ex / (b_k + slack)).max()))
        assert np.all(e_pl <= b_k + b_p + slack), (r, float((e_pl / (b_k + b_p + slack)).max()))
        assert abs(lse[0, 0, r] - lse_ex[0]) <= np.log(F_KERNEL) + 1e-3, r
        stats["exact"] = max(stats["exact"], float((e_ex / (b_k + slack)).max()))
        stats["plain"] = max(stats["plain"], float((e_pl / (b_k + b_p + slack)).max()))
        stats["plain_abs"] = max(stats["plain_abs"], float(e_pl.max()))
    return out, plain, rows, stats


@pytest.mark.parametrize("bk", [16, 32])
def test_attn_fp8_within_expcast_bound_of_plain_definition(bk):
    """Weighted lists (weights 1..8), several tiles per row: the kernel is within the
    derived ExpCast bound of the exact weighted attention and of the plain definition."""
    q, k, v = _bf16_inputs((1, 1, 640, 128), seed=40 + bk, offset=1.0)
    nqb, nkb = 5, 640 // bk
    idx, w, cnt = _lists(1, 1, nqb, nkb, 0.5, seed=bk)
    _, _, _, stats = _plain_case(q, k, v, bk, idx, w, cnt, rows_per_block=24, seed=bk)
    print(f"bk={bk}: largest error / bound: vs exact {stats['exact']:.3f}, vs plain {stats['plain']:.3f}; "
          f"largest |kernel - plain| {stats['plain_abs']:.4f}")


def test_attn_fp8_matches_plain_definition_when_first_tile_holds_the_maximum():
    """Lists whose first sub-block holds every row's largest weighted logit: the running
    reference starts at the row maximum, so the kernel's codes are those of the plain
    definition (up to a code step at an fp32 rounding boundary), and the kernel is held to
    the tight bound of the tiled comparison against attn_rows_fp8_plain."""
    g = torch.Generator().manual_seed(17)
    N, d, bk = 512, 128, 32
    u = torch.randn(d, generator=g)
    u = u / u.norm()
    q = (4.0 * u + 0.5 * torch.randn((1, 1, N, d), generator=g)).to(torch.bfloat16)
    k = (0.5 * torch.randn((1, 1, N, d), generator=g))
    k[0, 0, :bk] += 32.0 * u
    k = k.to(torch.bfloat16)
    v = torch.randn((1, 1, N, d), generator=g).to(torch.bfloat16)
    nqb, nkb = N // 128, N // bk
    idx, w, cnt = _hot_first_lists(nqb, nkb, 0.5, seed=3)
    out, plain, rows, _ = _plain_case(q, k, v, bk, idx, w, cnt, rows_per_block=128, seed=3)
    # the premise: sub-block 0 holds every checked row's largest weighted logit
    prep = fp8.prepare(q.float().numpy(), k.float().numpy(), v.float().numpy(), 128, bk)
    for r in rows:
        krows, _, xs = fp8._row_terms(prep, idx, w, cnt, 128, bk, desc_scale(d), 0, 0, r)
        assert krows[int(np.argmax(xs))] < bk, r
    o_ref = np.stack([plain[(0, 0, r)][0] for r in rows])
    got = out[0, 0, rows]
    assert np.all(np.abs(got - o_ref) <= TOL_ABS + TOL_REL * np.abs(o_ref))
    assert np.linalg.norm(got - o_ref) / np.linalg.norm(o_ref) <= TOL_RL2
