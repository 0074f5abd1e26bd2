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
# oracle is exact, so an ExpCast code can land one step away at a rounding
# boundary (a factor 2^(1/8) on one probability); outputs are compared within
#   |error| <= 2e-2 + 2^-7 |O| elementwise, relative L2 <= 1e-2 per query block,
#   |LSE error| <= 2e-3 max(1, |LSE|).
TOL_ABS, TOL_REL, TOL_RL2, TOL_LSE = 2e-2, 2.0 ** -7, 1e-2, 2e-3


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


def _check_attn(q, k, v, bk, density, seed, blocks=None, rows_per_block=None, empty_row=None):
    dev = _gpu()
    bq = 128
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    desc = ab.Desc.for_tensor(qd, bq, bk, 1)
    B, H, N, d = q.shape
    idx, w, cnt = _lists(B, H, desc.nqb, desc.nkb, density, seed, empty_row)
    ops = ab.ab_fp8_prepare(desc, qd, kd, vd)
    out, lse = ab.ab_attn_fwd_fp8(desc, ops, torch.from_numpy(idx).to(dev), torch.from_numpy(w).to(dev),
                                  torch.from_numpy(cnt).to(dev))
    torch.cuda.synchronize()
    out = out.float().cpu().numpy()
    lse = lse.cpu().numpy()
    heads = [(b, h) for b in range(B) for h in range(H)] if blocks is None else sorted({(b, h) for (b, h, _) in blocks})
    rng = np.random.default_rng(seed + 1)
    for (b, h) in heads:
        qs, ks, vs = (x[b:b + 1, h:h + 1].float().numpy() for x in (q, k, v))
        prep = fp8.prepare(qs, ks, vs, bq, bk)
        blist = range(desc.nqb) if blocks is None else [i for (bb, hh, i) in blocks if (bb, hh) == (b, h)]
        for i in blist:
            r0, r1 = i * bq, min(N, (i + 1) * bq)
            rows = list(range(r0, r1))
            if rows_per_block is not None:
                rows = sorted(set([r0, r1 - 1] + list(rng.choice(rows, min(rows_per_block, len(rows)), replace=False))))
            res = fp8.attn_rows_fp8(prep, idx[b:b + 1, h:h + 1], w[b:b + 1, h:h + 1], cnt[b:b + 1, h:h + 1],
                                    bq, bk, desc_scale(d), [(0, 0, r) for r in rows])
            o_ref = np.stack([res[(0, 0, r)][0] for r in rows])
            l_ref = np.array([res[(0, 0, r)][1] for r in rows])
            got = out[b, h, rows]
            err = np.abs(got - o_ref)
            assert np.all(err <= TOL_ABS + TOL_REL * np.abs(o_ref)), (b, h, i, float(err.max()))
            nrm = np.linalg.norm(o_ref)
            if nrm > 0:
                assert np.linalg.norm(got - o_ref) / nrm <= TOL_RL2, (b, h, i)
            else:
                assert not got.any()
            lg = lse[b, h, rows]
            fin = np.isfinite(l_ref)
            assert np.array_equal(np.isfinite(lg), fin)
            assert np.all(np.abs(lg[fin] - l_ref[fin]) <= TOL_LSE * np.maximum(1.0, np.abs(l_ref[fin]))), (b, h, i)


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


def test_attn_fp8_extreme_logits():
    """Query blocks whose logits reach +-200 in base-2 units, lie below -40 everywhere,
    or jump by more than 64 within a row's list (the inputs of the scorer's
    reference-path test), every block against the exact FP8 computation."""
    from test_gpu_parity import _reference_path_inputs

    q, k, v = (torch.from_numpy(x).to(torch.bfloat16) for x in _reference_path_inputs())
    _check_attn(q, k, v, 32, 0.5, seed=21)


@pytest.mark.parametrize("name", ["wan1.3b", "hunyuan"])
def test_attn_fp8_video_shape(name):
    """Full sequence length of the workload (its first and last head), sampled blocks
    and rows: the wan1.3b shape (k_block 32, 1024 sub-blocks a row) and the
    HunyuanVideo shape (k_block 16, 7425 sub-blocks a row, ragged tail)."""
    w = workloads.get(name)
    q, k, v = _two_heads(name)
    nqb = -(-w.N // w.q_block)
    blocks = [(0, 0, 0), (0, 0, nqb - 1), (0, 1, 77), (0, 1, nqb - 1)]
    _check_attn(q, k, v, w.k_block, w.density, seed=11, blocks=blocks, rows_per_block=6)
