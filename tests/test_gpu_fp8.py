"""GPU parity of the FP8 variant (VC-Attention page: 8-bit products, V-Smooth,
ExpCast-FP8) through the C ABI, against oracle/fp8.py.

ab_fp8_prepare: every output bit-exact (codes, scales, V-Smooth means and the
scaled-mean pairs): each is a fixed sequence of correctly rounded fp32 operations
and one E4M3 rounding, computed the same way on both sides.
"""

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


def test_prepare_video_shape_two_heads():
    w = workloads.get("wan1.3b")
    q, k, v = workloads.generate(w, seed=0)
    sel = [0, w.H - 1]
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x[:, sel])).to(torch.bfloat16) for x in (q, k, v))
    _check_prepare(q, k, v, w.q_block, w.k_block)
