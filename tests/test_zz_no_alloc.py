"""ab_score_noalloc (the allocation-free scorer) against ab_score, through the C ABI:
two calls in a row, the second on a smaller problem, must reproduce ab_score's scores
bit for bit (each head runs the same arithmetic with the same key splits); the first
call needs several chunks of heads, the second one."""

import numpy as np
import pytest
import torch

import block_sparse_attention_ibcs_amd as ab

pytestmark = pytest.mark.gpu


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _inputs(B, H, N, d, dtype, seed, dev):
    g = torch.Generator(device="cpu").manual_seed(seed)
    base = torch.randn((B, H, N, d), generator=g)
    q = (base + 0.5 * torch.randn((B, H, N, d), generator=g)).to(dtype).to(dev)
    k = (base + 0.5 * torch.randn((B, H, N, d), generator=g)).to(dtype).to(dev)
    return q, k


def test_noalloc_matches_ab_score_on_two_calls():
    dev = _gpu()
    cases = [
        # the 40-head, 75600-token shape: one head needs ~49 MB, so several chunks of heads
        (1, 40, 75600, 128, torch.bfloat16, 128, 32, 8),
        # smaller: two batch entries of six heads; chunks of three heads, so two chunk
        # boundaries fall inside a batch entry
        (2, 6, 75600, 128, torch.bfloat16, 128, 32, 8),
        # then a smaller, ragged problem in one chunk
        (2, 3, 5001, 64, torch.bfloat16, 64, 16, 4),
    ]
    for n_call, (B, H, N, d, dt, bq, bk, C) in enumerate(cases):
        print(f"no-alloc call {n_call}: B={B} H={H} N={N} d={d} {dt} Bq={bq} Bk={bk} C={C}", flush=True)
        q, k = _inputs(B, H, N, d, dt, 10 + n_call, dev)
        desc = ab.Desc.for_tensor(q, bq, bk, C)
        ref = ab.ab_score(desc, q, k)
        out = torch.full_like(ref, float("nan"))
        ab.ab_score_noalloc(desc, q, k, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (n_call, float((out - ref).abs().max()))
        del q, k, ref, out
        torch.cuda.empty_cache()


def test_noalloc_fp32_and_rejects_oversized_heads():
    dev = _gpu()
    q, k = _inputs(1, 2, 1000, 128, torch.float32, 3, dev)
    desc = ab.Desc.for_tensor(q, 128, 32, 8)
    ref = ab.ab_score(desc, q, k)
    out = torch.empty_like(ref)
    ab.ab_score_noalloc(desc, q, k, out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    # a head whose sub-block table alone exceeds the scratch: rejected before any launch
    big = ab.Desc(1, 1, 1 << 20, 128, ab.AB_BF16, 128, 16, 8)
    lib = ab.load_library()
    cd = big.c()
    dummy = torch.empty(16, dtype=torch.uint8, device=dev)
    import ctypes
    rc = lib.ab_score_noalloc(ctypes.byref(cd), ctypes.c_void_p(dummy.data_ptr()), ctypes.c_void_p(dummy.data_ptr()),
                              ctypes.c_void_p(dummy.data_ptr()), None)
    assert rc == -6 and b"allocation-free" in lib.ab_last_error()
