"""MI355X (gfx950) block-sparse attention for video diffusion transformers.

Thin ctypes binding over libabattn.so (see include/ab_attn.h). Every stage of
the path runs in the library's HIP kernels; this module only checks tensors,
allocates outputs with torch (device memory and streams are all torch is used
for) and passes pointers plus torch's current HIP stream.

Stages (AB-Attention abstract, paperdot search page, query "Xing Ma"):
  ab_score     IBCS block-importance estimates per (query block, key sub-block)
  ab_sample    SIP draw with inverse-inclusion-probability weights
  ab_sample_systematic  fixed-size systematic draw with the same inclusion probabilities
  ab_sample_topk  top-K truncation of the same scores (weight 1; for estimator comparisons)
  ab_intra_lists  INTRA's static Scatter / Gather relay patterns as kept lists (INTRA page)
  ab_attn_fwd  weighted block-sparse attention over the kept sub-blocks
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = [
    "Desc",
    "load_library",
    "library_path",
    "ab_abi_version",
    "ab_score_workspace_size",
    "ab_score",
    "ab_score_noalloc",
    "ab_score_debug",
    "ab_sample",
    "ab_sample_systematic",
    "ab_sample_topk",
    "ab_intra_lists",
    "ab_attn_fwd",
    "ab_attn_fwd_ordered",
    "AbError",
    "AB_INTRA_SCATTER",
    "AB_INTRA_GATHER",
    "AB_BF16",
    "AB_F32",
    "EXPORTED_SYMBOLS",
    "Fp8Operands",
    "ab_fp8_prepare",
    "ab_attn_fwd_fp8",
]

AB_BF16 = 0
AB_F32 = 1
AB_INTRA_SCATTER = 0
AB_INTRA_GATHER = 1
EXPORTED_SYMBOLS = (
    "ab_abi_version",
    "ab_status_str",
    "ab_last_error",
    "ab_score_workspace_size",
    "ab_score",
    "ab_score_noalloc",
    "ab_score_debug",
    "ab_sample",
    "ab_sample_systematic",
    "ab_sample_topk",
    "ab_intra_lists",
    "ab_attn_fwd",
    "ab_attn_fwd_ordered",
    "ab_fp8_workspace_size",
    "ab_fp8_prepare",
    "ab_attn_fwd_fp8",
)

_PKG = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_PKG, "libabattn.so")


class AbError(RuntimeError):
    def __init__(self, code: int, fn: str, msg: str):
        super().__init__(f"{fn} failed with {code}: {msg}")
        self.code = code


class _Desc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("N", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("q_block", ctypes.c_int32),
        ("k_block", ctypes.c_int32),
        ("n_clusters", ctypes.c_int32),
        ("kmeans_iters", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]


class Desc:
    """Problem descriptor (mirrors ab_desc)."""

    def __init__(self, B, H, N, d, dtype, q_block, k_block, n_clusters, kmeans_iters=4, scale=0.0):
        self.B, self.H, self.N, self.d = int(B), int(H), int(N), int(d)
        self.dtype = int(dtype)
        self.q_block, self.k_block = int(q_block), int(k_block)
        self.n_clusters, self.kmeans_iters = int(n_clusters), int(kmeans_iters)
        self.scale = float(scale)

    @classmethod
    def for_tensor(cls, q: torch.Tensor, q_block, k_block, n_clusters, kmeans_iters=4, scale=0.0):
        B, H, N, d = q.shape
        dt = AB_BF16 if q.dtype == torch.bfloat16 else AB_F32
        return cls(B, H, N, d, dt, q_block, k_block, n_clusters, kmeans_iters, scale)

    @property
    def nqb(self):
        return -(-self.N // self.q_block)

    @property
    def nkb(self):
        return -(-self.N // self.k_block)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == AB_BF16 else torch.float32

    def softmax_scale(self):
        return self.scale if self.scale > 0 else 1.0 / math.sqrt(self.d)

    def c(self) -> _Desc:
        return _Desc(self.B, self.H, self.N, self.d, self.dtype, self.q_block, self.k_block, self.n_clusters,
                     self.kmeans_iters, self.scale)


_lib = None


def load_library():
    """Load libabattn.so from this package (built by block_sparse_attention_ibcs_amd.build);
    the environment variable AB_ATTN_LIBRARY names another build of it (e.g. one with the
    host code compiled under sanitizers)."""
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("AB_ATTN_LIBRARY") or library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m block_sparse_attention_ibcs_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    D = ctypes.POINTER(_Desc)
    lib.ab_abi_version.restype = ctypes.c_int32
    lib.ab_status_str.restype = ctypes.c_char_p
    lib.ab_status_str.argtypes = [ctypes.c_int32]
    lib.ab_last_error.restype = ctypes.c_char_p
    lib.ab_score_workspace_size.restype = ctypes.c_size_t
    lib.ab_score_workspace_size.argtypes = [D]
    lib.ab_score.restype = ctypes.c_int32
    lib.ab_score.argtypes = [D, P, P, P, P, ctypes.c_size_t, P]
    lib.ab_score_noalloc.restype = ctypes.c_int32
    lib.ab_score_noalloc.argtypes = [D, P, P, P, P]
    lib.ab_score_debug.restype = ctypes.c_int32
    lib.ab_score_debug.argtypes = [D, P, P, P, P, P]
    lib.ab_sample.restype = ctypes.c_int32
    lib.ab_sample.argtypes = [D, P, ctypes.c_double, ctypes.c_uint64, P, P, P, P, P]
    lib.ab_sample_systematic.restype = ctypes.c_int32
    lib.ab_sample_systematic.argtypes = [D, P, ctypes.c_double, ctypes.c_uint64, P, P, P, P, P]
    lib.ab_sample_topk.restype = ctypes.c_int32
    lib.ab_sample_topk.argtypes = [D, P, ctypes.c_double, P, P, P, P, P]
    lib.ab_intra_lists.restype = ctypes.c_int32
    lib.ab_intra_lists.argtypes = [D, ctypes.c_int32, ctypes.c_int32, P, P, P, P, P]
    lib.ab_attn_fwd.restype = ctypes.c_int32
    lib.ab_attn_fwd.argtypes = [D, P, P, P, P, P, P, P, P, P]
    lib.ab_attn_fwd_ordered.restype = ctypes.c_int32
    lib.ab_attn_fwd_ordered.argtypes = [D, P, P, P, P, P, P, P, P, P, P]
    lib.ab_fp8_workspace_size.restype = ctypes.c_size_t
    lib.ab_fp8_workspace_size.argtypes = [D]
    lib.ab_fp8_prepare.restype = ctypes.c_int32
    lib.ab_fp8_prepare.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.ab_attn_fwd_fp8.restype = ctypes.c_int32
    lib.ab_attn_fwd_fp8.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P, P]
    _lib = lib
    return lib


def _check(rc: int, fn: str):
    if rc != 0:
        lib = load_library()
        raise AbError(rc, fn, lib.ab_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, shape, dtype):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def ab_abi_version() -> int:
    return int(load_library().ab_abi_version())


def ab_score_workspace_size(desc: Desc) -> int:
    lib = load_library()
    cd = desc.c()
    n = int(lib.ab_score_workspace_size(ctypes.byref(cd)))
    if n == 0:
        raise AbError(-2, "ab_score_workspace_size", lib.ab_last_error().decode())
    return n


def alloc_workspace(desc: Desc, device=None) -> torch.Tensor:
    """A device byte buffer large enough for ab_score (torch allocations are 256-byte aligned)."""
    return torch.empty(ab_score_workspace_size(desc), dtype=torch.uint8, device=device or "cuda")


def ab_score(desc: Desc, q, k, scores=None, workspace=None, stream=None):
    """IBCS scores, fp32 [B, H, NQB, NKB]."""
    lib = load_library()
    shp = (desc.B, desc.H, desc.N, desc.d)
    _need(q, "q", shp, desc.torch_dtype)
    _need(k, "k", shp, desc.torch_dtype)
    if scores is None:
        scores = torch.empty((desc.B, desc.H, desc.nqb, desc.nkb), dtype=torch.float32, device=q.device)
    _need(scores, "scores", (desc.B, desc.H, desc.nqb, desc.nkb), torch.float32)
    if workspace is None:
        workspace = alloc_workspace(desc, q.device)
    cd = desc.c()
    rc = lib.ab_score(ctypes.byref(cd), _ptr(q), _ptr(k), _ptr(scores), _ptr(workspace), workspace.numel(),
                      _stream(stream))
    _check(rc, "ab_score")
    return scores


AB_SCORE_NOALLOC_SCRATCH_BYTES = 256 << 20  # the library's fixed scratch for ab_score_noalloc, per GPU


def ab_score_noalloc(desc: Desc, q, k, scores, stream=None):
    """IBCS scores into a caller-given fp32 [B, H, NQB, NKB] tensor, with the library's
    fixed scratch instead of a workspace (no device allocation in the call)."""
    lib = load_library()
    shp = (desc.B, desc.H, desc.N, desc.d)
    _need(q, "q", shp, desc.torch_dtype)
    _need(k, "k", shp, desc.torch_dtype)
    _need(scores, "scores", (desc.B, desc.H, desc.nqb, desc.nkb), torch.float32)
    cd = desc.c()
    rc = lib.ab_score_noalloc(ctypes.byref(cd), _ptr(q), _ptr(k), _ptr(scores), _stream(stream))
    _check(rc, "ab_score_noalloc")
    return scores


def ab_score_debug(desc: Desc, q, stream=None):
    """k-means stage alone: (centroids fp32 [B,H,NQB,C,d], sizes int32 [B,H,NQB,C], assign uint8 [B,H,N])."""
    lib = load_library()
    _need(q, "q", (desc.B, desc.H, desc.N, desc.d), desc.torch_dtype)
    cent = torch.empty((desc.B, desc.H, desc.nqb, desc.n_clusters, desc.d), dtype=torch.float32, device=q.device)
    sizes = torch.empty((desc.B, desc.H, desc.nqb, desc.n_clusters), dtype=torch.int32, device=q.device)
    assign = torch.empty((desc.B, desc.H, desc.N), dtype=torch.uint8, device=q.device)
    cd = desc.c()
    rc = lib.ab_score_debug(ctypes.byref(cd), _ptr(q), _ptr(cent), _ptr(sizes), _ptr(assign), _stream(stream))
    _check(rc, "ab_score_debug")
    return cent, sizes, assign


def ab_sample(desc: Desc, scores, density: float, seed: int, idx=None, weights=None, counts=None, mask=None,
              want_mask=True, stream=None):
    """SIP draw: (idx int32, weights fp32 [B,H,NQB,NKB], counts int32 [B,H,NQB], mask uint32 or None)."""
    lib = load_library()
    rows = (desc.B, desc.H, desc.nqb)
    _need(scores, "scores", rows + (desc.nkb,), torch.float32)
    dev = scores.device
    if idx is None:
        idx = torch.empty(rows + (desc.nkb,), dtype=torch.int32, device=dev)
    if weights is None:
        weights = torch.empty(rows + (desc.nkb,), dtype=torch.float32, device=dev)
    if counts is None:
        counts = torch.empty(rows, dtype=torch.int32, device=dev)
    if mask is None and want_mask:
        mask = torch.empty(rows + (-(-desc.nkb // 32),), dtype=torch.int32, device=dev)
    cd = desc.c()
    rc = lib.ab_sample(ctypes.byref(cd), _ptr(scores), float(density), int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(idx),
                       _ptr(weights), _ptr(counts), _ptr(mask), _stream(stream))
    _check(rc, "ab_sample")
    return idx, weights, counts, mask


def ab_sample_systematic(desc: Desc, scores, density: float, seed: int, idx=None, weights=None, counts=None,
                         mask=None, want_mask=True, stream=None):
    """Systematic draw: (idx int32, weights fp32 [B,H,NQB,NKB], counts int32 [B,H,NQB], mask uint32 or None)."""
    lib = load_library()
    rows = (desc.B, desc.H, desc.nqb)
    _need(scores, "scores", rows + (desc.nkb,), torch.float32)
    dev = scores.device
    if idx is None:
        idx = torch.empty(rows + (desc.nkb,), dtype=torch.int32, device=dev)
    if weights is None:
        weights = torch.empty(rows + (desc.nkb,), dtype=torch.float32, device=dev)
    if counts is None:
        counts = torch.empty(rows, dtype=torch.int32, device=dev)
    if mask is None and want_mask:
        mask = torch.empty(rows + (-(-desc.nkb // 32),), dtype=torch.int32, device=dev)
    cd = desc.c()
    rc = lib.ab_sample_systematic(ctypes.byref(cd), _ptr(scores), float(density), int(seed) & 0xFFFFFFFFFFFFFFFF,
                                  _ptr(idx), _ptr(weights), _ptr(counts), _ptr(mask), _stream(stream))
    _check(rc, "ab_sample_systematic")
    return idx, weights, counts, mask


def ab_sample_topk(desc: Desc, scores, density: float, idx=None, weights=None, counts=None, mask=None,
                   want_mask=True, stream=None):
    """Top-K truncation: (idx int32, weights fp32 ones [B,H,NQB,NKB], counts int32 [B,H,NQB], mask or None)."""
    lib = load_library()
    rows = (desc.B, desc.H, desc.nqb)
    _need(scores, "scores", rows + (desc.nkb,), torch.float32)
    dev = scores.device
    if idx is None:
        idx = torch.empty(rows + (desc.nkb,), dtype=torch.int32, device=dev)
    if weights is None:
        weights = torch.empty(rows + (desc.nkb,), dtype=torch.float32, device=dev)
    if counts is None:
        counts = torch.empty(rows, dtype=torch.int32, device=dev)
    if mask is None and want_mask:
        mask = torch.empty(rows + (-(-desc.nkb // 32),), dtype=torch.int32, device=dev)
    cd = desc.c()
    rc = lib.ab_sample_topk(ctypes.byref(cd), _ptr(scores), float(density), _ptr(idx), _ptr(weights), _ptr(counts),
                            _ptr(mask), _stream(stream))
    _check(rc, "ab_sample_topk")
    return idx, weights, counts, mask


def ab_intra_lists(desc: Desc, layer: int, partition_tokens: int = 0, idx=None, weights=None, counts=None,
                   row_order=None, want_order=False, device=None, stream=None):
    """INTRA Scatter (layer 0) or Gather (layer 1) pattern: (idx int32, weights fp32 [B,H,NQB,NKB],
    counts int32 [B,H,NQB]), plus the processing order int32 [B*H*NQB] for ab_attn_fwd_ordered
    when want_order (or row_order is given); partition_tokens 0 selects q_block * ceil(sqrt(NQB))."""
    lib = load_library()
    rows = (desc.B, desc.H, desc.nqb)
    dev = device if device is not None else (idx.device if idx is not None else torch.device("cuda"))
    if idx is None:
        idx = torch.empty(rows + (desc.nkb,), dtype=torch.int32, device=dev)
    if weights is None:
        weights = torch.empty(rows + (desc.nkb,), dtype=torch.float32, device=dev)
    if counts is None:
        counts = torch.empty(rows, dtype=torch.int32, device=dev)
    _need(idx, "idx", rows + (desc.nkb,), torch.int32)
    _need(weights, "weights", rows + (desc.nkb,), torch.float32)
    _need(counts, "counts", rows, torch.int32)
    if row_order is None and want_order:
        row_order = torch.empty(desc.B * desc.H * desc.nqb, dtype=torch.int32, device=dev)
    if row_order is not None:
        _need(row_order, "row_order", (desc.B * desc.H * desc.nqb,), torch.int32)
    cd = desc.c()
    rc = lib.ab_intra_lists(ctypes.byref(cd), int(layer), int(partition_tokens), _ptr(idx), _ptr(weights),
                            _ptr(counts), _ptr(row_order), _stream(stream))
    _check(rc, "ab_intra_lists")
    return (idx, weights, counts, row_order) if row_order is not None else (idx, weights, counts)


def ab_attn_fwd(desc: Desc, q, k, v, idx, weights, counts, out=None, lse=None, want_lse=True, stream=None):
    """Weighted block-sparse attention: (out [B,H,N,d] in the input dtype, lse fp32 [B,H,N] or None)."""
    lib = load_library()
    shp = (desc.B, desc.H, desc.N, desc.d)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, shp, desc.torch_dtype)
    rows = (desc.B, desc.H, desc.nqb)
    _need(idx, "idx", rows + (desc.nkb,), torch.int32)
    _need(weights, "weights", rows + (desc.nkb,), torch.float32)
    _need(counts, "counts", rows, torch.int32)
    if out is None:
        out = torch.empty(shp, dtype=desc.torch_dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty(shp[:3], dtype=torch.float32, device=q.device)
    cd = desc.c()
    rc = lib.ab_attn_fwd(ctypes.byref(cd), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(weights), _ptr(counts),
                         _ptr(out), _ptr(lse), _stream(stream))
    _check(rc, "ab_attn_fwd")
    return out, lse


def ab_attn_fwd_ordered(desc: Desc, q, k, v, idx, weights, counts, row_order, out=None, lse=None, want_lse=True,
                        stream=None):
    """ab_attn_fwd with the query-block rows taken in row_order (int32 [B*H*NQB]); same outputs."""
    lib = load_library()
    shp = (desc.B, desc.H, desc.N, desc.d)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, shp, desc.torch_dtype)
    rows = (desc.B, desc.H, desc.nqb)
    _need(idx, "idx", rows + (desc.nkb,), torch.int32)
    _need(weights, "weights", rows + (desc.nkb,), torch.float32)
    _need(counts, "counts", rows, torch.int32)
    _need(row_order, "row_order", (desc.B * desc.H * desc.nqb,), torch.int32)
    if out is None:
        out = torch.empty(shp, dtype=desc.torch_dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty(shp[:3], dtype=torch.float32, device=q.device)
    cd = desc.c()
    rc = lib.ab_attn_fwd_ordered(ctypes.byref(cd), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(weights),
                                 _ptr(counts), _ptr(row_order), _ptr(out), _ptr(lse), _stream(stream))
    _check(rc, "ab_attn_fwd_ordered")
    return out, lse


class Fp8Operands:
    """Device tensors of ab_fp8_prepare's outputs (layouts as in include/ab_attn.h)."""

    def __init__(self, desc: Desc, device):
        B, H, N, d = desc.B, desc.H, desc.N, desc.d
        u8 = torch.uint8
        self.qcode = torch.empty((B, H, N, d), dtype=u8, device=device)
        self.qscale = torch.empty((B, H, desc.nqb), dtype=torch.float32, device=device)
        self.kcode = torch.empty((B, H, N, d), dtype=u8, device=device)
        self.kscale = torch.empty((B, H, desc.nkb), dtype=torch.float32, device=device)
        self.vcode = torch.empty((B, H, desc.nkb, 2, d, desc.k_block // 2), dtype=u8, device=device)
        self.vmean = torch.empty((B, H, desc.nkb, d), dtype=torch.bfloat16, device=device)
        self.vscale = torch.empty((B, H), dtype=torch.float32, device=device)
        self.vmean_scaled = torch.empty((B, H, desc.nkb, d), dtype=torch.int32, device=device)
        lib = load_library()
        cd = desc.c()
        nbytes = int(lib.ab_fp8_workspace_size(ctypes.byref(cd)))
        if nbytes == 0:
            raise AbError(-2, "ab_fp8_workspace_size", lib.ab_last_error().decode())
        self.ws = torch.empty((nbytes + 3) // 4, dtype=torch.int32, device=device)


def ab_fp8_prepare(desc: Desc, q, k, v, ops: "Fp8Operands" = None, stream=None) -> "Fp8Operands":
    """FP8 operands (E4M3 codes and scales, V-Smooth means) of q, k, v (bf16 [B,H,N,d])."""
    lib = load_library()
    shp = (desc.B, desc.H, desc.N, desc.d)
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, shp, torch.bfloat16)
    if ops is None:
        ops = Fp8Operands(desc, q.device)
    cd = desc.c()
    rc = lib.ab_fp8_prepare(ctypes.byref(cd), _ptr(q), _ptr(k), _ptr(v), _ptr(ops.qcode), _ptr(ops.qscale),
                            _ptr(ops.kcode), _ptr(ops.kscale), _ptr(ops.vcode), _ptr(ops.vmean), _ptr(ops.vscale),
                            _ptr(ops.vmean_scaled), _ptr(ops.ws), ops.ws.numel() * 4, _stream(stream))
    _check(rc, "ab_fp8_prepare")
    return ops


def ab_attn_fwd_fp8(desc: Desc, ops: "Fp8Operands", idx, weights, counts, out=None, lse=None, want_lse=True,
                    stream=None):
    """FP8 weighted block-sparse attention from ab_fp8_prepare's operands; (out bf16, lse fp32 or None)."""
    lib = load_library()
    rows = (desc.B, desc.H, desc.nqb)
    _need(idx, "idx", rows + (desc.nkb,), torch.int32)
    _need(weights, "weights", rows + (desc.nkb,), torch.float32)
    _need(counts, "counts", rows, torch.int32)
    dev = ops.qcode.device
    if out is None:
        out = torch.empty((desc.B, desc.H, desc.N, desc.d), dtype=torch.bfloat16, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((desc.B, desc.H, desc.N), dtype=torch.float32, device=dev)
    cd = desc.c()
    rc = lib.ab_attn_fwd_fp8(ctypes.byref(cd), _ptr(ops.qcode), _ptr(ops.qscale), _ptr(ops.kcode), _ptr(ops.kscale),
                             _ptr(ops.vcode), _ptr(ops.vscale), _ptr(ops.vmean_scaled), _ptr(idx), _ptr(weights),
                             _ptr(counts), _ptr(out), _ptr(lse), _stream(stream))
    _check(rc, "ab_attn_fwd_fp8")
    return out, lse
