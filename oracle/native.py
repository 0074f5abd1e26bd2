"""ctypes binding of oracle/csrc/oracle_c.c (test infrastructure only).

The C twin of two oracle steps - the exact-operation fp32 k-means of oracle/ibcs.py
and the integer SIP sampler of oracle/sip.py - for checks over every row of the
full-size workloads, where the numpy forms would take hours. It follows the same
specification operation by operation and is pinned to the numpy forms and to the
same golden values in tests/test_oracle_native.py. Built by build() (and here on
first use when missing) with gcc.
"""

import ctypes
import os
import shutil
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "oracle_c.c")
LIB = os.path.join(HERE, "liboracle_c.so")
_lib = None


def _cpu_has_fma():
    try:
        with open("/proc/cpuinfo") as f:
            return " fma " in f.read()
    except OSError:
        return False


def build(out=LIB):
    """Compile the C twin with gcc (-ffp-contract=off: no fused operations but the
    written fmaf calls)."""
    gcc = shutil.which("gcc")
    if gcc is None:
        raise RuntimeError("gcc is needed to build the oracle's C twin")
    cmd = [gcc, "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math"]
    if _cpu_has_fma():
        cmd.append("-mfma")
    tmp = out + ".tmp"
    subprocess.run(cmd + [SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    lib = ctypes.CDLL(LIB)
    P = ctypes.c_void_p
    lib.oc_kmeans_all.restype = ctypes.c_int
    lib.oc_kmeans_all.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, P, P, P]
    lib.oc_philox.restype = None
    lib.oc_philox.argtypes = [P, P, ctypes.c_int64, P]
    lib.oc_budget.restype = ctypes.c_int
    lib.oc_budget.argtypes = [ctypes.c_double, ctypes.c_int]
    lib.oc_sip_rows.restype = None
    lib.oc_sip_rows.argtypes = [P, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_uint64, P, P, P, P, P, P, P]
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def kmeans_all(Q, q_block, n_clusters, iters):
    """k-means of every query block. Q: float32 [B, H, N, d] (or [BH, N, d]).
    Returns mu float32 [B, H, NQB, C, d], sizes int32 [B, H, NQB, C], assign uint8 [B, H, N]."""
    Q = np.ascontiguousarray(Q, dtype=np.float32)
    lead = Q.shape[:-2]
    N, d = Q.shape[-2:]
    BH = int(np.prod(lead)) if lead else 1
    nqb = -(-N // q_block)
    mu = np.zeros(lead + (nqb, n_clusters, d), np.float32)
    sizes = np.zeros(lead + (nqb, n_clusters), np.int32)
    assign = np.zeros(lead + (N,), np.uint8)
    rc = load().oc_kmeans_all(_ptr(Q), BH, N, d, q_block, n_clusters, iters, _ptr(mu), _ptr(sizes), _ptr(assign))
    if rc != 0:
        raise ValueError("unsupported k-means size")
    return mu, sizes, assign


def budget(density, nkb):
    return int(load().oc_budget(float(density), int(nkb)))


def philox4x32_10(counter, key):
    """Philox4x32-10 of counters uint32 [n, 4] with keys uint32 [n, 2]."""
    c = np.ascontiguousarray(counter, dtype=np.uint32).reshape(-1, 4)
    k = np.ascontiguousarray(np.broadcast_to(key, (c.shape[0], 2)), dtype=np.uint32)
    out = np.empty_like(c)
    load().oc_philox(_ptr(c), _ptr(k), c.shape[0], _ptr(out))
    return out


def sample_all(scores, density, seed, with_thresholds=False, with_uniforms=False, heads=None):
    """SIP on every row of a score tensor float32 [B, H, NQB, NKB] (or, with heads = a
    list of (b, h), of [len(heads), NQB, NKB] holding those heads' rows). Returns a dict
    with counts int32, idx int32 and weight float32 (entries past the count are 0), mask
    uint32 bit words, and optionally the thresholds and the 24-bit uniforms, shaped like
    the input's leading axes."""
    s = np.ascontiguousarray(scores, dtype=np.float32)
    lead, nqb, nkb = s.shape[:-2], s.shape[-2], s.shape[-1]
    if heads is None:
        B, H = lead
        hb = [(b, h) for b in range(B) for h in range(H)]
    else:
        hb = [tuple(x) for x in heads]
        assert len(lead) == 1 and lead[0] == len(hb)
    rows = len(hb) * nqb
    bhi = np.ascontiguousarray(
        [(b, h, i) for (b, h) in hb for i in range(nqb)], dtype=np.int32).reshape(rows, 3)
    out = {
        "counts": np.zeros(lead + (nqb,), np.int32),
        "idx": np.zeros(lead + (nqb, nkb), np.int32),
        "weight": np.zeros(lead + (nqb, nkb), np.float32),
        "mask": np.zeros(lead + (nqb, -(-nkb // 32)), np.uint32),
    }
    th = np.zeros(lead + (nqb, nkb), np.uint32) if with_thresholds else None
    un = np.zeros(lead + (nqb, nkb), np.uint32) if with_uniforms else None
    K = budget(density, nkb)
    load().oc_sip_rows(_ptr(s), rows, nkb, K, int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(bhi), _ptr(out["counts"]),
                       _ptr(out["idx"]), _ptr(out["weight"]), _ptr(out["mask"]), _ptr(th), _ptr(un))
    if th is not None:
        out["thresh"] = th
    if un is not None:
        out["uniforms"] = un
    return out
