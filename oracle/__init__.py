"""fp64 CPU oracle of the IKBO hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package. It shares no code with the GPU library (``request_candidate_broadcast_amd``)
and never imports it.

The arithmetic lives in ``ikbo_oracle.c`` (plain C, fp64, threaded over candidates). It expands
every request-side tensor once per candidate -- the materialised broadcast the GPU path avoids --
then evaluates the definitions:

* ``dca``   candidate cross attention, ROCS Sec. 3.2 Eq. 13 (A^C) with request-batched K/V read
            through the candidate->request map (Sec. 4.3.1); two-pass softmax.
* ``glm``   the GLM-masked affine layer stack, Sec. 3.1.2 Eq. 4/6 (explicit zero block), with the
            per-group activation of Eq. 8, composed as in Sec. 3.1.5 Eq. 11. One layer is the
            IKBO-LCB linear form; two layers are the query MLP of Eq. 12.
* ``gelu``  exact GELU x * Phi(x) via libm erf.
* ``linear`` the request-side K/V projection, Sec. 4.1 (the DCA decomposition after Eq. 14):
            y = x W^T in fp64 with a library matmul on exactly decoded inputs (numpy).
* ``request_attention`` the request half A^R of Eq. 13: ``dca`` with one candidate per request.
* ``fm``    the GLM factorization machine, Sec. 3.1.4 Eq. 9-10 (two groups): request outputs
            X^R (X^R)^T, candidate outputs [X^C (X^R_m)^T, X^C (X^C)^T], in fp64 with the request
            rows expanded per candidate.
* ``dca_layer`` one DCA interaction layer, Sec. 3.2 Eq. 12-13: the query generator (``glm``), the
            K/V projections of the layer's sequence rows for both halves (``linear``), A^C
            (``dca``) and A^R (``request_attention``), each group's output the concatenation
            [Q | A] that the next layer reads; composed in fp64 with no rounding in between.
* ``lcb_emb`` the ROCSified LCB in its embedding-matrix (row-axis) form, Sec. 3.1.2 Eq. 5-6 (two
            groups): Y^R = W_RR X^R, Y^C = W_CR X^R_m + W_CC X^C, followed by the group-local
            normalisation of Sec. 3.1.3 Eq. 7 (LayerNorm or RMSNorm of each embedding row), in
            fp64 with the request embeddings expanded per candidate.

Parity status: every function here is pinned by ``tests/test_oracle_*.py`` against library
routines, closed forms, invariants and brute force on tiny inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libikbo_oracle.so")
SRC_PATH = os.path.join(_HERE, "ikbo_oracle.c")

F32, BF16, F64 = 0, 1, 2
ACT = {"none": 0, "gelu": 1}


def build_lib(force: bool = False) -> str:
    """Compile the oracle with gcc -O2 (no fast-math, no BLAS)."""
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
        tmp = LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               SRC_PATH, "-o", tmp, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


class _Layer(ctypes.Structure):
    _fields_ = [("w_rr", ctypes.c_void_p), ("w_cr", ctypes.c_void_p), ("w_cc", ctypes.c_void_p),
                ("b_r", ctypes.c_void_p), ("b_c", ctypes.c_void_p),
                ("k_req", ctypes.c_int32), ("k_cand", ctypes.c_int32),
                ("n_req", ctypes.c_int32), ("n_cand", ctypes.c_int32), ("act", ctypes.c_int32)]


_lib = None


def _get():
    global _lib
    if _lib is None:
        build_lib()
        lib = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.oracle_gelu.restype = dbl
        lib.oracle_gelu.argtypes = [dbl]
        lib.oracle_request_of.restype = i64
        lib.oracle_request_of.argtypes = [vp, vp, i64, i64, vp]
        lib.oracle_dca.restype = ctypes.c_int
        lib.oracle_dca.argtypes = [vp, i64, i32, vp, vp, i64, vp, i32, vp, vp, i32, i32, dbl, i32, i32,
                                   vp, i64, vp, ctypes.POINTER(ctypes.c_int64), i32]
        lib.oracle_glm.restype = ctypes.c_int
        lib.oracle_glm.argtypes = [vp, i64, vp, i64, vp, vp, i32, ctypes.POINTER(_Layer), i32,
                                   vp, i64, vp, vp, vp, ctypes.POINTER(ctypes.c_int64), i32]
        lib.oracle_index_violations.restype = i64
        lib.oracle_index_violations.argtypes = [vp, vp, i64, i64, i32]
        _lib = lib
    return _lib


class OracleError(RuntimeError):
    pass


def _threads(n: Optional[int]) -> int:
    return n if n else max(1, min(16, os.cpu_count() or 1))


def _dtype_code(arr: np.ndarray) -> int:
    if arr.dtype == np.uint16:
        return BF16
    if arr.dtype == np.float32:
        return F32
    raise TypeError("oracle inputs are bf16 bit patterns (uint16) or float32, got %s" % arr.dtype)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def gelu(x: float) -> float:
    return float(_get().oracle_gelu(float(x)))


def request_of(m, off, R: int, c: int) -> int:
    """Request of candidate c: from the offsets when given (they define the grouping), else from
    the map; -1 when it has none. A map that disagrees with the offsets is a violation (see
    ``index_violations``), not an error."""
    m, off = _i32(m), _i32(off)
    return int(_get().oracle_request_of(_ptr(m), _ptr(off), R, c, None))


def dca(q: np.ndarray, k: np.ndarray, v: np.ndarray, R: int, *, m=None, off=None, kv_cu=None,
        L: Optional[int] = None, scale: Optional[float] = None, cands: Optional[Sequence[int]] = None,
        nthreads: Optional[int] = None, return_violations: bool = False):
    """Cross attention of candidate queries over their request's K/V, fp64.

    q [C, Lq, H, d]; k, v [R, L, H, d] or varlen [sum L_r, H, d] with kv_cu [R+1].
    q, k and v may also be float64 (chained fp64 values). Returns [n, Lq, H, d] fp64 for the
    candidates `cands` (all when None)."""
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    dt = F64 if k.dtype == np.float64 else _dtype_code(k)
    assert (F64 if v.dtype == np.float64 else _dtype_code(v)) == dt
    qdt = F64 if q.dtype == np.float64 else _dtype_code(q)
    C, Lq, H, d = q.shape
    m, off, kv_cu = _i32(m), _i32(off), _i32(kv_cu)
    if kv_cu is None:
        Lu = k.shape[1] if k.ndim == 4 else (L if L is not None else 0)
    else:
        Lu = int(np.max(np.diff(kv_cu))) if R > 0 else 0
        if L is not None:
            Lu = max(Lu, L)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    cand_arr = None if cands is None else np.ascontiguousarray(cands, dtype=np.int64)
    n = C if cand_arr is None else len(cand_arr)
    out = np.zeros((n, Lq, H, d), dtype=np.float64)
    viol = ctypes.c_int64(0)
    rc = _get().oracle_dca(_ptr(q), C, Lq, _ptr(k), _ptr(v), R, _ptr(kv_cu), Lu, _ptr(m), _ptr(off),
                           H, d, float(scale), dt, qdt, _ptr(cand_arr), n, _ptr(out), ctypes.byref(viol),
                           _threads(nthreads))
    if rc != 0:
        raise OracleError("oracle_dca failed with code %d" % rc)
    return (out, viol.value) if return_violations else out


def glm(x_r: np.ndarray, x_c: np.ndarray, layers: Sequence[dict], *, m=None, off=None,
        cands: Optional[Sequence[int]] = None, want_request_per_cand: bool = False,
        want_request: bool = False, nthreads: Optional[int] = None, return_violations: bool = False):
    """GLM-masked layer stack, fp64.

    layers: dicts with w_rr [N_r,K_r], w_cr [N_c,K_r], w_cc [N_c,K_c] (bf16 bits or fp32),
    b_r, b_c fp32 (or None) and act ("none" | "gelu").
    Returns dict with y_c [n, N_c], and optionally y_r_c [n, N_r], y_r [R, N_r]."""
    x_r = np.ascontiguousarray(x_r)
    x_c = np.ascontiguousarray(x_c)
    dt = _dtype_code(x_r)
    assert _dtype_code(x_c) == dt
    R, C = x_r.shape[0], x_c.shape[0]
    keep = []
    arr = (_Layer * len(layers))()
    for i, ly in enumerate(layers):
        w_rr = np.ascontiguousarray(ly["w_rr"])
        w_cr = np.ascontiguousarray(ly["w_cr"])
        w_cc = np.ascontiguousarray(ly["w_cc"])
        for w in (w_rr, w_cr, w_cc):
            assert _dtype_code(w) == dt
        b_r = None if ly.get("b_r") is None else np.ascontiguousarray(ly["b_r"], dtype=np.float32)
        b_c = None if ly.get("b_c") is None else np.ascontiguousarray(ly["b_c"], dtype=np.float32)
        keep += [w_rr, w_cr, w_cc, b_r, b_c]
        arr[i] = _Layer(w_rr.ctypes.data, w_cr.ctypes.data, w_cc.ctypes.data,
                        None if b_r is None else b_r.ctypes.data,
                        None if b_c is None else b_c.ctypes.data,
                        w_rr.shape[1], w_cc.shape[1], w_rr.shape[0], w_cc.shape[0],
                        ACT[ly.get("act", "none")])
    m, off = _i32(m), _i32(off)
    cand_arr = None if cands is None else np.ascontiguousarray(cands, dtype=np.int64)
    n = C if cand_arr is None else len(cand_arr)
    nr, nc = int(arr[len(layers) - 1].n_req), int(arr[len(layers) - 1].n_cand)
    y_c = np.zeros((n, nc), dtype=np.float64)
    y_r_c = np.zeros((n, nr), dtype=np.float64) if want_request_per_cand else None
    y_r = np.zeros((R, nr), dtype=np.float64) if want_request else None
    viol = ctypes.c_int64(0)
    rc = _get().oracle_glm(_ptr(x_r), R, _ptr(x_c), C, _ptr(m), _ptr(off), len(layers), arr, dt,
                           _ptr(cand_arr), n, _ptr(y_c), _ptr(y_r_c), _ptr(y_r), ctypes.byref(viol),
                           _threads(nthreads))
    if rc != 0:
        raise OracleError("oracle_glm failed with code %d" % rc)
    out = {"y_c": y_c}
    if want_request_per_cand:
        out["y_r_c"] = y_r_c
    if want_request:
        out["y_r"] = y_r
    if return_violations:
        out["violations"] = viol.value
    return out


def decode(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) or float32 -> exact float64 values."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if a.dtype == np.float32:
        return a.astype(np.float64)
    raise TypeError("oracle inputs are bf16 bit patterns (uint16) or float32, got %s" % a.dtype)


def linear(x: np.ndarray, w: np.ndarray, *, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """y[i, n] = sum_k x[i, k] w[n, k] in fp64 (the projection S W of Sec. 4.1 with W stored as
    [d_out, d_in]); x [rows, d_in], w [d_out, d_in]. Returns the rows `rows` (all when None)."""
    xs = decode(x)
    if rows is not None:
        xs = xs[np.asarray(rows, dtype=np.int64)]
    return xs @ decode(w).T


def request_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, kv_cu=None, L: Optional[int] = None,
                      scale: Optional[float] = None, nthreads: Optional[int] = None) -> np.ndarray:
    """A^R: the queries of request r attend request r's K/V; q [R, Lq, H, d]."""
    R = q.shape[0]
    return dca(q, k, v, R, m=np.arange(R, dtype=np.int32), kv_cu=kv_cu, L=L, scale=scale, nthreads=nthreads)


def fm(x_r: np.ndarray, x_c: np.ndarray, *, m=None, off=None, cands: Optional[Sequence[int]] = None,
       want_request: bool = False):
    """GLM factorization machine, two groups (Eq. 10). x_r [R, n_r, d], x_c [C, n_c, d] (bf16 bits or
    fp32). Returns {"y_c": [n, n_c, n_r + n_c]} for the candidates `cands` (all when None) and, with
    want_request, "y_r": [R, n_r, n_r]. A candidate whose request is out of range (or not covered by
    the offsets) gets zeros."""
    xr, xc = decode(x_r), decode(x_c)
    R, n_r, _ = xr.shape
    C, n_c, _ = xc.shape
    ids = np.arange(C) if cands is None else np.asarray(cands, dtype=np.int64)
    y_c = np.zeros((len(ids), n_c, n_r + n_c), dtype=np.float64)
    mm, oo = _i32(m), _i32(off)
    for o, c in enumerate(ids):
        r = int(_get().oracle_request_of(_ptr(mm), _ptr(oo), R, int(c), None))
        if r < 0:
            continue
        y_c[o, :, :n_r] = xc[c] @ xr[r].T          # request-candidate interactions (the broadcast term)
        y_c[o, :, n_r:] = xc[c] @ xc[c].T          # candidate-candidate interactions
    out = {"y_c": y_c}
    if want_request:
        out["y_r"] = np.stack([xr[r] @ xr[r].T for r in range(R)]) if R else np.zeros((0, n_r, n_r))
    return out


def dca_layer(x_r: np.ndarray, x_c: np.ndarray, glm_layers: Sequence[dict], seq: np.ndarray, w_kc: np.ndarray,
              w_vc: np.ndarray, w_kr: np.ndarray, w_vr: np.ndarray, *, q_len: int, heads: int, m=None, off=None,
              kv_cu=None, scale: Optional[float] = None, cands: Optional[Sequence[int]] = None,
              nthreads: Optional[int] = None):
    """One DCA interaction layer (Eq. 12-13): y = [Q | A] per group, fp64.

    x_r [R, k_r], x_c [C, k_c], seq [rows, seq_dim] (R * L rows, or sum L_r with kv_cu), the
    glm layers' last widths W = q_len * heads * d, K/V weights [heads * d, seq_dim]. Returns
    {"y_c": [n, 2W]} for the candidates `cands` (all when None) and "y_r": [R, 2W]."""
    R = x_r.shape[0]
    g = glm(x_r, x_c, glm_layers, m=m, off=off, cands=cands, want_request=True, nthreads=nthreads)
    W = g["y_c"].shape[1]
    d = W // (q_len * heads)
    rows = seq.shape[0]
    kv_shape = (R, rows // R, heads, d) if kv_cu is None and R > 0 else (rows, heads, d)
    kc, vc = linear(seq, w_kc).reshape(kv_shape), linear(seq, w_vc).reshape(kv_shape)
    kr, vr = linear(seq, w_kr).reshape(kv_shape), linear(seq, w_vr).reshape(kv_shape)
    C = x_c.shape[0]
    ids = np.arange(C) if cands is None else np.asarray(cands, dtype=np.int64)
    # the candidates' requests, then A^C of exactly those query rows
    req = np.array([request_of(m, off, R, int(c)) for c in ids], dtype=np.int32)
    q_c = g["y_c"].reshape(len(ids), q_len, heads, d)
    a_c = dca(q_c, kc, vc, R, m=req, kv_cu=kv_cu, scale=scale, nthreads=nthreads).reshape(len(ids), W)
    q_r = g["y_r"].reshape(R, q_len, heads, d)
    a_r = request_attention(q_r, kr, vr, kv_cu=kv_cu, scale=scale, nthreads=nthreads).reshape(R, W)
    return {"y_c": np.concatenate([g["y_c"], a_c], axis=1), "y_r": np.concatenate([g["y_r"], a_r], axis=1)}


NORM = {"none": 0, "layer": 1, "rms": 2}


def _group_norm(y: np.ndarray, kind: str, gamma, beta, eps: float) -> np.ndarray:
    """Eq. 7 on one group's output: each embedding row (last axis, width d) normalised on its own
    values only. "layer": (y - mean) / sqrt(var + eps) with the biased variance; "rms":
    y / sqrt(mean(y^2) + eps); then * gamma + beta (gamma = 1, beta = 0 when None)."""
    if kind == "none":
        return y
    if kind == "layer":
        mu = y.mean(axis=-1, keepdims=True)
        var = ((y - mu) ** 2).mean(axis=-1, keepdims=True)
        z = (y - mu) / np.sqrt(var + eps)
    elif kind == "rms":
        z = y / np.sqrt((y ** 2).mean(axis=-1, keepdims=True) + eps)
    else:
        raise ValueError("norm must be one of %s" % sorted(NORM))
    if gamma is not None:
        z = z * np.asarray(gamma, dtype=np.float64)
    if beta is not None:
        z = z + np.asarray(beta, dtype=np.float64)
    return z


def lcb_emb(x_r: np.ndarray, x_c: np.ndarray, w_rr: np.ndarray, w_cr: np.ndarray, w_cc: np.ndarray, *,
            m=None, off=None, norm: str = "none", gamma_r=None, beta_r=None, gamma_c=None, beta_c=None,
            eps: float = 1e-5, cands: Optional[Sequence[int]] = None, want_request: bool = False,
            chunk: int = 4096):
    """ROCSified LCB, embedding form (Eq. 5-6, two groups), then the group-local norm (Eq. 7).

    x_r [R, n_r, d], x_c [C, n_c, d]; w_rr [k_r, n_r], w_cr [k_c, n_r], w_cc [k_c, n_c] (bf16 bits
    or fp32, all of one kind); gamma_*/beta_* fp32 [d] or None. Returns {"y_c": [n, k_c, d]} for
    the candidates `cands` (all when None) and, with want_request, "y_r": [R, k_r, d]. A candidate
    whose request is out of range (or not covered by the offsets) gets zeros."""
    xr, xc = decode(x_r), decode(x_c)
    wrr, wcr, wcc = decode(w_rr), decode(w_cr), decode(w_cc)
    R = xr.shape[0]
    ids = np.arange(xc.shape[0]) if cands is None else np.asarray(cands, dtype=np.int64)
    mm, oo = _i32(m), _i32(off)
    req = np.array([_get().oracle_request_of(_ptr(mm), _ptr(oo), R, int(c), None) for c in ids], dtype=np.int64)
    y_c = np.zeros((len(ids), wcc.shape[0], xc.shape[2]), dtype=np.float64)
    for s in range(0, len(ids), chunk):
        sl = slice(s, s + chunk)
        ok = req[sl] >= 0
        if not np.any(ok):
            continue
        rows = np.arange(s, min(s + chunk, len(ids)))[ok]
        x_req = xr[req[rows]]                       # the request embeddings expanded per candidate
        y = wcr @ x_req + wcc @ xc[ids[rows]]       # Eq. 6, candidate rows: W_CR X^R + W_CC X^C
        y_c[rows] = _group_norm(y, norm, gamma_c, beta_c, eps)
    out = {"y_c": y_c}
    if want_request:
        out["y_r"] = _group_norm(wrr @ xr, norm, gamma_r, beta_r, eps)   # Eq. 6, request rows: W_RR X^R
    return out


def index_violations(m, off, C: int, R: int, sorted_flag: bool = False) -> int:
    """Faults of an index, each counted once: with offsets, off[0] != 0 and off[R] != C (one each)
    and every decreasing step; with a map, every entry outside [0, R), with sorted_flag every entry
    below its predecessor, and with both, every valid entry whose candidate lies outside its
    request's offset range."""
    m, off = _i32(m), _i32(off)
    return int(_get().oracle_index_violations(_ptr(m), _ptr(off), C, R, 1 if sorted_flag else 0))
