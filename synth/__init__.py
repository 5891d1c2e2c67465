"""Seeded synthetic workloads for the IKBO hot path (inputs only, no method arithmetic).

Every tensor is drawn from its own counter-based SplitMix64 stream (``synth.c``), keyed by
(seed, tag). Any slice of any tensor can therefore be regenerated on its own, which lets the
oracle side rebuild just the rows it needs at full sizes.

Workloads (the five problem shapes of the IKBO kernels, by name):

* ``tiny``          R=4, candidates per request U{8..32}, L=64, H=2, d=64, Lq=1, fp32,
                    Q/K/V ~ N(0,1)/sqrt(d); GLM linear x_r [R,256], x_c [C,256], out 128,
                    W ~ N(0, 1/256), no activation.
* ``dca_fixed``     R=64 x 512 candidates, L=1024, H=4, d=128, Lq=4, bf16, N(0,1).
* ``dca_ragged``    R=256, candidates log-normal (median 256, sigma 1, clip [16, 2048]),
                    L_r ~ U{256..4096} varlen, H=8, d=64, Lq=1, bf16, N(0,1).
* ``lcb``           R=512 x 1024 candidates, x_r [R,8192], x_c [C,4096], out 1024, GELU, bf16.
* ``block``         R=128 x 2048 candidates; GLM-MLP [4096 | 2048] -> 2048 (GELU) -> 4096;
                    DCA L=8192, H=8, d=128, Lq=4; bf16, N(0,1).

Weights of a GLM block are N(0, 1/K) with K that block's reduction width; biases are drawn the
same way and kept in fp32.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")

_KIND = {"f64": 0, "f32": 1, "bf16": 2, "unif": 3}
_NP = {"f64": np.float64, "f32": np.float32, "bf16": np.uint16, "unif": np.float64}

# One stream tag per tensor role.
TAGS = {
    "counts": 1, "kv_len": 2, "q": 3, "k": 4, "v": 5,
    "x_r": 6, "x_c": 7, "w_rr": 8, "w_cr": 9, "w_cc": 10, "b_r": 11, "b_c": 12,
    "s": 13, "w_kc": 14, "w_vc": 15, "w_kr": 16, "w_vr": 17,
}


def layer_tag(layer: int, name: str) -> int:
    return 100 + 16 * layer + ("w_rr", "w_cr", "w_cc", "b_r", "b_c").index(name)


def build_lib(force: bool = False) -> str:
    src = os.path.join(_HERE, "synth.c")
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(src):
        import subprocess
        tmp = LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-pthread", src, "-o", tmp, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def _get():
    global _lib
    if _lib is None:
        build_lib()
        lib = ctypes.CDLL(LIB_PATH)
        lib.synth_stream_key.restype = ctypes.c_uint64
        lib.synth_stream_key.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_raw.restype = ctypes.c_uint64
        lib.synth_raw.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_fill.restype = None
        lib.synth_fill.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                                   ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
        _lib = lib
    return _lib


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def stream_key(seed: int, tag: int) -> int:
    return int(_get().synth_stream_key(seed, tag))


def raw(seed: int, tag: int, i: int) -> int:
    return int(_get().synth_raw(stream_key(seed, tag), i))


def draw(seed: int, tag: int, n: int, kind: str = "f64", scale: float = 1.0, start: int = 0,
         out: Optional[np.ndarray] = None) -> np.ndarray:
    """Draws start..start+n of stream (seed, tag): normals*scale as f64/f32/bf16 bits, or uniforms."""
    if out is None:
        out = np.empty(n, dtype=_NP[kind])
    assert out.dtype == _NP[kind] and out.flags.c_contiguous and out.size == n
    _get().synth_fill(stream_key(seed, tag), start, n, float(scale), _KIND[kind],
                      out.ctypes.data_as(ctypes.c_void_p), _threads())
    return out


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 round-to-nearest-even, as bit patterns (NaN kept quiet)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_to_f64(arr) if dtype == "bf16" else np.asarray(arr, dtype=np.float64)


# ----------------------------------------------------------------------------------------------
# Index layout helpers (grouping of candidates by request; no arithmetic of the method).

def offsets_from_counts(counts: np.ndarray) -> np.ndarray:
    off = np.zeros(len(counts) + 1, dtype=np.int64)
    np.cumsum(counts, out=off[1:])
    return off.astype(np.int32)


def cand_to_req_from_counts(counts: np.ndarray) -> np.ndarray:
    return np.repeat(np.arange(len(counts), dtype=np.int32), counts)


def uniform_ints(seed: int, tag: int, n: int, lo: int, hi: int) -> np.ndarray:
    """n integers uniform on {lo..hi} (inclusive), from floor(u * (hi - lo + 1))."""
    u = draw(seed, tag, n, "unif")
    return (lo + np.floor(u * (hi - lo + 1))).astype(np.int64)


def lognormal_ints(seed: int, tag: int, n: int, median: float, sigma: float, lo: int, hi: int):
    z = draw(seed, tag, n, "f64")
    return np.clip(np.rint(median * np.exp(sigma * z)), lo, hi).astype(np.int64)


# ----------------------------------------------------------------------------------------------
# Problem descriptions.

@dataclass
class DcaSpec:
    name: str
    seed: int
    R: int
    H: int
    d: int
    Lq: int
    dtype: str
    counts: np.ndarray                 # candidates per request [R]
    kv_lens: np.ndarray                # K/V length per request [R]
    varlen: bool
    value_scale: float = 1.0           # Q/K/V ~ N(0, value_scale^2)
    softmax_scale: float = 0.0         # 0 -> 1/sqrt(d)

    @property
    def C(self) -> int:
        return int(self.counts.sum())

    @property
    def L(self) -> int:
        return int(self.kv_lens.max()) if len(self.kv_lens) else 0

    @property
    def offsets(self) -> np.ndarray:
        return offsets_from_counts(self.counts)

    @property
    def cand_to_req(self) -> np.ndarray:
        return cand_to_req_from_counts(self.counts)

    @property
    def kv_cu(self) -> Optional[np.ndarray]:
        return offsets_from_counts(self.kv_lens) if self.varlen else None

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale > 0 else 1.0 / np.sqrt(self.d)

    @property
    def kv_rows(self) -> int:
        return int(self.kv_lens.sum()) if self.varlen else self.R * self.L

    def flops(self) -> float:
        """Effective FLOPs (no broadcast): 4 * Lq * H * d * sum_c L_{m(c)}."""
        return 4.0 * self.Lq * self.H * self.d * float(np.dot(self.counts, self.kv_lens))

    def q_shape(self):
        return (self.C, self.Lq, self.H, self.d)

    def kv_shape(self):
        return (self.kv_rows, self.H, self.d)


def dca_spec(name: str) -> DcaSpec:
    if name == "tiny":
        seed, R = 0, 4
        counts = uniform_ints(seed, TAGS["counts"], R, 8, 32)
        return DcaSpec(name, seed, R, 2, 64, 1, "f32", counts, np.full(R, 64, np.int64), False,
                       value_scale=1.0 / 8.0)
    if name == "dca_fixed":
        R = 64
        return DcaSpec(name, 1, R, 4, 128, 4, "bf16", np.full(R, 512, np.int64),
                       np.full(R, 1024, np.int64), False)
    if name == "dca_ragged":
        seed, R = 2, 256
        counts = lognormal_ints(seed, TAGS["counts"], R, 256.0, 1.0, 16, 2048)
        lens = uniform_ints(seed, TAGS["kv_len"], R, 256, 4096)
        return DcaSpec(name, seed, R, 8, 64, 1, "bf16", counts, lens, True)
    if name == "block":
        R = 128
        return DcaSpec(name, 4, R, 8, 128, 4, "bf16", np.full(R, 2048, np.int64),
                       np.full(R, 8192, np.int64), False)
    raise KeyError(name)


def custom_dca_spec(seed, counts, kv_lens, H, d, Lq, dtype="bf16", varlen=None, value_scale=1.0,
                    softmax_scale=0.0, name="custom") -> DcaSpec:
    counts = np.asarray(counts, dtype=np.int64)
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    if varlen is None:
        varlen = len(set(kv_lens.tolist())) > 1
    return DcaSpec(name, seed, len(counts), H, d, Lq, dtype, counts, kv_lens, varlen, value_scale,
                   softmax_scale)


def dca_q(spec: DcaSpec, cand_start: int = 0, cand_count: Optional[int] = None) -> np.ndarray:
    """Q rows of candidates [cand_start, cand_start + cand_count), shape [n, Lq, H, d]."""
    n = spec.C - cand_start if cand_count is None else cand_count
    row = spec.Lq * spec.H * spec.d
    a = draw(spec.seed, TAGS["q"], n * row, spec.dtype, spec.value_scale, start=cand_start * row)
    return a.reshape(n, spec.Lq, spec.H, spec.d)


def dca_kv(spec: DcaSpec, which: str, row_start: int = 0, row_count: Optional[int] = None):
    """K or V rows [row_start, row_start + row_count) of the flat [rows, H, d] store."""
    n = spec.kv_rows - row_start if row_count is None else row_count
    row = spec.H * spec.d
    a = draw(spec.seed, TAGS[which], n * row, spec.dtype, spec.value_scale, start=row_start * row)
    return a.reshape(n, spec.H, spec.d)


def dca_kv_request(spec: DcaSpec, which: str, r: int) -> np.ndarray:
    """The K or V block of request r, shape [L_r, H, d]."""
    if spec.varlen:
        cu = spec.kv_cu
        return dca_kv(spec, which, int(cu[r]), int(cu[r + 1] - cu[r]))
    return dca_kv(spec, which, r * spec.L, spec.L)


@dataclass
class GlmLayerSpec:
    k_req: int
    k_cand: int
    n_req: int
    n_cand: int
    act: str          # "none" | "gelu"


@dataclass
class GlmSpec:
    name: str
    seed: int
    counts: np.ndarray
    layers: list
    dtype: str

    @property
    def R(self) -> int:
        return len(self.counts)

    @property
    def C(self) -> int:
        return int(self.counts.sum())

    @property
    def offsets(self):
        return offsets_from_counts(self.counts)

    @property
    def cand_to_req(self):
        return cand_to_req_from_counts(self.counts)

    def flops(self) -> float:
        """Effective FLOPs: per layer 2*C*N_c*K_c + 2*R*(N_r + N_c)*K_r."""
        f = 0.0
        for ly in self.layers:
            f += 2.0 * self.C * ly.n_cand * ly.k_cand + 2.0 * self.R * (ly.n_req + ly.n_cand) * ly.k_req
        return f


def glm_spec(name: str) -> GlmSpec:
    if name == "tiny":
        seed, R = 0, 4
        counts = uniform_ints(seed, TAGS["counts"], R, 8, 32)
        return GlmSpec(name, seed, counts, [GlmLayerSpec(256, 256, 128, 128, "none")], "f32")
    if name == "lcb":
        return GlmSpec(name, 3, np.full(512, 1024, np.int64),
                       [GlmLayerSpec(8192, 4096, 1024, 1024, "gelu")], "bf16")
    if name == "block":
        return GlmSpec(name, 4, np.full(128, 2048, np.int64),
                       [GlmLayerSpec(4096, 2048, 2048, 2048, "gelu"),
                        GlmLayerSpec(2048, 2048, 4096, 4096, "none")], "bf16")
    raise KeyError(name)


def glm_x(spec: GlmSpec, which: str, row_start: int = 0, row_count: Optional[int] = None):
    ly = spec.layers[0]
    width = ly.k_req if which == "x_r" else ly.k_cand
    total = spec.R if which == "x_r" else spec.C
    n = total - row_start if row_count is None else row_count
    a = draw(spec.seed, TAGS[which], n * width, spec.dtype, 1.0, start=row_start * width)
    return a.reshape(n, width)


def glm_weights(spec: GlmSpec, layer: int) -> dict:
    """w_rr [N_r,K_r], w_cr [N_c,K_r], w_cc [N_c,K_c] in the run dtype; b_r, b_c fp32."""
    ly = spec.layers[layer]
    s, dt = spec.seed, spec.dtype
    sr, sc = 1.0 / np.sqrt(ly.k_req), 1.0 / np.sqrt(ly.k_cand)
    tag = (lambda nm: layer_tag(layer, nm)) if layer > 0 else (lambda nm: TAGS[nm])
    return {
        "w_rr": draw(s, tag("w_rr"), ly.n_req * ly.k_req, dt, sr).reshape(ly.n_req, ly.k_req),
        "w_cr": draw(s, tag("w_cr"), ly.n_cand * ly.k_req, dt, sr).reshape(ly.n_cand, ly.k_req),
        "w_cc": draw(s, tag("w_cc"), ly.n_cand * ly.k_cand, dt, sc).reshape(ly.n_cand, ly.k_cand),
        "b_r": draw(s, tag("b_r"), ly.n_req, "f32", sr),
        "b_c": draw(s, tag("b_c"), ly.n_cand, "f32", sc),
    }


# Width of the request-side sequence rows S that the K/V projections read. The pages give none;
# taken as num_heads * head_dim (a square projection).
def seq_width(spec: "DcaSpec") -> int:
    return spec.H * spec.d


def seq_rows(spec: "DcaSpec", row_start: int = 0, row_count: Optional[int] = None) -> np.ndarray:
    """Rows [row_start, row_start + row_count) of the stacked sequence rows S [kv_rows, seq_width],
    N(0, 1) in the spec's dtype."""
    n = spec.kv_rows - row_start if row_count is None else row_count
    w = seq_width(spec)
    return draw(spec.seed, TAGS["s"], n * w, spec.dtype, 1.0, start=row_start * w).reshape(n, w)


def kv_weight(spec: "DcaSpec", name: str) -> np.ndarray:
    """A K/V projection weight [H*d, seq_width] ("w_kc", "w_vc": the candidate half's W^C_K, W^C_V;
    "w_kr", "w_vr": the request half's), N(0, 1/seq_width)."""
    w = seq_width(spec)
    n = spec.H * spec.d
    return draw(spec.seed, TAGS[name], n * w, spec.dtype, 1.0 / np.sqrt(w)).reshape(n, w)


def block_specs():
    """The full ROCS block: the GLM-MLP that makes DCA queries, and the DCA it feeds."""
    return glm_spec("block"), dca_spec("block")
