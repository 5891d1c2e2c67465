"""MI355X-native IKBO hot path: In-Kernel Broadcast Optimization from ROCS (arXiv 2607.27744).

Python binding of ``libikbo.so`` (HIP kernels for gfx950 behind a C ABI, see ``include/ikbo.h``).
This module only marshals arguments: it turns torch tensors into device pointers, the current
HIP stream and workspace buffers, and calls the C entry points of the same names. Every step of
the computation runs in the library's kernels; there is no fallback. If the library is missing
the calls raise.

Entry points (tensor level):

* ``ikbo_dca_forward``      candidate cross attention over shared request K/V (ROCS Eq. 13, A^C)
* ``ikbo_lcb_forward``      GLM-masked linear layer with the request term gather-added (Eq. 6, 14)
* ``ikbo_glm_mlp_forward``  a stack of such layers (Eq. 11-12)
* ``ikbo_check_index``      device-side validation of the candidate -> request index
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libikbo.so")

IKBO_OK, IKBO_INVALID_ARGUMENT, IKBO_UNSUPPORTED, IKBO_MISALIGNED, IKBO_WORKSPACE_TOO_SMALL, IKBO_HIP_ERROR = range(6)
IKBO_F32, IKBO_BF16 = 0, 1
IKBO_ACT_NONE, IKBO_ACT_GELU = 0, 1
IKBO_INDEX_SORTED = 1
IKBO_NORM_NONE, IKBO_NORM_LAYER, IKBO_NORM_RMS = 0, 1, 2
IKBO_DCA_NOALLOC_SCRATCH_BYTES = 32 << 20      # the fixed scratch array of ikbo_dca_forward_noalloc

ACTIVATIONS = {"none": IKBO_ACT_NONE, "gelu": IKBO_ACT_GELU, None: IKBO_ACT_NONE}


class IkboError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (_STATUS_NAMES.get(status, str(status)), message))
        self.status = status


_STATUS_NAMES = {0: "IKBO_OK", 1: "IKBO_INVALID_ARGUMENT", 2: "IKBO_UNSUPPORTED", 3: "IKBO_MISALIGNED",
                 4: "IKBO_WORKSPACE_TOO_SMALL", 5: "IKBO_HIP_ERROR"}


class GlmLayer(ctypes.Structure):
    """Mirror of ``ikbo_glm_layer``."""
    _fields_ = [("w_rr", ctypes.c_void_p), ("w_cr", ctypes.c_void_p), ("w_cc", ctypes.c_void_p),
                ("b_r", ctypes.c_void_p), ("b_c", ctypes.c_void_p),
                ("k_req", ctypes.c_int32), ("k_cand", ctypes.c_int32),
                ("n_req_out", ctypes.c_int32), ("n_cand_out", ctypes.c_int32),
                ("activation", ctypes.c_int32)]


EXPORTS = ["ikbo_version", "ikbo_status_string", "ikbo_last_error_message",
           "ikbo_dca_workspace_size", "ikbo_dca_forward",
           "ikbo_lcb_workspace_size", "ikbo_lcb_forward",
           "ikbo_glm_mlp_workspace_size", "ikbo_glm_mlp_forward", "ikbo_check_index",
           "ikbo_kv_project", "ikbo_request_attention_workspace_size", "ikbo_request_attention",
           "ikbo_fm_forward", "ikbo_lcb_emb_workspace_size", "ikbo_lcb_emb_forward",
           "ikbo_dca_layer_workspace_size", "ikbo_dca_layer_forward", "ikbo_dca_forward_noalloc"]

_lib = None


PROBE_PATH = os.path.join(PKG_DIR, "libikbo_probe.so")
IKBO_PROBE_MFMA_BF16, IKBO_PROBE_EXP2, IKBO_PROBE_COPY, IKBO_PROBE_READ = 0, 1, 2, 3
IKBO_PROBE_LDS_B128, IKBO_PROBE_LDS_TR16 = 4, 5
_probe = None


def load_probe(path: str = PROBE_PATH) -> ctypes.CDLL:
    """The roofline ceiling probes (libikbo_probe.so, include/ikbo_probe.h); not part of the method."""
    global _probe
    if _probe is None:
        if not os.path.exists(path):
            raise RuntimeError("libikbo_probe.so is not built at %s" % path)
        lib = ctypes.CDLL(path)
        lib.ikbo_probe_launch.restype = ctypes.c_int
        lib.ikbo_probe_launch.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_void_p]
        _probe = lib
    return _probe


def ikbo_probe_launch(kind: int, buf: torch.Tensor, iters: int, blocks: int, stream=None) -> None:
    st = load_probe().ikbo_probe_launch(kind, _ptr(buf), buf.numel() * buf.element_size(), iters, blocks,
                                        _stream(stream))
    if st != 0:
        raise IkboError("ikbo_probe_launch(kind %d) failed with status %d" % (kind, st))


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libikbo.so and declare its C signatures. Raises when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libikbo.so is not built at %s; run `python -c 'import __graft_entry__ as g; g.build()'`"
                           % path)
    lib = ctypes.CDLL(path)
    vp, i64, i32, u32, f32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32,
                                  ctypes.c_float, ctypes.c_size_t)
    lib.ikbo_version.restype = ctypes.c_int
    lib.ikbo_version.argtypes = []
    lib.ikbo_status_string.restype = ctypes.c_char_p
    lib.ikbo_status_string.argtypes = [ctypes.c_int]
    lib.ikbo_last_error_message.restype = ctypes.c_char_p
    lib.ikbo_last_error_message.argtypes = []
    lib.ikbo_dca_workspace_size.restype = sz
    lib.ikbo_dca_workspace_size.argtypes = [i64, i64]
    lib.ikbo_dca_forward.restype = ctypes.c_int
    lib.ikbo_dca_forward.argtypes = [vp, i64, i32, vp, vp, i64, vp, i32, vp, vp, u32, i32, i32, f32, i32, i32, vp,
                                     vp, sz, vp]
    lib.ikbo_dca_forward_noalloc.restype = ctypes.c_int
    lib.ikbo_dca_forward_noalloc.argtypes = [vp, i64, i32, vp, vp, i64, vp, i32, vp, vp, u32, i32, i32, f32, i32, i32,
                                             vp, vp]
    lib.ikbo_lcb_workspace_size.restype = sz
    lib.ikbo_lcb_workspace_size.argtypes = [i64, i64, i32, i32, i32, i32, i32]
    lib.ikbo_lcb_forward.restype = ctypes.c_int
    lib.ikbo_lcb_forward.argtypes = [vp, i64, i32, vp, i64, i32, vp, vp, u32, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                     i32, vp, vp, vp, sz, vp]
    lib.ikbo_glm_mlp_workspace_size.restype = sz
    lib.ikbo_glm_mlp_workspace_size.argtypes = [i64, i64, i32, ctypes.POINTER(GlmLayer), i32]
    lib.ikbo_glm_mlp_forward.restype = ctypes.c_int
    lib.ikbo_glm_mlp_forward.argtypes = [vp, i64, vp, i64, vp, vp, u32, i32, ctypes.POINTER(GlmLayer), i32, i32, vp,
                                         vp, vp, sz, vp]
    lib.ikbo_check_index.restype = ctypes.c_int
    lib.ikbo_check_index.argtypes = [vp, vp, i64, i64, u32, vp, vp]
    lib.ikbo_kv_project.restype = ctypes.c_int
    lib.ikbo_kv_project.argtypes = [vp, i64, i32, vp, vp, i32, i32, i32, vp, vp, vp]
    lib.ikbo_request_attention_workspace_size.restype = sz
    lib.ikbo_request_attention_workspace_size.argtypes = [i64]
    lib.ikbo_fm_forward.restype = ctypes.c_int
    lib.ikbo_fm_forward.argtypes = [vp, i64, i32, vp, i64, i32, i32, vp, vp, u32, i32, i32, vp, vp, vp]
    lib.ikbo_lcb_emb_workspace_size.restype = sz
    lib.ikbo_lcb_emb_workspace_size.argtypes = [i64, i32, i32]
    lib.ikbo_lcb_emb_forward.restype = ctypes.c_int
    lib.ikbo_lcb_emb_forward.argtypes = [vp, i64, i32, vp, i64, i32, i32, vp, i32, vp, vp, i32, vp, vp, u32, i32,
                                         vp, vp, vp, vp, f32, i32, i32, vp, vp, vp, sz, vp]
    lib.ikbo_dca_layer_workspace_size.restype = sz
    lib.ikbo_dca_layer_workspace_size.argtypes = [i64, i64, i32, ctypes.POINTER(GlmLayer), i64, i32, i32, i32]
    lib.ikbo_dca_layer_forward.restype = ctypes.c_int
    lib.ikbo_dca_layer_forward.argtypes = [vp, i64, vp, i64, vp, vp, u32, i32, ctypes.POINTER(GlmLayer), vp, i64, i32,
                                           vp, i32, vp, vp, vp, vp, i32, i32, i32, f32, i32, vp, vp, vp, sz, vp]
    lib.ikbo_request_attention.restype = ctypes.c_int
    lib.ikbo_request_attention.argtypes = [vp, i64, i32, vp, vp, vp, i32, i32, i32, f32, i32, i32, vp, vp, sz, vp]
    _lib = lib
    return lib


def _check(status: int):
    if status != IKBO_OK:
        msg = load_library().ikbo_last_error_message().decode(errors="replace")
        raise IkboError(status, msg)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return IKBO_BF16
    if t.dtype == torch.float32:
        return IKBO_F32
    raise TypeError("IKBO kernels take bfloat16 or float32 tensors, got %s" % t.dtype)


def _torch_dtype(code: int):
    return torch.bfloat16 if code == IKBO_BF16 else torch.float32


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need_contig(name: str, t: Optional[torch.Tensor]):
    if t is not None and not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _index(t, name):
    if t is None:
        return None
    if t.dtype != torch.int32:
        raise TypeError("%s must be int32" % name)
    _need_contig(name, t)
    return t


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if workspace is not None:
        return workspace
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def version() -> int:
    return int(load_library().ikbo_version())


# ------------------------------------------------------------------------------------------------
def ikbo_dca_workspace_size(num_cand: int, num_req: int) -> int:
    return int(load_library().ikbo_dca_workspace_size(num_cand, num_req))


def ikbo_dca_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, num_req: Optional[int] = None,
                     cand_to_req: Optional[torch.Tensor] = None, req_cand_offsets: Optional[torch.Tensor] = None,
                     kv_cu_seqlens: Optional[torch.Tensor] = None, kv_len: Optional[int] = None,
                     sorted_index: bool = False, softmax_scale: float = 0.0, out_dtype=None,
                     out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """IKBO-DCA. q [C, Lq, H, d]; k, v [R, L, H, d] or varlen [sum L_r, H, d] with kv_cu_seqlens [R+1].

    Returns out [C, Lq, H, d] in out_dtype (default: q's dtype)."""
    lib = load_library()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _need_contig(n, t)
    C, Lq, H, d = q.shape
    cand_to_req = _index(cand_to_req, "cand_to_req")
    req_cand_offsets = _index(req_cand_offsets, "req_cand_offsets")
    kv_cu_seqlens = _index(kv_cu_seqlens, "kv_cu_seqlens")
    if num_req is None:
        if kv_cu_seqlens is not None:
            num_req = kv_cu_seqlens.numel() - 1
        elif req_cand_offsets is not None:
            num_req = req_cand_offsets.numel() - 1
        elif k.dim() == 4:
            num_req = k.shape[0]
        else:
            raise ValueError("num_req is needed")
    if kv_len is None:
        kv_len = k.shape[1] if (kv_cu_seqlens is None and k.dim() == 4) else 0
    in_code = _dt(q)
    out_code = in_code if out_dtype is None else _dt(torch.empty(0, dtype=out_dtype))
    if out is None:
        out = torch.empty((C, Lq, H, d), dtype=_torch_dtype(out_code), device=q.device)
    else:
        out_code = _dt(out)
    ws = _workspace(ikbo_dca_workspace_size(C, num_req), q.device, workspace)
    st = lib.ikbo_dca_forward(_ptr(q), C, Lq, _ptr(k), _ptr(v), num_req, _ptr(kv_cu_seqlens), kv_len,
                              _ptr(cand_to_req), _ptr(req_cand_offsets), IKBO_INDEX_SORTED if sorted_index else 0,
                              H, d, float(softmax_scale), in_code, out_code, _ptr(out), _ptr(ws),
                              0 if ws is None else ws.numel(), _stream(stream))
    _check(st)
    return out


# ------------------------------------------------------------------------------------------------
def ikbo_fm_forward(x_req: torch.Tensor, x_cand: torch.Tensor, *, cand_to_req: Optional[torch.Tensor] = None,
                    req_cand_offsets: Optional[torch.Tensor] = None, sorted_index: bool = False, out_dtype=None,
                    want_request_output: bool = True, y_req: Optional[torch.Tensor] = None,
                    y_cand: Optional[torch.Tensor] = None, stream=None):
    """GLM factorization machine (two groups). x_req [R, n_r, d], x_cand [C, n_c, d].
    Returns (y_req [R, n_r, n_r] or None, y_cand [C, n_c, n_r + n_c]) in out_dtype (default: input dtype)."""
    lib = load_library()
    _need_contig("x_req", x_req)
    _need_contig("x_cand", x_cand)
    R, n_r, d = x_req.shape
    C, n_c, d2 = x_cand.shape
    if d2 != d:
        raise ValueError("x_req and x_cand must share the embedding width")
    cand_to_req = _index(cand_to_req, "cand_to_req")
    req_cand_offsets = _index(req_cand_offsets, "req_cand_offsets")
    in_code = _dt(x_req)
    out_code = in_code if out_dtype is None else _dt(torch.empty(0, dtype=out_dtype))
    dev = x_cand.device
    if y_cand is None:
        y_cand = torch.empty((C, n_c, n_r + n_c), dtype=_torch_dtype(out_code), device=dev)
    if want_request_output and y_req is None:
        y_req = torch.empty((R, n_r, n_r), dtype=_torch_dtype(out_code), device=dev)
    if not want_request_output:
        y_req = None
    st = lib.ikbo_fm_forward(_ptr(x_req), R, n_r, _ptr(x_cand), C, n_c, d, _ptr(cand_to_req), _ptr(req_cand_offsets),
                             IKBO_INDEX_SORTED if sorted_index else 0, in_code, _dt(y_cand), _ptr(y_req), _ptr(y_cand),
                             _stream(stream))
    _check(st)
    return y_req, y_cand


def ikbo_lcb_emb_workspace_size(num_req: int, n_cand_out: int, dim: int) -> int:
    return int(load_library().ikbo_lcb_emb_workspace_size(num_req, n_cand_out, dim))


_NORMS = {"none": IKBO_NORM_NONE, "layer": IKBO_NORM_LAYER, "rms": IKBO_NORM_RMS}


def ikbo_lcb_emb_forward(x_req: torch.Tensor, x_cand: torch.Tensor, w_rr: torch.Tensor, w_cr: torch.Tensor,
                         w_cc: torch.Tensor, *, cand_to_req: Optional[torch.Tensor] = None,
                         req_cand_offsets: Optional[torch.Tensor] = None, sorted_index: bool = False,
                         norm: str = "none", gamma_req: Optional[torch.Tensor] = None,
                         beta_req: Optional[torch.Tensor] = None, gamma_cand: Optional[torch.Tensor] = None,
                         beta_cand: Optional[torch.Tensor] = None, eps: float = 1e-5, out_dtype=None,
                         want_request_output: bool = True, y_req: Optional[torch.Tensor] = None,
                         y_cand: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                         stream=None):
    """LCB, embedding form, with the group-local norm. x_req [R, n_r, d], x_cand [C, n_c, d];
    w_rr [k_r, n_r], w_cr [k_c, n_r], w_cc [k_c, n_c]; gamma/beta fp32 [d] or None; norm "none" |
    "layer" | "rms". Returns (y_req [R, k_r, d] or None, y_cand [C, k_c, d]) in out_dtype (default:
    input dtype)."""
    lib = load_library()
    for n, t in (("x_req", x_req), ("x_cand", x_cand), ("w_rr", w_rr), ("w_cr", w_cr), ("w_cc", w_cc),
                 ("gamma_req", gamma_req), ("beta_req", beta_req), ("gamma_cand", gamma_cand),
                 ("beta_cand", beta_cand)):
        if t is not None:
            _need_contig(n, t)
    R, n_r, d = x_req.shape
    C, n_c, d2 = x_cand.shape
    k_r, k_c = w_rr.shape[0], w_cc.shape[0]
    if d2 != d:
        raise ValueError("x_req and x_cand must share the embedding width")
    if w_rr.shape[1] != n_r or tuple(w_cr.shape) != (k_c, n_r) or w_cc.shape[1] != n_c:
        raise ValueError("weight shapes do not match the embedding counts")
    cand_to_req = _index(cand_to_req, "cand_to_req")
    req_cand_offsets = _index(req_cand_offsets, "req_cand_offsets")
    in_code = _dt(x_req)
    out_code = in_code if out_dtype is None else _dt(torch.empty(0, dtype=out_dtype))
    dev = x_cand.device
    if y_cand is None:
        y_cand = torch.empty((C, k_c, d), dtype=_torch_dtype(out_code), device=dev)
    if want_request_output and y_req is None:
        y_req = torch.empty((R, k_r, d), dtype=_torch_dtype(out_code), device=dev)
    if not want_request_output:
        y_req = None
    ws = _workspace(ikbo_lcb_emb_workspace_size(R, k_c, d), dev, workspace)
    st = lib.ikbo_lcb_emb_forward(_ptr(x_req), R, n_r, _ptr(x_cand), C, n_c, d, _ptr(w_rr), k_r, _ptr(w_cr),
                                  _ptr(w_cc), k_c, _ptr(cand_to_req), _ptr(req_cand_offsets),
                                  IKBO_INDEX_SORTED if sorted_index else 0, _NORMS[norm], _ptr(gamma_req),
                                  _ptr(beta_req), _ptr(gamma_cand), _ptr(beta_cand), eps, in_code, _dt(y_cand),
                                  _ptr(y_req), _ptr(y_cand), _ptr(ws), 0 if ws is None else ws.numel(),
                                  _stream(stream))
    _check(st)
    return y_req, y_cand


def ikbo_request_attention_workspace_size(num_req: int) -> int:
    return int(load_library().ikbo_request_attention_workspace_size(num_req))


def ikbo_request_attention(q_req: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *,
                           kv_cu_seqlens: Optional[torch.Tensor] = None, kv_len: Optional[int] = None,
                           softmax_scale: float = 0.0, out_dtype=None, out: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Request-side attention A^R. q_req [R, Lq, H, d]; k, v [R, L, H, d] or varlen [sum L_r, H, d] with
    kv_cu_seqlens [R+1]. Returns out [R, Lq, H, d] in out_dtype (default: q_req's dtype)."""
    lib = load_library()
    for n, t in (("q_req", q_req), ("k", k), ("v", v)):
        _need_contig(n, t)
    R, Lq, H, d = q_req.shape
    kv_cu_seqlens = _index(kv_cu_seqlens, "kv_cu_seqlens")
    if kv_len is None:
        kv_len = k.shape[1] if (kv_cu_seqlens is None and k.dim() == 4) else 0
    in_code = _dt(q_req)
    out_code = in_code if out_dtype is None else _dt(torch.empty(0, dtype=out_dtype))
    if out is None:
        out = torch.empty((R, Lq, H, d), dtype=_torch_dtype(out_code), device=q_req.device)
    else:
        out_code = _dt(out)
    ws = _workspace(ikbo_request_attention_workspace_size(R), q_req.device, workspace)
    st = lib.ikbo_request_attention(_ptr(q_req), R, Lq, _ptr(k), _ptr(v), _ptr(kv_cu_seqlens), kv_len, H, d,
                                    float(softmax_scale), in_code, out_code, _ptr(out), _ptr(ws),
                                    0 if ws is None else ws.numel(), _stream(stream))
    _check(st)
    return out


def ikbo_kv_project(s: torch.Tensor, w_k: torch.Tensor, w_v: torch.Tensor, *, out_dtype=None,
                    k_out: Optional[torch.Tensor] = None, v_out: Optional[torch.Tensor] = None, stream=None):
    """K/V projection at the request batch. s [rows, d_in]; w_k, w_v [d_out, d_in].
    Returns (k_out, v_out), each [rows, d_out] in out_dtype (default: s's dtype)."""
    lib = load_library()
    for n, t in (("s", s), ("w_k", w_k), ("w_v", w_v)):
        _need_contig(n, t)
    rows, d_in = s.shape
    d_out = w_k.shape[0]
    if tuple(w_k.shape) != (d_out, d_in) or tuple(w_v.shape) != (d_out, d_in):
        raise ValueError("w_k and w_v must be [d_out, d_in]")
    in_code = _dt(s)
    out_code = in_code if out_dtype is None else _dt(torch.empty(0, dtype=out_dtype))
    if k_out is None:
        k_out = torch.empty((rows, d_out), dtype=_torch_dtype(out_code), device=s.device)
    if v_out is None:
        v_out = torch.empty((rows, d_out), dtype=_torch_dtype(out_code), device=s.device)
    if k_out.dtype != v_out.dtype:
        raise TypeError("k_out and v_out must share a dtype")
    out_code = _dt(k_out)
    st = lib.ikbo_kv_project(_ptr(s), rows, d_in, _ptr(w_k), _ptr(w_v), d_out, in_code, out_code, _ptr(k_out),
                             _ptr(v_out), _stream(stream))
    _check(st)
    return k_out, v_out


# ------------------------------------------------------------------------------------------------
def ikbo_lcb_workspace_size(num_cand: int, num_req: int, k_req: int, k_cand: int, n_req_out: int, n_cand_out: int,
                            dtype=torch.bfloat16) -> int:
    code = _dt(torch.empty(0, dtype=dtype))
    return int(load_library().ikbo_lcb_workspace_size(num_cand, num_req, k_req, k_cand, n_req_out, n_cand_out, code))


def ikbo_lcb_forward(x_req: torch.Tensor, x_cand: torch.Tensor, w_rr: torch.Tensor, w_cr: torch.Tensor,
                     w_cc: torch.Tensor, *, b_r: Optional[torch.Tensor] = None, b_c: Optional[torch.Tensor] = None,
                     cand_to_req: Optional[torch.Tensor] = None, req_cand_offsets: Optional[torch.Tensor] = None,
                     sorted_index: bool = False, activation: str = "none", out_dtype=None,
                     want_request_output: bool = True, y_req: Optional[torch.Tensor] = None,
                     y_cand: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None):
    """IKBO-LCB. x_req [R, K_r], x_cand [C, K_c], w_rr [N_r, K_r], w_cr [N_c, K_r], w_cc [N_c, K_c].

    Returns (y_req [R, N_r] or None, y_cand [C, N_c])."""
    lib = load_library()
    for n, t in (("x_req", x_req), ("x_cand", x_cand), ("w_rr", w_rr), ("w_cr", w_cr), ("w_cc", w_cc),
                 ("b_r", b_r), ("b_c", b_c)):
        _need_contig(n, t)
    for n, t in (("b_r", b_r), ("b_c", b_c)):
        if t is not None and t.dtype != torch.float32:
            raise TypeError("%s must be float32" % n)
    R, K_r = x_req.shape
    C, K_c = x_cand.shape
    N_r, N_c = w_rr.shape[0], w_cc.shape[0]
    cand_to_req = _index(cand_to_req, "cand_to_req")
    req_cand_offsets = _index(req_cand_offsets, "req_cand_offsets")
    in_code = _dt(x_req)
    out_code = in_code if out_dtype is None else _dt(torch.empty(0, dtype=out_dtype))
    dev = x_cand.device
    if y_cand is None:
        y_cand = torch.empty((C, N_c), dtype=_torch_dtype(out_code), device=dev)
    if want_request_output and y_req is None:
        y_req = torch.empty((R, N_r), dtype=_torch_dtype(out_code), device=dev)
    ws = _workspace(ikbo_lcb_workspace_size(C, R, K_r, K_c, N_r, N_c, x_req.dtype), dev, workspace)
    st = lib.ikbo_lcb_forward(_ptr(x_req), R, K_r, _ptr(x_cand), C, K_c, _ptr(cand_to_req), _ptr(req_cand_offsets),
                              IKBO_INDEX_SORTED if sorted_index else 0, _ptr(w_rr), _ptr(w_cr), _ptr(w_cc),
                              _ptr(b_r), _ptr(b_c), N_r, N_c, ACTIVATIONS[activation], in_code, out_code,
                              _ptr(y_req), _ptr(y_cand), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
    _check(st)
    return y_req, y_cand


# ------------------------------------------------------------------------------------------------
def _layer_structs(layers: Sequence[dict]):
    arr = (GlmLayer * len(layers))()
    for i, ly in enumerate(layers):
        for n in ("w_rr", "w_cr", "w_cc", "b_r", "b_c"):
            _need_contig(n, ly.get(n))
        arr[i] = GlmLayer(_ptr(ly["w_rr"]), _ptr(ly["w_cr"]), _ptr(ly["w_cc"]), _ptr(ly.get("b_r")),
                          _ptr(ly.get("b_c")), ly["w_rr"].shape[1], ly["w_cc"].shape[1], ly["w_rr"].shape[0],
                          ly["w_cc"].shape[0], ACTIVATIONS[ly.get("act", "none")])
    return arr


def ikbo_glm_mlp_workspace_size(num_cand: int, num_req: int, layers: Sequence[dict], in_dtype) -> int:
    arr = _layer_structs(layers)
    return int(load_library().ikbo_glm_mlp_workspace_size(num_cand, num_req, len(layers), arr,
                                                          _dt(torch.empty(0, dtype=in_dtype))))


def ikbo_glm_mlp_forward(x_req: torch.Tensor, x_cand: torch.Tensor, layers: Sequence[dict], *,
                         cand_to_req: Optional[torch.Tensor] = None, req_cand_offsets: Optional[torch.Tensor] = None,
                         sorted_index: bool = False, out_dtype=None, want_request_output: bool = True,
                         y_req: Optional[torch.Tensor] = None, y_cand: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None):
    """GLM-MLP. layers: dicts with w_rr, w_cr, w_cc (input dtype), b_r, b_c (fp32 or None), act.

    Returns (y_req [R, N_r(last)] or None, y_cand [C, N_c(last)])."""
    lib = load_library()
    _need_contig("x_req", x_req)
    _need_contig("x_cand", x_cand)
    R, C = x_req.shape[0], x_cand.shape[0]
    cand_to_req = _index(cand_to_req, "cand_to_req")
    req_cand_offsets = _index(req_cand_offsets, "req_cand_offsets")
    in_code = _dt(x_req)
    out_code = in_code if out_dtype is None else _dt(torch.empty(0, dtype=out_dtype))
    arr = _layer_structs(layers)
    last = layers[-1]
    dev = x_cand.device
    if y_cand is None:
        y_cand = torch.empty((C, last["w_cc"].shape[0]), dtype=_torch_dtype(out_code), device=dev)
    if want_request_output and y_req is None:
        y_req = torch.empty((R, last["w_rr"].shape[0]), dtype=_torch_dtype(out_code), device=dev)
    nbytes = int(lib.ikbo_glm_mlp_workspace_size(C, R, len(layers), arr, in_code))
    ws = _workspace(nbytes, dev, workspace)
    st = lib.ikbo_glm_mlp_forward(_ptr(x_req), R, _ptr(x_cand), C, _ptr(cand_to_req), _ptr(req_cand_offsets),
                                  IKBO_INDEX_SORTED if sorted_index else 0, len(layers), arr, in_code, out_code,
                                  _ptr(y_req), _ptr(y_cand), _ptr(ws), 0 if ws is None else ws.numel(),
                                  _stream(stream))
    _check(st)
    return y_req, y_cand


def ikbo_dca_layer_forward(x_req: torch.Tensor, x_cand: torch.Tensor, glm_layers: Sequence[dict], seq: torch.Tensor,
                           w_k_cand: torch.Tensor, w_v_cand: torch.Tensor, w_k_req: torch.Tensor,
                           w_v_req: torch.Tensor, *, q_len: int, num_heads: int, head_dim: int,
                           cand_to_req: Optional[torch.Tensor] = None, req_cand_offsets: Optional[torch.Tensor] = None,
                           sorted_index: bool = False, kv_cu_seqlens: Optional[torch.Tensor] = None,
                           kv_len: Optional[int] = None, softmax_scale: float = 0.0,
                           y_req: Optional[torch.Tensor] = None, y_cand: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, stream=None):
    """One DCA interaction layer: y = [Q | A] per group (W = q_len * num_heads * head_dim columns each).
    x_req [R, k_req], x_cand [C, k_cand]; seq [rows, seq_dim] (R * kv_len rows, or sum L_r with
    kv_cu_seqlens); K/V weights [num_heads * head_dim, seq_dim]. Returns (y_req [R, 2W], y_cand [C, 2W])."""
    lib = load_library()
    for n, t in (("x_req", x_req), ("x_cand", x_cand), ("seq", seq), ("w_k_cand", w_k_cand), ("w_v_cand", w_v_cand),
                 ("w_k_req", w_k_req), ("w_v_req", w_v_req)):
        _need_contig(n, t)
    R, C = x_req.shape[0], x_cand.shape[0]
    rows, seq_dim = seq.shape
    cand_to_req = _index(cand_to_req, "cand_to_req")
    req_cand_offsets = _index(req_cand_offsets, "req_cand_offsets")
    kv_cu_seqlens = _index(kv_cu_seqlens, "kv_cu_seqlens")
    if kv_cu_seqlens is None and kv_len is None:
        kv_len = rows // max(R, 1)
    code = _dt(x_req)
    arr = _layer_structs(glm_layers)
    W = q_len * num_heads * head_dim
    dev = x_cand.device
    if y_cand is None:
        y_cand = torch.empty((C, 2 * W), dtype=_torch_dtype(code), device=dev)
    if y_req is None:
        y_req = torch.empty((R, 2 * W), dtype=_torch_dtype(code), device=dev)
    nbytes = int(lib.ikbo_dca_layer_workspace_size(C, R, len(glm_layers), arr, rows, num_heads, head_dim, code))
    ws = _workspace(nbytes, dev, workspace)
    st = lib.ikbo_dca_layer_forward(_ptr(x_req), R, _ptr(x_cand), C, _ptr(cand_to_req), _ptr(req_cand_offsets),
                                    IKBO_INDEX_SORTED if sorted_index else 0, len(glm_layers), arr, _ptr(seq), rows,
                                    seq_dim, _ptr(kv_cu_seqlens), 0 if kv_len is None else kv_len, _ptr(w_k_cand),
                                    _ptr(w_v_cand), _ptr(w_k_req), _ptr(w_v_req), q_len, num_heads, head_dim,
                                    softmax_scale, code, _ptr(y_req), _ptr(y_cand), _ptr(ws),
                                    0 if ws is None else ws.numel(), _stream(stream))
    _check(st)
    return y_req, y_cand


# ------------------------------------------------------------------------------------------------
def ikbo_check_index(num_cand: int, num_req: int, *, cand_to_req: Optional[torch.Tensor] = None,
                     req_cand_offsets: Optional[torch.Tensor] = None, sorted_index: bool = False,
                     stream=None) -> int:
    """Number of index violations (0 = valid). Synchronises the stream to read the count."""
    lib = load_library()
    cand_to_req = _index(cand_to_req, "cand_to_req")
    req_cand_offsets = _index(req_cand_offsets, "req_cand_offsets")
    dev = (cand_to_req if cand_to_req is not None else req_cand_offsets).device
    cnt = torch.empty(1, dtype=torch.int64, device=dev)
    st = lib.ikbo_check_index(_ptr(cand_to_req), _ptr(req_cand_offsets), num_cand, num_req,
                              IKBO_INDEX_SORTED if sorted_index else 0, _ptr(cnt), _stream(stream))
    _check(st)
    return int(cnt.item())
