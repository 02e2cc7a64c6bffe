"""Python binding of ``libtvp.so``, the tree-verification pass with W12 weights on MI355X.

Argument marshalling only: every step of the pass runs in the library's HIP
kernels.  PyTorch provides device memory and the current HIP stream.  The
functions carry the names of the C entry points declared in ``include/tvp.h``.

Importing this package loads the library and fails loudly when it has not
been built (``python -m tree_verification_pass_amd.build``); there is no
fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtvp.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python tree_verification_pass_amd/build.py`")
_lib = ctypes.CDLL(LIB_PATH)

# ----------------------------------------------------------------- constants
TVP_OK, TVP_ERR_ARG, TVP_ERR_SHAPE, TVP_ERR_TREE = 0, 1, 2, 3
TVP_ERR_CAPACITY, TVP_ERR_FORMAT, TVP_ERR_WORKSPACE, TVP_ERR_HIP = 4, 5, 6, 7
TVP_CHAN_PLAIN, TVP_CHAN_GATEUP, TVP_CHAN_QKV = 0, 1, 2
TVP_FMT_W12, TVP_FMT_HI8 = 0, 1
TVP_EPI_F32, TVP_EPI_BF16, TVP_EPI_RESID, TVP_EPI_SWIGLU, TVP_EPI_QKV, TVP_EPI_ARGMAX = range(6)
TVP_GEMM_COUNTERS = 256  # arrival counters of one GEMM call (tvp_gemm_epilogue.counters)

c_i32, c_i64, c_sz, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p


class TvpError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {tvp_status_string(status)} ({status})")


# ------------------------------------------------------------------ structs
class TvpW12(ctypes.Structure):
    _fields_ = [("n_out", c_i64), ("k_in", c_i64), ("n_esc", c_i64), ("hi", c_vp), ("lo", c_vp),
                ("base", c_vp), ("esc_ptr", c_vp), ("esc_idx", c_vp), ("esc_val", c_vp)]


class TvpW12Packed(ctypes.Structure):
    _fields_ = [("n_out", c_i64), ("k_in", c_i64), ("n_esc", c_i64), ("n_tiles", c_i32), ("n_kb", c_i32),
                ("chan_map", c_i32), ("map_a", c_i32), ("map_b", c_i32), ("map_c", c_i32), ("format", c_i32),
                ("blob", c_vp), ("bytes", c_sz), ("off_rec", c_sz), ("off_escoff", c_sz),
                ("off_esc", c_sz), ("off_b2", c_sz), ("off_rowmap", c_sz)]


class TvpLmheadI8(ctypes.Structure):
    _fields_ = [("vocab", c_i64), ("k_in", c_i64), ("q", c_vp), ("scale", c_vp), ("esc_col", c_vp),
                ("esc_val", c_vp), ("r", c_vp), ("r_eff", c_vp), ("tiles", TvpW12Packed)]


class TvpGemmEpilogue(ctypes.Structure):
    _fields_ = [("mode", c_i32), ("y", c_vp), ("ldy", c_i64), ("resid", c_vp), ("ldr", c_i64),
                ("pos", c_vp), ("slot", c_vp), ("k_cache", c_vp), ("v_cache", c_vp), ("s_stride", c_i64),
                ("rope_theta", ctypes.c_double), ("argmax", c_vp), ("logits", c_vp), ("ldl", c_i64),
                ("x_packed", c_i32), ("y_packed", c_i32), ("counters", c_vp)]


class TvpLayer(ctypes.Structure):
    _fields_ = [("wqkv", TvpW12Packed), ("wo", TvpW12Packed), ("wgu", TvpW12Packed),
                ("wdown", TvpW12Packed), ("attn_norm", c_vp), ("ffn_norm", c_vp), ("k_cache", c_vp),
                ("v_cache", c_vp)]


class TvpModelDesc(ctypes.Structure):
    _fields_ = [("n_layers", c_i32), ("hidden", c_i32), ("n_heads", c_i32), ("n_kv_heads", c_i32),
                ("head_dim", c_i32), ("ffn", c_i32), ("vocab", c_i32), ("rope_theta", ctypes.c_float),
                ("norm_eps", ctypes.c_float), ("s_max", c_i32), ("embed", c_vp), ("final_norm", c_vp),
                ("lm_head", TvpW12Packed), ("layers", ctypes.POINTER(TvpLayer))]


class TvpVerifyOut(ctypes.Structure):
    _fields_ = [("argmax", c_vp), ("path", c_vp), ("n_accepted", c_vp), ("bonus", c_vp),
                ("status", c_vp), ("logits", c_vp)]


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_lib_tvp_status_string = _sig("tvp_status_string", ctypes.c_char_p, [ctypes.c_int])
_lib_w12_encode_count = _sig("w12_encode_count", ctypes.c_int,
                             [c_vp, c_i64, c_i64, c_vp, c_vp, ctypes.POINTER(c_i64), c_vp])
_lib_w12_encode = _sig("w12_encode", ctypes.c_int, [c_vp, ctypes.POINTER(TvpW12), c_vp])
_lib_w12_decode = _sig("w12_decode", ctypes.c_int, [ctypes.POINTER(TvpW12), c_vp, c_vp])
_lib_w12_validate = _sig("w12_validate", ctypes.c_int, [c_vp, c_vp, c_vp, c_i64, c_i64, c_i64])
_lib_w12_pack_size = _sig("w12_pack_size", ctypes.c_int,
                          [c_i64, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32, ctypes.POINTER(TvpW12Packed)])
_lib_w12_pack_hi8_size = _sig("w12_pack_hi8_size", ctypes.c_int,
                              [c_i64, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32, ctypes.POINTER(TvpW12Packed)])
_lib_w12_pack_hi8 = _sig("w12_pack_hi8", ctypes.c_int,
                         [ctypes.POINTER(TvpW12), ctypes.POINTER(TvpW12Packed), c_vp, c_sz, c_vp])
_lib_w12_pack_workspace = _sig("w12_pack_workspace", c_sz, [c_i64, c_i64])
_lib_w12_pack = _sig("w12_pack", ctypes.c_int,
                     [ctypes.POINTER(TvpW12), ctypes.POINTER(TvpW12Packed), c_vp, c_sz, c_vp])
_lib_w12_gemm_workspace = _sig("w12_gemm_workspace", c_sz, [c_i64, ctypes.POINTER(TvpW12Packed)])
_lib_w12_gemm = _sig("w12_gemm", ctypes.c_int,
                     [c_vp, c_i64, c_i64, ctypes.POINTER(TvpW12Packed), c_vp, c_i64, ctypes.c_int, c_vp, c_sz,
                      c_vp])
_lib_w12_gemm_ex = _sig("w12_gemm_ex", ctypes.c_int,
                        [c_vp, c_i64, c_i64, ctypes.POINTER(TvpW12Packed), ctypes.POINTER(TvpGemmEpilogue),
                         c_vp, c_sz, c_vp])
_lib_w12_gemm_ex_noalloc = _sig("w12_gemm_ex_noalloc", ctypes.c_int,
                                [c_vp, c_i64, c_i64, ctypes.POINTER(TvpW12Packed), ctypes.POINTER(TvpGemmEpilogue),
                                 c_vp])
_lib_w12_packed_x_elems = _sig("w12_packed_x_elems", c_i64, [c_i64])
_lib_w12_pack_x = _sig("w12_pack_x", ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_vp])
_lib_w12_gemm_resid_norm_workspace = _sig("w12_gemm_resid_norm_workspace", c_sz,
                                          [c_i64, ctypes.POINTER(TvpW12Packed)])
_lib_w12_gemm_resid_norm = _sig("w12_gemm_resid_norm", ctypes.c_int,
                                [c_vp, c_i64, ctypes.POINTER(TvpW12Packed), c_vp, c_i64, c_vp, ctypes.c_float, c_vp,
                                 c_vp, c_sz, c_vp])
_lib_lmhead_i8_tiles_size = _sig("lmhead_i8_tiles_size", ctypes.c_int, [c_i64, c_i64, ctypes.POINTER(TvpW12Packed)])
_lib_lmhead_i8_encode_workspace = _sig("lmhead_i8_encode_workspace", c_sz, [c_i64, c_i64])
_lib_lmhead_i8_encode = _sig("lmhead_i8_encode", ctypes.c_int, [c_vp, ctypes.POINTER(TvpLmheadI8), c_vp, c_sz, c_vp])
_lib_lmhead_i8_argmax_workspace = _sig("lmhead_i8_argmax_workspace", c_sz, [c_i64, ctypes.POINTER(TvpLmheadI8)])
_lib_lmhead_i8_argmax = _sig("lmhead_i8_argmax", ctypes.c_int,
                             [c_vp, c_i64, ctypes.POINTER(TvpLmheadI8), ctypes.POINTER(TvpW12), c_vp, c_vp, c_vp,
                              c_vp, c_sz, c_vp])
_lib_tree_attention_workspace = _sig("tree_attention_workspace", c_sz, [c_i32, c_i32, c_i32, c_i32])
_lib_tree_attention = _sig("tree_attention", ctypes.c_int,
                           [c_vp, c_vp, c_vp, c_i64, c_i32, c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp,
                            c_sz, c_vp])
_lib_accept_path = _sig("accept_path", ctypes.c_int, [c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp])
_lib_tvp_plan_create = _sig("tvp_plan_create", ctypes.c_int,
                            [ctypes.POINTER(TvpModelDesc), c_i32, ctypes.POINTER(c_vp)])
_lib_tvp_plan_destroy = _sig("tvp_plan_destroy", None, [c_vp])
_lib_verify_step_workspace = _sig("verify_step_workspace", c_sz, [c_vp])
_lib_verify_step = _sig("verify_step", ctypes.c_int,
                        [c_vp, c_i32, c_vp, c_vp, c_i32, c_i32, ctypes.POINTER(TvpVerifyOut), c_vp, c_sz, c_vp])
_lib_verify_step_batched = _sig("verify_step_batched", ctypes.c_int,
                                [c_vp, c_i32, ctypes.POINTER(c_i32), ctypes.POINTER(c_i32), c_i32, c_vp, c_vp,
                                 c_i32, ctypes.POINTER(TvpVerifyOut), c_vp, c_sz, c_vp])
_lib_tvp_read_probe = _sig("tvp_read_probe", ctypes.c_int, [c_vp, c_sz, c_vp, c_vp])
_GDN_VERIFY_ARGS = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp]
_lib_gdn_tree_verify = _sig("gdn_tree_verify", ctypes.c_int, _GDN_VERIFY_ARGS)
_lib_gdn_path_verify = _sig("gdn_path_verify", ctypes.c_int, _GDN_VERIFY_ARGS)
_lib_gdn_commit = _sig("gdn_commit", ctypes.c_int,
                       [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp,
                        c_vp])

EXPORTED = ("tvp_status_string", "w12_encode_count", "w12_encode", "w12_decode", "w12_validate", "w12_pack_size",
            "w12_pack_workspace", "w12_pack", "w12_pack_hi8_size", "w12_pack_hi8", "w12_gemm_workspace", "w12_gemm", "w12_gemm_ex", "w12_gemm_ex_noalloc",
            "w12_packed_x_elems", "w12_pack_x", "w12_gemm_resid_norm_workspace", "w12_gemm_resid_norm",
            "lmhead_i8_tiles_size", "lmhead_i8_encode_workspace", "lmhead_i8_encode",
            "lmhead_i8_argmax_workspace", "lmhead_i8_argmax",
            "tree_attention_workspace", "tree_attention", "accept_path", "tvp_plan_create",
            "tvp_plan_destroy", "verify_step_workspace", "verify_step", "verify_step_batched",
            "tvp_read_probe", "gdn_tree_verify", "gdn_path_verify", "gdn_commit")


# ------------------------------------------------------------------ helpers
def tvp_status_string(status: int) -> str:
    return _lib_tvp_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != TVP_OK:
        raise TvpError(status, what)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device=None) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev_check(*ts: torch.Tensor) -> None:
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors passed to the library must be contiguous CUDA tensors")


class _Workspace:
    """Device scratch reused across calls (no initial contents are needed)."""

    def __init__(self):
        self._bufs: Dict[int, torch.Tensor] = {}

    def get(self, nbytes: int, device) -> torch.Tensor:
        dev = torch.device(device)
        key = dev.index if dev.index is not None else torch.cuda.current_device()
        buf = self._bufs.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=dev)
            self._bufs[key] = buf
        return buf


# one pool per entry point
_ws_gemm = _Workspace()
_ws_attn = _Workspace()


# ------------------------------------------------------------------ W12
@dataclass
class W12Tensor:
    """Canonical W12 tensor on the device (see ``tvp_w12`` in include/tvp.h)."""

    n_out: int
    k_in: int
    n_esc: int
    hi: torch.Tensor
    lo: torch.Tensor
    base: torch.Tensor
    esc_ptr: torch.Tensor
    esc_idx: torch.Tensor
    esc_val: torch.Tensor

    def struct(self) -> TvpW12:
        return TvpW12(self.n_out, self.k_in, self.n_esc, self.hi.data_ptr(), self.lo.data_ptr(),
                      self.base.data_ptr(), self.esc_ptr.data_ptr(), self.esc_idx.data_ptr(),
                      self.esc_val.data_ptr())

    def nbytes(self) -> int:
        return (self.hi.numel() + self.lo.numel() + self.base.numel() + 4 * self.esc_ptr.numel()
                + 4 * self.n_esc)


def w12_encode_count(w: torch.Tensor):
    """Phase 1 on device bf16 ``w [n_out, k_in]``: returns ``(base, esc_ptr, n_esc)``."""
    _dev_check(w)
    n, k = w.shape
    base = torch.empty(n, dtype=torch.uint8, device=w.device)
    esc_ptr = torch.empty(n + 1, dtype=torch.int32, device=w.device)
    cnt = c_i64(0)
    _check(_lib_w12_encode_count(_ptr(w), n, k, _ptr(base), _ptr(esc_ptr), ctypes.byref(cnt), _stream(w.device)),
           "w12_encode_count")
    return base, esc_ptr, int(cnt.value)


def w12_encode(w: torch.Tensor) -> W12Tensor:
    """Both encoder phases on device bf16 ``w [n_out, k_in]``."""
    base, esc_ptr, n_esc = w12_encode_count(w)
    n, k = w.shape
    dev = w.device
    t = W12Tensor(n, k, n_esc, torch.empty((n, k), dtype=torch.uint8, device=dev),
                  torch.empty((n, (k + 1) // 2), dtype=torch.uint8, device=dev), base, esc_ptr,
                  torch.empty(max(n_esc, 1), dtype=torch.int16, device=dev),
                  torch.empty(max(n_esc, 1), dtype=torch.int16, device=dev))
    s = t.struct()
    _check(_lib_w12_encode(_ptr(w), ctypes.byref(s), _stream(dev)), "w12_encode")
    return t


def w12_decode(t: W12Tensor) -> torch.Tensor:
    out = torch.empty((t.n_out, t.k_in), dtype=torch.bfloat16, device=t.hi.device)
    s = t.struct()
    _check(_lib_w12_decode(ctypes.byref(s), _ptr(out), _stream(t.hi.device)), "w12_decode")
    return out


def w12_validate(base, esc_ptr, esc_idx, k_in: int) -> int:
    """Host-side format check of a canonical tensor's side data (numpy arrays
    or CPU tensors: base uint8 [n], esc_ptr uint32/int32 [n+1], esc_idx
    uint16/int16 [n_esc]).  Returns the status code (TVP_OK or TVP_ERR_FORMAT)."""
    import numpy as np

    b = np.ascontiguousarray(np.asarray(base).astype(np.uint8, copy=False))
    p = np.ascontiguousarray(np.asarray(esc_ptr).view(np.uint32) if np.asarray(esc_ptr).dtype.itemsize == 4
                             else np.asarray(esc_ptr).astype(np.uint32))
    i = np.ascontiguousarray(np.asarray(esc_idx).view(np.uint16) if np.asarray(esc_idx).dtype.itemsize == 2
                             else np.asarray(esc_idx).astype(np.uint16))
    n = int(b.size)
    if p.size != n + 1:
        raise ValueError("esc_ptr needs n_out + 1 entries")
    n_esc = int(i.size)
    return int(_lib_w12_validate(b.ctypes.data_as(c_vp), p.ctypes.data_as(c_vp),
                                 i.ctypes.data_as(c_vp) if n_esc else None, n, int(k_in), n_esc))


@dataclass
class PackedW12:
    """Tiled GPU copy of a W12 tensor; ``blob`` owns the device memory."""

    desc: TvpW12Packed
    blob: torch.Tensor

    @property
    def n_out(self) -> int:
        return int(self.desc.n_out)

    @property
    def k_in(self) -> int:
        return int(self.desc.k_in)

    def stream_bytes(self) -> int:
        """Bytes one GEMM pass reads from the packed copy."""
        return int(self.desc.bytes)


def w12_pack_size(n_out: int, k_in: int, n_esc: int, chan_map: int = TVP_CHAN_PLAIN, map_a: int = 0,
                  map_b: int = 0, map_c: int = 0) -> TvpW12Packed:
    p = TvpW12Packed()
    _check(_lib_w12_pack_size(n_out, k_in, n_esc, chan_map, map_a, map_b, map_c, ctypes.byref(p)),
           "w12_pack_size")
    return p


def w12_pack(t: W12Tensor, chan_map: int = TVP_CHAN_PLAIN, map_a: int = 0, map_b: int = 0,
             map_c: int = 0, fmt: int = TVP_FMT_W12) -> PackedW12:
    """Tiled GPU copy of ``t``: the full records (TVP_FMT_W12) or only their
    8-bit leading view (TVP_FMT_HI8, the Q pass of two-level verification)."""
    dev = t.hi.device
    p = TvpW12Packed()
    size_fn, pack_fn = ((_lib_w12_pack_size, _lib_w12_pack) if fmt == TVP_FMT_W12
                        else (_lib_w12_pack_hi8_size, _lib_w12_pack_hi8))
    _check(size_fn(t.n_out, t.k_in, t.n_esc, chan_map, map_a, map_b, map_c, ctypes.byref(p)), "w12_pack_size")
    blob = torch.empty(int(p.bytes), dtype=torch.uint8, device=dev)
    p.blob = blob.data_ptr()
    need = _lib_w12_pack_workspace(t.n_out, t.k_in)
    ws = torch.empty(int(need), dtype=torch.uint8, device=dev)
    s = t.struct()
    _check(pack_fn(ctypes.byref(s), ctypes.byref(p), _ptr(ws), need, _stream(dev)), "w12_pack")
    torch.cuda.current_stream(dev).synchronize()
    return PackedW12(p, blob)


def w12_gemm_workspace(m: int, w: PackedW12) -> int:
    return int(_lib_w12_gemm_workspace(m, ctypes.byref(w.desc)))


def w12_gemm(x: torch.Tensor, w: PackedW12, out_fp32: bool = False, out: Optional[torch.Tensor] = None
             ) -> torch.Tensor:
    """``x [m, k_in]`` bf16 -> ``x @ W^T`` as ``[m, n_out]`` (bf16, or fp32)."""
    _dev_check(x)
    m, k = x.shape
    if k != w.k_in:
        raise ValueError("x has the wrong number of columns")
    if out is None:
        out = torch.empty((m, w.n_out), dtype=torch.float32 if out_fp32 else torch.bfloat16, device=x.device)
    need = w12_gemm_workspace(m, w)
    ws = _ws_gemm.get(need, x.device)
    _check(_lib_w12_gemm(_ptr(x), m, x.stride(0), ctypes.byref(w.desc), _ptr(out), out.stride(0),
                         1 if out_fp32 else 0, _ptr(ws), ws.numel(), _stream(x.device)), "w12_gemm")
    return out


def w12_gemm_ex(x: torch.Tensor, w: PackedW12, epi: TvpGemmEpilogue) -> None:
    _dev_check(x)
    m = x.shape[0]
    need = w12_gemm_workspace(m, w)
    ws = _ws_gemm.get(need, x.device)
    _check(_lib_w12_gemm_ex(_ptr(x), m, x.stride(0), ctypes.byref(w.desc), ctypes.byref(epi), _ptr(ws),
                            ws.numel(), _stream(x.device)), "w12_gemm_ex")


def w12_gemm_ex_noalloc(x: torch.Tensor, m: int, w: PackedW12, epi: TvpGemmEpilogue) -> None:
    """``w12_gemm_ex`` without a workspace: the library's own per-GPU scratch
    array (``x`` row-major, or packed when ``epi.x_packed`` is set)."""
    _dev_check(x)
    ldx = 0 if epi.x_packed else x.stride(0)
    _check(_lib_w12_gemm_ex_noalloc(_ptr(x), m, ldx, ctypes.byref(w.desc), ctypes.byref(epi), _stream(x.device)),
           "w12_gemm_ex_noalloc")


def w12_packed_x_elems(k_in: int) -> int:
    return int(_lib_w12_packed_x_elems(int(k_in)))


def w12_pack_x(x: torch.Tensor, k_in: int | None = None) -> torch.Tensor:
    """Row-major bf16 ``x [m, >= k_in]`` (m <= 32) -> the GEMM's packed
    activation layout, a flat bf16 tensor of ``w12_packed_x_elems(k_in)``."""
    _dev_check(x)
    m = x.shape[0]
    k_in = x.shape[1] if k_in is None else int(k_in)
    xp = torch.empty(max(w12_packed_x_elems(k_in), 8), dtype=torch.bfloat16, device=x.device)
    _check(_lib_w12_pack_x(_ptr(x), m, x.stride(0), k_in, _ptr(xp), _stream(x.device)), "w12_pack_x")
    return xp


def w12_gemm_px(xp: torch.Tensor, m: int, w: PackedW12, epi: TvpGemmEpilogue) -> None:
    """The GEMM on packed activations (``epi.x_packed`` is set here)."""
    _dev_check(xp)
    epi.x_packed = 1
    need = w12_gemm_workspace(m, w)
    ws = _ws_gemm.get(need, xp.device)
    _check(_lib_w12_gemm_ex(_ptr(xp), m, 0, ctypes.byref(w.desc), ctypes.byref(epi), _ptr(ws), ws.numel(),
                            _stream(xp.device)), "w12_gemm_ex")


def w12_gemm_resid_norm(xp: torch.Tensor, m: int, w: PackedW12, h: torch.Tensor, gain: torch.Tensor,
                        eps: float = 1e-6) -> torch.Tensor:
    """The verify pass's projection + residual + RMSNorm stage: ``h`` (bf16
    ``[m, n_out]``) is updated in place to ``bf16(h + x W^T)``; returns the
    normed rows in the packed activation layout."""
    _dev_check(xp, h, gain)
    yp = torch.empty(max(w12_packed_x_elems(w.n_out), 8), dtype=torch.bfloat16, device=xp.device)
    need = int(_lib_w12_gemm_resid_norm_workspace(m, ctypes.byref(w.desc)))
    ws = _ws_gemm.get(need, xp.device)
    _check(_lib_w12_gemm_resid_norm(_ptr(xp), m, ctypes.byref(w.desc), _ptr(h), h.stride(0), _ptr(gain), float(eps),
                                    _ptr(yp), _ptr(ws), ws.numel(), _stream(xp.device)), "w12_gemm_resid_norm")
    return yp


# ------------------------------------------------------- INT8 certified head
@dataclass
class LmheadI8:
    """Device INT8 LM head (see ``tvp_lmhead_i8``); the tensors own the memory."""

    desc: TvpLmheadI8
    q: torch.Tensor
    scale: torch.Tensor
    esc_col: torch.Tensor
    esc_val: torch.Tensor
    r: torch.Tensor
    r_eff: torch.Tensor
    tiles: torch.Tensor

    def stream_bytes(self) -> int:
        """Bytes the approximate pass streams: tiles, escapes, scales and radii."""
        return int(self.desc.tiles.bytes) + 8 * int(self.desc.vocab)


def lmhead_i8_encode(w: torch.Tensor) -> LmheadI8:
    """INT8 head of device bf16 ``w [vocab, k_in]``."""
    _dev_check(w)
    V, k = w.shape
    dev = w.device
    tp = TvpW12Packed()
    _check(_lib_lmhead_i8_tiles_size(V, k, ctypes.byref(tp)), "lmhead_i8_tiles_size")
    t = dict(q=torch.empty((V, k), dtype=torch.int8, device=dev), scale=torch.empty(V, dtype=torch.float32, device=dev),
             esc_col=torch.empty((V, 8), dtype=torch.int16, device=dev),
             esc_val=torch.empty((V, 8), dtype=torch.int16, device=dev),
             r=torch.empty(V, dtype=torch.float32, device=dev), r_eff=torch.empty(V, dtype=torch.float32, device=dev),
             tiles=torch.empty(int(tp.bytes), dtype=torch.uint8, device=dev))
    tp.blob = t["tiles"].data_ptr()
    d = TvpLmheadI8(V, k, t["q"].data_ptr(), t["scale"].data_ptr(), t["esc_col"].data_ptr(), t["esc_val"].data_ptr(),
                    t["r"].data_ptr(), t["r_eff"].data_ptr(), tp)
    need = int(_lib_lmhead_i8_encode_workspace(V, k))
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(_lib_lmhead_i8_encode(_ptr(w), ctypes.byref(d), _ptr(ws), need, _stream(dev)), "lmhead_i8_encode")
    torch.cuda.current_stream(dev).synchronize()
    return LmheadI8(d, **t)


def lmhead_i8_argmax(xp: torch.Tensor, m: int, head: LmheadI8, exact: W12Tensor, want_approx: bool = False):
    """Greedy tokens of the ``m`` rows of packed activations ``xp``: returns
    ``(argmax [m], candidates per row [m], approximate logits [m, vocab] or None)``."""
    _dev_check(xp)
    dev = xp.device
    V = int(head.desc.vocab)
    am = torch.empty(m, dtype=torch.int32, device=dev)
    nc = torch.empty(m, dtype=torch.int32, device=dev)
    apx = torch.empty((m, V), dtype=torch.float32, device=dev) if want_approx else None
    need = int(_lib_lmhead_i8_argmax_workspace(m, ctypes.byref(head.desc)))
    ws = _ws_gemm.get(need, dev)
    s = exact.struct()
    _check(_lib_lmhead_i8_argmax(_ptr(xp), m, ctypes.byref(head.desc), ctypes.byref(s), _ptr(am), _ptr(nc), _ptr(apx),
                                 _ptr(ws), ws.numel(), _stream(dev)), "lmhead_i8_argmax")
    return am, nc, apx


# --------------------------------------------------------------- attention
def tree_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, ctx_len: int,
                   parents: torch.Tensor):
    """``q [n, hq, d]``, caches ``[hkv, s, d]`` holding the context in slots
    ``[0, ctx_len)`` and the tree's keys/values in slots ``ctx_len + i``.
    Returns ``(out [n, hq, d], status)``."""
    _dev_check(q, k_cache, v_cache, parents)
    n, hq, d = q.shape
    hkv, s, _ = k_cache.shape
    out = torch.empty_like(q)
    status = torch.zeros(1, dtype=torch.int32, device=q.device)
    need = _lib_tree_attention_workspace(n, hq, d, ctx_len + n)
    ws = _ws_attn.get(need, q.device)
    _check(_lib_tree_attention(_ptr(q), _ptr(k_cache), _ptr(v_cache), s, ctx_len, _ptr(parents), n, hq, hkv, d,
                               _ptr(out), _ptr(status), _ptr(ws), ws.numel(), _stream(q.device)),
           "tree_attention")
    return out, status


def _gdn_verify(fn, name, q, k, v, g, beta, state, parents, out=None, status=None):
    _dev_check(q, k, v, g, beta, state, parents)
    n, hk, dk = q.shape
    hv, dv, _ = state.shape
    if out is None:
        out = torch.empty(n, hv, dv, dtype=torch.bfloat16, device=q.device)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=q.device)
    _dev_check(out, status)
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(parents), n, hk, hv, dk, dv,
              _ptr(out), _ptr(status), _stream(q.device)), name)
    return out, status


def gdn_tree_verify(q, k, v, g, beta, state, parents, out=None, status=None):
    """Gated DeltaNet layer over a draft tree, WY form (one solve for all
    paths).  ``q, k [n, hk, dk]`` and ``v [n, hv, dv]`` bf16, ``g, beta
    [n, hv]`` fp32, ``state [hv, dv, dk]`` fp32 (not modified), ``parents
    [n]`` int32.  Returns ``(out [n, hv, dv] bf16, status [1])`` (both may be
    passed in)."""
    return _gdn_verify(_lib_gdn_tree_verify, "gdn_tree_verify", q, k, v, g, beta, state, parents, out, status)


def gdn_path_verify(q, k, v, g, beta, state, parents, out=None, status=None):
    """The same outputs as ``gdn_tree_verify``, each leaf's root path replayed
    from the committed state."""
    return _gdn_verify(_lib_gdn_path_verify, "gdn_path_verify", q, k, v, g, beta, state, parents, out, status)


def gdn_commit(state, k, v, g, beta, path, n_accepted, status) -> None:
    """Replays ``path[0 .. n_accepted]`` into ``state [L, hv, dv, dk]`` (in
    place) for every layer; ``k [L, n, hk, dk]``, ``v [L, n, hv, dv]``,
    ``g, beta [L, n, hv]``.  Nothing changes unless ``status`` is TVP_OK."""
    _dev_check(state, k, v, g, beta, path, n_accepted, status)
    L, hv, dv, dk = state.shape
    _, n, hk, _ = k.shape
    _check(_lib_gdn_commit(_ptr(state), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), L, n, hk, hv, dk, dv, _ptr(path),
                           _ptr(n_accepted), _ptr(status), _stream(state.device)), "gdn_commit")


def accept_path(argmax: torch.Tensor, tokens: torch.Tensor, parents: torch.Tensor):
    """Returns device tensors ``(path [n], n_accepted [1], bonus [1], status [1])``."""
    _dev_check(argmax, tokens, parents)
    n = argmax.numel()
    dev = argmax.device
    path = torch.full((n,), -1, dtype=torch.int32, device=dev)
    n_acc = torch.zeros(1, dtype=torch.int32, device=dev)
    bonus = torch.zeros(1, dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    _check(_lib_accept_path(_ptr(argmax), _ptr(tokens), _ptr(parents), n, _ptr(path), _ptr(n_acc), _ptr(bonus),
                            _ptr(status), _stream(dev)), "accept_path")
    return path, n_acc, bonus, status


# ------------------------------------------------------------ verify pass
class Plan:
    """Owns a ``tvp_plan`` and references to every device buffer it points at."""

    def __init__(self, desc: TvpModelDesc, layers_arr, max_nodes: int, keepalive: list):
        self._keep = keepalive
        self._layers_arr = layers_arr
        self.desc = desc
        h = c_vp()
        _check(_lib_tvp_plan_create(ctypes.byref(desc), max_nodes, ctypes.byref(h)), "tvp_plan_create")
        self.handle = h
        self.max_nodes = max_nodes
        self.ws_bytes = int(_lib_verify_step_workspace(h))
        self.device = keepalive[0].device if keepalive else torch.device("cuda")
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=self.device)

    def __del__(self):
        h = getattr(self, "handle", None)
        try:
            if h is not None and h.value and _lib_tvp_plan_destroy is not None:
                _lib_tvp_plan_destroy(h)
                self.handle = c_vp()
        except Exception:  # interpreter shutdown
            pass


def tvp_plan_create(desc: TvpModelDesc, layers_arr, max_nodes: int, keepalive: list) -> Plan:
    return Plan(desc, layers_arr, max_nodes, keepalive)


@dataclass
class VerifyResult:
    argmax: torch.Tensor
    path: torch.Tensor
    n_accepted: torch.Tensor
    bonus: torch.Tensor
    status: torch.Tensor
    logits: Optional[torch.Tensor]


def _alloc_out(plan: Plan, n_nodes: int, n_req: int, want_logits: bool) -> VerifyResult:
    dev = plan.device
    vocab = int(plan.desc.vocab)
    return VerifyResult(torch.zeros(n_nodes, dtype=torch.int32, device=dev),
                        torch.full((n_nodes,), -1, dtype=torch.int32, device=dev),
                        torch.zeros(n_req, dtype=torch.int32, device=dev),
                        torch.zeros(n_req, dtype=torch.int32, device=dev),
                        torch.zeros(n_req, dtype=torch.int32, device=dev),
                        torch.zeros((n_nodes, vocab), dtype=torch.float32, device=dev) if want_logits else None)


def _out_struct(r: VerifyResult) -> TvpVerifyOut:
    return TvpVerifyOut(r.argmax.data_ptr(), r.path.data_ptr(), r.n_accepted.data_ptr(), r.bonus.data_ptr(),
                        r.status.data_ptr(), r.logits.data_ptr() if r.logits is not None else None)


def verify_step(plan: Plan, ctx_len: int, tokens: torch.Tensor, parents: torch.Tensor, commit: bool = True,
                want_logits: bool = False, out: Optional[VerifyResult] = None) -> VerifyResult:
    _dev_check(tokens, parents)
    n = tokens.numel()
    if out is None:
        out = _alloc_out(plan, n, 1, want_logits)
    o = _out_struct(out)
    _check(_lib_verify_step(plan.handle, ctx_len, _ptr(tokens), _ptr(parents), n, 1 if commit else 0,
                            ctypes.byref(o), _ptr(plan.ws), plan.ws_bytes, _stream(tokens.device)), "verify_step")
    return out


def verify_step_batched(plan: Plan, ctx_lens: Sequence[int], node_ptr: Sequence[int], s_req: int,
                        tokens: torch.Tensor, parents: torch.Tensor, commit: bool = True,
                        want_logits: bool = False, out: Optional[VerifyResult] = None) -> VerifyResult:
    _dev_check(tokens, parents)
    n_req = len(ctx_lens)
    n = tokens.numel()
    if out is None:
        out = _alloc_out(plan, n, n_req, want_logits)
    o = _out_struct(out)
    cl = (c_i32 * n_req)(*[int(x) for x in ctx_lens])
    npr = (c_i32 * (n_req + 1))(*[int(x) for x in node_ptr])
    _check(_lib_verify_step_batched(plan.handle, n_req, cl, npr, s_req, _ptr(tokens), _ptr(parents),
                                    1 if commit else 0, ctypes.byref(o), _ptr(plan.ws), plan.ws_bytes,
                                    _stream(tokens.device)), "verify_step_batched")
    return out


def tvp_read_probe(src: torch.Tensor, sink: torch.Tensor) -> None:
    """One streaming read of ``src`` (device, 16-byte aligned) on the current
    stream; ``sink`` is a device int32/uint32 tensor of >= 4096 words."""
    _dev_check(src, sink)
    if sink.numel() * sink.element_size() < 4096 * 4:
        raise ValueError("sink needs 4096 words")
    _check(_lib_tvp_read_probe(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(src.device)),
           "tvp_read_probe")


__all__ = [n for n in dir() if not n.startswith("_lib")]
