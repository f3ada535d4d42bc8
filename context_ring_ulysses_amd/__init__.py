"""Context-parallel attention hot path for AMD Instinct MI355X (gfx950).

A thin Python binding of the C ABI in include/cru.h (libcru.so, built from
the HIP sources in csrc/).  It only marshals arguments: torch tensors become
(pointer, shape, strides) descriptors, outputs are allocated with torch when
the caller passes none, and the current torch stream is handed over.  Every
step of the computation runs in the library's HIP kernels; there is no CPU
or PyTorch fallback, and importing the library fails loudly when it is not
built.

Entry points (same names as the C ABI without the ``cru_`` prefix):
    attn_fwd_lse, attn_merge_lse, ring_chunk_bounds, ring_workspace_bytes,
    ring_emulate, ring_emulate_noalloc, ulysses_head_bounds, ulysses_seq2head, ulysses_head2seq,
    usp_workspace_bytes, usp_emulate
plus ulysses_groups (views of the head groups of a packed buffer).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple, Union

import torch

__all__ = [
    "attn_fwd_lse", "attn_merge_lse", "ring_chunk_bounds", "ring_workspace_bytes",
    "ring_emulate", "ring_emulate_noalloc", "ulysses_head_bounds", "ulysses_seq2head", "ulysses_head2seq",
    "ulysses_groups", "usp_workspace_bytes", "usp_emulate", "ContextParallelConfig",
    "lib", "LIB_PATH", "CruError", "CruInvalid", "CruNotDivisible", "CruUnsupported",
    "CruDeviceError", "CruWorkspaceError", "CruHipError", "MAX_PARTS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcru.so")
MAX_PARTS = 64

F32, BF16 = 0, 1
_DTYPE_CODE = {torch.float32: F32, torch.bfloat16: BF16}


class CruTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("B", ctypes.c_int64), ("S", ctypes.c_int64),
                ("H", ctypes.c_int64), ("D", ctypes.c_int64), ("sb", ctypes.c_int64),
                ("ss", ctypes.c_int64), ("sh", ctypes.c_int64)]


class CruLse(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("B", ctypes.c_int64), ("H", ctypes.c_int64),
                ("S", ctypes.c_int64), ("sb", ctypes.c_int64), ("sh", ctypes.c_int64)]


class CruError(Exception):
    """A non-zero cru_status; ``status`` holds the code."""

    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class CruInvalid(CruError, ValueError):
    pass


class CruNotDivisible(CruError, ValueError):
    pass


class CruUnsupported(CruError, NotImplementedError):
    pass


class CruDeviceError(CruError, RuntimeError):
    pass


class CruWorkspaceError(CruError, ValueError):
    pass


class CruHipError(CruError, RuntimeError):
    pass


_ERRORS = {1: CruInvalid, 2: CruNotDivisible, 3: CruUnsupported, 4: CruDeviceError,
           5: CruWorkspaceError, 6: CruHipError}

_lib = None

_P = ctypes.POINTER


def lib() -> ctypes.CDLL:
    """The loaded libcru.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python context_ring_ulysses_amd/build.py` first")
    L = ctypes.CDLL(LIB_PATH)
    T, Lse = _P(CruTensor), _P(CruLse)
    st = ctypes.c_int
    vp = ctypes.c_void_p
    L.cru_attn_fwd_lse.argtypes = [T, T, T, T, Lse, ctypes.c_float, vp]
    L.cru_attn_fwd_lse.restype = st
    L.cru_attn_merge_lse.argtypes = [ctypes.c_int, T, Lse, T, Lse, vp]
    L.cru_attn_merge_lse.restype = st
    L.cru_ring_chunk_bounds.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                        _P(ctypes.c_int64)]
    L.cru_ring_chunk_bounds.restype = st
    L.cru_ring_workspace_bytes.argtypes = [T, ctypes.c_int, _P(ctypes.c_size_t)]
    L.cru_ring_workspace_bytes.restype = st
    L.cru_ring_emulate.argtypes = [T, T, T, ctypes.c_int, ctypes.c_int, _P(ctypes.c_int64),
                                   ctypes.c_int, ctypes.c_int, T, Lse, ctypes.c_float, vp,
                                   ctypes.c_size_t, vp]
    L.cru_ring_emulate.restype = st
    L.cru_ring_emulate_noalloc.argtypes = [T, T, T, ctypes.c_int, ctypes.c_int,
                                           _P(ctypes.c_int64), ctypes.c_int, ctypes.c_int, T, Lse,
                                           ctypes.c_float, vp]
    L.cru_ring_emulate_noalloc.restype = st
    L.cru_ulysses_head_bounds.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                          _P(ctypes.c_int64)]
    L.cru_ulysses_head_bounds.restype = st
    L.cru_ulysses_seq2head.argtypes = [ctypes.c_int, T, _P(vp), ctypes.c_int, ctypes.c_int, vp]
    L.cru_ulysses_seq2head.restype = st
    L.cru_ulysses_head2seq.argtypes = [ctypes.c_int, _P(vp), T, ctypes.c_int, ctypes.c_int, vp]
    L.cru_ulysses_head2seq.restype = st
    L.cru_usp_workspace_bytes.argtypes = [T, ctypes.c_int, ctypes.c_int, _P(ctypes.c_size_t)]
    L.cru_usp_workspace_bytes.restype = st
    L.cru_usp_emulate.argtypes = [T, T, T, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, T, Lse, ctypes.c_float, vp, ctypes.c_size_t, vp]
    L.cru_usp_emulate.restype = st
    L.cru_status_str.argtypes = [ctypes.c_int]
    L.cru_status_str.restype = ctypes.c_char_p
    L.cru_last_error.argtypes = []
    L.cru_last_error.restype = ctypes.c_char_p
    L.cru_abi_version.argtypes = []
    L.cru_abi_version.restype = ctypes.c_int
    _lib = L
    return L


def _check(status: int) -> None:
    if status != 0:
        L = lib()
        name = L.cru_status_str(status).decode()
        msg = L.cru_last_error().decode()
        raise _ERRORS.get(status, CruError)(status, f"{name}: {msg}")


# ------------------------------------------------------------ marshalling

def _desc(t: torch.Tensor, name: str) -> CruTensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() != 4:
        raise CruInvalid(1, f"{name} must be 4-d [B, S, H, D], got shape {tuple(t.shape)}")
    code = _DTYPE_CODE.get(t.dtype)
    if code is None:
        raise CruUnsupported(3, f"{name}: dtype {t.dtype} (supported: float32, bfloat16)")
    if t.numel() > 0 and t.stride(3) != 1:
        raise CruInvalid(1, f"{name}: the head dim must be contiguous (stride 1)")
    B, S, H, D = t.shape
    return CruTensor(t.data_ptr(), code, 0, B, S, H, D, t.stride(0), t.stride(1), t.stride(2))


def _lse_desc(t: Optional[torch.Tensor], name: str):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.dim() != 3 or t.dtype != torch.float32:
        raise CruInvalid(1, f"{name} must be a float32 [B, H, S] tensor")
    if t.numel() > 0 and t.stride(2) != 1:
        raise CruInvalid(1, f"{name}: the sequence dim must be contiguous (stride 1)")
    B, H, S = t.shape
    return CruLse(t.data_ptr(), B, H, S, t.stride(0), t.stride(1))


def _ref(x):
    return None if x is None else ctypes.byref(x)


def _stream(t: torch.Tensor) -> int:
    if t.is_cuda:
        return torch.cuda.current_stream(t.device).cuda_stream
    return 0


def _empty_lse(B, H, S, device):
    return torch.empty((B, H, S), dtype=torch.float32, device=device)


# -------------------------------------------------------------- entry points

def attn_fwd_lse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *,
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                 scale: Optional[float] = None, out_dtype: Optional[torch.dtype] = None,
                 return_lse: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """O = softmax(Q K^T * scale) V and its per-row LSE (natural log).

    q [B, Sq, H, D], k/v [B, Skv, H, D]; returns (o [B, Sq, H, D], lse [B, H, Sq]).
    """
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = _empty_lse(q.shape[0], q.shape[2], q.shape[1], q.device)
    qd, kd, vd, od = _desc(q, "q"), _desc(k, "k"), _desc(v, "v"), _desc(out, "out")
    ld = _lse_desc(lse, "lse")
    _check(lib().cru_attn_fwd_lse(qd, kd, vd, od, _ref(ld),
                                  ctypes.c_float(0.0 if scale is None else scale),
                                  _stream(q)))
    return out, lse


def attn_merge_lse(o_parts: Sequence[torch.Tensor], lse_parts: Sequence[torch.Tensor], *,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   out_dtype: torch.dtype = torch.bfloat16, return_lse: bool = True
                   ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Merge partial results over disjoint key sets, folded in ascending order.

    The partial outputs are all fp32, or all bf16 (the form ring steps leave
    without convert_to_fp32); the LSEs are fp32.  The sums are fp32 either way."""
    n = len(o_parts)
    if n == 0 or n != len(lse_parts):
        raise CruInvalid(1, "need one LSE per partial output, at least one")
    p0 = o_parts[0]
    if out is None:
        out = torch.empty(p0.shape, dtype=out_dtype, device=p0.device)
    if lse is None and return_lse:
        lse = _empty_lse(p0.shape[0], p0.shape[2], p0.shape[1], p0.device)
    parts = (CruTensor * n)(*[_desc(t, f"o_parts[{i}]") for i, t in enumerate(o_parts)])
    lparts = (CruLse * n)(*[_lse_desc(t, f"lse_parts[{i}]") for i, t in enumerate(lse_parts)])
    od, ld = _desc(out, "out"), _lse_desc(lse, "lse")
    _check(lib().cru_attn_merge_lse(n, parts, lparts, od, _ref(ld), _stream(p0)))
    return out, lse


def ring_chunk_bounds(S: int, n: int, anything: bool = False) -> List[Tuple[int, int]]:
    """The library's split of S rows into n chunks: [(start, end), ...]."""
    starts = (ctypes.c_int64 * (n + 1))()
    _check(lib().cru_ring_chunk_bounds(S, n, int(bool(anything)), starts))
    return [(starts[c], starts[c + 1]) for c in range(n)]


def ring_workspace_bytes(q_share: torch.Tensor, n_chunks: int) -> int:
    nbytes = ctypes.c_size_t(0)
    _check(lib().cru_ring_workspace_bytes(_desc(q_share, "q_share"), n_chunks,
                                          ctypes.byref(nbytes)))
    return nbytes.value


def ring_emulate(q_share: torch.Tensor, k: torch.Tensor, v: torch.Tensor, n_chunks: int, *,
                 anything: bool = False, chunk_sizes: Optional[Sequence[int]] = None,
                 fused: bool = False, convert_to_fp32: bool = True,
                 out: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                 scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None,
                 return_lse: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """One ring rank's share: q_share against every K/V chunk, folded in order.

    ``convert_to_fp32=False`` keeps each chunk's partial output in bf16 (the
    partial LSEs stay fp32)."""
    if out is None:
        out = torch.empty(q_share.shape, dtype=out_dtype or q_share.dtype, device=q_share.device)
    if lse is None and return_lse:
        lse = _empty_lse(q_share.shape[0], q_share.shape[2], q_share.shape[1], q_share.device)
    qd = _desc(q_share, "q_share")
    need = ring_workspace_bytes(q_share, n_chunks) if 1 <= n_chunks <= MAX_PARTS else 0
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q_share.device)
    sizes = None
    if chunk_sizes is not None:
        sizes = (ctypes.c_int64 * len(chunk_sizes))(*[int(x) for x in chunk_sizes])
        if len(chunk_sizes) != n_chunks:
            raise CruInvalid(1, f"{len(chunk_sizes)} chunk sizes for {n_chunks} chunks")
    kd, vd, od, ld = _desc(k, "k"), _desc(v, "v"), _desc(out, "out"), _lse_desc(lse, "lse")
    _check(lib().cru_ring_emulate(qd, kd, vd, n_chunks, int(bool(anything)), sizes,
                                  int(bool(fused)), int(bool(convert_to_fp32)), od, _ref(ld),
                                  ctypes.c_float(0.0 if scale is None else scale),
                                  workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                  _stream(q_share)))
    return out, lse


def ring_emulate_noalloc(q_share: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         n_chunks: int, *, anything: bool = False,
                         chunk_sizes: Optional[Sequence[int]] = None, fused: bool = False,
                         convert_to_fp32: bool = True, out: Optional[torch.Tensor] = None,
                         lse: Optional[torch.Tensor] = None,
                         out_dtype: Optional[torch.dtype] = None, scale: Optional[float] = None,
                         return_lse: bool = True
                         ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """ring_emulate with the partials in the library's static scratch array
    (no workspace; the C call allocates nothing).  Pass ``out`` (and ``lse``)
    to keep this wrapper from allocating them as well."""
    if out is None:
        out = torch.empty(q_share.shape, dtype=out_dtype or q_share.dtype, device=q_share.device)
    if lse is None and return_lse:
        lse = _empty_lse(q_share.shape[0], q_share.shape[2], q_share.shape[1], q_share.device)
    sizes = None
    if chunk_sizes is not None:
        if len(chunk_sizes) != n_chunks:
            raise CruInvalid(1, f"{len(chunk_sizes)} chunk sizes for {n_chunks} chunks")
        sizes = (ctypes.c_int64 * len(chunk_sizes))(*[int(x) for x in chunk_sizes])
    qd, kd, vd = _desc(q_share, "q_share"), _desc(k, "k"), _desc(v, "v")
    od, ld = _desc(out, "out"), _lse_desc(lse, "lse")
    _check(lib().cru_ring_emulate_noalloc(qd, kd, vd, n_chunks, int(bool(anything)), sizes,
                                          int(bool(fused)), int(bool(convert_to_fp32)), od,
                                          _ref(ld), ctypes.c_float(0.0 if scale is None else scale),
                                          _stream(q_share)))
    return out, lse


def _as_list(x) -> Tuple[List[torch.Tensor], bool]:
    if isinstance(x, torch.Tensor):
        return [x], True
    return list(x), False


def ulysses_head_bounds(H: int, P: int, anything: bool = False) -> List[Tuple[int, int]]:
    """Heads of each Ulysses group, [(start, end)] for p = 0..P-1 (the first
    H mod P groups hold one head more)."""
    starts = (ctypes.c_int64 * (max(P, 0) + 1))()
    _check(lib().cru_ulysses_head_bounds(H, P, int(bool(anything)), starts))
    return [(starts[p], starts[p + 1]) for p in range(P)]


def ulysses_groups(packed: torch.Tensor, B: int, S: int, H: int, D: int, P: int
                   ) -> List[torch.Tensor]:
    """The [B, S, Hp_p, D] views of the head groups in a packed buffer (as
    ulysses_seq2head writes it): group p starts at element B*S*D*h0_p."""
    flat = packed.reshape(-1)
    views = []
    for (h0, h1) in ulysses_head_bounds(H, P, anything=True):
        n = B * S * (h1 - h0) * D
        start = B * S * D * h0
        views.append(flat[start:start + n].view(B, S, h1 - h0, D))
    return views


def ulysses_seq2head(x: Union[torch.Tensor, Sequence[torch.Tensor]], P: int, *,
                     anything: bool = False, out: Optional[Sequence[torch.Tensor]] = None):
    """[B, S, H, D] -> [P, B, S, H/P, D] (group p = heads p*H/P .. (p+1)*H/P - 1).

    Accepts one tensor or up to 8 same-shaped tensors (one launch).  With
    ``anything`` (Ulysses Anything: H and S need not divide by P) the result
    is a flat buffer of B*S*H*D elements per tensor, the groups back to back
    (``ulysses_groups`` gives their views)."""
    xs, single = _as_list(x)
    if not xs:
        raise CruInvalid(1, "no tensors")
    descs = [_desc(t, f"x[{i}]") for i, t in enumerate(xs)]
    B, S, H, D = xs[0].shape
    even = P >= 1 and H % P == 0 and not anything
    if out is None:
        if anything:
            ys = [torch.empty(B * S * H * D, dtype=t.dtype, device=t.device) for t in xs]
        elif even:
            ys = [torch.empty((P, B, S, H // P, D), dtype=t.dtype, device=t.device) for t in xs]
        else:
            ys = [torch.empty(0, dtype=t.dtype, device=t.device) for t in xs]
    else:
        ys, _ = _as_list(out)
    if len(ys) != len(xs):
        raise CruInvalid(1, "one output per input")
    for y, t in zip(ys, xs):
        if anything:
            if y.numel() != B * S * H * D or not y.is_contiguous() or y.dtype != t.dtype:
                raise CruInvalid(1, f"output must be a contiguous {t.dtype} buffer of "
                                    f"{B * S * H * D} elements")
        elif even and (tuple(y.shape) != (P, B, S, H // P, D) or not y.is_contiguous()
                       or y.dtype != t.dtype):
            raise CruInvalid(1, f"output must be a contiguous {(P, B, S, H // P, D)} {t.dtype} tensor")
    n = len(xs)
    xarr = (CruTensor * n)(*descs)
    yarr = (ctypes.c_void_p * n)(*[y.data_ptr() for y in ys])
    _check(lib().cru_ulysses_seq2head(n, xarr, yarr, P, int(bool(anything)), _stream(xs[0])))
    return ys[0] if single else ys


def ulysses_head2seq(y: Union[torch.Tensor, Sequence[torch.Tensor]], P: int, *,
                     anything: bool = False, shape: Optional[Sequence[int]] = None,
                     out: Optional[Union[torch.Tensor, Sequence[torch.Tensor]]] = None):
    """[P, B, S, H/P, D] -> [B, S, H, D]; the inverse of ulysses_seq2head.

    With ``anything`` the inputs are packed buffers as ulysses_seq2head writes
    them, and the [B, S, H, D] shape comes from ``shape`` or ``out``."""
    ys, single = _as_list(y)
    if not ys:
        raise CruInvalid(1, "no tensors")
    if anything:
        if out is not None:
            xs, _ = _as_list(out)
            B, S, H, D = xs[0].shape
        elif shape is not None:
            B, S, H, D = (int(x) for x in shape)
            xs = [torch.empty((B, S, H, D), dtype=t.dtype, device=t.device) for t in ys]
        else:
            raise CruInvalid(1, "anything=True needs the [B, S, H, D] shape (shape= or out=)")
        for t in ys:
            if t.numel() != B * S * H * D or not t.is_contiguous():
                raise CruInvalid(1, f"input must be a contiguous buffer of {B * S * H * D} elements")
    else:
        for t in ys:
            if t.dim() != 5 or t.shape[0] != P or not t.is_contiguous():
                raise CruInvalid(1, f"input must be a contiguous [P={P}, B, S, H/P, D] tensor")
        _, B, S, hp, D = ys[0].shape
        H = P * hp
        if out is None:
            xs = [torch.empty((B, S, H, D), dtype=t.dtype, device=t.device) for t in ys]
        else:
            xs, _ = _as_list(out)
        for t in ys:
            if tuple(t.shape) != (P, B, S, hp, D):
                raise CruInvalid(1, "inputs must match in shape")
    if len(xs) != len(ys):
        raise CruInvalid(1, "one output per input")
    for t, x in zip(ys, xs):
        if x.dtype != t.dtype or tuple(x.shape) != (B, S, H, D):
            raise CruInvalid(1, "inputs and outputs must match in shape and dtype")
    n = len(ys)
    xarr = (CruTensor * n)(*[_desc(t, f"out[{i}]") for i, t in enumerate(xs)])
    yarr = (ctypes.c_void_p * n)(*[t.data_ptr() for t in ys])
    _check(lib().cru_ulysses_head2seq(n, yarr, xarr, P, int(bool(anything)), _stream(ys[0])))
    return xs[0] if single else xs


def usp_workspace_bytes(q: torch.Tensor, ulysses_degree: int, ring_degree: int) -> int:
    nbytes = ctypes.c_size_t(0)
    _check(lib().cru_usp_workspace_bytes(_desc(q, "q"), ulysses_degree, ring_degree,
                                         ctypes.byref(nbytes)))
    return nbytes.value


def usp_emulate(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, ulysses_degree: int,
                ring_degree: int, *, fused: bool = False, convert_to_fp32: bool = True,
                out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None,
                return_lse: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Unified (USP) attention on a ulysses_degree x ring_degree mesh, every
    device's share computed on this device: the full output and LSE."""
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = _empty_lse(q.shape[0], q.shape[2], q.shape[1], q.device)
    qd = _desc(q, "q")
    if workspace is None:
        need = usp_workspace_bytes(q, ulysses_degree, ring_degree)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    kd, vd, od, ld = _desc(k, "k"), _desc(v, "v"), _desc(out, "out"), _lse_desc(lse, "lse")
    _check(lib().cru_usp_emulate(qd, kd, vd, ulysses_degree, ring_degree, int(bool(fused)),
                                 int(bool(convert_to_fp32)), od,
                                 _ref(ld), ctypes.c_float(0.0 if scale is None else scale),
                                 workspace.data_ptr(),
                                 workspace.numel() * workspace.element_size(), _stream(q)))
    return out, lse


# ------------------------------------------------------------- configuration

@dataclass(frozen=True)
class ContextParallelConfig:
    """The per-rank view of diffusers' ContextParallelConfig (diffusers
    "Parallelism" API page): the fields that decide what one rank computes.

    Rules from the "Context parallelism" guide's variant table and the API
    page: degrees are >= 1; Ring Anything needs ring_degree > 1 and
    ulysses_degree == 1; Ulysses Anything needs ulysses_degree > 1 and
    ring_degree == 1.  Partials are fp32 with convert_to_fp32=True (the
    default) and bf16 otherwise (ring_emulate / usp_emulate take the same
    flag).  Both degrees > 1 is Unified attention (usp_emulate).
    """
    ring_degree: int = 1
    ulysses_degree: int = 1
    convert_to_fp32: bool = True
    ring_anything: bool = False
    ulysses_anything: bool = False

    def __post_init__(self):
        if self.ring_degree < 1 or self.ulysses_degree < 1:
            raise ValueError("ring_degree and ulysses_degree must be >= 1")
        if self.ring_anything and (self.ring_degree < 2 or self.ulysses_degree != 1):
            raise ValueError("ring_anything needs ring_degree > 1 and ulysses_degree == 1")
        if self.ulysses_anything and (self.ulysses_degree < 2 or self.ring_degree != 1):
            raise ValueError("ulysses_anything needs ulysses_degree > 1 and ring_degree == 1")
