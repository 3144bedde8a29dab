"""ctypes binding of libfsattn.so.

Argument marshalling only: every step of the attention path runs in the HIP
library. PyTorch provides device memory and the current stream. If the
library is not built, every call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
import re
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfsattn.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "fsattn.h")

# the layout of the structures below (FSATTN_ABI_VERSION of the header)
ABI_VERSION = 3

F32, BF16 = 0, 1
MODE_AUTO, MODE_FORCE_ONLINE, MODE_FORCE_FIXED, SHIFT_PER_ROW = 0, 1, 2, 4
DEFAULT_GAP_NATS = 30.0

STATUS_NAMES = {0: "FSATTN_OK", 1: "FSATTN_ERR_INVALID_ARGUMENT", 2: "FSATTN_ERR_BLOCK_GEOMETRY",
                3: "FSATTN_ERR_UNSUPPORTED", 4: "FSATTN_ERR_BUFFER_TOO_SMALL", 5: "FSATTN_ERR_HIP"}


class Mask(ctypes.Structure):
    _fields_ = [("num_frames", ctypes.c_int32), ("tokens_per_frame", ctypes.c_int32),
                ("window_before", ctypes.c_int32), ("window_after", ctypes.c_int32),
                ("ref_frame", ctypes.c_int32), ("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32),
                ("ref_queries_global", ctypes.c_int32), ("ref_count", ctypes.c_int32)]


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("stride_n", ctypes.c_int64)]


class HeadBound(ctypes.Structure):
    _fields_ = [("q_norm_max", ctypes.c_float), ("k_norm_max", ctypes.c_float), ("c_max", ctypes.c_float),
                ("bound", ctypes.c_float), ("gap_est", ctypes.c_float), ("eligible", ctypes.c_int32),
                ("pad", ctypes.c_int32 * 2)]


class FsattnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m frame_block_sparse_amd._build` "
                           "(or __graft_entry__.build()); there is no CPU fallback")
    L = ctypes.CDLL(LIB_PATH)
    c_i32p = ctypes.POINTER(ctypes.c_int32)
    c_i64p = ctypes.POINTER(ctypes.c_int64)
    L.fsattn_plan_size.argtypes = [ctypes.POINTER(Mask), c_i64p, c_i64p]
    L.fsattn_plan.argtypes = [ctypes.POINTER(Mask), c_i32p, ctypes.c_int64, c_i32p, ctypes.c_int64]
    L.fsattn_plan_device.argtypes = [ctypes.c_void_p, ctypes.POINTER(Mask), ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_void_p, ctypes.c_int64]
    L.fsattn_head_bounds_workspace_bytes.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Mask)]
    L.fsattn_head_bounds_workspace_bytes.restype = ctypes.c_size_t
    L.fsattn_head_bounds.argtypes = [ctypes.c_void_p, ctypes.POINTER(Shape), ctypes.POINTER(Mask), Tensor, Tensor,
                                     ctypes.c_float, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_size_t]
    L.fsattn_head_bounds_noalloc.argtypes = [ctypes.c_void_p, ctypes.POINTER(Shape), ctypes.POINTER(Mask), Tensor,
                                             Tensor, ctypes.c_float, ctypes.c_float, ctypes.c_void_p,
                                             ctypes.c_void_p]
    L.fsattn_head_bounds_noalloc_max_workspace.argtypes = []
    L.fsattn_head_bounds_noalloc_max_workspace.restype = ctypes.c_size_t
    L.fsattn_produce.argtypes = [ctypes.c_void_p, ctypes.POINTER(Shape), ctypes.POINTER(Mask), Tensor, Tensor,
                                 Tensor, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p,
                                 ctypes.c_void_p, Tensor, Tensor, Tensor, ctypes.c_float, ctypes.c_float,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t]
    L.fsattn_forward.argtypes = [ctypes.c_void_p, ctypes.POINTER(Shape), ctypes.POINTER(Mask),
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                 Tensor, Tensor, Tensor, Tensor, ctypes.c_int32, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_float, ctypes.c_uint32, ctypes.c_void_p]
    L.fsattn_forward_launch_info.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Mask), ctypes.c_uint32,
                                             c_i32p, c_i32p, c_i32p, c_i64p, c_i32p]
    L.fsattn_prior_art_forward.argtypes = [ctypes.c_void_p, ctypes.POINTER(Shape), ctypes.POINTER(Mask),
                                           Tensor, Tensor, Tensor, Tensor, ctypes.c_int32, ctypes.c_float,
                                           ctypes.c_void_p, ctypes.c_size_t]
    L.fsattn_prior_art_workspace_bytes.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Mask)]
    L.fsattn_prior_art_workspace_bytes.restype = ctypes.c_size_t
    L.fsattn_mfma_probe.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, c_i64p]
    L.fsattn_status_string.argtypes = [ctypes.c_int]
    L.fsattn_status_string.restype = ctypes.c_char_p
    L.fsattn_abi_version.argtypes = []
    if L.fsattn_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{LIB_PATH} has ABI {L.fsattn_abi_version()}, the binding expects {ABI_VERSION}: "
                           "rebuild it")
    for name in ("fsattn_plan_size", "fsattn_plan", "fsattn_plan_device", "fsattn_head_bounds",
                 "fsattn_head_bounds_noalloc", "fsattn_produce",
                 "fsattn_forward",
                 "fsattn_forward_launch_info", "fsattn_mfma_probe", "fsattn_prior_art_forward"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def status_string(st: int) -> str:
    return lib().fsattn_status_string(st).decode()


def abi_version() -> int:
    return lib().fsattn_abi_version()


def declared_functions():
    """Names of the functions include/fsattn.h declares."""
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w ]+?\*?\s*(fsattn_\w+)\s*\(", text, re.M)))


def _check(st: int, what: str):
    if st != 0:
        raise FsattnError(st, what)


def to_mask(mask) -> Mask:
    """A Mask from a Mask, a tuple of 7 to 9 integers (num_frames,
    tokens_per_frame, window_before, window_after, ref_frame, block_q,
    block_k [, ref_queries_global [, ref_count]]) or any object with a
    mask_tuple() method."""
    if isinstance(mask, Mask):
        return mask
    if hasattr(mask, "mask_tuple"):
        mask = mask.mask_tuple()
    vals = [int(x) for x in mask]
    if len(vals) not in (7, 8, 9):
        raise ValueError(f"a mask has 7 to 9 integers, got {len(vals)}")
    return Mask(*vals)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise FsattnError(3, f"unsupported tensor dtype {t.dtype}")


def _tensor(t: torch.Tensor) -> Tensor:
    if t.dim() != 4:
        raise FsattnError(1, "tensors must be [B, H, N, d]")
    if t.stride(3) != 1:
        raise FsattnError(1, "the head dimension must be contiguous")
    sb, sh, sn, _ = t.stride()
    return Tensor(t.data_ptr(), sb, sh, sn)


def _shape(q: torch.Tensor) -> Shape:
    B, H, N, d = q.shape
    return Shape(B, H, N, d, _dtype_code(q))


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


# Host-side checks of what the C ABI cannot see (the extent, dtype and
# device of each buffer): a mismatch would otherwise make a kernel read or
# write outside a buffer. Shapes and dtypes are checked first, then that
# every tensor is on the first operand's GPU.

def _same_operands(what: str, ref: torch.Tensor, *ts: torch.Tensor):
    if ref.dim() != 4:
        raise FsattnError(1, f"{what}: tensors must be [B, H, N, d], got shape {tuple(ref.shape)}")
    for t in ts:
        if tuple(t.shape) != tuple(ref.shape):
            raise FsattnError(1, f"{what}: operand of shape {tuple(t.shape)} beside {tuple(ref.shape)}")
        if t.dtype != ref.dtype:
            raise FsattnError(1, f"{what}: operand of dtype {t.dtype} beside {ref.dtype}")


def _f32_buffer(what: str, t: torch.Tensor, numel: int):
    if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() < numel:
        raise FsattnError(1, f"{what} must be a contiguous float32 tensor of at least {numel} elements")


def _bounds_buffers(what: str, b: "Bounds", B: int, H: int, d: int):
    _f32_buffer(f"{what}: key_mean", b.key_mean, B * H * d)
    _f32_buffer(f"{what}: rec", b.rec, B * H * 8)


def _nbytes(t: torch.Tensor) -> int:
    if not t.is_contiguous():
        raise FsattnError(1, "a workspace must be contiguous")
    return t.numel() * t.element_size()


def _on_gpu(what: str, ref: torch.Tensor, *ts: Optional[torch.Tensor]):
    if not ref.is_cuda:
        raise FsattnError(1, f"{what}: tensors must be on a GPU, got {ref.device}")
    for t in ts:
        if t is not None and t.device != ref.device:
            raise FsattnError(1, f"{what}: tensors on {t.device} and {ref.device}")


# ----------------------------------------------------------------- plan

def plan_size(mask) -> Tuple[int, int]:
    m = to_mask(mask)
    nqb, nnz = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().fsattn_plan_size(ctypes.byref(m), ctypes.byref(nqb), ctypes.byref(nnz)), "fsattn_plan_size")
    return nqb.value, nnz.value


def plan(mask) -> Tuple[torch.Tensor, torch.Tensor]:
    """(row_ptr, col_idx) as CPU int32 tensors."""
    m = to_mask(mask)
    nqb, nnz = plan_size(m)
    rp = torch.empty(nqb + 1, dtype=torch.int32)
    ci = torch.empty(max(nnz, 1), dtype=torch.int32)
    i32p = ctypes.POINTER(ctypes.c_int32)
    _check(lib().fsattn_plan(ctypes.byref(m), ctypes.cast(rp.data_ptr(), i32p), rp.numel(),
                             ctypes.cast(ci.data_ptr(), i32p), ci.numel()), "fsattn_plan")
    return rp, ci[:nnz]


@dataclass
class DevicePlan:
    mask: Mask
    row_ptr: torch.Tensor
    col_idx: torch.Tensor

    @property
    def nnz(self) -> int:
        return self.col_idx.numel()


def device_plan(mask, device) -> DevicePlan:
    """The host plan (fsattn_plan) copied to the device."""
    m = to_mask(mask)
    rp, ci = plan(m)
    if ci.numel() == 0:
        ci = torch.zeros(1, dtype=torch.int32)[:0]
    return DevicePlan(m, rp.to(device), ci.to(device))


def plan_on_device(mask, device=None, out: Optional[DevicePlan] = None) -> DevicePlan:
    """The plan written on the GPU by fsattn_plan_device, on the current
    stream; `out` reuses the device arrays of an earlier plan of the same
    mask. Both arrays live in one buffer (row_ptr, then col_idx)."""
    m = to_mask(mask)
    nqb, nnz = plan_size(m)
    if out is None:
        buf = torch.empty(nqb + 1 + nnz, dtype=torch.int32, device=device)
        out = DevicePlan(m, buf[:nqb + 1], buf[nqb + 1:])
    elif out.row_ptr.numel() != nqb + 1 or out.col_idx.numel() != nnz:
        raise ValueError("out holds a plan of another size")
    stream = torch.cuda.current_stream(out.row_ptr.device).cuda_stream
    _check(lib().fsattn_plan_device(stream, ctypes.byref(m), out.row_ptr.data_ptr(), out.row_ptr.numel(),
                                    out.col_idx.data_ptr(), out.col_idx.numel()), "fsattn_plan_device")
    return out


# ----------------------------------------------------------------- bounds

@dataclass
class Bounds:
    key_mean: torch.Tensor      # [B, H, d] fp32 (device)
    rec: torch.Tensor           # [B, H, 8] fp32 raw records (device)

    def host(self):
        """The records decoded on the host: dict of [B, H] numpy arrays."""
        r = self.rec.detach().cpu()
        return dict(q_norm_max=r[..., 0].numpy(), k_norm_max=r[..., 1].numpy(), c_max=r[..., 2].numpy(),
                    bound=r[..., 3].numpy(), gap_est=r[..., 4].numpy(),
                    eligible=r[..., 5].contiguous().view(torch.int32).numpy())


def head_bounds_workspace_bytes(q: torch.Tensor, mask) -> int:
    m = to_mask(mask)
    s = _shape(q)
    return lib().fsattn_head_bounds_workspace_bytes(ctypes.byref(s), ctypes.byref(m))


def head_bounds(q: torch.Tensor, k: torch.Tensor, mask, scale: Optional[float] = None,
                threshold: float = DEFAULT_GAP_NATS, workspace: Optional[torch.Tensor] = None,
                out: Optional[Bounds] = None) -> Bounds:
    m = to_mask(mask)
    _same_operands("fsattn_head_bounds", q, k)
    s = _shape(q)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is not None:
        _bounds_buffers("fsattn_head_bounds", out, B, H, d)
    _on_gpu("fsattn_head_bounds", q, k, workspace, *((out.key_mean, out.rec) if out is not None else ()))
    L = lib()
    need = L.fsattn_head_bounds_workspace_bytes(ctypes.byref(s), ctypes.byref(m))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if out is None:
        out = Bounds(torch.empty((B, H, d), dtype=torch.float32, device=q.device),
                     torch.empty((B, H, 8), dtype=torch.float32, device=q.device))
    _check(L.fsattn_head_bounds(_stream(q), ctypes.byref(s), ctypes.byref(m), _tensor(q), _tensor(k),
                                float(scale), float(threshold), out.key_mean.data_ptr(), out.rec.data_ptr(),
                                workspace.data_ptr(), _nbytes(workspace)), "fsattn_head_bounds")
    return out


def head_bounds_noalloc(q: torch.Tensor, k: torch.Tensor, mask, scale: Optional[float] = None,
                        threshold: float = DEFAULT_GAP_NATS, out: Optional[Bounds] = None) -> Bounds:
    """fsattn_head_bounds_noalloc: the same records with the library's
    device-resident workspace (no workspace argument; the outputs are still
    the caller's)."""
    m = to_mask(mask)
    _same_operands("fsattn_head_bounds_noalloc", q, k)
    s = _shape(q)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is not None:
        _bounds_buffers("fsattn_head_bounds_noalloc", out, B, H, d)
    _on_gpu("fsattn_head_bounds_noalloc", q, k, *((out.key_mean, out.rec) if out is not None else ()))
    if out is None:
        out = Bounds(torch.empty((B, H, d), dtype=torch.float32, device=q.device),
                     torch.empty((B, H, 8), dtype=torch.float32, device=q.device))
    _check(lib().fsattn_head_bounds_noalloc(_stream(q), ctypes.byref(s), ctypes.byref(m), _tensor(q), _tensor(k),
                                            float(scale), float(threshold), out.key_mean.data_ptr(),
                                            out.rec.data_ptr()), "fsattn_head_bounds_noalloc")
    return out


def noalloc_max_workspace() -> int:
    return lib().fsattn_head_bounds_noalloc_max_workspace()


def _f32_ptr(t: Optional[torch.Tensor], shape, what: str, device: torch.device) -> int:
    if t is None:
        return 0
    if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise FsattnError(1, f"{what} must be a contiguous float32 tensor of shape {tuple(shape)}")
    if t.device != device:
        raise FsattnError(1, f"{what} is on {t.device}, the operands on {device}")
    return t.data_ptr()


def produce(q_in: torch.Tensor, k_in: torch.Tensor, v_in: torch.Tensor, mask,
            gamma_q: Optional[torch.Tensor] = None, gamma_k: Optional[torch.Tensor] = None, eps: float = 1e-6,
            rope_cos: Optional[torch.Tensor] = None, rope_sin: Optional[torch.Tensor] = None,
            out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None, scale: Optional[float] = None,
            threshold: float = DEFAULT_GAP_NATS, workspace: Optional[torch.Tensor] = None,
            bounds: Optional[Bounds] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor, Bounds]:
    """fsattn_produce: Q, K (RMS-normalised with gamma [H, d], then rotated
    with the angle tables [N, d/2]) and V written through `out` (default:
    new contiguous [B, H, N, d] tensors), plus the bound records of the
    values written. Inputs may be any [B, H, N, d] views with a contiguous
    last axis, e.g. slices of a token-major QKV projection output."""
    m = to_mask(mask)
    _same_operands("fsattn_produce", q_in, k_in, v_in, *(out if out is not None else ()))
    if out is not None and len(out) != 3:
        raise FsattnError(1, "fsattn_produce: out holds Q, K and V")
    s = _shape(q_in)
    B, H, N, d = q_in.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if bounds is not None:
        _bounds_buffers("fsattn_produce", bounds, B, H, d)
    _on_gpu("fsattn_produce", q_in, k_in, v_in, workspace, *(out if out is not None else ()),
            *((bounds.key_mean, bounds.rec) if bounds is not None else ()))
    L = lib()
    if out is None:
        out = tuple(torch.empty((B, H, N, d), dtype=q_in.dtype, device=q_in.device) for _ in range(3))
    need = L.fsattn_head_bounds_workspace_bytes(ctypes.byref(s), ctypes.byref(m))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q_in.device)
    if bounds is None:
        bounds = Bounds(torch.empty((B, H, d), dtype=torch.float32, device=q_in.device),
                        torch.empty((B, H, 8), dtype=torch.float32, device=q_in.device))
    q, k, v = out
    _check(L.fsattn_produce(_stream(q_in), ctypes.byref(s), ctypes.byref(m), _tensor(q_in), _tensor(k_in),
                            _tensor(v_in), _f32_ptr(gamma_q, (H, d), "gamma_q", q_in.device),
                            _f32_ptr(gamma_k, (H, d), "gamma_k", q_in.device), float(eps),
                            _f32_ptr(rope_cos, (N, d // 2), "rope_cos", q_in.device),
                            _f32_ptr(rope_sin, (N, d // 2), "rope_sin", q_in.device), _tensor(q), _tensor(k),
                            _tensor(v), float(scale), float(threshold), bounds.key_mean.data_ptr(),
                            bounds.rec.data_ptr(), workspace.data_ptr(), _nbytes(workspace)), "fsattn_produce")
    return q, k, v, bounds


# ----------------------------------------------------------------- forward

_MODES = {"auto": MODE_AUTO, "online": MODE_FORCE_ONLINE, "fixed": MODE_FORCE_FIXED}


def make_flags(mode: str = "auto", per_row_shift: bool = False, waves: int = 0, rows_per_wave: int = 0,
               key_step: int = 0, ring: int = 0, deal: int = 0) -> int:
    """Flags word of fsattn_forward (see include/fsattn.h). deal: 0 library
    choice, 1..14 chunks of 2**(deal-1) tiles, 15 whole (frame, head) groups."""
    f = _MODES[mode]
    if per_row_shift:
        f |= SHIFT_PER_ROW
    f |= (waves & 15) << 8
    f |= ((rows_per_wave // 16) & 15) << 12
    f |= ((key_step // 16) & 15) << 16
    f |= (ring & 15) << 20
    f |= (deal & 15) << 24
    return f


def launch_info(q_shape, dtype: int, mask, flags: int = 0):
    """(waves, rows_per_wave, key_step, workgroups, lds_bytes) of a forward."""
    B, H, N, d = q_shape
    s = Shape(B, H, N, d, dtype)
    m = to_mask(mask)
    w, r, k, l = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    g = ctypes.c_int64()
    _check(lib().fsattn_forward_launch_info(ctypes.byref(s), ctypes.byref(m), flags, ctypes.byref(w),
                                            ctypes.byref(r), ctypes.byref(k), ctypes.byref(g), ctypes.byref(l)),
           "fsattn_forward_launch_info")
    return w.value, r.value, k.value, g.value, l.value


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dplan: DevicePlan,
            bounds: Optional[Bounds], scale: Optional[float] = None, flags: int = 0,
            out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
            lse: Optional[torch.Tensor] = None, stream: Optional[int] = None) -> torch.Tensor:
    """Attention over the plan's live blocks. Returns `out` ([B, H, N, d])."""
    _same_operands("fsattn_forward", q, k, v)
    s = _shape(q)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is not None:
        if tuple(out.shape) != tuple(q.shape) or out.dtype not in (q.dtype, torch.float32):
            raise FsattnError(1, f"fsattn_forward: out must be {tuple(q.shape)} of {q.dtype} or float32")
    if bounds is not None:
        _bounds_buffers("fsattn_forward", bounds, B, H, d)
    if lse is not None:
        _f32_buffer("fsattn_forward: lse", lse, B * H * N)
    nqb, nnz = plan_size(dplan.mask)
    for t, n, name in ((dplan.row_ptr, nqb + 1, "row_ptr"), (dplan.col_idx, nnz, "col_idx")):
        if t.dtype != torch.int32 or not t.is_contiguous() or t.numel() < n:
            raise FsattnError(1, f"fsattn_forward: {name} must be a contiguous int32 tensor of {n} elements")
    _on_gpu("fsattn_forward", q, k, v, out, lse, dplan.row_ptr, dplan.col_idx,
            *((bounds.key_mean, bounds.rec) if bounds is not None else ()))
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype or q.dtype, device=q.device)
    o_code = _dtype_code(out)
    km = bounds.key_mean.data_ptr() if bounds is not None else None
    rc = bounds.rec.data_ptr() if bounds is not None else None
    _check(lib().fsattn_forward(stream if stream is not None else _stream(q), ctypes.byref(s),
                                ctypes.byref(dplan.mask), dplan.row_ptr.data_ptr(), dplan.col_idx.data_ptr(),
                                dplan.nnz, _tensor(q), _tensor(k), _tensor(v), _tensor(out), o_code,
                                km, rc, float(scale), int(flags),
                                lse.data_ptr() if lse is not None else None), "fsattn_forward")
    return out


def mfma_probe(workgroups: int, iters: int, device=None, stream: Optional[int] = None) -> int:
    """Launches the pure-MFMA reference loop (fsattn_mfma_probe) on the
    current stream and returns the FLOPs it performs; time it with events."""
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    sink = torch.empty(max(1, workgroups), dtype=torch.float32, device=dev)
    flops = ctypes.c_int64()
    _check(lib().fsattn_mfma_probe(stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream,
                                   int(workgroups), int(iters), sink.data_ptr(), ctypes.byref(flops)),
           "fsattn_mfma_probe")
    return flops.value


def prior_art_workspace_bytes(q: torch.Tensor, mask) -> int:
    """Workspace bytes of fsattn_prior_art_forward for q's shape."""
    return int(lib().fsattn_prior_art_workspace_bytes(ctypes.byref(_shape(q)), ctypes.byref(to_mask(mask))))


def prior_art_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask, scale: Optional[float] = None,
                      out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                      workspace: Optional[torch.Tensor] = None, stream: Optional[int] = None) -> torch.Tensor:
    """The comparator (fsattn_prior_art_forward): the same attention with
    128-token tiles, window and reference-frame passes and a merge."""
    m = to_mask(mask)
    _same_operands("fsattn_prior_art_forward", q, k, v)
    s = _shape(q)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is not None:
        if tuple(out.shape) != tuple(q.shape) or out.dtype not in (q.dtype, torch.float32):
            raise FsattnError(1, f"fsattn_prior_art_forward: out must be {tuple(q.shape)} of {q.dtype} or float32")
    _on_gpu("fsattn_prior_art_forward", q, k, v, out, workspace)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype or q.dtype, device=q.device)
    need = prior_art_workspace_bytes(q, m)
    if workspace is None or _nbytes(workspace) < need:
        workspace = torch.empty(max(1, need), dtype=torch.uint8, device=q.device)
    _check(lib().fsattn_prior_art_forward(stream if stream is not None else _stream(q), ctypes.byref(s),
                                          ctypes.byref(m), _tensor(q), _tensor(k), _tensor(v), _tensor(out),
                                          _dtype_code(out), float(scale), workspace.data_ptr(), _nbytes(workspace)),
           "fsattn_prior_art_forward")
    return out
