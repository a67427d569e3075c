"""Python binding of libfd (split-KV decode attention for MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libfd.so``, reached through the C ABI of ``include/fd.h`` via
ctypes. PyTorch provides device memory and the stream. The functions carry
the C names. There is no fallback: if the library is missing or the call
fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "FD_F32", "FD_F16", "FD_BF16", "FD_MAX_SPLITS", "FdError", "library_path", "load_library",
    "fd_plan_splits", "fd_workspace_bytes", "fd_decode_attention", "fd_decode_split",
    "fd_decode_combine", "fd_status_string", "fd_last_error", "fd_set_kernel_path", "kv_layout",
    "FD_PATH_AUTO", "FD_PATH_VALU", "FD_PATH_MFMA", "FD_PATH_UNPACKED", "workspace_views",
    "fd_workspace_bytes_unnorm", "fd_decode_split_unnorm", "fd_decode_combine_unnorm",
    "fd_decode_attention_unnorm", "workspace_views_unnorm", "fd_decode_attention_noalloc",
    "FD_NOALLOC_SCRATCH_BYTES", "fd_set_schedule", "fd_plan_schedule", "FD_SCHED_AUTO", "FD_SCHED_STATIC",
    "FD_SCHED_QUEUE", "FD_SCHED_STEAL", "fd_set_combine", "FD_COMBINE_SEPARATE", "FD_COMBINE_FUSED",
    "fd_plan_time_us",
]

FD_F32, FD_F16, FD_BF16 = 0, 1, 2
FD_MAX_SPLITS = 16384
FD_NOALLOC_SCRATCH_BYTES = 16 << 20
FD_PATH_AUTO, FD_PATH_VALU, FD_PATH_MFMA, FD_PATH_UNPACKED = 0, 1, 2, 3
FD_SCHED_AUTO, FD_SCHED_STATIC, FD_SCHED_QUEUE, FD_SCHED_STEAL = 0, 1, 2, 3
FD_COMBINE_SEPARATE, FD_COMBINE_FUSED = 0, 1
_STATUS = {0: "FD_OK", 1: "FD_ERR_INVALID_ARG", 2: "FD_ERR_UNSUPPORTED",
           3: "FD_ERR_EMPTY_SPLIT", 4: "FD_ERR_HIP", 5: "FD_ERR_SCRATCH"}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class FdError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        lib = load_library()
        msg = lib.fd_status_string(status).decode()
        extra = lib.fd_last_error().decode() if status in (4, 5) else ""
        super().__init__(f"{where}: {_STATUS.get(status, status)} ({msg}) {extra}".strip())


class FdKvLayout(ctypes.Structure):
    _fields_ = [("batch_stride", ctypes.c_int64), ("head_stride", ctypes.c_int64),
                ("token_stride", ctypes.c_int64), ("cu_stride", ctypes.c_int64)]


def library_path() -> str:
    return os.path.join(_HERE, "libfd.so")


def load_library():
    """Load libfd.so (built by ``decode_attention_09_amd.build``); raises if absent."""
    global _LIB
    if _LIB is not None:
        return _LIB
    # torch ships its own HIP runtime under the same soname as the system one.
    # Import it first so libfd binds to the runtime that owns the tensors and
    # streams it is handed (loading libfd first would bring in a second HIP
    # runtime, on which the device is not visible).
    import torch  # noqa: F401
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() or "
                           "python -m decode_attention_09_amd.build")
    lib = ctypes.CDLL(path)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lay = ctypes.POINTER(FdKvLayout)
    lib.fd_plan_splits.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(ctypes.c_int32), i32,
                                   i32, ctypes.POINTER(ctypes.c_int)]
    lib.fd_plan_splits.restype = i32
    lib.fd_plan_schedule.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(ctypes.c_int32),
                                     i32, i32, ctypes.POINTER(ctypes.c_int),
                                     ctypes.POINTER(ctypes.c_int)]
    lib.fd_plan_schedule.restype = i32
    lib.fd_plan_time_us.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(ctypes.c_int32), i32,
                                    i32]
    lib.fd_plan_time_us.restype = ctypes.c_double
    lib.fd_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.fd_workspace_bytes.restype = ctypes.c_size_t
    lib.fd_decode_attention.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, vp, vp, vp,
                                        i32, lay]
    lib.fd_decode_attention.restype = i32
    lib.fd_decode_split.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, vp, vp, i32, lay]
    lib.fd_decode_split.restype = i32
    lib.fd_decode_combine.argtypes = [vp, i32, i32, i32, i32, vp, vp, i32]
    lib.fd_decode_combine.restype = i32
    lib.fd_workspace_bytes_unnorm.argtypes = [i32, i32, i32, i32]
    lib.fd_workspace_bytes_unnorm.restype = ctypes.c_size_t
    lib.fd_decode_attention_unnorm.argtypes = lib.fd_decode_attention.argtypes
    lib.fd_decode_attention_unnorm.restype = i32
    lib.fd_decode_split_unnorm.argtypes = lib.fd_decode_split.argtypes
    lib.fd_decode_split_unnorm.restype = i32
    lib.fd_decode_combine_unnorm.argtypes = lib.fd_decode_combine.argtypes
    lib.fd_decode_combine_unnorm.restype = i32
    lib.fd_decode_attention_noalloc.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, vp,
                                                vp, i32, lay]
    lib.fd_decode_attention_noalloc.restype = i32
    lib.fd_status_string.argtypes = [i32]
    lib.fd_status_string.restype = ctypes.c_char_p
    lib.fd_last_error.argtypes = []
    lib.fd_last_error.restype = ctypes.c_char_p
    lib.fd_set_kernel_path.argtypes = [i32]
    lib.fd_set_kernel_path.restype = i32
    lib.fd_set_schedule.argtypes = [i32]
    lib.fd_set_schedule.restype = i32
    lib.fd_set_combine.argtypes = [i32]
    lib.fd_set_combine.restype = i32
    _LIB = lib
    return lib


def _check(status: int, where: str):
    if status != 0:
        raise FdError(status, where)


def fd_status_string(status: int) -> str:
    return load_library().fd_status_string(int(status)).decode()


def fd_last_error() -> str:
    return load_library().fd_last_error().decode()


def fd_set_kernel_path(path: int) -> int:
    """Select the split kernel (FD_PATH_AUTO / _VALU / _MFMA / _UNPACKED) for
    later calls from this thread; returns the previous setting."""
    prev = load_library().fd_set_kernel_path(int(path))
    if prev < 0:
        raise ValueError(f"unknown kernel path {path}")
    return prev


def fd_set_schedule(sched: int) -> int:
    """Select how split launches from this thread hand segments to
    workgroups (FD_SCHED_AUTO / _STATIC / _QUEUE / _STEAL); returns the
    previous setting. Static and queue results are bitwise identical; the
    steal schedule (whole calls only) merges other key ranges, so its
    results differ by rounding."""
    prev = load_library().fd_set_schedule(int(sched))
    if prev < 0:
        raise ValueError(f"unknown schedule {sched}")
    return prev


def fd_set_combine(mode: int) -> int:
    """Select where fd_decode_attention calls from this thread merge the
    partials (FD_COMBINE_SEPARATE: the combine kernel; FD_COMBINE_FUSED: the
    last split workgroup of each (sequence, KV head), one launch); returns
    the previous setting. A fused call needs the workspace's arrival counters
    at zero: workspaces this binding allocates are zero-filled, and a caller's
    own workspace must be zeroed once when allocated."""
    prev = load_library().fd_set_combine(int(mode))
    if prev < 0:
        raise ValueError(f"unknown combine mode {mode}")
    return prev


# ----------------------------------------------------------- marshalling --
def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: FD_F32, torch.float16: FD_F16, torch.bfloat16: FD_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _torch_stream(stream, device):
    """The stream the kernels run on, as a torch stream: None -> torch's
    current stream of `device`; a raw hipStream_t handle (int) is wrapped."""
    import torch
    if stream is None:
        return torch.cuda.current_stream(device)
    if hasattr(stream, "cuda_stream"):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _handle(ts):
    return ctypes.c_void_p(ts.cuda_stream)


def kv_layout(k, layout: str = "packed"):
    """Strides (elements) of a K or V tensor for the C ABI.

    "packed": k is [total_kv, kv_heads, dim]; "bhsd": k is
    [batch, kv_heads, max_len, dim]; "bshd": k is [batch, max_len, kv_heads,
    dim]. Views are fine (the tensor's own strides are used); the last dim
    must be contiguous.
    """
    if k.stride(-1) != 1:
        raise ValueError("the head dim of K/V must be contiguous")
    if layout == "packed":
        if k.dim() != 3:
            raise ValueError("packed K/V must be [total_kv, kv_heads, dim]")
        return FdKvLayout(0, k.stride(1), k.stride(0), k.stride(0))
    if layout == "bhsd":
        if k.dim() != 4:
            raise ValueError("bhsd K/V must be [batch, kv_heads, max_len, dim]")
        return FdKvLayout(k.stride(0), k.stride(1), k.stride(2), 0)
    if layout == "bshd":
        if k.dim() != 4:
            raise ValueError("bshd K/V must be [batch, max_len, kv_heads, dim]")
        return FdKvLayout(k.stride(0), k.stride(2), k.stride(1), 0)
    raise ValueError(f"unknown layout {layout!r}")


def fd_plan_splits(batch: int, heads: int, kv_heads: int, dim: int, dtype: int, seqlens,
                   num_cus: int = 0, max_splits: int = 0) -> int:
    lib = load_library()
    lens = [int(x) for x in seqlens]
    arr = (ctypes.c_int32 * max(1, len(lens)))(*lens)
    out = ctypes.c_int(0)
    _check(lib.fd_plan_splits(batch, heads, kv_heads, dim, dtype, arr, num_cus, max_splits,
                              ctypes.byref(out)), "fd_plan_splits")
    return out.value


def fd_plan_schedule(batch: int, heads: int, kv_heads: int, dim: int, dtype: int, seqlens,
                     num_cus: int = 0, max_splits: int = 0) -> tuple[int, int]:
    """(schedule, num_splits) the library recommends for the batch: the
    steal schedule with its layout where it measured faster, else the
    static schedule with fd_plan_splits's count. Set the schedule with
    fd_set_schedule before the call."""
    lib = load_library()
    lens = [int(x) for x in seqlens]
    arr = (ctypes.c_int32 * max(1, len(lens)))(*lens)
    sched, ns = ctypes.c_int(0), ctypes.c_int(0)
    _check(lib.fd_plan_schedule(batch, heads, kv_heads, dim, dtype, arr, num_cus, max_splits,
                                ctypes.byref(sched), ctypes.byref(ns)), "fd_plan_schedule")
    return sched.value, ns.value


def fd_plan_time_us(batch: int, heads: int, kv_heads: int, dim: int, dtype: int, seqlens,
                    num_splits: int, num_cus: int = 0) -> float:
    """The planner's modelled time (us) of one call with num_splits splits."""
    lens = [int(x) for x in seqlens]
    arr = (ctypes.c_int32 * max(1, len(lens)))(*lens)
    t = load_library().fd_plan_time_us(batch, heads, kv_heads, dim, dtype, arr, num_cus,
                                       int(num_splits))
    if t < 0:
        raise ValueError("fd_plan_time_us: bad arguments")
    return float(t)


def fd_workspace_bytes(batch: int, heads: int, num_splits: int, dim: int) -> int:
    return int(load_library().fd_workspace_bytes(batch, heads, num_splits, dim))


def fd_workspace_bytes_unnorm(batch: int, heads: int, num_splits: int, dim: int) -> int:
    return int(load_library().fd_workspace_bytes_unnorm(batch, heads, num_splits, dim))


# Axis of the KV-head index in K/V, per layout name of kv_layout.
_KV_HEAD_AXIS = {"packed": 1, "bhsd": 1, "bshd": 2}


def _sizes(q, k, v, cu, layout):
    """Sizes for the C call, after checking that q, k, v and cu agree: the C
    ABI applies one stride set to K and V and reads everything on one
    device, so mismatches are refused here rather than misread there."""
    import torch
    if q.dim() != 3:
        raise ValueError("q must be [batch, heads, dim]")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    if layout not in _KV_HEAD_AXIS:
        raise ValueError(f"unknown layout {layout!r}")
    batch, heads, dim = q.shape
    if k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("k and v must have the same shape and strides")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must have the same dtype")
    if k.shape[-1] != dim:
        raise ValueError("the head dim of K/V must equal that of q")
    if not (q.device == k.device == v.device == cu.device):
        raise ValueError("q, k, v and cu_seqlens_k must be on one device")
    if cu.dtype != torch.int32 or not cu.is_contiguous():
        raise TypeError("cu_seqlens_k must be a contiguous int32 tensor")
    kv_heads = k.shape[_KV_HEAD_AXIS[layout]]
    if cu.numel() != batch + 1:
        raise ValueError("cu_seqlens_k must have batch + 1 entries")
    return batch, heads, kv_heads, dim


def _check_out(out, q):
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() \
            or out.device != q.device:
        raise ValueError("out must be a contiguous tensor like q ([batch, heads, dim], same dtype)")


def _workspace(q, batch, heads, dim, num_splits, workspace, unnorm=False):
    import torch
    size = fd_workspace_bytes_unnorm if unnorm else fd_workspace_bytes
    need = size(batch, heads, num_splits, dim)
    if workspace is None:
        # zero-filled: the arrival counters of a fused call must start at zero
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace too small: need {need} bytes")
    return workspace


def _plan_from_device_lengths(q, cu, heads, kv_heads, dim) -> int:
    """fd_plan_splits on the lengths in cu_seqlens_k (copied to the host,
    which waits for the device). Empty sequences are left out of the plan:
    the kernels write zero rows for them under any split count."""
    lens = (cu[1:] - cu[:-1]).tolist()
    live = [L for L in lens if L > 0]
    if not live:
        return 1
    return fd_plan_splits(len(live), heads, kv_heads, dim, _dtype_code(q), live)


def _attention(name, unnorm, q, k, v, cu_seqlens_k, num_splits, scale, out, workspace, layout,
               stream):
    import torch
    batch, heads, kv_heads, dim = _sizes(q, k, v, cu_seqlens_k, layout)
    if out is not None:
        _check_out(out, q)
    lay = kv_layout(k, layout)
    if scale is None:
        scale = 1.0 / math.sqrt(dim)
    ts = _torch_stream(stream, q.device)
    # Buffers made here (out, workspace) belong to the stream the kernels
    # run on, so the caching allocator cannot hand them to work on another
    # stream while these kernels still use them.
    with torch.cuda.stream(ts):
        if num_splits is None:
            num_splits = _plan_from_device_lengths(q, cu_seqlens_k, heads, kv_heads, dim)
        if out is None:
            out = torch.empty_like(q)
        if num_splits > 1:
            workspace = _workspace(q, batch, heads, dim, num_splits, workspace, unnorm)
    _check(getattr(load_library(), name)(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_k), batch, heads, kv_heads, dim,
        int(num_splits), float(scale), _ptr(out), _ptr(workspace), _handle(ts),
        _dtype_code(q), ctypes.byref(lay)), name)
    return out


def _split(name, unnorm, q, k, v, cu_seqlens_k, num_splits, scale, workspace, layout, stream):
    import torch
    batch, heads, kv_heads, dim = _sizes(q, k, v, cu_seqlens_k, layout)
    if scale is None:
        scale = 1.0 / math.sqrt(dim)
    lay = kv_layout(k, layout)
    ts = _torch_stream(stream, q.device)
    with torch.cuda.stream(ts):
        workspace = _workspace(q, batch, heads, dim, num_splits, workspace, unnorm)
    _check(getattr(load_library(), name)(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_k), batch, heads, kv_heads, dim,
        int(num_splits), float(scale), _ptr(workspace), _handle(ts),
        _dtype_code(q), ctypes.byref(lay)), name)
    return workspace


def _combine(name, workspace, batch, heads, dim, num_splits, out, stream):
    if tuple(out.shape) != (batch, heads, dim) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [batch, heads, dim] tensor")
    size = fd_workspace_bytes_unnorm if name.endswith("_unnorm") else fd_workspace_bytes
    if workspace.numel() * workspace.element_size() < size(batch, heads, num_splits, dim):
        raise ValueError("workspace smaller than the split launch wrote")
    if workspace.device != out.device:
        raise ValueError("workspace and out must be on one device")
    _check(getattr(load_library(), name)(
        _ptr(workspace), batch, heads, dim, int(num_splits), _ptr(out),
        _handle(_torch_stream(stream, out.device)), _dtype_code(out)), name)
    return out


def fd_decode_attention(q, k, v, cu_seqlens_k, num_splits: int | None, scale: float | None = None,
                        out=None, workspace=None, layout: str = "packed", stream=None):
    """out[b,h] = softmax(scale q[b,h].K_b^T) V_b through libfd's two launches.

    num_splits=None asks fd_plan_splits for the count, on the lengths in
    cu_seqlens_k; reading them to the host waits for the device, so pass the
    count (planned once from host-side lengths) where that matters."""
    return _attention("fd_decode_attention", False, q, k, v, cu_seqlens_k, num_splits, scale,
                      out, workspace, layout, stream)


def fd_decode_split(q, k, v, cu_seqlens_k, num_splits: int, scale: float | None = None,
                    workspace=None, layout: str = "packed", stream=None):
    """First launch only; returns the workspace (uint8 tensor)."""
    return _split("fd_decode_split", False, q, k, v, cu_seqlens_k, num_splits, scale,
                  workspace, layout, stream)


def fd_decode_combine(workspace, batch: int, heads: int, dim: int, num_splits: int, out,
                      stream=None):
    """Second launch only: merge the workspace into out [batch, heads, dim]."""
    return _combine("fd_decode_combine", workspace, batch, heads, dim, num_splits, out, stream)


def fd_decode_attention_noalloc(q, k, v, cu_seqlens_k, num_splits: int, out,
                                scale: float | None = None, layout: str = "packed", stream=None):
    """fd_decode_attention without a workspace: the partials go to the
    library's static per-GPU scratch (FD_NOALLOC_SCRATCH_BYTES). Nothing is
    allocated, here or in the library: `out` and `num_splits` are required.
    Calls that overlap in time on one GPU share that scratch and race."""
    batch, heads, kv_heads, dim = _sizes(q, k, v, cu_seqlens_k, layout)
    _check_out(out, q)
    lay = kv_layout(k, layout)
    if scale is None:
        scale = 1.0 / math.sqrt(dim)
    name = "fd_decode_attention_noalloc"
    _check(getattr(load_library(), name)(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_k), batch, heads, kv_heads, dim,
        int(num_splits), float(scale), _ptr(out), _handle(_torch_stream(stream, q.device)),
        _dtype_code(q), ctypes.byref(lay)), name)
    return out


def fd_decode_attention_unnorm(q, k, v, cu_seqlens_k, num_splits: int | None,
                               scale: float | None = None, out=None, workspace=None,
                               layout: str = "packed", stream=None):
    """The same attention with ceil-equal bounds and (m, l, acc) partials
    (num_splits=None: as in fd_decode_attention)."""
    return _attention("fd_decode_attention_unnorm", True, q, k, v, cu_seqlens_k, num_splits,
                      scale, out, workspace, layout, stream)


def fd_decode_split_unnorm(q, k, v, cu_seqlens_k, num_splits: int, scale: float | None = None,
                           workspace=None, layout: str = "packed", stream=None):
    """Split launch of the (m, l, acc) format; returns the workspace."""
    return _split("fd_decode_split_unnorm", True, q, k, v, cu_seqlens_k, num_splits, scale,
                  workspace, layout, stream)


def fd_decode_combine_unnorm(workspace, batch: int, heads: int, dim: int, num_splits: int, out,
                             stream=None):
    """Combine launch of the (m, l, acc) format."""
    return _combine("fd_decode_combine_unnorm", workspace, batch, heads, dim, num_splits, out,
                    stream)


def _f32_view(flat, off, shape):
    import torch
    n = 1
    for x in shape:
        n *= x
    return flat[off:off + n * 4].view(torch.float32).view(*shape)


def workspace_views(workspace, batch: int, heads: int, dim: int, num_splits: int):
    """(Opart [B,H,ns,D], LSE [B,ns,H]) fp32 views of a workspace, per the
    layout documented in include/fd.h."""
    import torch
    flat = workspace.view(torch.uint8)
    n_o = batch * heads * num_splits * dim
    off = ((n_o * 4 + 255) // 256) * 256
    return (_f32_view(flat, 0, (batch, heads, num_splits, dim)),
            _f32_view(flat, off, (batch, num_splits, heads)))


def workspace_views_unnorm(workspace, batch: int, heads: int, dim: int, num_splits: int):
    """(ACC [B,H,ns,D], M [B,H,ns], L [B,H,ns]) fp32 views of an
    unnormalised-format workspace, per the layout documented in include/fd.h."""
    import torch
    flat = workspace.view(torch.uint8)
    rows = batch * heads * num_splits
    off_m = ((rows * dim * 4 + 255) // 256) * 256
    off_l = off_m + ((rows * 4 + 255) // 256) * 256
    return (_f32_view(flat, 0, (batch, heads, num_splits, dim)),
            _f32_view(flat, off_m, (batch, heads, num_splits)),
            _f32_view(flat, off_l, (batch, heads, num_splits)))
