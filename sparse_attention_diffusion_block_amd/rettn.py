"""Python binding of librettn (include/rettn.h): argument marshalling only.

PyTorch supplies device memory and the current HIP stream; every step of the
path runs in the library's gfx950 kernels.  There is no fallback: if the
library is not built, or a call is rejected, an exception is raised.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librettn.so")

RETTN_F32, RETTN_BF16 = 0, 1
MASK_DIAG, MASK_BAND, MASK_COGVIDEO3D, MASK_FULL = 0, 1, 2, 3
RESIDUAL_MASKED, RESIDUAL_DIFFERENCE = 0, 1
EXPORTED = ("rettn_mask_build", "rettn_index_build", "rettn_index_build_sliced", "rettn_dynamic_workspace_bytes",
            "rettn_dynamic_index", "rettn_dynamic_index_noalloc", "rettn_calibrate", "rettn_calibrate_residual",
            "rettn_calibrate_workspace_bytes", "rettn_calibrate_ws", "rettn_sparse", "rettn_sparse_workspace_bytes",
            "rettn_sparse_ws", "rettn_status_str")
STATUS_ESCRATCH = 4
NOALLOC_SCRATCH_BYTES = 32 << 20   # RETTN_NOALLOC_SCRATCH_BYTES


class Desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("L", ctypes.c_int32), ("d", ctypes.c_int32),
                ("block", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64), ("stride_l", ctypes.c_int64)]


class MaskSpec(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("nb", ctypes.c_int32), ("w", ctypes.c_int32),
                ("text_blocks", ctypes.c_int32), ("tshift", ctypes.c_int32)]


class Index(ctypes.Structure):
    _fields_ = [("nqb", ctypes.c_int32), ("nkb", ctypes.c_int32), ("nnz", ctypes.c_int32),
                ("row_ptr", ctypes.c_void_p), ("col_idx", ctypes.c_void_p), ("mask", ctypes.c_void_p),
                ("slices", ctypes.c_int32), ("col_stride", ctypes.c_int32)]


class RettnError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {lib().rettn_status_str(status).decode()}")


_lib = None


def lib():
    """Load librettn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run sparse_attention_diffusion_block_amd.build.build()")
        # torch first: it loads the HIP runtime it ships with, and the library must bind to that
        # same runtime (loaded first, the library would pull in the system one, whose streams and
        # allocations are foreign to torch's)
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        L.rettn_status_str.argtypes = [ctypes.c_int]
        L.rettn_status_str.restype = ctypes.c_char_p
        L.rettn_mask_build.argtypes = [ctypes.POINTER(MaskSpec), vp]
        L.rettn_mask_build.restype = ctypes.c_int
        L.rettn_index_build.argtypes = [vp, i32, i32, vp, vp, ctypes.POINTER(i32), vp]
        L.rettn_index_build.restype = ctypes.c_int
        L.rettn_index_build_sliced.argtypes = [vp, i32, i32, i32, vp, vp, ctypes.POINTER(i32), vp]
        L.rettn_index_build_sliced.restype = ctypes.c_int
        L.rettn_dynamic_workspace_bytes.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(ctypes.c_size_t)]
        L.rettn_dynamic_workspace_bytes.restype = ctypes.c_int
        L.rettn_dynamic_index.argtypes = [ctypes.POINTER(Desc), vp, vp, i32, vp, ctypes.c_size_t, vp, vp, vp, vp]
        L.rettn_dynamic_index.restype = ctypes.c_int
        L.rettn_dynamic_index_noalloc.argtypes = [ctypes.POINTER(Desc), vp, vp, i32, vp, vp, vp, vp]
        L.rettn_dynamic_index_noalloc.restype = ctypes.c_int
        L.rettn_calibrate.argtypes = [ctypes.POINTER(Desc), vp, vp, vp, ctypes.POINTER(Index), vp, vp, vp, vp]
        L.rettn_calibrate.restype = ctypes.c_int
        L.rettn_calibrate_residual.argtypes = [ctypes.POINTER(Desc), vp, vp, vp, ctypes.POINTER(Index), vp, vp, vp,
                                               ctypes.c_int, vp]
        L.rettn_calibrate_residual.restype = ctypes.c_int
        L.rettn_calibrate_workspace_bytes.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(ctypes.c_size_t)]
        L.rettn_calibrate_workspace_bytes.restype = ctypes.c_int
        L.rettn_calibrate_ws.argtypes = [ctypes.POINTER(Desc), vp, vp, vp, ctypes.POINTER(Index), vp, ctypes.c_size_t,
                                         vp, vp, vp, ctypes.c_int, vp]
        L.rettn_calibrate_ws.restype = ctypes.c_int
        L.rettn_sparse.argtypes = [ctypes.POINTER(Desc), vp, vp, vp, ctypes.POINTER(Index), vp, vp,
                                   ctypes.c_float, i32, vp, vp]
        L.rettn_sparse.restype = ctypes.c_int
        L.rettn_sparse_workspace_bytes.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(Index),
                                                   ctypes.POINTER(ctypes.c_size_t)]
        L.rettn_sparse_workspace_bytes.restype = ctypes.c_int
        L.rettn_sparse_ws.argtypes = [ctypes.POINTER(Desc), vp, vp, vp, ctypes.POINTER(Index), vp, vp,
                                      ctypes.c_float, i32, vp, ctypes.c_size_t, vp, vp]
        L.rettn_sparse_ws.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status, what):
    if status != 0:
        raise RettnError(status, what)


def mask_build(kind, nb, w=0, text_blocks=0, tshift=0):
    """Static block mask [nb, nb] (uint8 0/1) built by the library on the host."""
    out = np.zeros((nb, nb), dtype=np.uint8)
    spec = MaskSpec(kind, nb, w, text_blocks, tshift)
    _check(lib().rettn_mask_build(ctypes.byref(spec), out.ctypes.data_as(ctypes.c_void_p)), "rettn_mask_build")
    return out


class BlockIndex:
    """A block mask on the device and its CSR index (kept key blocks per query block).

    `mask` is [nqb, nkb] (one mask for every head) or [S, nqb, nkb] with S = H (one per head) or
    S = B*H (one per (batch, head) slice, slice b*H + h); row_ptr is [S, nqb + 1] and slice s's
    column ids start at s * col_stride.  nnz is the largest slice's count."""

    def __init__(self, mask, row_ptr, col_idx, nnz, block, col_stride=0):
        self.mask, self.row_ptr, self.col_idx, self.nnz, self.block = mask, row_ptr, col_idx, nnz, block
        self.nqb, self.nkb = mask.shape[-2:]
        self.slices = mask.shape[0] if mask.dim() == 3 else 1
        self.col_stride = col_stride

    def c_struct(self):
        return Index(self.nqb, self.nkb, self.nnz, self.row_ptr.data_ptr(), self.col_idx.data_ptr(),
                     self.mask.data_ptr(), self.slices, self.col_stride)


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def index_build(mask, block):
    """Compact a uint8 mask (host array or device tensor) on the GPU; synchronises once.

    [nqb, nkb]: one mask for every (batch, head); [S, nqb, nkb]: one per head (S = H) or per
    (batch, head) slice (S = B*H)."""
    import torch
    m = torch.as_tensor(np.asarray(mask) if not isinstance(mask, torch.Tensor) else mask)
    m = m.to(device="cuda", dtype=torch.uint8).contiguous()
    nnz = ctypes.c_int32(0)
    if m.dim() == 2:
        nqb, nkb = m.shape
        row_ptr = torch.empty(nqb + 1, dtype=torch.int32, device=m.device)
        col_idx = torch.empty(max(nqb * nkb, 1), dtype=torch.int32, device=m.device)
        _check(lib().rettn_index_build(m.data_ptr(), nqb, nkb, row_ptr.data_ptr(), col_idx.data_ptr(),
                                       ctypes.byref(nnz), _stream(m.device)), "rettn_index_build")
        return BlockIndex(m, row_ptr, col_idx, nnz.value, block)
    if m.dim() != 3:
        raise ValueError("mask must be [nqb, nkb] or [slices, nqb, nkb]")
    S, nqb, nkb = m.shape
    row_ptr = torch.empty((S, nqb + 1), dtype=torch.int32, device=m.device)
    col_idx = torch.empty(max(S * nqb * nkb, 1), dtype=torch.int32, device=m.device)
    _check(lib().rettn_index_build_sliced(m.data_ptr(), S, nqb, nkb, row_ptr.data_ptr(), col_idx.data_ptr(),
                                          ctypes.byref(nnz), _stream(m.device)), "rettn_index_build_sliced")
    return BlockIndex(m, row_ptr, col_idx, nnz.value, block, col_stride=nqb * nkb)


def dynamic_workspace_bytes(q, block):
    """Device workspace that dynamic_index needs for tensors shaped like q."""
    n = ctypes.c_size_t(0)
    desc = _desc(q, block)
    _check(lib().rettn_dynamic_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)), "rettn_dynamic_workspace_bytes")
    return n.value


def dynamic_index(q, k, keep, block, workspace=None, out=None):
    """Dynamic block masks of this step's Q and K, one per (batch, head) slice, and their CSR.

    Row a of every slice keeps block a and the keep - 1 other key blocks whose mean key has the
    largest dot product with the block's mean query.  Asynchronous (no host wait).  `workspace`
    (uint8 device tensor of at least dynamic_workspace_bytes) and `out` (a BlockIndex from an
    earlier call of the same shape) may be passed to reuse memory."""
    import torch
    q, k = _prep((q, k))
    B, H, L, d = q.shape
    if keep < 1:
        raise ValueError("keep must be at least 1")
    nb = -(-L // block)
    kk = min(int(keep), nb)
    need = dynamic_workspace_bytes(q, block)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        mask = torch.empty((B * H, nb, nb), dtype=torch.uint8, device=q.device)
        row_ptr = torch.empty((B * H, nb + 1), dtype=torch.int32, device=q.device)
        col_idx = torch.empty(B * H * nb * kk, dtype=torch.int32, device=q.device)
        out = BlockIndex(mask, row_ptr, col_idx, nb * kk, block, col_stride=nb * kk)
    elif out.mask.shape != (B * H, nb, nb) or out.col_stride != nb * kk or out.block != block:
        raise ValueError("`out` was built for another shape or keep")
    desc = _desc(q, block)
    _check(lib().rettn_dynamic_index(ctypes.byref(desc), q.data_ptr(), k.data_ptr(), int(keep), workspace.data_ptr(),
                                     workspace.numel() * workspace.element_size(), out.mask.data_ptr(),
                                     out.row_ptr.data_ptr(), out.col_idx.data_ptr(), _stream(q.device)),
           "rettn_dynamic_index")
    return out


def dynamic_index_noalloc(q, k, keep, block, out):
    """dynamic_index through the entry point that allocates nothing: the block means live in the
    library's static per-GPU scratch.  `out` (a BlockIndex from dynamic_index of the same shape and
    keep) receives the result; nothing is allocated here either.  Calls that overlap on one GPU
    share the scratch and must be ordered by the caller."""
    if not (q.is_cuda and k.is_cuda and q.dim() == 4 and q.shape == k.shape and q.dtype == k.dtype
            and q.stride() == k.stride() and q.stride(3) == 1):
        raise ValueError("Q and K must be CUDA tensors of one [B, H, L, d] layout with d contiguous")
    B, H, L, d = q.shape
    nb = -(-L // block)
    kk = min(int(keep), nb)
    if out.mask.shape != (B * H, nb, nb) or out.col_stride != nb * kk or out.block != block:
        raise ValueError("`out` was built for another shape or keep")
    desc = _desc(q, block)
    _check(lib().rettn_dynamic_index_noalloc(ctypes.byref(desc), q.data_ptr(), k.data_ptr(), int(keep),
                                             out.mask.data_ptr(), out.row_ptr.data_ptr(), out.col_idx.data_ptr(),
                                             _stream(q.device)), "rettn_dynamic_index_noalloc")
    return out


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return RETTN_BF16
    if t.dtype == torch.float32:
        return RETTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16")


def _prep(tensors):
    """Tensors sharing one [B,H,L,d] layout with d contiguous (copied to contiguous otherwise)."""
    ts = list(tensors)
    for t in ts:
        if not t.is_cuda or t.dim() != 4:
            raise ValueError("expected CUDA tensors of shape [B, H, L, d]")
        if t.shape != ts[0].shape or t.dtype != ts[0].dtype:
            raise ValueError("Q, K, V (and R) must share shape and dtype")
    if any(t.stride() != ts[0].stride() for t in ts) or ts[0].stride(3) != 1:
        ts = [t.contiguous() for t in ts]
    return ts


def _check_out(t, like, what):
    """An output tensor the kernels write with `like`'s layout: same device, shape, dtype and strides."""
    if (not t.is_cuda or t.device != like.device or t.shape != like.shape or t.dtype != like.dtype
            or t.stride() != like.stride()):
        raise ValueError(f"{what} must match Q's device, shape, dtype and strides "
                         f"({tuple(like.shape)}, {like.dtype}, strides {like.stride()})")


def _check_rho(rho, q):
    import torch
    if (not rho.is_cuda or rho.device != q.device or rho.dtype != torch.float32 or not rho.is_contiguous()
            or tuple(rho.shape) != tuple(q.shape[:3])):
        raise ValueError("rho must be a contiguous float32 [B, H, L] tensor on Q's device")


def _desc(t, block):
    B, H, L, d = t.shape
    sb, sh, sl, _ = t.stride()
    return Desc(B, H, L, d, block, _dtype_code(t), sb, sh, sl)


def calibrate_workspace_bytes(q, block):
    """Device workspace (bytes) rettn_calibrate_ws needs for tensors shaped and strided like q (0: none)."""
    desc = _desc(q, block)
    n = ctypes.c_size_t(0)
    _check(lib().rettn_calibrate_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)),
           "rettn_calibrate_workspace_bytes")
    return int(n.value)


def calibrate(q, k, v, index, out=None, residual="masked", workspace=None):
    """Full-attention calibration step -> (O, rho, R).  O and R have q's dtype; rho is float32 [B,H,L].

    residual="masked" gives Re-ttention's R (the masked keys' share of O); "difference" gives
    the DiTFastAttn comparator's residual (full minus window attention).

    workspace: None allocates the device workspace rettn_calibrate_ws needs (V in float16); a
    uint8 tensor of at least calibrate_workspace_bytes(q, block) bytes on q's device is used as
    given; False calls rettn_calibrate_residual, which takes no workspace (same results)."""
    import torch
    q, k, v = _prep((q, k, v))
    B, H, L, d = q.shape
    if out is None:
        o = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
        r = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
        rho = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    else:
        o, rho, r = out
        _check_out(o, q, "out[0] (O)")
        _check_out(r, q, "out[2] (R)")
        _check_rho(rho, q)
    desc = _desc(q, index.block)
    idx = index.c_struct()
    kind = {"masked": RESIDUAL_MASKED, "difference": RESIDUAL_DIFFERENCE}[residual]
    if workspace is False:
        _check(lib().rettn_calibrate_residual(ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                              ctypes.byref(idx), o.data_ptr(), rho.data_ptr(), r.data_ptr(), kind,
                                              _stream(q.device)), "rettn_calibrate_residual")
        return o, rho, r
    need = calibrate_workspace_bytes(q, index.block)
    ws_ptr, ws_bytes = None, 0
    if need:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        elif (not workspace.is_cuda or workspace.device != q.device or workspace.dtype != torch.uint8
              or not workspace.is_contiguous() or workspace.numel() < need):
            raise ValueError(f"workspace must be a contiguous uint8 tensor of at least {need} bytes on Q's device")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    _check(lib().rettn_calibrate_ws(ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(idx),
                                    ws_ptr, ws_bytes, o.data_ptr(), rho.data_ptr(), r.data_ptr(), kind,
                                    _stream(q.device)), "rettn_calibrate_ws")
    return o, rho, r


def sparse_workspace_bytes(q, index):
    """Device workspace (bytes) rettn_sparse_ws takes for tensors like q and this index (0: none)."""
    desc = _desc(q, index.block)
    idx = index.c_struct()
    n = ctypes.c_size_t(0)
    _check(lib().rettn_sparse_workspace_bytes(ctypes.byref(desc), ctypes.byref(idx), ctypes.byref(n)),
           "rettn_sparse_workspace_bytes")
    return int(n.value)


def sparse(q, k, v, index, rho, r, lam=0.04, step=1, out=None, workspace=None):
    """Sparse step `step` after a calibration: min(1, rho (1 + lam step)) * window attention + R.

    workspace: None allocates what rettn_sparse_ws takes (V in float16, only for dense 128-token-block
    indices; usually nothing); a uint8 tensor of at least sparse_workspace_bytes(q, index) bytes is
    used as given; False calls rettn_sparse, which takes no workspace (same results)."""
    import torch
    q, k, v, r = _prep((q, k, v, r))
    _check_rho(rho, q)
    if out is not None:
        _check_out(out, q, "out")
    o = out if out is not None else torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    desc = _desc(q, index.block)
    idx = index.c_struct()
    if workspace is False:
        _check(lib().rettn_sparse(ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(idx),
                                  rho.data_ptr(), r.data_ptr(), float(lam), int(step), o.data_ptr(),
                                  _stream(q.device)), "rettn_sparse")
        return o
    need = sparse_workspace_bytes(q, index)
    ws_ptr, ws_bytes = None, 0
    if need:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        elif (not workspace.is_cuda or workspace.device != q.device or workspace.dtype != torch.uint8
              or not workspace.is_contiguous() or workspace.numel() < need):
            raise ValueError(f"workspace must be a contiguous uint8 tensor of at least {need} bytes on Q's device")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    _check(lib().rettn_sparse_ws(ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(idx),
                                 rho.data_ptr(), r.data_ptr(), float(lam), int(step), ws_ptr, ws_bytes, o.data_ptr(),
                                 _stream(q.device)), "rettn_sparse_ws")
    return o
