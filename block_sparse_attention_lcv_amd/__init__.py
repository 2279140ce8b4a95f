"""Python binding of liblcv_bsa: LongCat-Video block-sparse 3D self-attention on MI355X.

Argument marshalling only: every step of the computation runs in the HIP kernels of the
C-ABI library (include/lcv_bsa.h).  PyTorch provides device memory and streams.  The
library must be built (``python -m block_sparse_attention_lcv_amd._build`` or
``__graft_entry__.build()``); nothing falls back to another implementation when it is
missing.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "liblcv_bsa.so"

ROPE_Q = 1
ROPE_K = 2

STATUS_NAMES = {0: "OK", 1: "ERR_NULL", 2: "ERR_INVALID_ARG", 3: "ERR_SHAPE", 5: "ERR_LAYOUT_MISMATCH",
                6: "ERR_UNSUPPORTED", 7: "ERR_OOM", 8: "ERR_HIP"}

# Every symbol include/lcv_bsa.h declares.
EXPORTED = ("lcv_bsa_layout_query", "lcv_bsa_build_layout", "lcv_bsa_layout_get_info", "lcv_bsa_layout_copy_csr",
            "lcv_bsa_layout_destroy", "lcv_rope3d_apply", "lcv_qk_rmsnorm_rope3d",
            "lcv_qk_rmsnorm_rope3d_backward_workspace", "lcv_qk_rmsnorm_rope3d_backward",
            "lcv_qk_rmsnorm_rope3d_backward_noalloc", "lcv_bsa_forward",
            "lcv_bsa_forward_cached", "lcv_bsa_forward_rows", "lcv_bsa_backward_workspace", "lcv_bsa_backward",
            "lcv_cross_attention",
            "lcv_cross_attention_backward_workspace", "lcv_cross_attention_backward", "lcv_attn_merge",
            "lcv_last_error", "lcv_abi_version")


class LayoutParams(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int32), ("block", ctypes.c_int32), ("local_blocks", ctypes.c_int32),
                ("global_stride", ctypes.c_int32), ("cond_len", ctypes.c_int32)]


class Rope3dGrid(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("W", ctypes.c_int32), ("theta", ctypes.c_float)]


class LayoutInfo(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int32), ("n_blocks", ctypes.c_int32), ("local_blocks", ctypes.c_int32),
                ("global_stride", ctypes.c_int32), ("cond_len", ctypes.c_int32), ("max_row_len", ctypes.c_int32),
                ("nnz", ctypes.c_int64), ("attended_pairs", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class LcvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load liblcv_bsa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise RuntimeError(f"{LIB_PATH} is missing: build it with python -m block_sparse_attention_lcv_amd._build")
    # PyTorch ships its own HIP runtime with the same soname as ROCm's; loading torch first
    # makes the dynamic linker bind this library to that one runtime instead of a second copy.
    import torch  # noqa: F401
    L = ctypes.CDLL(str(LIB_PATH))
    vp, i32, i64, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
    sig = {
        "lcv_bsa_layout_query": (i32, [ctypes.POINTER(LayoutParams), ctypes.POINTER(LayoutInfo)]),
        "lcv_bsa_build_layout": (i32, [ctypes.POINTER(LayoutParams), vp, ctypes.POINTER(vp)]),
        "lcv_bsa_layout_get_info": (i32, [vp, ctypes.POINTER(LayoutInfo)]),
        "lcv_bsa_layout_copy_csr": (i32, [vp, vp, vp, vp]),
        "lcv_bsa_layout_destroy": (None, [vp]),
        "lcv_rope3d_apply": (i32, [vp, vp, i64, i32, i32, ctypes.POINTER(Rope3dGrid), vp]),
        "lcv_qk_rmsnorm_rope3d": (i32, [vp, vp, vp, ctypes.c_float, i64, i32, i32, ctypes.POINTER(Rope3dGrid), vp]),
        "lcv_qk_rmsnorm_rope3d_backward_workspace": (i64, [i64, i32]),
        "lcv_qk_rmsnorm_rope3d_backward": (i32, [vp, vp, vp, ctypes.c_float, i64, i32, i32, ctypes.POINTER(Rope3dGrid),
                                                 vp, vp, vp, i64, vp]),
        "lcv_qk_rmsnorm_rope3d_backward_noalloc": (i32, [vp, vp, vp, ctypes.c_float, i64, i32, i32,
                                                         ctypes.POINTER(Rope3dGrid), vp, vp, vp]),
        "lcv_bsa_forward": (i32, [vp, vp, vp, i32, i32, vp, i32, u32, ctypes.POINTER(Rope3dGrid), vp, vp, vp]),
        "lcv_bsa_forward_cached": (i32, [vp, vp, vp, vp, vp, i32, i32, vp, i32, u32, ctypes.POINTER(Rope3dGrid),
                                         vp, vp, vp]),
        "lcv_bsa_forward_rows": (i32, [vp, vp, vp, i32, i32, vp, i32, u32, ctypes.POINTER(Rope3dGrid), i32, i32, vp, vp,
                                       vp]),
        "lcv_bsa_backward_workspace": (i64, [i32, i32, i32]),
        "lcv_bsa_backward": (i32, [vp, vp, vp, vp, vp, vp, i32, i32, vp, i32, vp, vp, vp, vp, i64, vp]),
        "lcv_cross_attention": (i32, [vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp]),
        "lcv_cross_attention_backward_workspace": (i64, [i32, i32, i32, i32]),
        "lcv_cross_attention_backward": (i32, [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, i64,
                                               vp]),
        "lcv_attn_merge": (i32, [ctypes.POINTER(vp), ctypes.POINTER(vp), i32, i64, vp, vp, vp]),
        "lcv_last_error": (ctypes.c_char_p, []),
        "lcv_abi_version": (i32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(status: int) -> None:
    if status != 0:
        raise LcvError(status, lib().lcv_last_error().decode())


def _params(n_tokens: int, local_blocks: int, global_stride: int, cond_len: int) -> LayoutParams:
    return LayoutParams(n_tokens, 64, local_blocks, global_stride, cond_len)


def layout_query(n_tokens: int, local_blocks: int = 2, global_stride: int = 4, cond_len: int = 0) -> dict:
    """Closed-form layout sizes, computed on the host (no GPU needed)."""
    info = LayoutInfo()
    _check(lib().lcv_bsa_layout_query(ctypes.byref(_params(n_tokens, local_blocks, global_stride, cond_len)),
                                      ctypes.byref(info)))
    return info.as_dict()


def _stream_ptr(stream) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


class Layout:
    """A built block layout (device CSR + the forward kernel's per-workgroup lists)."""

    def __init__(self, n_tokens: int, local_blocks: int = 2, global_stride: int = 4, cond_len: int = 0, stream=None):
        handle = ctypes.c_void_p()
        params = _params(n_tokens, local_blocks, global_stride, cond_len)
        _check(lib().lcv_bsa_build_layout(ctypes.byref(params), _stream_ptr(stream), ctypes.byref(handle)))
        self._h = handle
        info = LayoutInfo()
        _check(lib().lcv_bsa_layout_get_info(self._h, ctypes.byref(info)))
        self.info = info.as_dict()

    @property
    def handle(self) -> ctypes.c_void_p:
        return self._h

    @property
    def n_tokens(self) -> int:
        return self.info["n_tokens"]

    @property
    def cond_len(self) -> int:
        return self.info["cond_len"]

    def csr(self, stream=None):
        """(row_ptr, col_idx) as int32 device tensors (copies)."""
        import torch
        row_ptr = torch.empty(self.info["n_blocks"] + 1, dtype=torch.int32, device="cuda")
        col_idx = torch.empty(max(self.info["nnz"], 1), dtype=torch.int32, device="cuda")
        _check(lib().lcv_bsa_layout_copy_csr(self._h, row_ptr.data_ptr(), col_idx.data_ptr(), _stream_ptr(stream)))
        return row_ptr, col_idx[: self.info["nnz"]]

    def close(self) -> None:
        if self._h:
            lib().lcv_bsa_layout_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def build_layout(n_tokens: int, local_blocks: int = 2, global_stride: int = 4, cond_len: int = 0,
                 stream=None) -> Layout:
    return Layout(n_tokens, local_blocks, global_stride, cond_len, stream)


@dataclass(frozen=True)
class Grid:
    T: int
    H: int
    W: int
    theta: float = 10000.0

    def c(self) -> Rope3dGrid:
        return Rope3dGrid(self.T, self.H, self.W, self.theta)


def _as_grid(grid) -> Grid | None:
    if grid is None or isinstance(grid, Grid):
        return grid
    return Grid(*grid)


def _bf16(t, name: str):
    import torch
    if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous bfloat16 CUDA tensor")
    return t.data_ptr()


def _check_shape(t, shape, name: str) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have the shape {tuple(shape)} (got {tuple(t.shape)})")


def _check_f32(t, shape, name: str) -> None:
    """A float32 output or input the library reads or writes: contiguous, on the GPU, of
    exactly this shape (the library only receives its address)."""
    import torch
    _check_shape(t, shape, name)
    if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 CUDA tensor")


def _check_devices(ref, named) -> None:
    """Every tensor on the device of ref (the library launches on the current device and
    receives raw addresses)."""
    for name, t in named:
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, expected {ref.device}")


def rope3d_apply(x, grid, token_offset: int = 0, out=None, stream=None):
    """3D-RoPE of x[..., n_tokens, 64] (bf16); out may be x for in-place use."""
    import torch
    g = _as_grid(grid)
    if x.shape[-1] != 64:
        raise ValueError("last dimension must be 64")
    y = torch.empty_like(x) if out is None else out
    if y.shape != x.shape:
        raise ValueError("out must have the shape of x")
    n_tokens = x.shape[-2]
    n_outer = x.numel() // (64 * n_tokens) if n_tokens else 0
    _check(lib().lcv_rope3d_apply(_bf16(x, "x"), _bf16(y, "out"), n_outer, n_tokens, token_offset,
                                  ctypes.byref(g.c()), _stream_ptr(stream)))
    return y


def qk_rmsnorm_rope3d(x, gamma, eps: float = 1e-6, grid=None, token_offset: int = 0, out=None, stream=None):
    """RMSNorm of each 64-channel row of x[..., n_tokens, 64] (bf16) with the gain gamma[64]
    (float32 CUDA tensor), then the 3D-RoPE when grid is given; out may be x."""
    import torch
    g = _as_grid(grid)
    if x.shape[-1] != 64:
        raise ValueError("last dimension must be 64")
    if gamma.dtype != torch.float32 or not gamma.is_cuda or not gamma.is_contiguous() or gamma.numel() != 64:
        raise ValueError("gamma must be a contiguous float32 CUDA tensor of 64 values")
    y = torch.empty_like(x) if out is None else out
    if y.shape != x.shape:
        raise ValueError("out must have the shape of x")
    n_tokens = x.shape[-2]
    n_outer = x.numel() // (64 * n_tokens) if n_tokens else 0
    _check(lib().lcv_qk_rmsnorm_rope3d(_bf16(x, "x"), _bf16(y, "out"), gamma.data_ptr(), float(eps), n_outer,
                                       n_tokens, token_offset, ctypes.byref(g.c()) if g is not None else None,
                                       _stream_ptr(stream)))
    return y


def qk_rmsnorm_rope3d_backward(x, dy, gamma, eps: float = 1e-6, grid=None, token_offset: int = 0, dx=None,
                               dgamma=None, workspace=None, stream=None):
    """Gradients (dx, dgamma) of qk_rmsnorm_rope3d(x, gamma, eps, grid, token_offset) for the
    upstream gradient dy (bf16, the shape of x); dx may be x or dy."""
    import torch
    g = _as_grid(grid)
    if x.shape[-1] != 64 or dy.shape != x.shape:
        raise ValueError("x and dy must share the shape [..., n_tokens, 64]")
    if gamma.dtype != torch.float32 or not gamma.is_cuda or not gamma.is_contiguous() or gamma.numel() != 64:
        raise ValueError("gamma must be a contiguous float32 CUDA tensor of 64 values")
    n_tokens = x.shape[-2]
    n_outer = x.numel() // (64 * n_tokens) if n_tokens else 0
    dx = torch.empty_like(x) if dx is None else dx
    if dx.shape != x.shape:
        raise ValueError("dx must have the shape of x")
    dgamma = torch.empty(64, dtype=torch.float32, device=x.device) if dgamma is None else dgamma
    need = int(lib().lcv_qk_rmsnorm_rope3d_backward_workspace(n_outer, n_tokens))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.float32, device=x.device)
    _check(lib().lcv_qk_rmsnorm_rope3d_backward(_bf16(x, "x"), _bf16(dy, "dy"), gamma.data_ptr(), float(eps), n_outer,
                                                n_tokens, token_offset, ctypes.byref(g.c()) if g is not None else None,
                                                _bf16(dx, "dx"), dgamma.data_ptr(), workspace.data_ptr(),
                                                workspace.numel(), _stream_ptr(stream)))
    return dx, dgamma


def qk_rmsnorm_rope3d_backward_noalloc(x, dy, gamma, eps: float = 1e-6, grid=None, token_offset: int = 0, dx=None,
                                       dgamma=None, stream=None):
    """qk_rmsnorm_rope3d_backward with the library's static scratch instead of a workspace (no
    device allocation inside the call when dx and dgamma are given; calls that overlap on one
    GPU race on that scratch)."""
    import torch
    g = _as_grid(grid)
    if x.shape[-1] != 64 or dy.shape != x.shape:
        raise ValueError("x and dy must share the shape [..., n_tokens, 64]")
    if gamma.dtype != torch.float32 or not gamma.is_cuda or not gamma.is_contiguous() or gamma.numel() != 64:
        raise ValueError("gamma must be a contiguous float32 CUDA tensor of 64 values")
    n_tokens = x.shape[-2]
    n_outer = x.numel() // (64 * n_tokens) if n_tokens else 0
    dx = torch.empty_like(x) if dx is None else dx
    if dx.shape != x.shape:
        raise ValueError("dx must have the shape of x")
    dgamma = torch.empty(64, dtype=torch.float32, device=x.device) if dgamma is None else dgamma
    _check_f32(dgamma, (64,), "dgamma")
    _check(lib().lcv_qk_rmsnorm_rope3d_backward_noalloc(
        _bf16(x, "x"), _bf16(dy, "dy"), gamma.data_ptr(), float(eps), n_outer, n_tokens, token_offset,
        ctypes.byref(g.c()) if g is not None else None, _bf16(dx, "dx"), dgamma.data_ptr(), _stream_ptr(stream)))
    return dx, dgamma


def _flags(rope_q: bool, rope_k: bool) -> int:
    return (ROPE_Q if rope_q else 0) | (ROPE_K if rope_k else 0)


def forward(q, k, v, layout: Layout, grid=None, rope_q: bool = True, rope_k: bool = True, out=None, lse=None,
            with_lse: bool = True, stream=None):
    """Block-sparse attention of q, k, v [B, H, N, 64] (bf16).  Returns (out, lse)."""
    import torch
    B, Hh, N, D = q.shape
    if D != 64 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share the shape [B, H, N, 64]")
    if N != layout.n_tokens:
        raise ValueError(f"q holds {N} tokens, the layout {layout.n_tokens}")
    if out is not None:
        _check_shape(out, q.shape, "out")
    if lse is not None:
        _check_f32(lse, (B, Hh, N), "lse")
    _check_devices(q, (("k", k), ("v", v), ("out", out), ("lse", lse)))
    g = _as_grid(grid)
    flags = _flags(rope_q, rope_k) if g is not None else 0
    out = torch.empty_like(q) if out is None else out
    if with_lse and lse is None:
        lse = torch.empty((B, Hh, N), dtype=torch.float32, device=q.device)
    lse_ptr = None if lse is None else lse.data_ptr()
    _check(lib().lcv_bsa_forward(_bf16(q, "q"), _bf16(k, "k"), _bf16(v, "v"), B, Hh, layout.handle,
                                 layout.cond_len, flags, ctypes.byref(g.c()) if g is not None else None,
                                 _bf16(out, "out"), lse_ptr, _stream_ptr(stream)))
    return out, lse


def forward_rows(q_rows, k, v, layout: Layout, row_begin: int, row_end: int, grid=None, rope_q: bool = True,
                 rope_k: bool = True, out=None, lse=None, with_lse: bool = True, stream=None):
    """Rows [row_begin, row_end) of forward(): q_rows [B, H, row_end - row_begin, 64], k, v the
    full [B, H, N, 64] tensors.  Returns (out, lse) of the range's rows."""
    import torch
    B, Hh, M, D = q_rows.shape
    if D != 64 or M != row_end - row_begin:
        raise ValueError(f"q_rows must be [B, H, {row_end - row_begin}, 64]")
    if k.shape != (B, Hh, layout.n_tokens, 64) or v.shape != k.shape:
        raise ValueError(f"k, v must be [B, H, {layout.n_tokens}, 64]")
    if out is not None:
        _check_shape(out, q_rows.shape, "out")
    if lse is not None:
        _check_f32(lse, (B, Hh, M), "lse")
    _check_devices(q_rows, (("k", k), ("v", v), ("out", out), ("lse", lse)))
    g = _as_grid(grid)
    flags = _flags(rope_q, rope_k) if g is not None else 0
    out = torch.empty_like(q_rows) if out is None else out
    if with_lse and lse is None:
        lse = torch.empty((B, Hh, M), dtype=torch.float32, device=q_rows.device)
    _check(lib().lcv_bsa_forward_rows(_bf16(q_rows, "q_rows"), _bf16(k, "k"), _bf16(v, "v"), B, Hh, layout.handle,
                                      layout.cond_len, flags, ctypes.byref(g.c()) if g is not None else None,
                                      row_begin, row_end, _bf16(out, "out"), None if lse is None else lse.data_ptr(),
                                      _stream_ptr(stream)))
    return out, lse


def forward_cached(q_noise, k_noise, v_noise, k_cond, v_cond, layout: Layout, grid=None, rope_q: bool = True,
                   rope_k: bool = True, out=None, lse=None, with_lse: bool = True, stream=None):
    """Noise rows [C, N) with the condition K/V [B, H, C, 64] taken from a cache."""
    import torch
    B, Hh, M, D = q_noise.shape
    if D != 64 or k_noise.shape != q_noise.shape or v_noise.shape != q_noise.shape:
        raise ValueError("q_noise, k_noise, v_noise must share the shape [B, H, N-C, 64]")
    C = layout.cond_len
    if M != layout.n_tokens - C:
        raise ValueError(f"noise tensors must hold N-C = {layout.n_tokens - C} tokens")
    if C > 0 and (k_cond.shape != (B, Hh, C, 64) or v_cond.shape != (B, Hh, C, 64)):
        raise ValueError("k_cond, v_cond must be [B, H, C, 64]")
    if out is not None:
        _check_shape(out, q_noise.shape, "out")
    if lse is not None:
        _check_f32(lse, (B, Hh, M), "lse")
    _check_devices(q_noise, (("k_noise", k_noise), ("v_noise", v_noise), ("k_cond", k_cond if C > 0 else None),
                             ("v_cond", v_cond if C > 0 else None), ("out", out), ("lse", lse)))
    g = _as_grid(grid)
    flags = _flags(rope_q, rope_k) if g is not None else 0
    out = torch.empty_like(q_noise) if out is None else out
    if with_lse and lse is None:
        lse = torch.empty((B, Hh, M), dtype=torch.float32, device=q_noise.device)
    lse_ptr = None if lse is None else lse.data_ptr()
    kc = _bf16(k_cond, "k_cond") if C > 0 else None
    vc = _bf16(v_cond, "v_cond") if C > 0 else None
    _check(lib().lcv_bsa_forward_cached(_bf16(q_noise, "q_noise"), _bf16(k_noise, "k_noise"),
                                        _bf16(v_noise, "v_noise"), kc, vc, B, Hh, layout.handle, C, flags,
                                        ctypes.byref(g.c()) if g is not None else None, _bf16(out, "out"),
                                        lse_ptr, _stream_ptr(stream)))
    return out, lse


def backward(q, k, v, out, lse, dout, layout: Layout, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Gradients (dq, dk, dv) of the block-sparse attention for the upstream gradient dout.
    q, k as they entered the scores (rotated), out and lse [B, H, N] (float32) from forward."""
    import torch
    B, Hh, N, D = q.shape
    for name, t in (("k", k), ("v", v), ("out", out), ("dout", dout)):
        if t.shape != q.shape:
            raise ValueError(f"{name} must have the shape of q [B, H, N, 64]")
    if D != 64 or N != layout.n_tokens:
        raise ValueError(f"q must be [B, H, {layout.n_tokens}, 64]")
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is not None and t.shape != q.shape:
            raise ValueError(f"{name} must have the shape of q")
    if lse.dtype != torch.float32 or not lse.is_cuda or not lse.is_contiguous() or lse.shape != (B, Hh, N):
        raise ValueError("lse must be a contiguous float32 CUDA tensor [B, H, N]")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    _check_devices(q, (("k", k), ("v", v), ("out", out), ("lse", lse), ("dout", dout), ("dq", dq), ("dk", dk),
                       ("dv", dv), ("workspace", workspace)))
    need = backward_workspace(B, Hh, N)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.float32, device=q.device)
    if (workspace.dtype != torch.float32 or not workspace.is_cuda or not workspace.is_contiguous()
            or workspace.numel() < need):
        raise ValueError(f"workspace must be a contiguous float32 CUDA tensor of at least {need} values")
    _check(lib().lcv_bsa_backward(_bf16(q, "q"), _bf16(k, "k"), _bf16(v, "v"), _bf16(out, "out"), lse.data_ptr(),
                                  _bf16(dout, "dout"), B, Hh, layout.handle, layout.cond_len, _bf16(dq, "dq"),
                                  _bf16(dk, "dk"), _bf16(dv, "dv"), workspace.data_ptr(), workspace.numel(),
                                  _stream_ptr(stream)))
    return dq, dk, dv


def backward_workspace(batch: int, heads: int, n_tokens: int) -> int:
    """fp32 values of scratch that backward needs for these sizes."""
    n = lib().lcv_bsa_backward_workspace(batch, heads, n_tokens)
    if n < 0:
        raise ValueError("invalid sizes")
    return n


def cross_attention(q, k, v, kv_lens=None, out=None, lse=None, with_lse: bool = True, stream=None):
    """Cross-attention of video queries q [B, H, N, 64] over text keys/values k, v [B, H, L, 64]
    (bf16); kv_lens: optional int32 CUDA tensor [B] of valid text lengths.  Returns (out, lse)."""
    import torch
    B, Hh, N, D = q.shape
    if D != 64 or k.shape[:2] != (B, Hh) or k.shape[3] != 64 or v.shape != k.shape:
        raise ValueError("q must be [B, H, N, 64] and k, v [B, H, L, 64]")
    L = k.shape[2]
    if kv_lens is not None and (kv_lens.dtype != torch.int32 or not kv_lens.is_cuda or kv_lens.numel() != B
                                or not kv_lens.is_contiguous()):
        raise ValueError("kv_lens must be a contiguous int32 CUDA tensor of B values")
    out = torch.empty_like(q) if out is None else out
    if out.shape != q.shape:
        raise ValueError("out must have the shape of q")
    if lse is not None:
        _check_f32(lse, (B, Hh, N), "lse")
    _check_devices(q, (("k", k), ("v", v), ("out", out), ("lse", lse), ("kv_lens", kv_lens)))
    if with_lse and lse is None:
        lse = torch.empty((B, Hh, N), dtype=torch.float32, device=q.device)
    def ptr(t, name):   # tensors without rows may be empty (NULL)
        p = _bf16(t, name)
        return p if t.numel() else None

    _check(lib().lcv_cross_attention(ptr(q, "q"), ptr(k, "k"), ptr(v, "v"), B, Hh, N, L,
                                     None if kv_lens is None else kv_lens.data_ptr(), ptr(out, "out"),
                                     None if lse is None or lse.numel() == 0 else lse.data_ptr(),
                                     _stream_ptr(stream)))
    return out, lse


def cross_attention_backward_workspace(batch: int, heads: int, n_q: int, kv_len: int) -> int:
    """fp32 values of scratch that cross_attention_backward needs for these sizes."""
    n = lib().lcv_cross_attention_backward_workspace(batch, heads, n_q, kv_len)
    if n < 0:
        raise ValueError("invalid sizes")
    return n


def cross_attention_backward(q, k, v, out, lse, dout, kv_lens=None, dq=None, dk=None, dv=None, workspace=None,
                             stream=None):
    """Gradients (dq, dk, dv) of cross_attention for the upstream gradient dout: q, out, dout
    [B, H, N, 64], k, v [B, H, L, 64] (bf16), lse [B, H, N] (float32) from cross_attention."""
    import torch
    B, Hh, N, D = q.shape
    if D != 64 or k.shape[:2] != (B, Hh) or k.shape[3] != 64 or v.shape != k.shape:
        raise ValueError("q must be [B, H, N, 64] and k, v [B, H, L, 64]")
    L = k.shape[2]
    for name, t in (("out", out), ("dout", dout)):
        if t.shape != q.shape:
            raise ValueError(f"{name} must have the shape of q")
    if lse.dtype != torch.float32 or not lse.is_cuda or not lse.is_contiguous() or lse.shape != (B, Hh, N):
        raise ValueError("lse must be a contiguous float32 CUDA tensor [B, H, N]")
    if kv_lens is not None and (kv_lens.dtype != torch.int32 or not kv_lens.is_cuda or kv_lens.numel() != B
                                or not kv_lens.is_contiguous()):
        raise ValueError("kv_lens must be a contiguous int32 CUDA tensor of B values")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != k.shape:
        raise ValueError("dq must have the shape of q, dk and dv that of k")
    _check_devices(q, (("k", k), ("v", v), ("out", out), ("lse", lse), ("dout", dout), ("kv_lens", kv_lens),
                       ("dq", dq), ("dk", dk), ("dv", dv), ("workspace", workspace)))
    need = cross_attention_backward_workspace(B, Hh, N, L)
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.float32, device=q.device)
    if workspace.dtype != torch.float32 or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous float32 CUDA tensor")
    def ptr(t, name):   # tensors of a side without rows may be empty (NULL)
        p = _bf16(t, name)
        return p if t.numel() else None

    _check(lib().lcv_cross_attention_backward(
        ptr(q, "q"), ptr(k, "k"), ptr(v, "v"), ptr(out, "out"), lse.data_ptr() if lse.numel() else None,
        ptr(dout, "dout"), B, Hh, N, L, None if kv_lens is None else kv_lens.data_ptr(), ptr(dq, "dq"), ptr(dk, "dk"),
        ptr(dv, "dv"), workspace.data_ptr(), workspace.numel(), _stream_ptr(stream)))
    return dq, dk, dv


def attn_merge(outs, lses, out=None, lse=None, with_lse: bool = True, stream=None):
    """Merge attention results over disjoint key sets: outs (bf16 [..., N, 64]) and lses
    (float32 [..., N]) of each part -> (out, lse) of the attention over the union."""
    import torch
    if not 1 <= len(outs) <= 8 or len(lses) != len(outs):
        raise ValueError("1 to 8 parts, one lse per out")
    shape = outs[0].shape
    if shape[-1] != 64:
        raise ValueError("last dimension must be 64")
    for o, l in zip(outs, lses):
        if o.shape != shape or tuple(l.shape) != tuple(shape[:-1]):
            raise ValueError("every part must have the same shape [..., N, 64] with lse [..., N]")
        if l.dtype != torch.float32 or not l.is_cuda or not l.is_contiguous():
            raise ValueError("lse parts must be contiguous float32 CUDA tensors")
    out = torch.empty_like(outs[0]) if out is None else out
    if out.shape != shape:
        raise ValueError("out must have the parts' shape")
    if with_lse and lse is None:
        lse = torch.empty(shape[:-1], dtype=torch.float32, device=outs[0].device)
    rows = outs[0].numel() // 64
    n = len(outs)
    optr = (ctypes.c_void_p * n)(*[_bf16(o, "outs[i]") for o in outs])
    lptr = (ctypes.c_void_p * n)(*[l.data_ptr() for l in lses])
    _check(lib().lcv_attn_merge(optr, lptr, n, rows, _bf16(out, "out"), None if lse is None else lse.data_ptr(),
                                _stream_ptr(stream)))
    return out, lse
