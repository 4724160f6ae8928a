"""Python binding of the gfx950 FP8 grouped (ragged) matmul library ``libgmm_fp8.so``.

Argument marshalling only: every computation runs in the HIP kernels behind the C ABI
declared in ``include/gmm_fp8.h``.  PyTorch provides device memory and the current
stream; outputs and workspaces are allocated here with ``torch.empty`` and filled by
the library.  There is no fallback: if the shared library is missing, ``load()``
raises, and so does every call.

Functions (same names as the C ABI):
  gmm_fwd, gmm_fwd_noalloc, gmm_dlhs, tgmm_drhs, gmm_dynamic_scales, gmm_quantize, gmm_quantize_rhs,
  gmm_static_scale_from_bound, gmm_workspace_size, gmm_status_string, gmm_version.

fp8 codes travel as ``torch.uint8`` tensors; bf16 values as ``torch.bfloat16``.
"""

import ctypes
import os

__all__ = [
    "load", "library_path", "GmmError", "gmm_fwd", "gmm_fwd_noalloc", "gmm_dlhs", "tgmm_drhs", "gmm_quantize",
    "gmm_dynamic_scales", "gmm_fwd_swiglu", "gmm_fwd_swiglu_fp8",
    "gmm_fwd_swiglu_fp8_subchannel", "gmm_swiglu_bwd",
    "gmm_permute", "gmm_unpermute", "gmm_fwd_local", "gmm_dlhs_local", "tgmm_drhs_local",
    "gmm_fwd_blockwise", "gmm_dlhs_blockwise", "gmm_quantize_subchannel",
    "gmm_quantize_rhs_blockwise", "gmm_quantize_rhs_blockwise_dlhs",
    "gmm_quantize_folded",
    "gmm_quantize_rhs", "gmm_static_scale_from_bound", "gmm_workspace_size",
    "gmm_status_string", "gmm_version", "E4M3", "E5M2", "STATIC", "DYNAMIC", "BLOCK_ROWS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgmm_fp8.so")
_lib = None

# enum values of include/gmm_fp8.h
GMM_OK = 0
E4M3, E5M2 = 0, 1
STATIC, DYNAMIC, DYNAMIC_GIVEN = 0, 1, 2
KIND_BF16, KIND_FP8 = 0, 1
OUT_BF16, OUT_F32 = 0, 1
RHS_KN, RHS_NK = 0, 1
OP_FWD, OP_DLHS, OP_TGMM, OP_FWD_FUSED, OP_DLHS_FUSED, OP_QUANTIZE, OP_FWD_SWIGLU = 0, 1, 2, 3, 4, 5, 6
BLOCK_ROWS = 128

_FMT = {"e4m3": E4M3, "e5m2": E5M2, E4M3: E4M3, E5M2: E5M2}
_SCALING = {"static": STATIC, "dynamic": DYNAMIC, "dynamic_given": DYNAMIC_GIVEN,
            STATIC: STATIC, DYNAMIC: DYNAMIC, DYNAMIC_GIVEN: DYNAMIC_GIVEN}
_LAYOUT = {"kn": RHS_KN, "nk": RHS_NK, RHS_KN: RHS_KN, RHS_NK: RHS_NK}


class GmmError(ValueError):
    """A library call returned an error status."""

    def __init__(self, status, what):
        super().__init__(f"{what}: {gmm_status_string(status)} (status {status})")
        self.status = status


class Operand(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("format", ctypes.c_int32),
                ("scaling", ctypes.c_int32), ("static_scale", ctypes.c_float)]


_P = ctypes.c_void_p
_I32, _I64, _SZ, _F = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
_OPP = ctypes.POINTER(Operand)

_SIGNATURES = {
    "gmm_fwd": [_OPP, _I32, _I32, _I32, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P],
    "gmm_fwd_noalloc": [_OPP, _I32, _I32, _I32, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P],
    "gmm_dlhs": [_OPP, _I32, _I32, _I32, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P],
    "tgmm_drhs": [_OPP, _OPP, _I32, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P],
    "gmm_fwd_swiglu": [_OPP, _I32, _I32, _I32, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P],
    "gmm_fwd_swiglu_fp8": [_OPP, _I32, _I32, _I32, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _OPP, _P, _P, _SZ, _P],
    "gmm_fwd_swiglu_fp8_subchannel": [_OPP, _I32, _I32, _I32, _I64, _I64, _I64, _I32, _P, _P, _P,
                                      _P, _P, _P, _I32, _P, _P, _P, _SZ, _P],
    "gmm_swiglu_bwd": [_I64, _I64, _P, _P, _P, _P],
    "gmm_dlhs_swiglu_bwd": [_OPP, _I32, _I32, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P,
                            _I32, _P, _P, _SZ, _P],
    "gmm_permute_workspace_size": [_I64, _I32, _I32],
    "gmm_fwd_blockwise": [_I32, _I32, _I64, _I64, _I64, _I32, _I64, _P, _P, _P, _P, _P, _P, _P],
    "gmm_dlhs_blockwise": [_I32, _I32, _I64, _I64, _I64, _I32, _I64, _P, _P, _P, _P, _P, _P, _P],
    "gmm_quantize_subchannel": [_I32, _I64, _I64, _I64, _P, _P, _P, _P],
    "gmm_quantize_rhs_blockwise": [_I32, _I32, _I64, _I64, _I64, _I64, _P, _P, _P, _P],
    "gmm_quantize_folded": [_I32, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P],
    "gmm_fwd_local": [_OPP, _I32, _I32, _I32, _I64, _I64, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P],
    "gmm_dlhs_local": [_OPP, _I32, _I32, _I32, _I64, _I64, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P],
    "tgmm_drhs_local": [_OPP, _OPP, _I32, _I64, _I64, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P],
    "gmm_permute": [_I64, _I32, _I32, _P, _I64, _P, _P, _P, _P, _P, _P, _SZ, _P],
    "gmm_unpermute": [_I64, _I32, _I64, _P, _P, _P, _P, _P],
    "gmm_workspace_size": [_I32, _OPP, _OPP, _I64, _I64, _I64, _I32, ctypes.POINTER(_SZ)],
    "gmm_dynamic_scales": [_I32, _I64, _I64, _P, _P, _P, _SZ, _P],
    "gmm_quantize": [_OPP, _I64, _I64, _P, _P, _P, _P, _SZ, _P],
    "gmm_quantize_rhs": [_I32, _I32, _I32, _I64, _I64, _I64, _P, _P, _P, _P],
    "gmm_static_scale_from_bound": [_F, _F, _I32, ctypes.POINTER(_F)],
    "gmm_status_string": [_I32],
    "gmm_version": [],
}
EXPORTED = tuple(_SIGNATURES)


def library_path():
    return _LIB_PATH


def load(path=None):
    """Load (once) and return the shared library; raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} is missing: build it with `python -m fp8_grouped_gemm_ragged_amd.build` "
            "(there is no fallback implementation)")
    # torch first: the library then binds to the HIP runtime torch has loaded (the one its
    # tensors and streams live in), not to a second copy that would reject torch's streams
    import torch  # noqa: F401

    lib = ctypes.CDLL(p)
    for name, args in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = (ctypes.c_char_p if name in ("gmm_status_string", "gmm_version") else
                      ctypes.c_size_t if name == "gmm_permute_workspace_size" else ctypes.c_int32)
    _lib = lib
    return lib


def gmm_status_string(status):
    return load().gmm_status_string(int(status)).decode()


def gmm_version():
    return load().gmm_version().decode()


def _check(status, what):
    if status != GMM_OK:
        raise GmmError(status, what)


def _operand(kind, fmt, scaling, static_scale):
    return Operand(kind, _FMT[fmt], _SCALING[scaling],
                   float(static_scale) if static_scale is not None else 0.0)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, dtype, name, ndim=None):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")


def _shape(t, shape, name):
    """Reject a tensor whose shape differs from the one the call reads or writes: the C ABI
    sees only pointers, so an undersized buffer would be accessed past its end."""
    if tuple(t.shape) != tuple(int(d) for d in shape):
        raise ValueError(f"{name} must have shape {tuple(int(d) for d in shape)}, got {tuple(t.shape)}")


def _block_scales(t, rows, name):
    """Per-128-row-block scales: a 1-D f32 tensor with at least ceil(rows / 128) entries."""
    import torch

    _need(t, torch.float32, name, 1)
    if t.shape[0] < _nblocks(rows):
        raise ValueError(f"{name} needs {_nblocks(rows)} block scales for {rows} rows, got {t.shape[0]}")


def _group_sizes(gs, G, name="group_sizes"):
    if gs.shape[0] != G:
        raise ValueError(f"{name} must hold one size per expert ({G}), got {gs.shape[0]}")


def gmm_static_scale_from_bound(lo, hi, fmt="e4m3"):
    """Per-tensor scale of a fixed symmetric range [lo, hi] = [-b, b]: RNE(b / qmax)."""
    out = _F()
    _check(load().gmm_static_scale_from_bound(float(lo), float(hi), _FMT[fmt], ctypes.byref(out)),
           "gmm_static_scale_from_bound")
    return out.value


def gmm_workspace_size(op, a_fmt, a_scaling, rows, cols_a=0, cols_b=0, b_fmt="e5m2",
                       b_scaling="dynamic", a_kind=KIND_BF16, static_scale=1.0, groups=1):
    a = _operand(a_kind, a_fmt, a_scaling, static_scale)
    b = _operand(KIND_BF16, b_fmt, b_scaling, static_scale)
    n = _SZ()
    _check(load().gmm_workspace_size(int(op), ctypes.byref(a), ctypes.byref(b), int(rows),
                                     int(cols_a), int(cols_b), int(groups), ctypes.byref(n)),
           "gmm_workspace_size")
    return n.value


def _workspace(nbytes, device):
    import torch

    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device) if nbytes else None


def _nblocks(rows):
    return (rows + BLOCK_ROWS - 1) // BLOCK_ROWS


def _gemm(cname, a, rhs, rhs_scales, group_sizes, fmt, scaling, static_scale, a_scales,
          rhs_layout, out_dtype, out, contraction_dim, out_cols, fused, group_offset=None,
          gu=None, gu_scales=None, gu_fmt=0):
    import torch

    lib = load()
    prequant = a.dtype == torch.uint8
    _need(a, torch.uint8 if prequant else torch.bfloat16, "lhs/grad", 2)
    _need(rhs, torch.uint8, "rhs", 3)
    _need(rhs_scales, torch.float32, "rhs_scales", 2)
    _need(group_sizes, torch.int32, "group_sizes", 1)
    M = a.shape[0]
    G = rhs.shape[0]
    K_or_N = a.shape[1]
    # logical (K, N) of the weight from its layout
    if _LAYOUT[rhs_layout] == RHS_KN:
        K, N = rhs.shape[1], rhs.shape[2]
    else:
        N, K = rhs.shape[1], rhs.shape[2]
    if K_or_N != (K if contraction_dim == "K" else N):
        raise ValueError("operand width does not match the rhs contraction dimension")
    odt = torch.float32 if out_dtype == torch.float32 else torch.bfloat16
    n_out = N if out_cols == "N" else K
    _shape(rhs_scales, (G, n_out), "rhs_scales")
    if group_offset is None:
        _group_sizes(group_sizes, G)
    elif not 0 <= int(group_offset) <= group_sizes.shape[0] - G:
        raise ValueError("the local window group_offset .. group_offset + G must lie inside group_sizes")
    # with gu (the SwiGLU backward in the dlhs epilogue) the output is d_gu [M, 2 I], bf16
    out_w = n_out
    if gu is not None:
        if odt != torch.bfloat16:
            raise ValueError("the SwiGLU backward writes bf16")
        _need(gu, torch.bfloat16, "gu", 2)
        _shape(gu, (M, 2 * n_out), "gu")
        out_w = 2 * n_out
    if out is None:
        out = torch.empty((M, out_w), dtype=odt, device=a.device)
    else:
        _need(out, odt, "out", 2)
        _shape(out, (M, out_w), "out")
    op = _operand(KIND_FP8 if prequant else KIND_BF16, fmt, scaling, static_scale)
    mode = _SCALING[scaling]
    if mode != STATIC and a_scales is None:
        if prequant or mode == DYNAMIC_GIVEN:
            raise ValueError("this recipe needs the operand's block scales as an input")
        a_scales = torch.empty(_nblocks(M), dtype=torch.float32, device=a.device)
    if a_scales is not None:
        _block_scales(a_scales, M, "scales")
    ws_n = _SZ()
    if cname == "gmm_fwd":
        wop = OP_FWD_FUSED if fused else OP_FWD
    else:
        wop = OP_DLHS_FUSED if fused else OP_DLHS
    _check(lib.gmm_workspace_size(wop, ctypes.byref(op), ctypes.byref(op), M, K_or_N, n_out,
                                  G, ctypes.byref(ws_n)), "gmm_workspace_size")
    ws = _workspace(ws_n.value, a.device)
    odt_code = OUT_F32 if odt == torch.float32 else OUT_BF16
    if gu is not None:
        _check(lib.gmm_dlhs_swiglu_bwd(ctypes.byref(op), E4M3, _LAYOUT[rhs_layout], M, K, N, G,
                                       _ptr(a), _ptr(a_scales), _ptr(rhs), _ptr(rhs_scales),
                                       _ptr(group_sizes), _ptr(gu), _ptr(out), int(gu_fmt),
                                       _ptr(gu_scales), _ptr(ws), ws_n.value, _stream()),
               "gmm_dlhs_swiglu_bwd")
    elif group_offset is None:
        _check(getattr(lib, cname)(ctypes.byref(op), E4M3, _LAYOUT[rhs_layout], odt_code, M, K, N,
                                   G, _ptr(a), _ptr(a_scales), _ptr(rhs), _ptr(rhs_scales),
                                   _ptr(group_sizes), _ptr(out), _ptr(ws), ws_n.value, _stream()),
               cname)
    else:
        # local-expert window: rhs holds the G experts from group_offset on
        _check(getattr(lib, cname + "_local")(
            ctypes.byref(op), E4M3, _LAYOUT[rhs_layout], odt_code, M, K, N, group_sizes.shape[0],
            int(group_offset), G, _ptr(a), _ptr(a_scales), _ptr(rhs), _ptr(rhs_scales),
            _ptr(group_sizes), _ptr(out), _ptr(ws), ws_n.value, _stream()), cname + "_local")
    return out, a_scales


def gmm_fwd(lhs, rhs, rhs_scales, group_sizes, *, lhs_format="e4m3", lhs_scaling="dynamic",
            static_scale=None, lhs_scales=None, rhs_layout="nk", out_dtype=None, out=None,
            return_scales=False, fused=False):
    """Forward grouped matmul: out[M, N] = q(lhs)[rows of g] . rhs[g] (scales applied).

    lhs: bf16 [M, K] (quantized in-kernel) or uint8 fp8 codes [M, K] (pre-quantized,
    then ``lhs_scales`` holds its block scales when dynamic).  lhs_scaling "static",
    "dynamic" (block scales computed by the call; returned with return_scales) or
    "dynamic_given" (block scales from an earlier call in ``lhs_scales``).  rhs: uint8 codes,
    [G, N, K] for rhs_layout "nk" or [G, K, N] for "kn"; rhs_scales f32 [G, N].
    fused=True hands the call only the workspace of the in-kernel quantization route
    (a bf16 lhs is then quantized inside the product kernel even for wide outputs).
    """
    o, s = _gemm("gmm_fwd", lhs, rhs, rhs_scales, group_sizes, lhs_format, lhs_scaling,
                 static_scale, lhs_scales, rhs_layout, out_dtype, out, "K", "N", fused)
    return (o, s) if return_scales else o


def gmm_fwd_noalloc(lhs, rhs, rhs_scales, group_sizes, *, lhs_format="e4m3",
                    lhs_scaling="dynamic", static_scale=None, lhs_scales=None, rhs_layout="nk",
                    out_dtype=None, out=None):
    """gmm_fwd without a workspace: the library's device scratch array holds the dynamic
    scales' abs-max partials (M <= GMM_NOALLOC_MAX_ROWS).  With `out` (and `lhs_scales`
    when the recipe needs or returns them) given, nothing is allocated here either."""
    import torch

    lib = load()
    prequant = lhs.dtype == torch.uint8
    _need(lhs, torch.uint8 if prequant else torch.bfloat16, "lhs", 2)
    _need(rhs, torch.uint8, "rhs", 3)
    _need(rhs_scales, torch.float32, "rhs_scales", 2)
    _need(group_sizes, torch.int32, "group_sizes", 1)
    M, K = lhs.shape
    G = rhs.shape[0]
    if _LAYOUT[rhs_layout] == RHS_KN:
        Kw, N = rhs.shape[1], rhs.shape[2]
    else:
        N, Kw = rhs.shape[1], rhs.shape[2]
    if Kw != K:
        raise ValueError("operand width does not match the rhs contraction dimension")
    _shape(rhs_scales, (G, N), "rhs_scales")
    _group_sizes(group_sizes, G)
    odt = torch.float32 if out_dtype == torch.float32 else torch.bfloat16
    if out is None:
        out = torch.empty((M, N), dtype=odt, device=lhs.device)
    else:
        _need(out, odt, "out", 2)
        _shape(out, (M, N), "out")
    mode = _SCALING[lhs_scaling]
    if mode != STATIC and (prequant or mode == DYNAMIC_GIVEN) and lhs_scales is None:
        raise ValueError("this recipe needs the operand's block scales as an input")
    if lhs_scales is not None:
        _block_scales(lhs_scales, M, "scales")
    op = _operand(KIND_FP8 if prequant else KIND_BF16, lhs_format, lhs_scaling, static_scale)
    _check(lib.gmm_fwd_noalloc(ctypes.byref(op), E4M3, _LAYOUT[rhs_layout],
                               OUT_F32 if odt == torch.float32 else OUT_BF16, M, K, N, G,
                               _ptr(lhs), _ptr(lhs_scales), _ptr(rhs), _ptr(rhs_scales),
                               _ptr(group_sizes), _ptr(out), _stream()), "gmm_fwd_noalloc")
    return out


def gmm_fwd_local(lhs, rhs, rhs_scales, group_sizes, group_offset, *, lhs_format="e4m3",
                  lhs_scaling="dynamic", static_scale=None, lhs_scales=None, rhs_layout="nk",
                  out_dtype=None, out=None, return_scales=False, fused=False):
    """gmm_fwd over a local-expert window: group_sizes has every expert, rhs / rhs_scales the
    rhs.shape[0] local ones from group_offset on; rows of other experts come out zero."""
    o, s = _gemm("gmm_fwd", lhs, rhs, rhs_scales, group_sizes, lhs_format, lhs_scaling,
                 static_scale, lhs_scales, rhs_layout, out_dtype, out, "K", "N", fused,
                 group_offset)
    return (o, s) if return_scales else o


def gmm_dlhs_local(grad, rhs, rhs_scales, group_sizes, group_offset, *, grad_format="e5m2",
                   grad_scaling="dynamic", static_scale=None, grad_scales=None,
                   rhs_layout="kn", out_dtype=None, out=None, return_scales=False, fused=False):
    """gmm_dlhs over a local-expert window (as gmm_fwd_local)."""
    o, s = _gemm("gmm_dlhs", grad, rhs, rhs_scales, group_sizes, grad_format, grad_scaling,
                 static_scale, grad_scales, rhs_layout, out_dtype, out, "N", "K", fused,
                 group_offset)
    return (o, s) if return_scales else o


def gmm_dlhs(grad, rhs, rhs_scales, group_sizes, *, grad_format="e5m2", grad_scaling="dynamic",
             static_scale=None, grad_scales=None, rhs_layout="kn", out_dtype=None, out=None,
             return_scales=False, fused=False):
    """lhs gradient: dlhs[M, K] = q(grad)[rows of g] . rhs[g]^T; rhs_scales f32 [G, K].
    fused: as for gmm_fwd."""
    o, s = _gemm("gmm_dlhs", grad, rhs, rhs_scales, group_sizes, grad_format, grad_scaling,
                 static_scale, grad_scales, rhs_layout, out_dtype, out, "N", "K", fused)
    return (o, s) if return_scales else o


def gmm_dlhs_swiglu_bwd(grad, rhs, rhs_scales, group_sizes, gu, *, grad_format="e5m2",
                        grad_scaling="dynamic", static_scale=None, grad_scales=None,
                        rhs_layout="kn", out=None, return_scales=False, fused=False,
                        d_gu_format=None):
    """The down projection's dlhs with the SwiGLU backward in its epilogue: d_gu [M, 2I]
    bf16 = gmm_swiglu_bwd(gmm_dlhs(grad, rhs, ...) in bf16, gu), bit for bit, without the
    [M, I] dh in between.  rhs: the down weight's dlhs copy ([G, I, H] for "kn"),
    rhs_scales f32 [G, I]; gu bf16 [M, 2I] from gmm_fwd_swiglu.  With d_gu_format ("e4m3"
    or "e5m2") the call also returns d_gu's dynamic 128-row block scales (those
    gmm_dynamic_scales gives on d_gu): (d_gu, scales); return_scales appends the grad's."""
    import torch

    gsc, fmt = None, 0
    if d_gu_format is not None:
        fmt = _FMT[d_gu_format]
        gsc = torch.empty(_nblocks(grad.shape[0]), dtype=torch.float32, device=grad.device)
    o, s = _gemm("gmm_dlhs", grad, rhs, rhs_scales, group_sizes, grad_format, grad_scaling,
                 static_scale, grad_scales, rhs_layout, None, out, "N", "K", fused, gu=gu,
                 gu_scales=gsc, gu_fmt=fmt)
    r = (o,) if gsc is None else (o, gsc)
    if return_scales:
        r = r + (s,)
    return r[0] if len(r) == 1 else r


def tgmm_drhs_local(lhs, grad, group_sizes, group_offset, num_local, **kw):
    """tgmm_drhs over a local-expert window: drhs [num_local, K, N] for the experts
    group_offset .. group_offset + num_local - 1 of group_sizes."""
    return tgmm_drhs(lhs, grad, group_sizes, _window=(int(group_offset), int(num_local)), **kw)


def tgmm_drhs(lhs, grad, group_sizes, *, lhs_format="e4m3", lhs_scaling="dynamic",
              lhs_static_scale=None, lhs_scales=None, grad_format="e5m2",
              grad_scaling="dynamic", grad_static_scale=None, grad_scales=None,
              out_dtype=None, out=None, return_scales=False, _window=None):
    """Weight gradient: drhs[g] = q(lhs)_g^T . q(grad)_g, [G, K, N]; empty groups give zeros.

    lhs / grad are bf16 values, or uint8 fp8 codes quantized beforehand (then their
    block scales, or the static scale, are an input)."""
    import torch

    lib = load()
    a_codes = isinstance(lhs, torch.Tensor) and lhs.dtype == torch.uint8
    g_codes = isinstance(grad, torch.Tensor) and grad.dtype == torch.uint8
    _need(lhs, torch.uint8 if a_codes else torch.bfloat16, "lhs", 2)
    _need(grad, torch.uint8 if g_codes else torch.bfloat16, "grad", 2)
    _need(group_sizes, torch.int32, "group_sizes", 1)
    M, K = lhs.shape
    if grad.shape[0] != M:
        raise ValueError("lhs and grad must have the same number of rows")
    N = grad.shape[1]
    G_total = group_sizes.shape[0]
    offset, G = _window if _window else (0, G_total)
    if not (G >= 1 and 0 <= offset <= G_total - G):
        raise ValueError("the local window group_offset .. group_offset + num_local must lie inside group_sizes")
    odt = torch.float32 if out_dtype == torch.float32 else torch.bfloat16
    if out is None:
        out = torch.empty((G, K, N), dtype=odt, device=lhs.device)
    else:
        _need(out, odt, "out", 3)
        _shape(out, (G, K, N), "out")
    aop = _operand(KIND_FP8 if a_codes else KIND_BF16, lhs_format, lhs_scaling, lhs_static_scale)
    bop = _operand(KIND_FP8 if g_codes else KIND_BF16, grad_format, grad_scaling, grad_static_scale)
    def scales_for(mode, given, codes):
        if _SCALING[mode] == DYNAMIC_GIVEN or (codes and _SCALING[mode] == DYNAMIC):
            if given is None:
                raise ValueError("this recipe needs the operand's block scales as an input")
            _block_scales(given, M, "scales")
            return given
        if _SCALING[mode] == DYNAMIC:
            if given is not None:
                _block_scales(given, M, "scales")
                return given
            return torch.empty(_nblocks(M), dtype=torch.float32, device=lhs.device)
        return None

    sa = scales_for(lhs_scaling, lhs_scales, a_codes)
    sg = scales_for(grad_scaling, grad_scales, g_codes)
    ws_n = _SZ()
    _check(lib.gmm_workspace_size(OP_TGMM, ctypes.byref(aop), ctypes.byref(bop), M, K, N, G,
                                  ctypes.byref(ws_n)), "gmm_workspace_size")
    ws = _workspace(ws_n.value, lhs.device)
    odt_code = OUT_F32 if odt == torch.float32 else OUT_BF16
    if _window:
        _check(lib.tgmm_drhs_local(ctypes.byref(aop), ctypes.byref(bop), odt_code, M, K, N, G_total,
                                   offset, G, _ptr(lhs), _ptr(sa), _ptr(grad), _ptr(sg),
                                   _ptr(group_sizes), _ptr(out), _ptr(ws), ws_n.value, _stream()),
               "tgmm_drhs_local")
    else:
        _check(lib.tgmm_drhs(ctypes.byref(aop), ctypes.byref(bop), odt_code, M, K, N, G, _ptr(lhs),
                             _ptr(sa), _ptr(grad), _ptr(sg), _ptr(group_sizes), _ptr(out),
                             _ptr(ws), ws_n.value, _stream()), "tgmm_drhs")
    return (out, sa, sg) if return_scales else out


def gmm_fwd_swiglu(lhs, rhs, rhs_scales, group_sizes, *, lhs_format="e4m3",
                   lhs_scaling="dynamic", static_scale=None, lhs_scales=None, out_dtype=None,
                   out=None, gu=False, return_scales=False):
    """Merged gate|up forward with SwiGLU: h[M, I] = silu(x[:, :I]) * x[:, I:] where x is the
    gmm_fwd product over rhs [G, 2I, K] (layout "nk") with rhs_scales [G, 2I].

    lhs: bf16 [M, K] (quantized once in the call) or uint8 codes (then lhs_scales holds its
    block scales when dynamic).  gu=True also returns x itself ([M, 2I], the backward's
    input); returns h, or (h, x) with gu=True, with the lhs scales appended when
    return_scales."""
    return _swiglu_fwd(lhs, rhs, rhs_scales, group_sizes, lhs_format, lhs_scaling,
                       static_scale, lhs_scales, out_dtype, out, gu, return_scales, None)


def gmm_fwd_swiglu_fp8(lhs, rhs, rhs_scales, group_sizes, h_scale, *, h_format="e4m3",
                       lhs_format="e4m3", lhs_scaling="dynamic", static_scale=None,
                       lhs_scales=None, gu_dtype=None, out=None, gu=False,
                       return_scales=False):
    """gmm_fwd_swiglu with h returned as uint8 fp8 codes [M, I] (format h_format) under the
    static per-tensor scale h_scale: code = fp8(clamp(RNE_f32(h * RNE_f32(1/h_scale)))).
    The codes feed gmm_fwd(h_codes, ..., lhs_scaling="static", static_scale=h_scale).
    gu=True also returns the product x in gu_dtype (bf16 unless torch.float32)."""
    return _swiglu_fwd(lhs, rhs, rhs_scales, group_sizes, lhs_format, lhs_scaling,
                       static_scale, lhs_scales, gu_dtype, out, gu, return_scales,
                       (h_format, h_scale))


def gmm_fwd_swiglu_fp8_subchannel(lhs, rhs, rhs_scales, group_sizes, *, h_format="e4m3",
                                  lhs_format="e4m3", lhs_scaling="dynamic", static_scale=None,
                                  lhs_scales=None, gu_dtype=None, out=None, h_scales=None,
                                  gu=False, return_scales=False):
    """gmm_fwd_swiglu with h returned as uint8 fp8 codes [M, I] under dynamic scales f32
    [M, I/128], one per row and block of 128 channels (s = RNE(amax / qmax) over the
    block's float32 |h|).  Returns (h_codes, h_scales[, gu][, lhs_scales]).  The pair
    feeds gmm_fwd_blockwise(h_codes, h_scales, ..., bk=128) as its sub-channel lhs."""
    import torch

    I = rhs.shape[1] // 2
    if h_scales is None:
        h_scales = torch.empty((lhs.shape[0], I // 128), dtype=torch.float32, device=lhs.device)
    else:
        _need(h_scales, torch.float32, "h_scales", 2)
        _shape(h_scales, (lhs.shape[0], I // 128), "h_scales")
    res = _swiglu_fwd(lhs, rhs, rhs_scales, group_sizes, lhs_format, lhs_scaling,
                      static_scale, lhs_scales, gu_dtype, out, gu, return_scales,
                      (h_format, None), h_scales)
    res = res if isinstance(res, tuple) else (res,)
    return (res[0], h_scales) + res[1:]


def _swiglu_fwd(lhs, rhs, rhs_scales, group_sizes, lhs_format, lhs_scaling, static_scale,
                lhs_scales, out_dtype, out, gu, return_scales, h_fp8, h_scales=None):
    import torch

    lib = load()
    prequant = lhs.dtype == torch.uint8
    _need(lhs, torch.uint8 if prequant else torch.bfloat16, "lhs", 2)
    _need(rhs, torch.uint8, "rhs", 3)
    _need(rhs_scales, torch.float32, "rhs_scales", 2)
    _need(group_sizes, torch.int32, "group_sizes", 1)
    M, K = lhs.shape
    G, N2 = rhs.shape[0], rhs.shape[1]
    if rhs.shape[2] != K or N2 % 2:
        raise ValueError("rhs must be [G, 2I, K] codes matching the lhs width")
    I = N2 // 2
    _shape(rhs_scales, (G, N2), "rhs_scales")
    _group_sizes(group_sizes, G)
    odt = torch.float32 if out_dtype == torch.float32 else torch.bfloat16
    hdt = torch.uint8 if h_fp8 else odt
    if out is None:
        out = torch.empty((M, I), dtype=hdt, device=lhs.device)
    else:
        _need(out, hdt, "out", 2)
        _shape(out, (M, I), "out")
    x = torch.empty((M, N2), dtype=odt, device=lhs.device) if gu else None
    op = _operand(KIND_FP8 if prequant else KIND_BF16, lhs_format, lhs_scaling, static_scale)
    mode = _SCALING[lhs_scaling]
    if mode != STATIC and lhs_scales is None:
        if prequant or mode == DYNAMIC_GIVEN:
            raise ValueError("this recipe needs the operand's block scales as an input")
        lhs_scales = torch.empty(_nblocks(M), dtype=torch.float32, device=lhs.device)
    if lhs_scales is not None:
        _block_scales(lhs_scales, M, "scales")
    ws_n = _SZ()
    _check(lib.gmm_workspace_size(OP_FWD_SWIGLU, ctypes.byref(op), ctypes.byref(op), M, K, N2, 1,
                                  ctypes.byref(ws_n)), "gmm_workspace_size")
    ws = _workspace(ws_n.value, lhs.device)
    odt_code = OUT_F32 if odt == torch.float32 else OUT_BF16
    head = (ctypes.byref(op), E4M3, RHS_NK, odt_code, M, K, I, G, _ptr(lhs), _ptr(lhs_scales),
            _ptr(rhs), _ptr(rhs_scales), _ptr(group_sizes), _ptr(x))
    if h_scales is not None:
        _check(lib.gmm_fwd_swiglu_fp8_subchannel(*head, _FMT[h_fp8[0]], _ptr(out), _ptr(h_scales),
                                                 _ptr(ws), ws_n.value, _stream()),
               "gmm_fwd_swiglu_fp8_subchannel")
    elif h_fp8:
        hop = _operand(KIND_FP8, h_fp8[0], "static", h_fp8[1])
        _check(lib.gmm_fwd_swiglu_fp8(*head, ctypes.byref(hop), _ptr(out), _ptr(ws), ws_n.value,
                                      _stream()), "gmm_fwd_swiglu_fp8")
    else:
        _check(lib.gmm_fwd_swiglu(*head, _ptr(out), _ptr(ws), ws_n.value, _stream()),
               "gmm_fwd_swiglu")
    res = (out, x) if gu else (out,)
    if return_scales:
        res = res + (lhs_scales,)
    return res if len(res) > 1 else res[0]


def gmm_swiglu_bwd(dh, gu, out=None):
    """d_gu [M, 2I] bf16 = [dL/dg | dL/du] of h = silu(g) * u, from dh [M, I] and gu = [g | u]."""
    import torch

    lib = load()
    _need(dh, torch.bfloat16, "dh", 2)
    _need(gu, torch.bfloat16, "gu", 2)
    M, I = dh.shape
    if tuple(gu.shape) != (M, 2 * I):
        raise ValueError("gu must be [M, 2I] for dh [M, I]")
    if out is None:
        out = torch.empty((M, 2 * I), dtype=torch.bfloat16, device=dh.device)
    else:
        _need(out, torch.bfloat16, "out", 2)
        _shape(out, (M, 2 * I), "out")
    _check(lib.gmm_swiglu_bwd(M, I, _ptr(dh), _ptr(gu), _ptr(out), _stream()), "gmm_swiglu_bwd")
    return out


def gmm_dynamic_scales(x, fmt="e4m3"):
    """Per-128-row-block scales of a bf16 matrix [R, C] (the abs-max prepass alone)."""
    import torch

    lib = load()
    _need(x, torch.bfloat16, "x", 2)
    R, C = x.shape
    scales = torch.empty(_nblocks(R), dtype=torch.float32, device=x.device)
    op = _operand(KIND_BF16, fmt, "dynamic", None)
    ws_n = _SZ()
    _check(lib.gmm_workspace_size(OP_QUANTIZE, ctypes.byref(op), ctypes.byref(op), R, C, 0, 1,
                                  ctypes.byref(ws_n)), "gmm_workspace_size")
    ws = _workspace(ws_n.value, x.device)
    _check(lib.gmm_dynamic_scales(_FMT[fmt], R, C, _ptr(x), _ptr(scales), _ptr(ws), ws_n.value,
                                  _stream()), "gmm_dynamic_scales")
    return scales


def gmm_quantize(x, fmt="e4m3", scaling="dynamic", static_scale=None, scales=None):
    """Stand-alone quantization of bf16 [R, C] -> (uint8 codes [R, C], f32 scales or None).

    scaling "dynamic_given" takes the block scales in ``scales``."""
    import torch

    lib = load()
    _need(x, torch.bfloat16, "x", 2)
    R, C = x.shape
    op = _operand(KIND_BF16, fmt, scaling, static_scale)
    codes = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    mode = _SCALING[scaling]
    if mode == DYNAMIC_GIVEN and scales is None:
        raise ValueError("dynamic_given needs the block scales")
    if mode == DYNAMIC and scales is None:
        scales = torch.empty(_nblocks(R), dtype=torch.float32, device=x.device)
    if scales is not None and mode != STATIC:
        _block_scales(scales, R, "scales")
    ws_n = _SZ()
    _check(lib.gmm_workspace_size(OP_QUANTIZE, ctypes.byref(op), ctypes.byref(op), R, C, 0, 1,
                                  ctypes.byref(ws_n)), "gmm_workspace_size")
    ws = _workspace(ws_n.value, x.device)
    _check(lib.gmm_quantize(ctypes.byref(op), R, C, _ptr(x), _ptr(codes), _ptr(scales), _ptr(ws),
                            ws_n.value, _stream()), "gmm_quantize")
    return codes, scales


def gmm_quantize_rhs(w, fmt="e4m3", channel_axis=0, layout="kn"):
    """Per-channel quantization of a bf16 weight [G, K, N].

    channel_axis 0 -> scales [G, N] (forward); 1 -> scales [G, K] (dlhs).
    layout "kn" -> codes [G, K, N]; "nk" -> codes [G, N, K].
    """
    import torch

    lib = load()
    _need(w, torch.bfloat16, "w", 3)
    G, K, N = w.shape
    shape = (G, K, N) if _LAYOUT[layout] == RHS_KN else (G, N, K)
    codes = torch.empty(shape, dtype=torch.uint8, device=w.device)
    scales = torch.empty((G, N) if channel_axis == 0 else (G, K), dtype=torch.float32, device=w.device)
    _check(lib.gmm_quantize_rhs(_FMT[fmt], int(channel_axis), _LAYOUT[layout], G, K, N, _ptr(w),
                                _ptr(codes), _ptr(scales), _stream()), "gmm_quantize_rhs")
    return codes, scales


def gmm_permute(expert_ids, num_groups, x=None, x_perm=None):
    """Sort token slots by expert: expert_ids int32 [T, k] (ids outside [0, num_groups) are
    dropped).  Returns (group_sizes [G], row_of_slot [T, k], slot_of_row [T * k]) and, when
    x ([T, ...], any dtype, 16-byte rows) is given, x_perm [T * k, ...] first: row r holds
    x[slot_of_row[r] // k]; rows past sum(group_sizes) are left as allocated."""
    import torch

    lib = load()
    _need(expert_ids, torch.int32, "expert_ids", 2)
    T, k = expert_ids.shape
    G = int(num_groups)
    dev = expert_ids.device
    gs = torch.empty(G, dtype=torch.int32, device=dev)
    ros = torch.empty((T, k), dtype=torch.int32, device=dev)
    sor = torch.empty(T * k, dtype=torch.int32, device=dev)
    row_bytes = 0
    if x is not None:
        if x.device != dev or not x.is_contiguous() or x.shape[0] != T:
            raise ValueError("x must be a contiguous [T, ...] tensor on the ids' device")
        row_bytes = x.element_size()
        for d in x.shape[1:]:
            row_bytes *= int(d)
        if x_perm is None:
            x_perm = torch.empty((T * k,) + tuple(x.shape[1:]), dtype=x.dtype, device=dev)
        elif (x_perm.dtype != x.dtype or tuple(x_perm.shape) != (T * k,) + tuple(x.shape[1:])
              or not x_perm.is_contiguous() or x_perm.device != dev):
            raise ValueError("x_perm must be a contiguous [T * k, ...] tensor of x's dtype")
    ws_n = lib.gmm_permute_workspace_size(T, k, G)
    ws = _workspace(ws_n, dev)
    _check(lib.gmm_permute(T, k, G, _ptr(expert_ids), row_bytes, _ptr(x), _ptr(x_perm), _ptr(gs),
                           _ptr(ros), _ptr(sor), _ptr(ws), ws_n, _stream()), "gmm_permute")
    return (x_perm, gs, ros, sor) if x is not None else (gs, ros, sor)


def gmm_unpermute(y, row_of_slot, weights=None, out=None):
    """out [T, H] bf16 = sum over j of weights[t, j] * y[row_of_slot[t, j]] (fp32 in j order;
    dropped slots skipped); y bf16 [T * k, H]; weights f32 [T, k] or None (all 1)."""
    import torch

    lib = load()
    _need(y, torch.bfloat16, "y", 2)
    _need(row_of_slot, torch.int32, "row_of_slot", 2)
    T, k = row_of_slot.shape
    H = y.shape[1]
    if y.shape[0] != T * k:
        raise ValueError("y must have T * k rows")
    if weights is not None:
        _need(weights, torch.float32, "weights", 2)
        if tuple(weights.shape) != (T, k):
            raise ValueError("weights must be [T, k]")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    else:
        _need(out, torch.bfloat16, "out", 2)
        _shape(out, (T, H), "out")
    _check(lib.gmm_unpermute(T, k, H, _ptr(y), _ptr(row_of_slot), _ptr(weights), _ptr(out),
                             _stream()), "gmm_unpermute")
    return out


def gmm_quantize_subchannel(x, bk=128, fmt="e4m3"):
    """bf16 x [M, K] -> (uint8 codes [M, K], f32 scales [M, K / bk]): one dynamic scale per
    row and block of bk columns (bk 128, 256 or 512)."""
    import torch

    lib = load()
    _need(x, torch.bfloat16, "x", 2)
    M, K = x.shape
    codes = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    scales = torch.empty((M, K // bk if bk else 0), dtype=torch.float32, device=x.device)
    _check(lib.gmm_quantize_subchannel(_FMT[fmt], M, K, int(bk), _ptr(x), _ptr(codes), _ptr(scales),
                                       _stream()), "gmm_quantize_subchannel")
    return codes, scales


def gmm_quantize_rhs_blockwise(w, bk=128, fmt="e4m3", layout="nk"):
    """bf16 w [G, K, N] -> (uint8 codes [G, N, K] ("nk") or [G, K, N] ("kn"), f32 scales
    [G, K / bk, N]): one dynamic scale per expert, block of bk contraction rows and column."""
    import torch

    lib = load()
    _need(w, torch.bfloat16, "w", 3)
    G, K, N = w.shape
    lay = _LAYOUT[layout]
    codes = torch.empty((G, N, K) if lay == RHS_NK else (G, K, N), dtype=torch.uint8, device=w.device)
    scales = torch.empty((G, K // bk if bk else 0, N), dtype=torch.float32, device=w.device)
    _check(lib.gmm_quantize_rhs_blockwise(_FMT[fmt], lay, G, K, N, int(bk), _ptr(w), _ptr(codes),
                                          _ptr(scales), _stream()), "gmm_quantize_rhs_blockwise")
    return codes, scales


def gmm_quantize_rhs_blockwise_dlhs(w, bk=128, fmt="e4m3"):
    """bf16 w [G, K, N] -> (uint8 codes [G, K, N], f32 scales [G, K, N / bk]): the weight copy
    of gmm_dlhs_blockwise, one dynamic scale per expert, output channel k and block of bk
    columns n (gmm_quantize_subchannel of w viewed as [G * K, N])."""
    import torch

    _need(w, torch.bfloat16, "w", 3)
    G, K, N = w.shape
    codes, scales = gmm_quantize_subchannel(w.reshape(G * K, N), bk, fmt)
    return codes.view(G, K, N), scales.view(G, K, N // bk)


def gmm_dlhs_blockwise(grad, grad_scales, rhs, rhs_scales, group_sizes, bk=128, *,
                       grad_format="e5m2", out_dtype=None, out=None):
    """lhs gradient with block-wise scales along its contraction: grad uint8 codes [M, N]
    with grad_scales f32 [M, N / bk], rhs uint8 codes [G, K, N] with rhs_scales f32
    [G, K, N / bk] (gmm_quantize_rhs_blockwise_dlhs); returns dlhs [M, K]."""
    import torch

    lib = load()
    _need(grad, torch.uint8, "grad", 2)
    _need(rhs, torch.uint8, "rhs", 3)
    _need(grad_scales, torch.float32, "grad_scales", 2)
    _need(rhs_scales, torch.float32, "rhs_scales", 3)
    _need(group_sizes, torch.int32, "group_sizes", 1)
    M, N = grad.shape
    G, K = rhs.shape[0], rhs.shape[1]
    if rhs.shape[2] != N or N % bk:
        raise ValueError("rhs must be [G, K, N] codes matching the grad width, N a multiple of bk")
    _shape(grad_scales, (M, N // bk), "grad_scales")
    _shape(rhs_scales, (G, K, N // bk), "rhs_scales")
    _group_sizes(group_sizes, G)
    odt = torch.float32 if out_dtype == torch.float32 else torch.bfloat16
    if out is None:
        out = torch.empty((M, K), dtype=odt, device=grad.device)
    else:
        _need(out, odt, "out", 2)
        _shape(out, (M, K), "out")
    _check(lib.gmm_dlhs_blockwise(_FMT[grad_format], OUT_F32 if odt == torch.float32 else OUT_BF16,
                                  M, K, N, G, bk, _ptr(grad), _ptr(grad_scales), _ptr(rhs),
                                  _ptr(rhs_scales), _ptr(group_sizes), _ptr(out), _stream()),
           "gmm_dlhs_blockwise")
    return out


def gmm_fwd_blockwise(lhs, lhs_scales, rhs, rhs_scales, group_sizes, bk=128, *,
                      lhs_format="e4m3", out_dtype=None, out=None):
    """Forward grouped matmul with block-wise scales: lhs uint8 codes [M, K] with
    lhs_scales f32 [M, K / bk], rhs uint8 codes [G, N, K] with rhs_scales f32
    [G, K / bk, N]; every block of bk contraction elements is scaled on its own."""
    import torch

    lib = load()
    _need(lhs, torch.uint8, "lhs", 2)
    _need(lhs_scales, torch.float32, "lhs_scales", 2)
    _need(rhs, torch.uint8, "rhs", 3)
    _need(rhs_scales, torch.float32, "rhs_scales", 3)
    _need(group_sizes, torch.int32, "group_sizes", 1)
    M, K = lhs.shape
    G, N = rhs.shape[0], rhs.shape[1]
    if rhs.shape[2] != K:
        raise ValueError("rhs must be [G, N, K] codes matching the lhs width")
    if bk <= 0 or K % bk:
        raise ValueError("bk must be a positive divisor of K")
    _shape(lhs_scales, (M, K // bk), "lhs_scales")
    _shape(rhs_scales, (G, K // bk, N), "rhs_scales")
    _group_sizes(group_sizes, G)
    odt = torch.float32 if out_dtype == torch.float32 else torch.bfloat16
    if out is None:
        out = torch.empty((M, N), dtype=odt, device=lhs.device)
    else:
        _need(out, odt, "out", 2)
        _shape(out, (M, N), "out")
    _check(lib.gmm_fwd_blockwise(_FMT[lhs_format], OUT_F32 if odt == torch.float32 else OUT_BF16,
                                 M, K, N, G, int(bk), _ptr(lhs), _ptr(lhs_scales), _ptr(rhs),
                                 _ptr(rhs_scales), _ptr(group_sizes), _ptr(out), _stream()),
           "gmm_fwd_blockwise")
    return out


def gmm_quantize_folded(grad, col_scales, group_sizes, fmt="e5m2"):
    """The folded gradient of the one-weight-copy dlhs: codes and 128-row-block scales of
    RNE_f32(grad[m, n] * col_scales[g(m), n]).  grad bf16 [M, N], col_scales f32 [G, N]
    (the forward's per-channel weight scales).  Feed the result to gmm_dlhs with
    grad_scales=scales, the forward's codes laid out [G, K, N] and all-one rhs_scales."""
    import torch

    lib = load()
    _need(grad, torch.bfloat16, "grad", 2)
    _need(col_scales, torch.float32, "col_scales", 2)
    _need(group_sizes, torch.int32, "group_sizes", 1)
    M, N = grad.shape
    G = group_sizes.shape[0]
    if tuple(col_scales.shape) != (G, N):
        raise ValueError("col_scales must be [G, N]")
    codes = torch.empty((M, N), dtype=torch.uint8, device=grad.device)
    scales = torch.empty(_nblocks(M), dtype=torch.float32, device=grad.device)
    ws_n = _nblocks(M) * 32
    ws = _workspace(ws_n, grad.device)
    _check(lib.gmm_quantize_folded(_FMT[fmt], M, N, G, _ptr(grad), _ptr(col_scales),
                                   _ptr(group_sizes), _ptr(codes), _ptr(scales), _ptr(ws), ws_n,
                                   _stream()), "gmm_quantize_folded")
    return codes, scales
