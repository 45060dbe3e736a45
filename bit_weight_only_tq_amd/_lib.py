"""ctypes binding of libtq.so: argument marshalling only.

Every function here forwards to the C ABI declared in include/tq.h with the
same name; tensors are torch tensors on the current HIP device (torch is used
for device memory and the current stream, nothing else).  There is no CPU
fallback: if libtq.so is missing or cannot be loaded, every call raises.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtq.so")

# tq_status
STATUS_NAMES = {
    0: "TQ_OK", 1: "TQ_ERR_NULL", 2: "TQ_ERR_SHAPE", 3: "TQ_ERR_ALIGN", 4: "TQ_ERR_DTYPE",
    5: "TQ_ERR_GROUP", 6: "TQ_ERR_NONFINITE", 7: "TQ_ERR_RANGE", 8: "TQ_ERR_BAD_CODE",
    9: "TQ_ERR_HIP", 10: "TQ_ERR_PATH", 11: "TQ_ERR_SCRATCH",
}
# tq_dtype
TQ_F16, TQ_BF16 = 0, 1
# tq_path
PATHS = {"auto": 0, "gemv": 1, "stream_mfma": 2, "gemm": 3}
PATH_NAMES = {v: k for k, v in PATHS.items()}

# every symbol include/tq.h declares, with (restype, argtypes)
_i64, _vp, _i32, _sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "tq_pack": (_i32, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "tq_unpack": (_i32, [_vp, _vp, _i64, _i64, _vp, _vp, _vp]),
    "w4a16_pack": (_i32, [_vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "w4a16_unpack": (_i32, [_vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "tq_gemm": (_i32, [_vp, _i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp]),
    "tq_gemm_ex": (_i32, [_vp, _i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _i32]),
    "tq_gemm_ws": (_i32, [_vp, _i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _i32]),
    "tq_gemm_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32, _i32]),
    "tq_gemm_noalloc": (_i32, [_vp, _i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _i32]),
    "tq_gemm_noalloc_scratch_bytes": (_sz, []),
    "w4a16_gemm": (_i32, [_vp, _i32, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _vp]),
    "w4a16_gemm_ex": (_i32, [_vp, _i32, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _vp, _i32]),
    "w4a16_gemm_ws": (_i32, [_vp, _i32, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp, _i32]),
    "w4a16_gemm_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32, _i64]),
    "w4a16_pack_asym": (_i32, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "w4a16_unpack_asym": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "w4a16_gemm_asym": (_i32, [_vp, _i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp,
                               _i32]),
    "w4a16_gemm_asym_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32, _i64, _i32]),
    "tq_diag_stream_read": (_i32, [_vp, _sz, _vp, _i64, _vp]),
    "tq_diag_gemv": (_i32, [_vp, _i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _i32]),
    "tq_select_path": (_i32, [_i32, _i64, _i64, _i64, _i32]),
    "tq_status_str": (ctypes.c_char_p, [_i32]),
    "tq_abi_version": (_i32, []),
}


class TQError(RuntimeError):
    """A libtq call returned a status other than TQ_OK."""

    def __init__(self, fn: str, status: int, msg: str):
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{fn}: {self.name} ({msg})")


_lib = None


def load(path: str = LIB_PATH):
    """Load libtq.so once and declare its prototypes; raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libtq.so not built: {path} is missing "
                           "(run `python -m bit_weight_only_tq_amd.build`)")
    # torch ships its own HIP runtime under another file name; loading it
    # first makes libtq.so bind to that copy.  Loaded the other way round the
    # process would hold two runtimes, and torch's device pointers and
    # streams would be foreign to the library's.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != 0:
        msg = load().tq_status_str(status).decode()
        raise TQError(fn, status, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device=None):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_enum(t):
    import torch
    if t.dtype == torch.float16:
        return TQ_F16
    if t.dtype == torch.bfloat16:
        return TQ_BF16
    raise TypeError(f"activations must be float16 or bfloat16, got {t.dtype}")


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous device tensors")
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"tensors must live on one device, got {sorted(str(d) for d in devs)}")


# Shape and dtype checks before any call: the C ABI takes bare pointers and
# cannot check buffer sizes, so a mismatched tensor would make a kernel read
# or write out of bounds.

def _check_activations(A):
    import torch
    if A.dim() != 2:
        raise ValueError(f"A must be 2-D [M, K], got shape {tuple(A.shape)}")
    if A.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError(f"activations must be float16 or bfloat16, got {A.dtype}")
    return A.shape


def _check_out_bias(A, N, bias, out):
    M = A.shape[0]
    if bias is not None and (bias.dtype != A.dtype or tuple(bias.shape) != (N,)):
        raise ValueError(f"bias must be {A.dtype} ({N},), got {bias.dtype} {tuple(bias.shape)}")
    if out is not None and (out.dtype != A.dtype or tuple(out.shape) != (M, N)):
        raise ValueError(f"out must be {A.dtype} ({M}, {N}), got {out.dtype} {tuple(out.shape)}")


def _ternary_layout(codes, scale, K):
    from .layout import TernaryLayout
    if codes.dim() != 2:
        raise ValueError(f"codes must be 2-D [N, ceil(K/4)], got shape {tuple(codes.shape)}")
    lay = TernaryLayout(int(codes.shape[0]), int(K))
    lay.validate(codes, scale)
    return lay


def _w4_layout(qweight, scales, K, group_size, zeros=None, perm=None):
    import torch
    from .layout import W4Layout
    if qweight.dim() != 2:
        raise ValueError(f"qweight must be 2-D [N, K/8], got shape {tuple(qweight.shape)}")
    lay = W4Layout(int(qweight.shape[0]), int(K), int(group_size))
    lay.validate(qweight, scales)
    if zeros is not None and (zeros.dtype != torch.uint8 or tuple(zeros.shape) != lay.scales_shape):
        raise ValueError(f"zeros must be uint8 {lay.scales_shape}, got {zeros.dtype} {tuple(zeros.shape)}")
    if perm is not None and (perm.dtype != torch.int32 or tuple(perm.shape) != (lay.K,)):
        raise ValueError(f"perm must be int32 ({lay.K},), got {perm.dtype} {tuple(perm.shape)}")
    return lay


# ------------------------------------------------------------------ prepare

def tq_pack(W):
    """fp32 [N, K] -> (codes uint8 [N, ceil(K/4)], scale fp16 [N])."""
    import torch
    _need_cuda(W)
    if W.dtype != torch.float32 or W.dim() != 2:
        raise TypeError("W must be a 2-D float32 tensor")
    N, K = W.shape
    codes = torch.empty((N, (K + 3) // 4), dtype=torch.uint8, device=W.device)
    scale = torch.empty((N,), dtype=torch.float16, device=W.device)
    _check("tq_pack", load().tq_pack(_ptr(W), N, K, _ptr(codes), _ptr(scale), _stream(W.device)))
    return codes, scale


def tq_unpack(codes, scale, K: int, want_t: bool = True, want_wdq: bool = True):
    """-> (t int8 [N, K] or None, wdq fp16 [N, K] or None)."""
    import torch
    N = _ternary_layout(codes, scale, K).N
    _need_cuda(codes, scale)
    t = torch.empty((N, K), dtype=torch.int8, device=codes.device) if want_t else None
    w = torch.empty((N, K), dtype=torch.float16, device=codes.device) if want_wdq else None
    _check("tq_unpack", load().tq_unpack(_ptr(codes), _ptr(scale), N, K, _ptr(t), _ptr(w), _stream(codes.device)))
    return t, w


def w4a16_pack(W, group_size: int = 128):
    """fp32 [N, K] -> (qweight int32 [N, K/8], scales fp16 [N, K/group])."""
    import torch
    _need_cuda(W)
    if W.dtype != torch.float32 or W.dim() != 2:
        raise TypeError("W must be a 2-D float32 tensor")
    N, K = W.shape
    q = torch.empty((N, K // 8), dtype=torch.int32, device=W.device)
    s = torch.empty((N, max(K // max(group_size, 1), 1)), dtype=torch.float16, device=W.device)
    _check("w4a16_pack", load().w4a16_pack(_ptr(W), N, K, group_size, _ptr(q), _ptr(s), _stream(W.device)))
    return q, s


def w4a16_unpack(qweight, scales, K: int, group_size: int = 128, want_q: bool = True, want_wdq: bool = True):
    """-> (q uint8 [N, K] or None, wdq fp16 [N, K] or None)."""
    import torch
    N = _w4_layout(qweight, scales, K, group_size).N
    _need_cuda(qweight, scales)
    q = torch.empty((N, K), dtype=torch.uint8, device=qweight.device) if want_q else None
    w = torch.empty((N, K), dtype=torch.float16, device=qweight.device) if want_wdq else None
    _check("w4a16_unpack", load().w4a16_unpack(_ptr(qweight), _ptr(scales), N, K, group_size,
                                               _ptr(q), _ptr(w), _stream(qweight.device)))
    return q, w


def w4a16_pack_asym(W, g_idx=None, group_size: int = 128):
    """fp32 [N, K] (+ g_idx int32 [K]) -> (qweight int32 [N, K/8], scales fp16 [N, G],
    zeros uint8 [N, G], perm int32 [K] or None); columns packed in group order."""
    import torch
    _need_cuda(W, g_idx)
    if W.dtype != torch.float32 or W.dim() != 2:
        raise TypeError("W must be a 2-D float32 tensor")
    if g_idx is not None and (g_idx.dtype != torch.int32 or g_idx.numel() != W.shape[1]):
        raise TypeError("g_idx must be an int32 tensor of K entries")
    N, K = W.shape
    G = max(K // max(group_size, 1), 1)
    q = torch.empty((N, K // 8), dtype=torch.int32, device=W.device)
    s = torch.empty((N, G), dtype=torch.float16, device=W.device)
    z = torch.empty((N, G), dtype=torch.uint8, device=W.device)
    perm = torch.empty((K,), dtype=torch.int32, device=W.device) if g_idx is not None else None
    _check("w4a16_pack_asym", load().w4a16_pack_asym(_ptr(W), N, K, group_size, _ptr(g_idx), _ptr(q), _ptr(s),
                                                     _ptr(z), _ptr(perm), _stream(W.device)))
    return q, s, z, perm


def w4a16_unpack_asym(qweight, scales, zeros, K: int, perm=None, group_size: int = 128, want_q: bool = True,
                      want_wdq: bool = True):
    """-> (q uint8 [N, K] packed order or None, wdq fp16 [N, K] input order or None)."""
    import torch
    if zeros is None:
        raise ValueError("zeros are required")
    N = _w4_layout(qweight, scales, K, group_size, zeros, perm).N
    _need_cuda(qweight, scales, zeros, perm)
    q = torch.empty((N, K), dtype=torch.uint8, device=qweight.device) if want_q else None
    w = torch.empty((N, K), dtype=torch.float16, device=qweight.device) if want_wdq else None
    _check("w4a16_unpack_asym", load().w4a16_unpack_asym(_ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(perm), N,
                                                         K, group_size, _ptr(q), _ptr(w), _stream(qweight.device)))
    return q, w


# -------------------------------------------------------------------- apply

# Bytes of split arrival counters at the front of every workspace (include/tq.h)
TQ_WORKSPACE_FLAG_BYTES = 16384


def new_workspace(nbytes: int, device):
    """A device workspace of nbytes bytes from torch's allocator (None for 0)
    whose arrival counters, the first TQ_WORKSPACE_FLAG_BYTES bytes, are zero
    (the library leaves them zero after every call, so a reused workspace
    needs this once)."""
    import torch
    if not nbytes:
        return None
    ws = torch.empty((nbytes,), dtype=torch.uint8, device=device)
    ws[:TQ_WORKSPACE_FLAG_BYTES].zero_()
    return ws


def tq_gemm_workspace_bytes(M: int, N: int, K: int, dtype: str = "f16", path: str = "auto") -> int:
    """Bytes of workspace tq_gemm_ws uses for its fastest schedule (0: none)."""
    d = {"f16": TQ_F16, "bf16": TQ_BF16}[dtype]
    return int(load().tq_gemm_workspace_bytes(M, N, K, d, PATHS[path]))


def tq_gemm(A, codes, scale, bias=None, out=None, path: str = "auto", workspace="auto"):
    """C = A @ dequant(codes, scale)^T (+ bias); A [M, K] fp16/bf16.

    workspace: "auto" takes the bytes tq_gemm_workspace_bytes asks for from
    torch's allocator (stream-ordered, so overlapping calls never share it)
    and zeroes its arrival counters; None runs without one; or a contiguous
    device tensor whose first TQ_WORKSPACE_FLAG_BYTES bytes are zero (see
    new_workspace)."""
    import torch
    M, K = _check_activations(A)
    N = _ternary_layout(codes, scale, K).N
    _check_out_bias(A, N, bias, out)
    _need_cuda(A, codes, scale, bias, out)
    dt = _dtype_enum(A)
    C = out if out is not None else torch.empty((M, N), dtype=A.dtype, device=A.device)
    if isinstance(workspace, str):
        nbytes = int(load().tq_gemm_workspace_bytes(M, N, K, dt, PATHS[path]))
        workspace = new_workspace(nbytes, A.device)
    ws_bytes = 0
    if workspace is not None:
        _need_cuda(A, workspace)
        ws_bytes = workspace.numel() * workspace.element_size()
    _check("tq_gemm", load().tq_gemm_ws(_ptr(A), dt, M, N, K, _ptr(codes), _ptr(scale), _ptr(bias), _ptr(C),
                                         _ptr(workspace), ws_bytes, _stream(A.device), PATHS[path]))
    return C


def tq_gemm_noalloc(A, codes, scale, bias=None, out=None, path: str = "auto"):
    """tq_gemm through the entry point that allocates nothing (its split-K
    partials go to the library's per-device scratch; see include/tq.h)."""
    import torch
    M, K = _check_activations(A)
    N = _ternary_layout(codes, scale, K).N
    _check_out_bias(A, N, bias, out)
    _need_cuda(A, codes, scale, bias, out)
    dt = _dtype_enum(A)
    C = out if out is not None else torch.empty((M, N), dtype=A.dtype, device=A.device)
    _check("tq_gemm_noalloc", load().tq_gemm_noalloc(_ptr(A), dt, M, N, K, _ptr(codes), _ptr(scale), _ptr(bias),
                                                     _ptr(C), _stream(A.device), PATHS[path]))
    return C


def w4a16_gemm_workspace_bytes(M: int, N: int, K: int, dtype: str = "f16", group_size: int = 128) -> int:
    """Bytes of workspace w4a16_gemm_ws uses for its fastest schedule (0: none)."""
    d = {"f16": TQ_F16, "bf16": TQ_BF16}[dtype]
    return int(load().w4a16_gemm_workspace_bytes(M, N, K, d, group_size))


def w4a16_gemm_asym_workspace_bytes(M: int, N: int, K: int, dtype: str = "f16", group_size: int = 128,
                                    with_perm: bool = False) -> int:
    """Bytes of workspace w4a16_gemm_asym uses for its fastest schedule."""
    d = {"f16": TQ_F16, "bf16": TQ_BF16}[dtype]
    return int(load().w4a16_gemm_asym_workspace_bytes(M, N, K, d, group_size, 1 if with_perm else 0))


def w4a16_gemm(A, qweight, scales, bias=None, out=None, group_size: int = 128, path: str = "auto",
               workspace="auto", zeros=None, perm=None):
    """C = A @ dequant(qweight, scales[, zeros])^T (+ bias); A [M, K] fp16/bf16.

    zeros / perm: the zero points and column order of w4a16_pack_asym (both
    optional); with either, the zero-point entry point runs.
    workspace: as for tq_gemm ("auto", None or a contiguous device tensor)."""
    import torch
    M, K = _check_activations(A)
    N = _w4_layout(qweight, scales, K, group_size, zeros, perm).N
    _check_out_bias(A, N, bias, out)
    _need_cuda(A, qweight, scales, bias, zeros, perm, out)
    dt = _dtype_enum(A)
    C = out if out is not None else torch.empty((M, N), dtype=A.dtype, device=A.device)
    asym = zeros is not None or perm is not None
    if isinstance(workspace, str):
        if asym:
            nbytes = int(load().w4a16_gemm_asym_workspace_bytes(M, N, K, dt, group_size, 1 if perm is not None else 0))
        else:
            nbytes = int(load().w4a16_gemm_workspace_bytes(M, N, K, dt, group_size))
        workspace = new_workspace(nbytes, A.device)
    ws_bytes = 0
    if workspace is not None:
        _need_cuda(A, workspace)
        ws_bytes = workspace.numel() * workspace.element_size()
    if asym:
        _check("w4a16_gemm_asym", load().w4a16_gemm_asym(
            _ptr(A), dt, M, N, K, _ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(perm), group_size, _ptr(bias),
            _ptr(C), _ptr(workspace), ws_bytes, _stream(A.device), PATHS[path]))
        return C
    _check("w4a16_gemm", load().w4a16_gemm_ws(_ptr(A), dt, M, N, K, _ptr(qweight), _ptr(scales), group_size,
                                               _ptr(bias), _ptr(C), _ptr(workspace), ws_bytes, _stream(A.device),
                                               PATHS[path]))
    return C


def tq_select_path(fmt: str, M: int, N: int, K: int, dtype: str = "f16") -> str:
    """The dispatcher's kernel choice for a shape ("gemv", "stream_mfma", "gemm")."""
    f = {"ternary": 0, "w4a16": 1}[fmt]
    d = {"f16": TQ_F16, "bf16": TQ_BF16}[dtype]
    return PATH_NAMES[load().tq_select_path(f, M, N, K, d)]


def tq_diag_stream_read(src, blocks: int, sink=None):
    """Launch the plain streaming read over all of `src` (a contiguous
    device tensor); returns the sink tensor it may write."""
    import torch
    _need_cuda(src)
    nbytes = src.numel() * src.element_size()
    if sink is None:
        sink = torch.empty((blocks,), dtype=torch.int32, device=src.device)
    _check("tq_diag_stream_read", load().tq_diag_stream_read(_ptr(src), nbytes, _ptr(sink), blocks,
                                                             _stream(src.device)))
    return sink


def tq_diag_gemv(A, codes, scale, variant: int, out=None):
    """The M = 1 decode kernel in measurement form (0 as tq_gemm, 1 codes
    from the cache, 2 codes from the cache without the multiply)."""
    import torch
    M, K = _check_activations(A)
    N = _ternary_layout(codes, scale, K).N
    _check_out_bias(A, N, None, out)
    _need_cuda(A, codes, scale, out)
    C = out if out is not None else torch.empty((M, N), dtype=A.dtype, device=A.device)
    _check("tq_diag_gemv", load().tq_diag_gemv(_ptr(A), _dtype_enum(A), M, N, K, _ptr(codes), _ptr(scale), None,
                                               _ptr(C), _stream(A.device), variant))
    return C


def tq_abi_version() -> int:
    return load().tq_abi_version()
