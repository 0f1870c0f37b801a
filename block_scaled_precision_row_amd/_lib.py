"""Thin ctypes binding of libbsq.so, with the C entry points' names.

Two layers:
  * ``lib`` -- the loaded library with argument / return types declared for
    every symbol of include/bsq.h (raw pointers and sizes);
  * functions named like the C entry points that take torch tensors, check
    dtype / shape / device, allocate outputs and workspaces with torch when
    the caller passes none, and call the library on the current stream.
No arithmetic of the method happens here. Importing this module raises if
the library has not been built (there is no fallback path).
"""
import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbsq.so")

BSQ_FMT_FP8R = 1
BSQ_FMT_NVFP4 = 2
BSQ_WEIGHT_ONLY = 0x1
BSQ_NOALLOC_MAX_BYTES = 64 << 20  # scratch of bsq_gemm_fp8r_noalloc (include/bsq.h)

STATUS = {0: "BSQ_OK", 1: "BSQ_ERR_NULL", 2: "BSQ_ERR_SHAPE", 3: "BSQ_ERR_ALIGN", 4: "BSQ_ERR_WORKSPACE",
          5: "BSQ_ERR_DEVICE", 6: "BSQ_ERR_HIP", 7: "BSQ_ERR_ARG"}

_p, _i64, _u32, _sz, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t, ctypes.c_int
_f32 = ctypes.c_float

BSQ_MAX_GROUP = 8


class GemmProblem(ctypes.Structure):
    """bsq_gemm_problem: one linear of a grouped launch (device pointers as integers)."""
    _fields_ = [("xq", _p), ("x_scale", _p), ("input_scale", _p), ("w", _p), ("w_scale", _p), ("w_scale2", _p),
                ("y", _p), ("ldy", _i64), ("M", _i64), ("N", _i64), ("K", _i64)]


class WeightOnlyProblem(ctypes.Structure):
    """bsq_weight_only_problem: one weight-only linear of a grouped launch (device pointers as integers)."""
    _fields_ = [("x", _p), ("ldx", _i64), ("w", _p), ("w_scale", _p), ("w_scale2", _p), ("y", _p), ("ldy", _i64),
                ("M", _i64), ("N", _i64), ("K", _i64)]


# symbol -> (restype, argtypes); mirrors include/bsq.h
SIGNATURES = {
    "bsq_abi_version": (_int, []),
    "bsq_status_string": (ctypes.c_char_p, [_int]),
    "bsq_last_hip_error": (ctypes.c_char_p, []),
    "bsq_quantize_act_fp8r": (_int, [_p, _i64, _i64, _i64, _p, _p, _p]),
    "bsq_quantize_act_nvfp4": (_int, [_p, _i64, _i64, _i64, _p, _p, _p, _p]),
    "bsq_calibrate_workspace_bytes": (_sz, [_i64, _i64]),
    "bsq_calibrate_global_scale": (_int, [_p, _i64, _i64, _i64, _p, _p, _sz, _p]),
    "bsq_gemm_workspace_bytes": (_sz, [_int, _i64, _i64, _i64, _u32]),
    "bsq_gemm_fp8r": (_int, [_p, _i64, _p, _p, _p, _i64, _i64, _i64, _i64, _u32, _p, _sz, _p]),
    "bsq_gemm_fp8r_noalloc": (_int, [_p, _i64, _p, _p, _p, _i64, _i64, _i64, _i64, _u32, _p]),
    "bsq_gemm_nvfp4": (_int, [_p, _i64, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _u32, _p, _sz, _p]),
    "bsq_dequant_to_bf16": (_int, [_int, _p, _p, _p, _i64, _i64, _p, _p]),
    "bsq_gemm_fp8r_q": (_int, [_p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _p]),
    "bsq_gemm_nvfp4_q": (_int, [_p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _p]),
    "bsq_gemm_grouped_q": (_int, [_int, ctypes.POINTER(GemmProblem), _int, _p]),
    "bsq_gemm_grouped_weight_only": (_int, [_int, ctypes.POINTER(WeightOnlyProblem), _int, _p]),
    "bsq_gemm_nvfp4_quantize_y_workspace_bytes": (_sz, [_i64, _i64, _i64, _int]),
    "bsq_gemm_nvfp4_q_quantize_y": (_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _p, _sz,
                                           _p]),
    "bsq_gemm_quantize_y_workspace_bytes": (_sz, [_int, _i64, _i64, _int]),
    "bsq_gemm_fp8r_q_quantize_y": (_int, [_p, _p, _p, _p, _int, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _p, _sz,
                                          _p]),
    "bsq_gemm_nvfp4_q_quantize_y_fp8r": (_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _p, _sz,
                                                _p]),
    "bsq_gemm_weight_only_quantize_y": (_int, [_int, _p, _i64, _p, _p, _p, _int, _p, _p, _p, _p, _i64, _i64, _i64,
                                                _i64, _p, _sz, _p]),
    "bsq_lora_workspace_bytes": (_sz, [_int, _i64, _i64, _i64, _i64, _u32]),
    "bsq_gemm_fp8r_lora": (_int, [_p, _i64, _p, _p, _p, _p, _i64, _f32, _p, _i64, _i64, _i64, _i64, _u32, _p, _sz,
                                  _p]),
    "bsq_gemm_nvfp4_lora": (_int, [_p, _i64, _p, _p, _p, _p, _p, _p, _i64, _f32, _p, _i64, _i64, _i64, _i64, _u32,
                                   _p, _sz, _p]),
    "bsq_lora_down_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "bsq_lora_down": (_int, [_p, _i64, _p, _i64, _i64, _i64, _f32, _p, _p, _sz, _p]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libbsq.so is not built at %s; run `python -m block_scaled_precision_row_amd.build`"
                          % LIB_PATH)
    so = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(so, name)
        fn.restype = res
        fn.argtypes = args
    return so


lib = _load()


class BsqError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = "%s returned %s (%s)" % (fn, STATUS.get(status, status), lib.bsq_status_string(status).decode())
        if status == 6:
            msg += ": " + lib.bsq_last_hip_error().decode()
        super().__init__(msg)


def _check(fn, status):
    if status != 0:
        raise BsqError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _rows(x, dtype, name):
    if x.dtype != dtype or x.dim() != 2 or not x.is_cuda:
        raise ValueError("%s must be a 2-D %s tensor on the GPU" % (name, dtype))
    if x.stride(1) != 1:
        raise ValueError("%s must have unit stride along its last dimension" % name)
    return x.shape[0], x.shape[1], (x.stride(0) if x.shape[0] > 1 else x.shape[1])


def _dense(x, dtype, shape, name):
    if x.dtype != dtype or tuple(x.shape) != tuple(shape) or not x.is_cuda or not x.is_contiguous():
        raise ValueError("%s must be a contiguous %s tensor of shape %s on the GPU" % (name, dtype, tuple(shape)))


def _scalar(t, name):
    if t is None:
        return None
    _dense(t, torch.float32, (1,), name)
    return t


# ---- entry points -------------------------------------------------------------

def bsq_quantize_act_fp8r(x, xq=None, x_scale=None):
    """bf16 x [M, K] -> (E4M3 codes uint8 [M, K], fp32 row scales [M])."""
    M, K, ldx = _rows(x, torch.bfloat16, "x")
    xq = torch.empty((M, K), dtype=torch.uint8, device=x.device) if xq is None else xq
    x_scale = torch.empty((M,), dtype=torch.float32, device=x.device) if x_scale is None else x_scale
    _dense(xq, torch.uint8, (M, K), "xq")
    _dense(x_scale, torch.float32, (M,), "x_scale")
    _check("bsq_quantize_act_fp8r", lib.bsq_quantize_act_fp8r(_ptr(x), M, K, ldx, _ptr(xq), _ptr(x_scale), _stream()))
    return xq, x_scale


def bsq_quantize_act_nvfp4(x, global_scale, xq=None, x_bscale=None):
    """bf16 x [M, K], fp32 global scale [1] -> (packed E2M1 uint8 [M, K/2], E4M3 block scales uint8 [M, K/16])."""
    M, K, ldx = _rows(x, torch.bfloat16, "x")
    _scalar(global_scale, "global_scale")
    xq = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device) if xq is None else xq
    x_bscale = torch.empty((M, K // 16), dtype=torch.uint8, device=x.device) if x_bscale is None else x_bscale
    _dense(xq, torch.uint8, (M, K // 2), "xq")
    _dense(x_bscale, torch.uint8, (M, K // 16), "x_bscale")
    _check("bsq_quantize_act_nvfp4", lib.bsq_quantize_act_nvfp4(_ptr(x), M, K, ldx, _ptr(global_scale), _ptr(xq),
                                                                _ptr(x_bscale), _stream()))
    return xq, x_bscale


def bsq_calibrate_global_scale(x, out=None, workspace=None):
    """bf16 x [M, K] -> fp32 [1] holding amax(x) / 2688 (1.0 for an all-zero x)."""
    M, K, ldx = _rows(x, torch.bfloat16, "x")
    out = torch.empty((1,), dtype=torch.float32, device=x.device) if out is None else out
    _scalar(out, "out")
    nbytes = lib.bsq_calibrate_workspace_bytes(M, K)
    if workspace is None:
        workspace = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=x.device)
    _check("bsq_calibrate_global_scale", lib.bsq_calibrate_global_scale(
        _ptr(x), M, K, ldx, _ptr(out), _ptr(workspace), _nbytes(workspace), _stream()))
    return out


def bsq_gemm_workspace_bytes(fmt, M, N, K, flags=0):
    return lib.bsq_gemm_workspace_bytes(fmt, M, N, K, flags)


def _workspace(fmt, M, N, K, flags, workspace, device):
    nbytes = lib.bsq_gemm_workspace_bytes(fmt, M, N, K, flags)
    if workspace is None and nbytes:
        workspace = torch.empty((nbytes,), dtype=torch.uint8, device=device)
    return workspace, _nbytes(workspace)


def _nbytes(t):
    """Size in bytes of a caller's workspace tensor of any dtype (0 for None)."""
    return 0 if t is None else t.numel() * t.element_size()


def bsq_gemm_fp8r(x, w, w_scale, flags=0, y=None, workspace=None):
    """bf16 x [M, K], E4M3 w [N, K], fp32 w_scale [N] -> bf16 y [M, N]."""
    M, K, ldx = _rows(x, torch.bfloat16, "x")
    N = w.shape[0]
    _dense(w, torch.uint8, (N, K), "w")
    _dense(w_scale, torch.float32, (N,), "w_scale")
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device) if y is None else y
    _, _, ldy = _rows(y, torch.bfloat16, "y")
    ws, nbytes = _workspace(BSQ_FMT_FP8R, M, N, K, flags, workspace, x.device)
    _check("bsq_gemm_fp8r", lib.bsq_gemm_fp8r(_ptr(x), ldx, _ptr(w), _ptr(w_scale), _ptr(y), ldy, M, N, K, flags,
                                              _ptr(ws), nbytes, _stream()))
    return y


def bsq_gemm_fp8r_noalloc(x, w, w_scale, flags=0, y=None):
    """bsq_gemm_fp8r on the library's own device scratch (no workspace; y must be passed in to
    allocate nothing at all)."""
    M, K, ldx = _rows(x, torch.bfloat16, "x")
    N = w.shape[0]
    _dense(w, torch.uint8, (N, K), "w")
    _dense(w_scale, torch.float32, (N,), "w_scale")
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device) if y is None else y
    _, _, ldy = _rows(y, torch.bfloat16, "y")
    _check("bsq_gemm_fp8r_noalloc", lib.bsq_gemm_fp8r_noalloc(_ptr(x), ldx, _ptr(w), _ptr(w_scale), _ptr(y), ldy,
                                                              M, N, K, flags, _stream()))
    return y


def bsq_gemm_nvfp4(x, w, w_bscale, w_scale2, input_scale=None, flags=0, y=None, workspace=None):
    """bf16 x [M, K], packed E2M1 w [N, K/2], E4M3 w_bscale [N, K/16], fp32 w_scale2 [1],
    fp32 input_scale [1] (None with BSQ_WEIGHT_ONLY) -> bf16 y [M, N]."""
    M, K, ldx = _rows(x, torch.bfloat16, "x")
    N = w.shape[0]
    _dense(w, torch.uint8, (N, K // 2), "w")
    _dense(w_bscale, torch.uint8, (N, K // 16), "w_bscale")
    _scalar(w_scale2, "w_scale2")
    _scalar(input_scale, "input_scale")
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device) if y is None else y
    _, _, ldy = _rows(y, torch.bfloat16, "y")
    ws, nbytes = _workspace(BSQ_FMT_NVFP4, M, N, K, flags, workspace, x.device)
    _check("bsq_gemm_nvfp4", lib.bsq_gemm_nvfp4(_ptr(x), ldx, _ptr(w), _ptr(w_bscale), _ptr(w_scale2),
                                                _ptr(input_scale), _ptr(y), ldy, M, N, K, flags, _ptr(ws), nbytes,
                                                _stream()))
    return y


def _adapter(lora_a, lora_b, N, K):
    rank = lora_a.shape[0]
    _dense(lora_a, torch.bfloat16, (rank, K), "lora_a")
    _dense(lora_b, torch.bfloat16, (N, rank), "lora_b")
    return rank


def _lora_workspace(fmt, M, N, K, rank, flags, workspace, device):
    nbytes = lib.bsq_lora_workspace_bytes(fmt, M, N, K, rank, flags)
    if workspace is None and nbytes:
        workspace = torch.empty((nbytes,), dtype=torch.uint8, device=device)
    return workspace, _nbytes(workspace)


def bsq_lora_workspace_bytes(fmt, M, N, K, rank, flags=0):
    return lib.bsq_lora_workspace_bytes(fmt, M, N, K, rank, flags)


def bsq_lora_down(x, lora_a, lora_scale, t=None, workspace=None):
    """bf16 x [M, K], bf16 lora_a [rank, K], float scale -> bf16 t = scale * x lora_a^T [M, rank]."""
    M, K, ldx = _rows(x, torch.bfloat16, "x")
    rank = lora_a.shape[0]
    _dense(lora_a, torch.bfloat16, (rank, K), "lora_a")
    t = torch.empty((M, rank), dtype=torch.bfloat16, device=x.device) if t is None else t
    _dense(t, torch.bfloat16, (M, rank), "t")
    nbytes = lib.bsq_lora_down_workspace_bytes(M, K, rank)
    if workspace is None and nbytes:
        workspace = torch.empty((nbytes,), dtype=torch.uint8, device=x.device)
    _check("bsq_lora_down", lib.bsq_lora_down(_ptr(x), ldx, _ptr(lora_a), M, K, rank, float(lora_scale), _ptr(t),
                                              _ptr(workspace), _nbytes(workspace),
                                              _stream()))
    return t


def bsq_gemm_fp8r_lora(x, w, w_scale, lora_a, lora_b, lora_scale, flags=0, y=None, workspace=None):
    """bsq_gemm_fp8r plus a LoRA: y = linear(x) + scale * (x lora_a^T) lora_b^T, with
    lora_a [rank, K] and lora_b [N, rank] bf16."""
    M, K, ldx = _rows(x, torch.bfloat16, "x")
    N = w.shape[0]
    _dense(w, torch.uint8, (N, K), "w")
    _dense(w_scale, torch.float32, (N,), "w_scale")
    rank = _adapter(lora_a, lora_b, N, K)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device) if y is None else y
    _, _, ldy = _rows(y, torch.bfloat16, "y")
    ws, nbytes = _lora_workspace(BSQ_FMT_FP8R, M, N, K, rank, flags, workspace, x.device)
    _check("bsq_gemm_fp8r_lora", lib.bsq_gemm_fp8r_lora(
        _ptr(x), ldx, _ptr(w), _ptr(w_scale), _ptr(lora_a), _ptr(lora_b), rank, float(lora_scale), _ptr(y), ldy,
        M, N, K, flags, _ptr(ws), nbytes, _stream()))
    return y


def bsq_gemm_nvfp4_lora(x, w, w_bscale, w_scale2, input_scale, lora_a, lora_b, lora_scale, flags=0, y=None,
                        workspace=None):
    """bsq_gemm_nvfp4 plus a LoRA: y = linear(x) + scale * (x lora_a^T) lora_b^T, with
    lora_a [rank, K] and lora_b [N, rank] bf16 (input_scale None with BSQ_WEIGHT_ONLY)."""
    M, K, ldx = _rows(x, torch.bfloat16, "x")
    N = w.shape[0]
    _dense(w, torch.uint8, (N, K // 2), "w")
    _dense(w_bscale, torch.uint8, (N, K // 16), "w_bscale")
    _scalar(w_scale2, "w_scale2")
    _scalar(input_scale, "input_scale")
    rank = _adapter(lora_a, lora_b, N, K)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device) if y is None else y
    _, _, ldy = _rows(y, torch.bfloat16, "y")
    ws, nbytes = _lora_workspace(BSQ_FMT_NVFP4, M, N, K, rank, flags, workspace, x.device)
    _check("bsq_gemm_nvfp4_lora", lib.bsq_gemm_nvfp4_lora(
        _ptr(x), ldx, _ptr(w), _ptr(w_bscale), _ptr(w_scale2), _ptr(input_scale), _ptr(lora_a), _ptr(lora_b), rank,
        float(lora_scale), _ptr(y), ldy, M, N, K, flags, _ptr(ws), nbytes, _stream()))
    return y


def bsq_gemm_fp8r_q(xq, x_scale, w, w_scale, y=None):
    """E4M3 xq [M, K] with fp32 row scales [M], E4M3 w [N, K], fp32 w_scale [N] -> bf16 y [M, N]."""
    M, K = xq.shape
    N = w.shape[0]
    _dense(xq, torch.uint8, (M, K), "xq")
    _dense(x_scale, torch.float32, (M,), "x_scale")
    _dense(w, torch.uint8, (N, K), "w")
    _dense(w_scale, torch.float32, (N,), "w_scale")
    y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device) if y is None else y
    _, _, ldy = _rows(y, torch.bfloat16, "y")
    _check("bsq_gemm_fp8r_q", lib.bsq_gemm_fp8r_q(_ptr(xq), _ptr(x_scale), _ptr(w), _ptr(w_scale), _ptr(y), ldy,
                                                  M, N, K, _stream()))
    return y


def bsq_gemm_nvfp4_q(xq, x_bscale, input_scale, w, w_bscale, w_scale2, y=None):
    """packed E2M1 xq [M, K/2] + E4M3 x_bscale [M, K/16] + input_scale [1], nvfp4 weights -> bf16 y [M, N]."""
    M, K = xq.shape[0], xq.shape[1] * 2
    N = w.shape[0]
    _dense(xq, torch.uint8, (M, K // 2), "xq")
    _dense(x_bscale, torch.uint8, (M, K // 16), "x_bscale")
    _scalar(input_scale, "input_scale")
    _dense(w, torch.uint8, (N, K // 2), "w")
    _dense(w_bscale, torch.uint8, (N, K // 16), "w_bscale")
    _scalar(w_scale2, "w_scale2")
    y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device) if y is None else y
    _, _, ldy = _rows(y, torch.bfloat16, "y")
    _check("bsq_gemm_nvfp4_q", lib.bsq_gemm_nvfp4_q(_ptr(xq), _ptr(x_bscale), _ptr(input_scale), _ptr(w),
                                                    _ptr(w_bscale), _ptr(w_scale2), _ptr(y), ldy, M, N, K,
                                                    _stream()))
    return y


def bsq_gemm_grouped_q(fmt, problems, ys=None):
    """Several pre-quantized linears of one scheme in one launch (bsq_gemm_grouped_q).
    fmt BSQ_FMT_FP8R: each problem is (xq [M, K], x_scale [M], w [N, K], w_scale [N]);
    fmt BSQ_FMT_NVFP4: (xq [M, K/2], x_bscale [M, K/16], input_scale [1], w [N, K/2], w_bscale [N, K/16],
    w_scale2 [1]). Returns the bf16 outputs [M, N], each bit for bit what bsq_gemm_fp8r_q /
    bsq_gemm_nvfp4_q returns for that problem."""
    if fmt not in (BSQ_FMT_FP8R, BSQ_FMT_NVFP4):
        raise ValueError("fmt must be BSQ_FMT_FP8R or BSQ_FMT_NVFP4")
    if len(problems) > BSQ_MAX_GROUP:
        raise ValueError("at most %d problems per group" % BSQ_MAX_GROUP)
    arr = (GemmProblem * max(len(problems), 1))()
    out = []
    for i, p in enumerate(problems):
        if fmt == BSQ_FMT_FP8R:
            xq, xs, w, ws = p
            M, K = xq.shape
            N = w.shape[0]
            _dense(xq, torch.uint8, (M, K), "xq")
            _dense(xs, torch.float32, (M,), "x_scale")
            _dense(w, torch.uint8, (N, K), "w")
            _dense(ws, torch.float32, (N,), "w_scale")
            gx = gw = None
        else:
            xq, xs, gx, w, ws, gw = p
            M, K = xq.shape[0], xq.shape[1] * 2
            N = w.shape[0]
            _dense(xq, torch.uint8, (M, K // 2), "xq")
            _dense(xs, torch.uint8, (M, K // 16), "x_bscale")
            _scalar(gx, "input_scale")
            _dense(w, torch.uint8, (N, K // 2), "w")
            _dense(ws, torch.uint8, (N, K // 16), "w_bscale")
            _scalar(gw, "w_scale2")
        y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device) if ys is None else ys[i]
        _, _, ldy = _rows(y, torch.bfloat16, "y")
        arr[i] = GemmProblem(xq.data_ptr(), xs.data_ptr(), None if gx is None else gx.data_ptr(), w.data_ptr(),
                             ws.data_ptr(), None if gw is None else gw.data_ptr(), y.data_ptr(), ldy, M, N, K)
        out.append(y)
    _check("bsq_gemm_grouped_q", lib.bsq_gemm_grouped_q(fmt, arr, len(problems), _stream()))
    return out


def bsq_gemm_grouped_weight_only(fmt, problems, ys=None):
    """Several weight-only linears (bf16 activations) of one scheme in one launch
    (bsq_gemm_grouped_weight_only). fmt BSQ_FMT_FP8R: each problem is (x [M, K] bf16, w [N, K] E4M3,
    w_scale [N] fp32); fmt BSQ_FMT_NVFP4: (x, w [N, K/2] packed E2M1, w_bscale [N, K/16] E4M3,
    w_scale2 [1]). Returns the bf16 outputs [M, N]."""
    if fmt not in (BSQ_FMT_FP8R, BSQ_FMT_NVFP4):
        raise ValueError("fmt must be BSQ_FMT_FP8R or BSQ_FMT_NVFP4")
    if len(problems) > BSQ_MAX_GROUP:
        raise ValueError("at most %d problems per group" % BSQ_MAX_GROUP)
    arr = (WeightOnlyProblem * max(len(problems), 1))()
    out = []
    for i, p in enumerate(problems):
        x = p[0]
        M, K, ldx = _rows(x, torch.bfloat16, "x")
        if fmt == BSQ_FMT_FP8R:
            _, w, ws = p
            N = w.shape[0]
            _dense(w, torch.uint8, (N, K), "w")
            _dense(ws, torch.float32, (N,), "w_scale")
            g2 = None
        else:
            _, w, ws, g2 = p
            N = w.shape[0]
            _dense(w, torch.uint8, (N, K // 2), "w")
            _dense(ws, torch.uint8, (N, K // 16), "w_bscale")
            _scalar(g2, "w_scale2")
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device) if ys is None else ys[i]
        _, _, ldy = _rows(y, torch.bfloat16, "y")
        arr[i] = WeightOnlyProblem(x.data_ptr(), ldx, w.data_ptr(), ws.data_ptr(),
                                   None if g2 is None else g2.data_ptr(), y.data_ptr(), ldy, M, N, K)
        out.append(y)
    _check("bsq_gemm_grouped_weight_only", lib.bsq_gemm_grouped_weight_only(fmt, arr, len(problems), _stream()))
    return out


def bsq_gemm_nvfp4_q_quantize_y(xq, x_bscale, input_scale, w, w_bscale, w_scale2, y_scale, with_y=False,
                                yq=None, y_bscale=None, y=None, workspace=None):
    """W4A4 GEMM as bsq_gemm_nvfp4_q whose output is also (or only) returned in nvfp4 with global scale
    y_scale [1]: (yq uint8 [M, N/2], y_bscale uint8 [M, N/16], bf16 y [M, N] or None)."""
    M, K = xq.shape[0], xq.shape[1] * 2
    N = w.shape[0]
    _dense(xq, torch.uint8, (M, K // 2), "xq")
    _dense(x_bscale, torch.uint8, (M, K // 16), "x_bscale")
    _scalar(input_scale, "input_scale")
    _dense(w, torch.uint8, (N, K // 2), "w")
    _dense(w_bscale, torch.uint8, (N, K // 16), "w_bscale")
    _scalar(w_scale2, "w_scale2")
    _scalar(y_scale, "y_scale")
    dev = xq.device
    yq = torch.empty((M, N // 2), dtype=torch.uint8, device=dev) if yq is None else yq
    y_bscale = torch.empty((M, N // 16), dtype=torch.uint8, device=dev) if y_bscale is None else y_bscale
    _dense(yq, torch.uint8, (M, N // 2), "yq")
    _dense(y_bscale, torch.uint8, (M, N // 16), "y_bscale")
    ldy = 0
    if with_y or y is not None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if y is None else y
        _, _, ldy = _rows(y, torch.bfloat16, "y")
    nws = lib.bsq_gemm_nvfp4_quantize_y_workspace_bytes(M, N, K, 1 if y is not None else 0)
    if workspace is None and nws:
        workspace = torch.empty(nws, dtype=torch.uint8, device=dev)
    _check("bsq_gemm_nvfp4_q_quantize_y",
           lib.bsq_gemm_nvfp4_q_quantize_y(_ptr(xq), _ptr(x_bscale), _ptr(input_scale), _ptr(w), _ptr(w_bscale),
                                           _ptr(w_scale2), _ptr(y_scale), _ptr(yq), _ptr(y_bscale),
                                           _ptr(y) if y is not None else None, ldy, M, N, K,
                                           _ptr(workspace) if workspace is not None else None,
                                           _nbytes(workspace), _stream()))
    return yq, y_bscale, y


def _quantized_output(out_format, M, N, y_global, with_y, yq, yq_scale, y, dev):
    """Output tensors of the quantized-output linears: (yq, yq_scale, y or None, ldy)."""
    if out_format == BSQ_FMT_NVFP4:
        _scalar(y_global, "y_global")
        yq = torch.empty((M, N // 2), dtype=torch.uint8, device=dev) if yq is None else yq
        yq_scale = torch.empty((M, N // 16), dtype=torch.uint8, device=dev) if yq_scale is None else yq_scale
        _dense(yq, torch.uint8, (M, N // 2), "yq")
        _dense(yq_scale, torch.uint8, (M, N // 16), "yq_scale")
    else:
        if y_global is not None:
            raise ValueError("an fp8r output takes no global scale")
        yq = torch.empty((M, N), dtype=torch.uint8, device=dev) if yq is None else yq
        yq_scale = torch.empty((M,), dtype=torch.float32, device=dev) if yq_scale is None else yq_scale
        _dense(yq, torch.uint8, (M, N), "yq")
        _dense(yq_scale, torch.float32, (M,), "yq_scale")
    ldy = 0
    if with_y or y is not None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if y is None else y
        _, _, ldy = _rows(y, torch.bfloat16, "y")
    return yq, yq_scale, y, ldy


def _quantize_y_workspace(out_format, M, N, y, workspace, dev):
    n = lib.bsq_gemm_quantize_y_workspace_bytes(out_format, M, N, 1 if y is not None else 0)
    if workspace is None and n:
        workspace = torch.empty((n,), dtype=torch.uint8, device=dev)
    return workspace


def bsq_gemm_fp8r_q_quantize_y(xq, x_scale, w, w_scale, out_format, y_global=None, with_y=False, yq=None,
                               yq_scale=None, y=None, workspace=None):
    """W8A8 GEMM as bsq_gemm_fp8r_q whose output is also returned encoded for the next linear:
    (yq, yq_scale, bf16 y or None) -- nvfp4 (uint8 [M, N/2], uint8 [M, N/16]; y_global [1]) or
    fp8r (uint8 [M, N], fp32 [M])."""
    M, K = xq.shape
    N = w.shape[0]
    _dense(xq, torch.uint8, (M, K), "xq")
    _dense(x_scale, torch.float32, (M,), "x_scale")
    _dense(w, torch.uint8, (N, K), "w")
    _dense(w_scale, torch.float32, (N,), "w_scale")
    yq, yq_scale, y, ldy = _quantized_output(out_format, M, N, y_global, with_y, yq, yq_scale, y, xq.device)
    ws = _quantize_y_workspace(out_format, M, N, y, workspace, xq.device)
    _check("bsq_gemm_fp8r_q_quantize_y", lib.bsq_gemm_fp8r_q_quantize_y(
        _ptr(xq), _ptr(x_scale), _ptr(w), _ptr(w_scale), out_format, _ptr(y_global), _ptr(yq), _ptr(yq_scale),
        _ptr(y), ldy, M, N, K, _ptr(ws), _nbytes(ws), _stream()))
    return yq, yq_scale, y


def bsq_gemm_nvfp4_q_quantize_y_fp8r(xq, x_bscale, input_scale, w, w_bscale, w_scale2, with_y=False, yq=None,
                                     y_rowscale=None, y=None, workspace=None):
    """W4A4 GEMM as bsq_gemm_nvfp4_q whose output is also returned in fp8r for the next linear:
    (E4M3 yq uint8 [M, N], fp32 row scales [M], bf16 y or None)."""
    M, K = xq.shape[0], xq.shape[1] * 2
    N = w.shape[0]
    _dense(xq, torch.uint8, (M, K // 2), "xq")
    _dense(x_bscale, torch.uint8, (M, K // 16), "x_bscale")
    _scalar(input_scale, "input_scale")
    _dense(w, torch.uint8, (N, K // 2), "w")
    _dense(w_bscale, torch.uint8, (N, K // 16), "w_bscale")
    _scalar(w_scale2, "w_scale2")
    yq, y_rowscale, y, ldy = _quantized_output(BSQ_FMT_FP8R, M, N, None, with_y, yq, y_rowscale, y, xq.device)
    ws = _quantize_y_workspace(BSQ_FMT_FP8R, M, N, y, workspace, xq.device)
    _check("bsq_gemm_nvfp4_q_quantize_y_fp8r", lib.bsq_gemm_nvfp4_q_quantize_y_fp8r(
        _ptr(xq), _ptr(x_bscale), _ptr(input_scale), _ptr(w), _ptr(w_bscale), _ptr(w_scale2), _ptr(yq),
        _ptr(y_rowscale), _ptr(y), ldy, M, N, K, _ptr(ws), _nbytes(ws), _stream()))
    return yq, y_rowscale, y


def bsq_gemm_weight_only_quantize_y(w_format, x, w, w_scale, w_scale2, out_format, y_global=None, with_y=False,
                                    yq=None, yq_scale=None, y=None, workspace=None):
    """Weight-only linear (bf16 x [M, K]; nvfp4 w [N, K/2] with uint8 block scales [N, K/16] and
    w_scale2 [1], or E4M3 w [N, K] with fp32 row scales [N] and w_scale2 None) whose output is
    also returned encoded for the next linear: (yq, yq_scale, bf16 y or None), as
    bsq_gemm_fp8r_q_quantize_y."""
    M, K, ldx = _rows(x, torch.bfloat16, "x")
    N = w.shape[0]
    if w_format == BSQ_FMT_NVFP4:
        _dense(w, torch.uint8, (N, K // 2), "w")
        _dense(w_scale, torch.uint8, (N, K // 16), "w_scale")
        _scalar(w_scale2, "w_scale2")
    else:
        _dense(w, torch.uint8, (N, K), "w")
        _dense(w_scale, torch.float32, (N,), "w_scale")
    yq, yq_scale, y, ldy = _quantized_output(out_format, M, N, y_global, with_y, yq, yq_scale, y, x.device)
    ws = _quantize_y_workspace(out_format, M, N, y, workspace, x.device)
    _check("bsq_gemm_weight_only_quantize_y", lib.bsq_gemm_weight_only_quantize_y(
        w_format, _ptr(x), ldx, _ptr(w), _ptr(w_scale), _ptr(w_scale2), out_format, _ptr(y_global), _ptr(yq),
        _ptr(yq_scale), _ptr(y), ldy, M, N, K, _ptr(ws), _nbytes(ws), _stream()))
    return yq, yq_scale, y


def bsq_dequant_to_bf16(fmt, w, w_scale, w_scale2=None, out=None):
    """Dequantize fp8r (w [N, K], w_scale fp32 [N]) or nvfp4 (w [N, K/2], w_scale uint8 [N, K/16],
    w_scale2 fp32 [1]) weights to bf16 [N, K]."""
    N = w.shape[0]
    K = w.shape[1] * (2 if fmt == BSQ_FMT_NVFP4 else 1)
    _dense(w, torch.uint8, tuple(w.shape), "w")
    if fmt == BSQ_FMT_NVFP4:
        _dense(w_scale, torch.uint8, (N, K // 16), "w_scale")
        _scalar(w_scale2, "w_scale2")
    else:
        _dense(w_scale, torch.float32, (N,), "w_scale")
    out = torch.empty((N, K), dtype=torch.bfloat16, device=w.device) if out is None else out
    _dense(out, torch.bfloat16, (N, K), "out")
    _check("bsq_dequant_to_bf16", lib.bsq_dequant_to_bf16(fmt, _ptr(w), _ptr(w_scale), _ptr(w_scale2), N, K,
                                                          _ptr(out), _stream()))
    return out
