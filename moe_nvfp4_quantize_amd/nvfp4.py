"""Python binding of libnvfp4.so (C ABI in include/nvfp4.h).

Argument marshalling only: every function here checks tensor placement and
dtypes, allocates outputs and workspaces with torch when the caller did not pass
them, and calls the C entry point of the same name on torch's current HIP
stream.  All arithmetic runs in the library's HIP kernels; if the library is
missing, the first call raises -- there is no fallback.

Layouts follow the C header: an NVFP4 tensor is ``(q, s, g)`` with q uint8
[rows, cols/2] (two E2M1 codes per byte, even element in the low nibble),
s uint8 [rows, cols/16] (E4M3FN block scale codes) and g float32 [1] (the global
decode scale), all on the GPU.
"""

import atexit
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

NVFP4_OK, NVFP4_ERR_INVALID_ARG, NVFP4_ERR_UNSUPPORTED, NVFP4_ERR_HIP = 0, 1, 2, 3
NVFP4_F32, NVFP4_BF16 = 0, 1
NVFP4_EPI_NONE, NVFP4_EPI_SILU_GATE = 0, 1

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t

# name -> (restype, argtypes); the order follows include/nvfp4.h
SIGNATURES = {
    "nvfp4_abi_version": (ctypes.c_int, []),
    "nvfp4_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "nvfp4_quantize_workspace_size": (_SZ, [_I64, _I64]),
    "nvfp4_quantize": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _I64, _P, _P, _P, ctypes.c_int,
                                      _P, _SZ, _P]),
    "nvfp4_quantize_noalloc": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _I64, _P, _P, _P,
                                              ctypes.c_int, _P]),
    "nvfp4_quantize_batched_workspace_size": (_SZ, [_I64, _I64, _I64]),
    "nvfp4_quantize_batched": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _I64, _P, _P, _P, _P,
                                              _SZ, _P]),
    "nvfp4_qdq": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _I64, _P, _I64, _P, ctypes.c_int, _P,
                                 _SZ, _P]),
    "nvfp4_quantize_4over6": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _I64, _P, _P, _P, _P,
                                             _SZ, _P]),
    "nvfp4_gemm": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, ctypes.c_int, _I64,
                                  _P]),
    "nvfp4_fp8_quantize_workspace_size": (_SZ, [_I64, _I64]),
    "nvfp4_fp8_quantize": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _I64, _P, _P, ctypes.c_int, _P,
                                          _SZ, _P]),
    "nvfp4_fp8_gemm": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _P, ctypes.c_int, _I64, _P]),
    "nvfp4_moe_route_workspace_size": (_SZ, [_I64, _I32, _I32]),
    "nvfp4_moe_route": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "nvfp4_moe_grouped_gemm": (ctypes.c_int, [_P, _P, _P, _I64, _P, _P, _I32, _I64, _P, _P, _P,
                                              _I64, _I64, _P, ctypes.c_int, ctypes.c_int, _P]),
    "nvfp4_moe_grouped_gemm_silu_nvfp4": (ctypes.c_int, [_P, _P, _P, _I64, _P, _P, _I32, _I64, _P, _P,
                                                         _P, _I64, _I64, _P, _P, _P, _P]),
    "nvfp4_moe_combine": (ctypes.c_int, [_P, ctypes.c_int, _P, _P, _I64, _I32, _I64, _I64, _P,
                                         ctypes.c_int, _P]),
}

_lib = None


class NVFP4Error(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)}")


def load_library(path=LIB_PATH):
    """Load libnvfp4.so (once) and declare every exported signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m moe_nvfp4_quantize_amd.build` "
            "(hipcc for gfx950); there is no fallback implementation")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status):
    return load_library().nvfp4_status_string(int(status)).decode()


def _check(fn, status):
    if status != NVFP4_OK:
        raise NVFP4Error(fn, status)


def _torch_stream(stream=None):
    return torch.cuda.current_stream() if stream is None else stream


def _stream(stream=None):
    return ctypes.c_void_p(_torch_stream(stream).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _dtype_code(dtype):
    if dtype == torch.float32:
        return NVFP4_F32
    if dtype == torch.bfloat16:
        return NVFP4_BF16
    raise TypeError(f"unsupported dtype {dtype}; float32 or bfloat16 expected")


def _on_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")


def _ws(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# nvfp4_quantize's workspace must start zero-filled and then be reused: one per
# (device, stream), grown (zero-filled again) when a larger one is needed.  It is
# allocated and filled on the stream the kernels run on, so the fill is ordered
# before them, and the caching allocator only hands a replaced buffer to later
# work on that same stream, after the kernels that still read it.
_QWS = {}


def _quantize_ws(nbytes, device, stream):
    s = _torch_stream(stream)
    key = (torch.device(device).index, int(s.cuda_stream))
    ws = _QWS.get(key)
    if ws is None or ws.numel() < nbytes:
        with torch.cuda.stream(s):
            ws = torch.zeros(max(int(nbytes), 4096), dtype=torch.uint8, device=device)
        _QWS[key] = ws
    return ws


@atexit.register
def _release_workspaces():
    """Drop the cached workspaces while the runtime is fully up: wait for the
    kernels that use them, then release the tensors (before interpreter
    teardown frees module state in no particular order)."""
    if not _QWS:
        return
    try:
        for dev in {k[0] for k in _QWS}:
            torch.cuda.synchronize(dev)
    except Exception:  # teardown: nothing left to protect
        pass
    _QWS.clear()


# ------------------------------------------------------------------ quantize


def nvfp4_quantize(x, g=None, out=None, stream=None):
    """Quantize a 2-D f32/bf16 GPU tensor along its last dim -> (q, s, g).

    ``g=None``: dynamic global scale (amax/2688), written into the returned g.
    ``g`` given (float32 [1] GPU tensor): static global scale, used as is.
    ``out``: optional preallocated (q, s, g).
    """
    lib = load_library()
    _on_gpu(x)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit stride along the last dim")
    rows, cols = x.shape
    if out is None:
        q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
        s = torch.empty((rows, cols // 16), dtype=torch.uint8, device=x.device)
        gg = torch.empty(1, dtype=torch.float32, device=x.device)
    else:
        q, s, gg = out
    static = g is not None
    if static and gg.data_ptr() != g.data_ptr():
        gg.copy_(g.reshape(1))
    hs = _stream(stream)
    ws = _quantize_ws(lib.nvfp4_quantize_workspace_size(rows, cols), x.device, stream)
    st = lib.nvfp4_quantize(_ptr(x), _dtype_code(x.dtype), rows, cols, x.stride(0) if rows else cols,
                            _ptr(q), _ptr(s), _ptr(gg), int(static), _ptr(ws), ws.numel(), hs)
    _check("nvfp4_quantize", st)
    return q, s, gg


def nvfp4_quantize_noalloc(x, g=None, out=None, stream=None):
    """nvfp4_quantize through the allocation-free entry point: the library's own
    per-GPU scratch replaces the workspace (calls overlapping on one GPU race).
    Arguments and results as for :func:`nvfp4_quantize`; with ``out`` given,
    nothing is allocated at all."""
    lib = load_library()
    _on_gpu(x)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit stride along the last dim")
    rows, cols = x.shape
    if out is None:
        q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
        s = torch.empty((rows, cols // 16), dtype=torch.uint8, device=x.device)
        gg = torch.empty(1, dtype=torch.float32, device=x.device)
    else:
        q, s, gg = out
    static = g is not None
    if static and gg.data_ptr() != g.data_ptr():
        gg.copy_(g.reshape(1))
    st = lib.nvfp4_quantize_noalloc(_ptr(x), _dtype_code(x.dtype), rows, cols,
                                    x.stride(0) if rows else cols, _ptr(q), _ptr(s), _ptr(gg),
                                    int(static), _stream(stream))
    _check("nvfp4_quantize_noalloc", st)
    return q, s, gg


def nvfp4_qdq(x, g=None, out=None, stream=None):
    """Quantize-dequantize a 2-D f32/bf16 GPU tensor -> (y of x's dtype, g).

    ``g=None``: dynamic global scale (written into the returned g); a float32 [1] GPU
    tensor: frozen global scale.  ``out`` may be x itself (in place)."""
    lib = load_library()
    _on_gpu(x)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit stride along the last dim")
    rows, cols = x.shape
    y = torch.empty_like(x) if out is None else out
    if y.shape != x.shape or y.dtype != x.dtype or y.stride(1) != 1:
        raise ValueError("out must match x in shape and dtype")
    static = g is not None
    gg = g.reshape(1) if static else torch.empty(1, dtype=torch.float32, device=x.device)
    hs = _stream(stream)
    ws = _quantize_ws(lib.nvfp4_quantize_workspace_size(rows, cols), x.device, stream)
    st = lib.nvfp4_qdq(_ptr(x), _dtype_code(x.dtype), rows, cols, x.stride(0) if rows else cols,
                       _ptr(y), y.stride(0) if rows else cols, _ptr(gg), int(static), _ptr(ws),
                       ws.numel(), hs)
    _check("nvfp4_qdq", st)
    return y, gg


def nvfp4_quantize_4over6(x, stream=None):
    """Offline quantize with four-over-six block scales of a 2-D [rows, cols] or batched
    [B, rows, cols] contiguous GPU tensor -> (q, s, g); one global scale per matrix."""
    lib = load_library()
    _on_gpu(x)
    if not x.is_contiguous() or x.dim() not in (2, 3):
        raise ValueError("x must be a contiguous 2-D or 3-D tensor")
    single = x.dim() == 2
    xb = x.unsqueeze(0) if single else x
    B, rows, cols = xb.shape
    q = torch.empty((B, rows, cols // 2), dtype=torch.uint8, device=x.device)
    s = torch.empty((B, rows, cols // 16), dtype=torch.uint8, device=x.device)
    g = torch.empty(B, dtype=torch.float32, device=x.device)
    ws = _ws(lib.nvfp4_quantize_batched_workspace_size(B, rows, cols), x.device)
    st = lib.nvfp4_quantize_4over6(_ptr(xb), _dtype_code(x.dtype), B, rows, cols, _ptr(q), _ptr(s),
                                   _ptr(g), _ptr(ws), ws.numel(), _stream(stream))
    _check("nvfp4_quantize_4over6", st)
    return (q[0], s[0], g[:1]) if single else (q, s, g)


def nvfp4_quantize_batched(x, stream=None):
    """Quantize each matrix of a contiguous [B, rows, cols] tensor with its own global scale."""
    lib = load_library()
    _on_gpu(x)
    if x.dim() != 3 or not x.is_contiguous():
        raise ValueError("x must be a contiguous 3-D tensor")
    b, rows, cols = x.shape
    q = torch.empty((b, rows, cols // 2), dtype=torch.uint8, device=x.device)
    s = torch.empty((b, rows, cols // 16), dtype=torch.uint8, device=x.device)
    g = torch.empty(b, dtype=torch.float32, device=x.device)
    ws = _ws(lib.nvfp4_quantize_batched_workspace_size(b, rows, cols), x.device)
    st = lib.nvfp4_quantize_batched(_ptr(x), _dtype_code(x.dtype), b, rows, cols, _ptr(q), _ptr(s),
                                    _ptr(g), _ptr(ws), ws.numel(), _stream(stream))
    _check("nvfp4_quantize_batched", st)
    return q, s, g


# ---------------------------------------------------------------------- GEMM


def nvfp4_gemm(a, b, out_dtype=torch.bfloat16, out=None, stream=None):
    """C = A_hat @ B_hat^T for NVFP4 tensors a = (q, s, g) [M, K], b = (q, s, g) [N, K]."""
    lib = load_library()
    a_q, a_s, a_g = a
    b_q, b_s, b_g = b
    _on_gpu(a_q, a_s, a_g, b_q, b_s, b_g)
    M, K = a_q.shape[0], a_q.shape[1] * 2
    N = b_q.shape[0]
    if b_q.shape[1] * 2 != K:
        raise ValueError("K mismatch between A and B")
    for t in (a_q, a_s, b_q, b_s):
        if not t.is_contiguous():
            raise ValueError("q and s must be contiguous")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a_q.device)
    st = lib.nvfp4_gemm(_ptr(a_q), _ptr(a_s), _ptr(a_g), _ptr(b_q), _ptr(b_s), _ptr(b_g), M, N, K,
                        _ptr(out), _dtype_code(out.dtype), out.stride(0) if M else N,
                        _stream(stream))
    _check("nvfp4_gemm", st)
    return out


# ----------------------------------------------------------------------- FP8


def nvfp4_fp8_quantize(x, g=None, out=None, stream=None):
    """FP8 W8A8 quantize of a 2-D f32/bf16 GPU tensor -> (q uint8 [rows, cols], g float32 [1]).

    ``g=None``: dynamic per-tensor scale (amax/448), written into the returned g;
    a float32 [1] GPU tensor: static scale, used as is.  ``out``: optional (q, g)."""
    lib = load_library()
    _on_gpu(x)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit stride along the last dim")
    rows, cols = x.shape
    if out is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
        gg = torch.empty(1, dtype=torch.float32, device=x.device)
    else:
        q, gg = out
    static = g is not None
    if static and gg.data_ptr() != g.data_ptr():
        gg.copy_(g.reshape(1))
    hs = _stream(stream)
    ws = _quantize_ws(lib.nvfp4_fp8_quantize_workspace_size(rows, cols), x.device, stream)
    st = lib.nvfp4_fp8_quantize(_ptr(x), _dtype_code(x.dtype), rows, cols, x.stride(0) if rows else cols,
                                _ptr(q), _ptr(gg), int(static), _ptr(ws), ws.numel(), hs)
    _check("nvfp4_fp8_quantize", st)
    return q, gg


def nvfp4_fp8_gemm(a, b, out_dtype=torch.bfloat16, out=None, stream=None):
    """C = A_hat @ B_hat^T for FP8 tensors a = (q, g) [M, K], b = (q, g) [N, K]."""
    lib = load_library()
    a_q, a_g = a
    b_q, b_g = b
    _on_gpu(a_q, a_g, b_q, b_g)
    M, K = a_q.shape
    N = b_q.shape[0]
    if b_q.shape[1] != K:
        raise ValueError("K mismatch between A and B")
    if not (a_q.is_contiguous() and b_q.is_contiguous()):
        raise ValueError("q must be contiguous")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a_q.device)
    st = lib.nvfp4_fp8_gemm(_ptr(a_q), _ptr(a_g), _ptr(b_q), _ptr(b_g), M, N, K, _ptr(out),
                            _dtype_code(out.dtype), out.stride(0) if M else N, _stream(stream))
    _check("nvfp4_fp8_gemm", st)
    return out


# ----------------------------------------------------------------------- MoE


def nvfp4_moe_route(logits, k, stream=None):
    """Top-k routing + permutation -> dict(topk_ids, topk_w, offsets, src_row, inv)."""
    lib = load_library()
    _on_gpu(logits)
    if logits.dtype != torch.float32 or not logits.is_contiguous():
        raise ValueError("logits must be contiguous float32")
    T, E = logits.shape
    dev = logits.device
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    src_row = torch.empty(T * k, dtype=torch.int32, device=dev)
    inv = torch.empty((T, k), dtype=torch.int32, device=dev)
    ws = _ws(lib.nvfp4_moe_route_workspace_size(T, E, k), dev)
    st = lib.nvfp4_moe_route(_ptr(logits), T, E, k, _ptr(ids), _ptr(w), _ptr(offsets),
                             _ptr(src_row), _ptr(inv), _ptr(ws), ws.numel(), _stream(stream))
    _check("nvfp4_moe_route", st)
    return dict(topk_ids=ids, topk_w=w, offsets=offsets, src_row=src_row, inv=inv)


def nvfp4_moe_grouped_gemm(a, src_row, offsets, R, w, epilogue=NVFP4_EPI_NONE,
                           out_dtype=torch.float32, out=None, stream=None):
    """Grouped GEMM over expert segments; a = (q, s, g) source rows, w = stacked expert weights."""
    lib = load_library()
    a_q, a_s, a_g = a
    w_q, w_s, w_g = w
    _on_gpu(a_q, a_s, a_g, src_row, offsets, w_q, w_s, w_g)
    E, N, khalf = w_q.shape
    K = khalf * 2
    if a_q.shape[1] * 2 != K:
        raise ValueError("K mismatch between activations and expert weights")
    n_out = N // 2 if epilogue == NVFP4_EPI_SILU_GATE else N
    if out is None:
        out = torch.empty((R, n_out), dtype=out_dtype, device=a_q.device)
    st = lib.nvfp4_moe_grouped_gemm(_ptr(a_q), _ptr(a_s), _ptr(a_g), a_q.shape[0], _ptr(src_row),
                                    _ptr(offsets), E, R, _ptr(w_q), _ptr(w_s), _ptr(w_g), N, K,
                                    _ptr(out), _dtype_code(out.dtype), epilogue, _stream(stream))
    _check("nvfp4_moe_grouped_gemm", st)
    return out


def nvfp4_moe_grouped_gemm_silu_nvfp4(a, src_row, offsets, R, w, h_g, out=None, stream=None):
    """Grouped gate_up GEMM whose SiLU-gate epilogue writes h = SiLU(gate) * up as NVFP4 under the
    static global scale h_g (a one-element float32 device tensor).  Returns (h_q, h_s, h_g)."""
    lib = load_library()
    a_q, a_s, a_g = a
    w_q, w_s, w_g = w
    _on_gpu(a_q, a_s, a_g, src_row, offsets, w_q, w_s, w_g, h_g)
    E, N, khalf = w_q.shape
    K = khalf * 2
    if a_q.shape[1] * 2 != K:
        raise ValueError("K mismatch between activations and expert weights")
    I = N // 2
    if out is None:
        out = (torch.empty((R, I // 2), dtype=torch.uint8, device=a_q.device),
               torch.empty((R, I // 16), dtype=torch.uint8, device=a_q.device))
    h_q, h_s = out
    st = lib.nvfp4_moe_grouped_gemm_silu_nvfp4(_ptr(a_q), _ptr(a_s), _ptr(a_g), a_q.shape[0],
                                               _ptr(src_row), _ptr(offsets), E, R, _ptr(w_q),
                                               _ptr(w_s), _ptr(w_g), N, K, _ptr(h_q), _ptr(h_s),
                                               _ptr(h_g), _stream(stream))
    _check("nvfp4_moe_grouped_gemm_silu_nvfp4", st)
    return h_q, h_s, h_g


def nvfp4_moe_combine(y, topk_w, inv, out_dtype=torch.bfloat16, out=None, stream=None):
    """out[t] = sum_j topk_w[t, j] * y[inv[t, j]]."""
    lib = load_library()
    _on_gpu(y, topk_w, inv)
    T, k = inv.shape
    R, H = y.shape
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=y.device)
    st = lib.nvfp4_moe_combine(_ptr(y), _dtype_code(y.dtype), _ptr(topk_w), _ptr(inv), T, k, H, R,
                               _ptr(out), _dtype_code(out.dtype), _stream(stream))
    _check("nvfp4_moe_combine", st)
    return out


def moe_layer(x, logits, k, w_gate_up, w_down, stream=None, keep=False, inter_dtype=torch.float32):
    """The routed-expert layer as a sequence of library calls.

    x bf16/f32 [T, H]; w_gate_up and w_down are quantized expert stacks
    (q, s, g) for [E, 2I, H] and [E, H, I].  ``inter_dtype`` (float32 or
    bfloat16) is the storage type of the intermediates h and y.  Returns the
    bf16 output, or with ``keep=True`` a dict of every intermediate.
    """
    T = x.shape[0]
    r = nvfp4_moe_route(logits, k, stream=stream)
    R = T * k
    xq = nvfp4_quantize(x, stream=stream)
    h = nvfp4_moe_grouped_gemm(xq, r["src_row"], r["offsets"], R, w_gate_up,
                               epilogue=NVFP4_EPI_SILU_GATE, out_dtype=inter_dtype, stream=stream)
    hq = nvfp4_quantize(h, stream=stream)
    y = nvfp4_moe_grouped_gemm(hq, None, r["offsets"], R, w_down, out_dtype=inter_dtype,
                               stream=stream)
    out = nvfp4_moe_combine(y, r["topk_w"], r["inv"], stream=stream)
    if keep:
        return dict(r, xq=xq, h=h, hq=hq, y=y, out=out)
    return out
