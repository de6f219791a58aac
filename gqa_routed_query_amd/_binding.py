"""ctypes binding of libgqa.so: argument marshalling only.

Each wrapper checks the torch tensors it is given (device, dtype, layout,
shape), allocates outputs when the caller passes none, and calls the C entry
point of the same name with raw device pointers and the current HIP stream.
No attention arithmetic happens here, and there is no fallback: if the library
is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_PKG_DIR, "libgqa.so")

GQA_F32 = 0
GQA_BF16 = 1
_STATUS = {0: "GQA_OK", 1: "GQA_ERR_INVALID_ARG", 2: "GQA_ERR_UNSUPPORTED",
           3: "GQA_ERR_WORKSPACE", 4: "GQA_ERR_NO_DEVICE", 5: "GQA_ERR_HIP"}


class GqaError(RuntimeError):
    """A libgqa entry point returned a non-OK status."""

    def __init__(self, fn: str, status: int, detail: str):
        self.status = status
        super().__init__(f"{fn}: {_STATUS.get(status, status)}: {detail}")


def _load():
    if not os.path.exists(lib_path):
        raise ImportError(
            f"{lib_path} is not built; run `python gqa_routed_query_amd/build.py` "
            "(hipcc, gfx950)")
    lib = ctypes.CDLL(lib_path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.gqa_abi_version.restype = i32
    lib.gqa_abi_version.argtypes = []
    lib.gqa_prefill.restype = i32
    lib.gqa_prefill.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp]
    lib.gqa_decode_workspace_bytes.restype = sz
    lib.gqa_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.gqa_decode.restype = i32
    lib.gqa_decode.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32,
                               vp, sz, vp]
    lib.gqa_decode_noalloc.restype = i32
    lib.gqa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, vp]
    lib.gqe_routed_prefill.restype = i32
    lib.gqe_routed_prefill.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32,
                                       i32, i32, i32, f32, i32, vp, sz, vp]
    lib.gqe_workspace_bytes.restype = sz
    lib.gqe_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.gqe_routed_decode.restype = i32
    lib.gqe_routed_decode.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32,
                                      i32, i32, i32, f32, vp, sz, vp]
    lib.gqa_peak_hbm_read.restype = i32
    lib.gqa_peak_hbm_read.argtypes = [vp, sz, vp, vp]
    lib.gqa_peak_mfma_bf16.restype = i32
    lib.gqa_peak_mfma_bf16.argtypes = [vp, i32, vp, ctypes.POINTER(ctypes.c_double), vp]
    lib.gqa_peak_attn_tile.restype = i32
    lib.gqa_peak_attn_tile.argtypes = [vp, i32, f32, vp, ctypes.POINTER(ctypes.c_double), vp]
    lib.gqe_prefill_build.restype = i32
    lib.gqe_prefill_build.argtypes = [vp, vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, i32, i32,
                                      i32, i32, i32, i32, i32, f32, i32, vp]
    lib.gqe_router.restype = i32
    lib.gqe_router.argtypes = [vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    lib.gqa_kv_cache_bytes.restype = ctypes.c_uint64
    lib.gqa_kv_cache_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.gqa_status_string.restype = ctypes.c_char_p
    lib.gqa_status_string.argtypes = [i32]
    lib.gqa_last_error.restype = ctypes.c_char_p
    lib.gqa_last_error.argtypes = []
    return lib


_lib = _load()

_DT = {torch.float32: GQA_F32, torch.bfloat16: GQA_BF16}


def abi_version() -> int:
    return int(_lib.gqa_abi_version())


def status_string(status: int) -> str:
    return _lib.gqa_status_string(status).decode()


def last_error() -> str:
    return _lib.gqa_last_error().decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise GqaError(fn, status, last_error())


def _dt(t: torch.Tensor, name: str) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"{name}: dtype {t.dtype} is not float32 or bfloat16")
    return _DT[t.dtype]


def _dev(*tensors):
    dev = tensors[0].device
    for t in tensors:
        if t.device.type != "cuda":
            raise ValueError("libgqa tensors must live on the GPU")
        if t.device != dev:
            raise ValueError("all tensors must be on the same device")
        if not t.is_contiguous():
            raise ValueError("libgqa tensors must be contiguous")
    return dev


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def gqa_kv_cache_bytes(B: int, n_kv: int, T: int, d: int, dtype=torch.bfloat16) -> int:
    """Bytes of a one-layer KV cache: 2 * n_kv * d * T * sizeof(dtype) * B."""
    return int(_lib.gqa_kv_cache_bytes(B, n_kv, T, d, _DT[dtype]))


def gqa_decode_workspace_bytes(B: int, h: int, g: int, T_max: int, d: int) -> int:
    return int(_lib.gqa_decode_workspace_bytes(B, h, g, T_max, d))


def gqa_prefill(q, k, v, causal: bool = True, scale: float | None = None, out=None,
                out_dtype=None):
    """GQA prefill. q [B,h,T,d], k/v [B,g,T,d] -> out [B,h,T,d]."""
    dev = _dev(q, k, v)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("expected q [B,h,T,d] and k, v [B,g,T,d]")
    B, h, T, d = q.shape
    if k.shape[0] != B or k.shape[2:] != (T, d):
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    g = k.shape[1]
    out_dtype = out_dtype or (out.dtype if out is not None else q.dtype)
    if out is None:
        out = torch.empty((B, h, T, d), dtype=out_dtype, device=dev)
    elif out.shape != q.shape or out.dtype != out_dtype:
        raise ValueError("out must be [B,h,T,d] of out_dtype")
    _dev(q, out)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = _lib.gqa_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                          B, h, g, T, d, _dt(q, "q"), _dt(out, "out"), scale,
                          int(bool(causal)), _stream(dev))
    _check("gqa_prefill", st)
    return out


def gqa_decode(q, k_cache, v_cache, lens, scale: float | None = None, out=None,
               out_dtype=None, workspace=None):
    """GQA decode. q [B,h,d], caches [B,g,T_max,d], lens [B] int32 -> out [B,h,d]."""
    dev = _dev(q, k_cache, v_cache, lens)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("expected q [B,h,d] and caches [B,g,T_max,d]")
    B, h, d = q.shape
    if k_cache.shape[0] != B or k_cache.shape[3] != d:
        raise ValueError("cache shape does not match q")
    if lens.dtype != torch.int32 or lens.shape != (B,):
        raise ValueError("lens must be int32 [B]")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and the caches must share one dtype")
    g, T_max = k_cache.shape[1], k_cache.shape[2]
    out_dtype = out_dtype or (out.dtype if out is not None else q.dtype)
    if out is None:
        out = torch.empty((B, h, d), dtype=out_dtype, device=dev)
    elif out.shape != q.shape or out.dtype != out_dtype:
        raise ValueError("out must be [B,h,d] of out_dtype")
    _dev(q, out)
    need = gqa_decode_workspace_bytes(B, h, g, T_max, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = _lib.gqa_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), lens.data_ptr(),
                         out.data_ptr(), B, h, g, T_max, d, _dt(q, "q"), _dt(out, "out"),
                         scale, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                         _stream(dev))
    _check("gqa_decode", st)
    return out


def gqa_decode_noalloc(q, k_cache, v_cache, lens, out, scale: float | None = None):
    """GQA decode with the split partials in the library's static device
    scratch (the entry point allocates nothing; ``out`` [B,h,d] is the
    caller's). Calls that overlap on one device race."""
    dev = _dev(q, k_cache, v_cache, lens, out)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("expected q [B,h,d] and caches [B,g,T_max,d]")
    B, h, d = q.shape
    if k_cache.shape[0] != B or k_cache.shape[3] != d:
        raise ValueError("cache shape does not match q")
    if lens.dtype != torch.int32 or lens.shape != (B,):
        raise ValueError("lens must be int32 [B]")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and the caches must share one dtype")
    if out.shape != q.shape:
        raise ValueError("out must be [B,h,d]")
    g, T_max = k_cache.shape[1], k_cache.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = _lib.gqa_decode_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), lens.data_ptr(),
                                 out.data_ptr(), B, h, g, T_max, d, _dt(q, "q"), _dt(out, "out"), scale,
                                 _stream(dev))
    _check("gqa_decode_noalloc", st)
    return out


def gqe_workspace_bytes(B: int, h: int, g: int, T: int, d: int, top_k: int) -> int:
    """Bytes of workspace gqe_routed_prefill can use at this shape (0: none)."""
    return int(_lib.gqe_workspace_bytes(B, h, g, T, d, top_k))


def gqe_routed_prefill(q, k, v, router_logits, top_k: int, causal: bool = True,
                       scale: float | None = None, out=None, out_dtype=None, workspace=True):
    """GQE routed prefill -> (out [B,h,T,d], idx [B,T,g,k] int32, gate [B,T,g,k] fp32).

    workspace: True (default) allocates the gqe_workspace_bytes(...) the call
    can use, None or False passes none, or a uint8 device tensor to use."""
    dev = _dev(q, k, v, router_logits)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("expected q [B,h,T,d] and k, v [B,g,T,d]")
    B, h, T, d = q.shape
    g = k.shape[1]
    if k.shape[0] != B or k.shape[2:] != (T, d):
        raise ValueError("k/v shape does not match q")
    if router_logits.dtype != torch.float32 or router_logits.shape != (B, T, h):
        raise ValueError("router_logits must be float32 [B,T,h]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    out_dtype = out_dtype or (out.dtype if out is not None else q.dtype)
    if out is None:
        out = torch.empty((B, h, T, d), dtype=out_dtype, device=dev)
    elif out.shape != q.shape or out.dtype != out_dtype:
        raise ValueError("out must be [B,h,T,d] of out_dtype")
    _dev(q, out)
    kk = max(int(top_k), 1)
    idx = torch.empty((B, T, g, kk), dtype=torch.int32, device=dev)
    gate = torch.empty((B, T, g, kk), dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if workspace is True:
        nbytes = gqe_workspace_bytes(B, h, g, T, d, int(top_k)) if 1 <= top_k <= h // max(g, 1) else 0
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None
    elif workspace is False:
        workspace = None
    if workspace is not None:
        _dev(q, workspace)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _lib.gqe_routed_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                 router_logits.data_ptr(), int(top_k), out.data_ptr(),
                                 idx.data_ptr(), gate.data_ptr(), B, h, g, T, d,
                                 _dt(q, "q"), _dt(out, "out"), scale, int(bool(causal)),
                                 ws_ptr, ws_bytes, _stream(dev))
    _check("gqe_routed_prefill", st)
    return out, idx, gate


def gqe_routed_decode(q, k_cache, v_cache, lens, router_logits, top_k: int,
                      scale: float | None = None, out=None, out_dtype=None, workspace=None):
    """GQE routed decode. q [B,h,d], caches [B,g,T_max,d], lens [B] int32,
    router_logits [B,h] float32 -> (out [B,h,d], idx [B,g,k] int32, gate [B,g,k] fp32)."""
    dev = _dev(q, k_cache, v_cache, lens, router_logits)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("expected q [B,h,d] and caches [B,g,T_max,d]")
    B, h, d = q.shape
    if k_cache.shape[0] != B or k_cache.shape[3] != d:
        raise ValueError("cache shape does not match q")
    if lens.dtype != torch.int32 or lens.shape != (B,):
        raise ValueError("lens must be int32 [B]")
    if router_logits.dtype != torch.float32 or router_logits.shape != (B, h):
        raise ValueError("router_logits must be float32 [B,h]")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and the caches must share one dtype")
    g, T_max = k_cache.shape[1], k_cache.shape[2]
    out_dtype = out_dtype or (out.dtype if out is not None else q.dtype)
    if out is None:
        out = torch.empty((B, h, d), dtype=out_dtype, device=dev)
    elif out.shape != q.shape or out.dtype != out_dtype:
        raise ValueError("out must be [B,h,d] of out_dtype")
    _dev(q, out)
    kk = max(int(top_k), 1)
    idx = torch.empty((B, g, kk), dtype=torch.int32, device=dev)
    gate = torch.empty((B, g, kk), dtype=torch.float32, device=dev)
    need = gqa_decode_workspace_bytes(B, h, g, T_max, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = _lib.gqe_routed_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                lens.data_ptr(), router_logits.data_ptr(), int(top_k),
                                out.data_ptr(), idx.data_ptr(), gate.data_ptr(), B, h, g, T_max, d,
                                _dt(q, "q"), _dt(out, "out"), scale, workspace.data_ptr(),
                                workspace.numel() * workspace.element_size(), _stream(dev))
    _check("gqe_routed_decode", st)
    return out, idx, gate


def gqe_router(x, w_r, g: int, top_k: int, return_logits: bool = True):
    """GQE router with its projection. x [..., d_model] bf16 (tokens),
    w_r [h, d_model] bf16 -> (logits [..., h] fp32 or None, idx [..., g, k] int32,
    gate [..., g, k] fp32)."""
    dev = _dev(x, w_r)
    if w_r.dim() != 2 or x.shape[-1] != w_r.shape[1]:
        raise ValueError("expected x [..., d_model] and w_r [h, d_model]")
    if x.dtype != w_r.dtype:
        raise TypeError("x and w_r must share one dtype")
    if not x.is_contiguous() or not w_r.is_contiguous():
        raise ValueError("x and w_r must be contiguous")
    lead = tuple(x.shape[:-1])
    n_tok = 1
    for s_ in lead:
        n_tok *= s_
    h, d_model = w_r.shape
    kk = max(int(top_k), 1)
    idx = torch.empty(lead + (g, kk), dtype=torch.int32, device=dev)
    gate = torch.empty(lead + (g, kk), dtype=torch.float32, device=dev)
    logits = torch.empty(lead + (h,), dtype=torch.float32, device=dev) if return_logits else None
    st = _lib.gqe_router(x.data_ptr(), w_r.data_ptr(), int(top_k),
                         logits.data_ptr() if logits is not None else None, idx.data_ptr(),
                         gate.data_ptr(), n_tok, d_model, h, int(g), _dt(x, "x"), _stream(dev))
    _check("gqe_router", st)
    return logits, idx, gate


def peak_hbm_read(buf, xor_out=None):
    """Peak microbenchmark: read every 16-byte word of buf (a contiguous device
    tensor, nbytes a multiple of 16) once. Returns xor_out, an int32 [1] device
    tensor into which the XOR of all 32-bit words of buf is folded (zeroed here
    when not given)."""
    dev = _dev(buf)
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    if xor_out is None:
        xor_out = torch.zeros(1, dtype=torch.int32, device=dev)
    st = _lib.gqa_peak_hbm_read(buf.data_ptr(), buf.numel() * buf.element_size(), xor_out.data_ptr(),
                                _stream(dev))
    _check("gqa_peak_hbm_read", st)
    return xor_out


def peak_mfma_bf16(operands, iters: int, sum_out=None):
    """Peak microbenchmark: the MFMA-only loop. operands: bf16 device tensor of
    1024 values (64 A fragments of 8, then 64 B fragments). Returns (sum_out,
    flops): sum_out, a float32 [1] device tensor, receives the sum of all
    accumulators; flops is the work the launch performs."""
    dev = _dev(operands)
    if operands.dtype != torch.bfloat16 or operands.numel() != 1024 or not operands.is_contiguous():
        raise ValueError("operands must be 1024 contiguous bf16 values")
    if sum_out is None:
        sum_out = torch.zeros(1, dtype=torch.float32, device=dev)
    flops = ctypes.c_double(0.0)
    st = _lib.gqa_peak_mfma_bf16(operands.data_ptr(), int(iters), sum_out.data_ptr(), ctypes.byref(flops),
                                 _stream(dev))
    _check("gqa_peak_mfma_bf16", st)
    return sum_out, flops.value


def peak_attn_tile(qkv, iters: int, scale: float | None = None, out=None):
    """Peak microbenchmark: the prefill's attention tile loop on register
    operands. qkv: bf16 device tensor [3, 32, 128] (q, k, v of one tile).
    Returns (out, flops): out [32, 128] float32, the attention of the 32
    queries over the 32 keys as one wave computed it; flops, the work of the
    launch."""
    dev = _dev(qkv)
    if qkv.dtype != torch.bfloat16 or tuple(qkv.shape) != (3, 32, 128):
        raise ValueError("qkv must be a contiguous bf16 tensor [3, 32, 128]")
    if out is None:
        out = torch.empty((32, 128), dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(128) if scale is None else float(scale)
    flops = ctypes.c_double(0.0)
    st = _lib.gqa_peak_attn_tile(qkv.data_ptr(), int(iters), scale, out.data_ptr(), ctypes.byref(flops),
                                 _stream(dev))
    _check("gqa_peak_attn_tile", st)
    return out, flops.value


def gqe_prefill_build(q, q_shared, k, v, router_logits, top_k: int, shared_kv: int = 0,
                      causal: bool = True, scale: float | None = None, out_dtype=None):
    """GQE output build. q [B,h,T,d], q_shared [B,T,d], k/v [B,g,T,d], router_logits
    [B,T,h] -> (concat [B,T,g,k,d], wsum [B,T,g,d], shared [B,T,d], idx, gate)."""
    dev = _dev(q, q_shared, k, v, router_logits)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("expected q [B,h,T,d] and k, v [B,g,T,d]")
    B, h, T, d = q.shape
    g = k.shape[1]
    if k.shape[0] != B or k.shape[2:] != (T, d) or q_shared.shape != (B, T, d):
        raise ValueError("k/v or q_shared shape does not match q")
    if router_logits.dtype != torch.float32 or router_logits.shape != (B, T, h):
        raise ValueError("router_logits must be float32 [B,T,h]")
    if k.dtype != q.dtype or v.dtype != q.dtype or q_shared.dtype != q.dtype:
        raise TypeError("q, q_shared, k and v must share one dtype")
    out_dtype = out_dtype or q.dtype
    kk = max(int(top_k), 1)
    concat = torch.empty((B, T, g, kk, d), dtype=out_dtype, device=dev)
    wsum = torch.empty((B, T, g, d), dtype=out_dtype, device=dev)
    shared = torch.empty((B, T, d), dtype=out_dtype, device=dev)
    idx = torch.empty((B, T, g, kk), dtype=torch.int32, device=dev)
    gate = torch.empty((B, T, g, kk), dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = _lib.gqe_prefill_build(q.data_ptr(), q_shared.data_ptr(), k.data_ptr(), v.data_ptr(),
                                router_logits.data_ptr(), int(top_k), int(shared_kv),
                                concat.data_ptr(), wsum.data_ptr(), shared.data_ptr(),
                                idx.data_ptr(), gate.data_ptr(), B, h, g, T, d, _dt(q, "q"),
                                _DT[out_dtype], scale, int(bool(causal)), _stream(dev))
    _check("gqe_prefill_build", st)
    return concat, wsum, shared, idx, gate
