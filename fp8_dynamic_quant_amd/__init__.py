"""FP8 (OCP E4M3) dynamically quantized linear layers for AMD MI355X (gfx950).

Python binding of libdq.so. Each function here has the name of the C entry point it calls and
only marshals arguments: it checks tensor devices, dtypes and shapes, allocates outputs with
torch (device memory only) when the caller passes none, and calls the library on the current
stream. Every step of the computation runs in the HIP kernels of libdq; there is no fallback.

    q, scale   = dq_quantize_fp8(x)                # x: bf16 [M, K] on the GPU
    qw, w_scale = dq_quantize_weight_fp8(w)        # w: bf16 [N, K], once per weight
    out = dq_linear_fp8(q, scale, qw, w_scale, bias, "gelu_tanh")
    q, scale, y = dq_layernorm_modulate_quantize_fp8(h, mod_scale, mod_shift)  # LN + modulate
    oq, ok, ov = dq_linear_qkv_fp8(q, scale, qw, w_scale, heads, bias, norm_qk, cos, sin)
    o = dq_attention_fp8(*quantize_qkv_heads_fp8(oq, ok, ov))     # [S, heads, 128]

dq_linear_fp8 takes a workspace that lets workgroups share tiles (see include/dq.h). By default
the binding keeps one zero-filled workspace per (device, stream) and grows it when a larger
problem needs more; pass workspace=None to run without one, or a uint8 tensor of your own.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdq.so")

(DQ_OK, DQ_ERR_NULL, DQ_ERR_SHAPE, DQ_ERR_ALIGN, DQ_ERR_ALIAS, DQ_ERR_EPILOGUE, DQ_ERR_HIP,
 DQ_ERR_WORKSPACE, DQ_ERR_VALUE) = range(9)
EPILOGUES = {"bias": 0, "gelu_tanh": 1, "gated_residual": 2}


class DQError(RuntimeError):
    """A nonzero status from libdq."""

    def __init__(self, status: int, where: str):
        self.status = status
        self.hip_error = lib().dq_last_hip_error() if status == DQ_ERR_HIP else 0
        msg = lib().dq_status_string(status).decode()
        extra = f" (hipError {self.hip_error})" if self.hip_error else ""
        super().__init__(f"{where}: status {status}: {msg}{extra}")


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded libdq.so. Raises if it was not built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python fp8_dynamic_quant_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.dq_quantize_fp8.argtypes = [vp, i64, i64, vp, vp, vp]
        L.dq_quantize_fp8.restype = i32
        L.dq_quantize_weight_fp8.argtypes = [vp, i64, i64, vp, vp, vp]
        L.dq_quantize_weight_fp8.restype = i32
        L.dq_linear_fp8.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, i32, vp, vp, vp, vp,
                                    ctypes.c_uint64, vp]
        L.dq_linear_fp8.restype = i32
        L.dq_linear_fp8_noalloc.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, i32, vp, vp, vp,
                                            vp]
        L.dq_linear_fp8_noalloc.restype = i32
        L.dq_linear_fp8_segmented.argtypes = [vp, vp, i64, i64, vp, vp, vp, i64, vp, i32, vp, vp,
                                              vp, vp, ctypes.c_uint64, vp]
        L.dq_linear_fp8_segmented.restype = i32
        L.dq_linear_fp8_segmented_workspace_size.argtypes = [i64, vp, i64, i64]
        L.dq_linear_fp8_segmented_workspace_size.restype = ctypes.c_uint64
        L.dq_layernorm_modulate_quantize_fp8.argtypes = [vp, i64, i64, vp, vp, ctypes.c_float,
                                                         vp, vp, vp, vp]
        L.dq_layernorm_modulate_quantize_fp8.restype = i32
        L.dq_linear_qkv_fp8.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, vp, vp, vp,
                                        ctypes.c_float, vp, vp, vp, vp, ctypes.c_uint64, vp]
        L.dq_linear_qkv_fp8.restype = i32
        L.dq_linear_qkv_fp8_attn.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, vp, vp, vp,
                                             ctypes.c_float, vp, vp, vp, vp, vp, vp, vp,
                                             ctypes.c_uint64, vp]
        L.dq_linear_qkv_fp8_attn.restype = i32
        L.dq_quantize_v_fp8.argtypes = [vp, i64, i64, vp, vp, vp]
        L.dq_quantize_v_fp8.restype = i32
        L.dq_attention_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, vp, vp,
                                       ctypes.c_uint64, i64, vp]
        L.dq_attention_fp8.restype = i32
        L.dq_attention_fp8_workspace_size.argtypes = [i64, i64]
        L.dq_attention_fp8_workspace_size.restype = ctypes.c_uint64
        L.dq_quantize_mx_fp8.argtypes = [vp, i64, i64, vp, vp, vp]
        L.dq_quantize_mx_fp8.restype = i32
        L.dq_linear_mx_fp8.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, i32, vp, vp]
        L.dq_linear_mx_fp8.restype = i32
        L.dq_quantize_mxfp4.argtypes = [vp, i64, i64, vp, vp, vp]
        L.dq_quantize_mxfp4.restype = i32
        L.dq_linear_mxfp4.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, i32, vp, vp, vp, vp]
        L.dq_linear_mxfp4.restype = i32
        L.dq_linear_mxfp4_segmented.argtypes = [vp, vp, i64, i64, vp, vp, vp, i64, vp, i32, vp,
                                                vp, vp, vp]
        L.dq_linear_mxfp4_segmented.restype = i32
        L.dq_linear_fp8_workspace_size.argtypes = [i64, i64, i64]
        L.dq_linear_fp8_workspace_size.restype = ctypes.c_uint64
        L.dq_status_string.argtypes = [i32]
        L.dq_status_string.restype = ctypes.c_char_p
        L.dq_last_hip_error.argtypes = []
        L.dq_last_hip_error.restype = i32
        L.dq_abi_version.argtypes = []
        L.dq_abi_version.restype = i32
        _LIB = L
    return _LIB


lib()  # fail at import when the library is missing


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check(status, where):
    if status != DQ_OK:
        raise DQError(status, where)


def _quantize(fn, where, x, q, scale, stream):
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError(f"{where}: input must be a 2-D tensor")
    if x.device.type != "cuda":
        raise ValueError(f"{where}: input must be on a GPU")
    R, K = x.shape
    dev = x.device
    _need(x, "input", torch.bfloat16, (R, K), dev)
    q = torch.empty((R, K), dtype=torch.uint8, device=dev) if q is None else q
    scale = torch.empty((R,), dtype=torch.float32, device=dev) if scale is None else scale
    _need(q, "codes", torch.uint8, (R, K), dev)
    _need(scale, "scale", torch.float32, (R,), dev)
    with torch.cuda.device(dev):
        _check(fn(_ptr(x), R, K, _ptr(q), _ptr(scale), _stream(stream, dev)), where)
    return q, scale


def dq_quantize_fp8(x, q=None, scale=None, stream=None):
    """Per-token FP8 quantization: x bf16 [M, K] -> (codes uint8 [M, K], scale float32 [M])."""
    return _quantize(lib().dq_quantize_fp8, "dq_quantize_fp8", x, q, scale, stream)


def dq_quantize_weight_fp8(w, qw=None, w_scale=None, stream=None):
    """Per-output-channel FP8 quantization: w bf16 [N, K] -> (codes [N, K], scale [N])."""
    return _quantize(lib().dq_quantize_weight_fp8, "dq_quantize_weight_fp8", w, qw, w_scale, stream)


def dq_layernorm_modulate_quantize_fp8(x, mod_scale, mod_shift, eps=1e-6, store_y=True, q=None,
                                       scale=None, y=None, stream=None):
    """LayerNorm (no affine) + modulation + per-token FP8 quantization in one pass.

    x bf16 [M, K]; mod_scale, mod_shift bf16 [K]. Returns (codes uint8 [M, K], scale float32
    [M], y bf16 [M, K] or None): y = bf16(LN(x) * (1 + mod_scale) + mod_shift), and the codes
    are y's per-row quantization. store_y=False skips writing y.
    """
    where = "dq_layernorm_modulate_quantize_fp8"
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError(f"{where}: input must be a 2-D tensor")
    if x.device.type != "cuda":
        raise ValueError(f"{where}: input must be on a GPU")
    M, K = x.shape
    dev = x.device
    _need(x, "input", torch.bfloat16, (M, K), dev)
    _need(mod_scale, "mod_scale", torch.bfloat16, (K,), dev)
    _need(mod_shift, "mod_shift", torch.bfloat16, (K,), dev)
    q = torch.empty((M, K), dtype=torch.uint8, device=dev) if q is None else q
    scale = torch.empty((M,), dtype=torch.float32, device=dev) if scale is None else scale
    _need(q, "codes", torch.uint8, (M, K), dev)
    _need(scale, "scale", torch.float32, (M,), dev)
    if store_y:
        y = torch.empty((M, K), dtype=torch.bfloat16, device=dev) if y is None else y
        _need(y, "y", torch.bfloat16, (M, K), dev)
    else:
        y = None
    with torch.cuda.device(dev):
        _check(lib().dq_layernorm_modulate_quantize_fp8(
            _ptr(x), M, K, _ptr(mod_scale), _ptr(mod_shift), float(eps), _ptr(y), _ptr(q),
            _ptr(scale), _stream(stream, dev)), where)
    return q, scale, y


def dq_linear_fp8_workspace_size(M, K, N):
    """Bytes of workspace the schedule dq_linear_fp8 prefers for an M x K -> N problem on the
    current device (0: no workspace needed, or invalid sizes)."""
    return int(lib().dq_linear_fp8_workspace_size(int(M), int(K), int(N)))


_WORKSPACES = {}


def _resolve_workspace(workspace, dev, st, M, K, N):
    """(workspace tensor or None, its size in bytes) for the 'auto' / None / tensor forms."""
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError(f"workspace must be 'auto', None or a tensor, not {workspace!r}")
        need = dq_linear_fp8_workspace_size(M, K, N)
        workspace = _cached_workspace(dev, st, need) if (need and M > 0) else None
    if workspace is None:
        return None, 0
    if not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8 \
            or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the device")
    return workspace, workspace.numel()


def _cached_workspace(dev, stream, nbytes, kind="linear"):
    """The zero-filled workspace of (device, stream, kind), grown to at least nbytes. Every
    completed call leaves its workspace's counters zeroed, and calls on one stream run in order,
    so it is reused. The linear layers and attention keep separate workspaces (their counters
    sit at different places)."""
    key = (dev.index, stream.cuda_stream, kind)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        with torch.cuda.stream(stream):
            ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        _WORKSPACES[key] = ws
    return ws


def dq_linear_fp8(q, scale, qw, w_scale, bias=None, epilogue="bias", gate=None, residual=None,
                  out=None, stream=None, workspace="auto"):
    """W8A8 GEMM + fused epilogue -> bf16 [M, N].

    epilogue: "bias" | "gelu_tanh" | "gated_residual" (needs gate [N] and residual [M, N];
    out may be residual itself for an in-place update).
    workspace: "auto" (a cached zero-filled buffer per device and stream, of the size the
    preferred schedule uses), None (no tile is cut), or a uint8 tensor whose first 4096 bytes
    hold zeros before its first use; its size is a budget (include/dq.h).
    """
    dev, M, K, N, gate, residual, out = _linear_args(q, scale, qw, w_scale, bias, epilogue, gate,
                                                     residual, out)
    with torch.cuda.device(dev):
        st = stream if stream is not None else torch.cuda.current_stream(dev)
        workspace, ws_bytes = _resolve_workspace(workspace, dev, st, M, K, N)
        _check(lib().dq_linear_fp8(_ptr(q), _ptr(scale), M, K, _ptr(qw), _ptr(w_scale), N,
                                   _ptr(bias), EPILOGUES[epilogue], _ptr(gate), _ptr(residual),
                                   _ptr(out), _ptr(workspace), ws_bytes,
                                   ctypes.c_void_p(st.cuda_stream)), "dq_linear_fp8")
    return out


def dq_linear_fp8_noalloc(q, scale, qw, w_scale, bias=None, epilogue="bias", gate=None,
                          residual=None, out=None, stream=None):
    """dq_linear_fp8 on the library's own device scratch: the library allocates nothing (pass
    `out` to allocate nothing here either). Calls that may overlap on one GPU race."""
    dev, M, K, N, gate, residual, out = _linear_args(q, scale, qw, w_scale, bias, epilogue, gate,
                                                     residual, out)
    with torch.cuda.device(dev):
        st = stream if stream is not None else torch.cuda.current_stream(dev)
        _check(lib().dq_linear_fp8_noalloc(_ptr(q), _ptr(scale), M, K, _ptr(qw), _ptr(w_scale), N,
                                           _ptr(bias), EPILOGUES[epilogue], _ptr(gate),
                                           _ptr(residual), _ptr(out),
                                           ctypes.c_void_p(st.cuda_stream)),
               "dq_linear_fp8_noalloc")
    return out


def dq_linear_fp8_segmented_workspace_size(seg_rows, K, N):
    """Bytes of workspace the preferred schedule of a segmented linear uses (0: none, or invalid
    sizes)."""
    rows = (ctypes.c_int64 * len(seg_rows))(*[int(r) for r in seg_rows])
    return int(lib().dq_linear_fp8_segmented_workspace_size(len(seg_rows), rows, int(K), int(N)))


def dq_linear_fp8_segmented(q, scale, seg_rows, qws, w_scales, biases, epilogue="bias",
                            gates=None, residual=None, out=None, stream=None, workspace="auto"):
    """The linear over row segments with one weight each, in one launch -> bf16 [M, N].

    q uint8 [M, K], scale f32 [M] for the whole sequence; seg_rows: row counts summing to M;
    qws / w_scales / biases (/ gates for "gated_residual"): one tensor per segment (a bias may
    be None). residual and out cover all M rows (out may be residual).
    """
    where = "dq_linear_fp8_segmented"
    nseg = len(seg_rows)
    if not (1 <= nseg <= 4) or len(qws) != nseg or len(w_scales) != nseg or len(biases) != nseg:
        raise ValueError(f"{where}: 1 to 4 segments, one weight, scale and bias each")
    if epilogue == "gated_residual" and (gates is None or len(gates) != nseg):
        raise ValueError(f"{where}: gated_residual needs one gate per segment")
    M = sum(int(r) for r in seg_rows)
    if not isinstance(q, torch.Tensor) or q.dim() != 2 or q.shape[0] != M:
        raise ValueError(f"{where}: q must be [sum(seg_rows), K]")
    for i in range(nseg):   # each segment's tensors against the shared ones
        dev, _, K, N, _, residual, out = _linear_args(
            q, scale, qws[i], w_scales[i], biases[i], epilogue,
            gates[i] if epilogue == "gated_residual" else None, residual, out)
    VP = ctypes.c_void_p * nseg
    rows = (ctypes.c_int64 * nseg)(*[int(r) for r in seg_rows])
    ptrs = [VP(*[t.data_ptr() if t is not None else None for t in ts])
            for ts in (qws, w_scales, biases)]
    gp = VP(*[t.data_ptr() for t in gates]) if epilogue == "gated_residual" else None
    with torch.cuda.device(dev):
        st = stream if stream is not None else torch.cuda.current_stream(dev)
        if isinstance(workspace, str):
            if workspace != "auto":
                raise ValueError(f"workspace must be 'auto', None or a tensor, not {workspace!r}")
            need = dq_linear_fp8_segmented_workspace_size(seg_rows, K, N)
            workspace = _cached_workspace(dev, st, need) if (need and M > 0) else None
        workspace, ws_bytes = _resolve_workspace(workspace, dev, st, M, K, N)
        _check(lib().dq_linear_fp8_segmented(_ptr(q), _ptr(scale), K, nseg, rows, ptrs[0],
                                             ptrs[1], N, ptrs[2], EPILOGUES[epilogue], gp,
                                             _ptr(residual), _ptr(out), _ptr(workspace),
                                             ws_bytes, ctypes.c_void_p(st.cuda_stream)), where)
    return out


def _linear_args(q, scale, qw, w_scale, bias, epilogue, gate, residual, out):
    """Checks of dq_linear_fp8's tensors; allocates out when None. Returns (device, M, K, N,
    gate, residual, out)."""
    if epilogue not in EPILOGUES:
        raise ValueError(f"unknown epilogue {epilogue!r}")
    if not isinstance(q, torch.Tensor) or q.dim() != 2 or not isinstance(qw, torch.Tensor) \
            or qw.dim() != 2:
        raise ValueError("dq_linear_fp8: q and qw must be 2-D tensors")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("dq_linear_fp8: tensors must be on a GPU")
    M, K = q.shape
    N = qw.shape[0]
    _need(q, "q", torch.uint8, (M, K), dev)
    _need(scale, "scale", torch.float32, (M,), dev)
    _need(qw, "qw", torch.uint8, (N, K), dev)
    _need(w_scale, "w_scale", torch.float32, (N,), dev)
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, (N,), dev)
    if epilogue == "gated_residual":
        if gate is None or residual is None:
            raise ValueError("gated_residual needs gate and residual")
        _need(gate, "gate", torch.bfloat16, (N,), dev)
        _need(residual, "residual", torch.bfloat16, (M, N), dev)
    else:
        gate = residual = None
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if out is None else out
    _need(out, "out", torch.bfloat16, (M, N), dev)
    return dev, M, K, N, gate, residual, out


HEAD_DIM = 128


def dq_linear_qkv_fp8(q, scale, qw, w_scale, heads, bias, norm_qk, rope_cos, rope_sin, eps=1e-6,
                      out=None, stream=None, workspace="auto"):
    """W8A8 QKV projection with per-head query/key RMS norm and rotary embedding fused.

    q uint8 [M, K], scale f32 [M], qw uint8 [3 heads 128, K], w_scale f32 [N], bias bf16 [N] or
    None, norm_qk bf16 [2, 128] (query then key weights), rope_cos / rope_sin f32 [M, 64].
    Returns (out_q, out_k, out_v), bf16 [heads, M, 128] each; `out` may supply the three.
    """
    where = "dq_linear_qkv_fp8"
    if not isinstance(q, torch.Tensor) or q.dim() != 2 or not isinstance(qw, torch.Tensor) \
            or qw.dim() != 2:
        raise ValueError(f"{where}: q and qw must be 2-D tensors")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError(f"{where}: tensors must be on a GPU")
    M, K = q.shape
    heads = int(heads)
    N = 3 * heads * HEAD_DIM
    _need(q, "q", torch.uint8, (M, K), dev)
    _need(scale, "scale", torch.float32, (M,), dev)
    _need(qw, "qw", torch.uint8, (N, K), dev)
    _need(w_scale, "w_scale", torch.float32, (N,), dev)
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, (N,), dev)
    _need(norm_qk, "norm_qk", torch.bfloat16, (2, HEAD_DIM), dev)
    _need(rope_cos, "rope_cos", torch.float32, (M, HEAD_DIM // 2), dev)
    _need(rope_sin, "rope_sin", torch.float32, (M, HEAD_DIM // 2), dev)
    if out is None:
        out = tuple(torch.empty((heads, M, HEAD_DIM), dtype=torch.bfloat16, device=dev)
                    for _ in range(3))
    for t, name in zip(out, ("out_q", "out_k", "out_v")):
        _need(t, name, torch.bfloat16, (heads, M, HEAD_DIM), dev)
    with torch.cuda.device(dev):
        st = stream if stream is not None else torch.cuda.current_stream(dev)
        workspace, ws_bytes = _resolve_workspace(workspace, dev, st, M, K, N)
        _check(lib().dq_linear_qkv_fp8(_ptr(q), _ptr(scale), M, K, _ptr(qw), _ptr(w_scale), heads,
                                       _ptr(bias), _ptr(norm_qk), _ptr(rope_cos), _ptr(rope_sin),
                                       float(eps), _ptr(out[0]), _ptr(out[1]), _ptr(out[2]),
                                       _ptr(workspace), ws_bytes, ctypes.c_void_p(st.cuda_stream)),
               where)
    return tuple(out)


def dq_linear_qkv_fp8_attn(q, scale, qw, w_scale, heads, bias, norm_qk, rope_cos, rope_sin,
                           eps=1e-6, out=None, stream=None, workspace="auto"):
    """dq_linear_qkv_fp8 with its outputs as FP8 codes and per-(head, token) scales, the operands
    of dq_attention_fp8 (M a multiple of 16).

    Arguments as dq_linear_qkv_fp8. Returns (q8 uint8 [heads, M, 128], q_scale f32 [heads, M],
    k8, k_scale, vt8 uint8 [heads, 128, M] (values transposed), v_scale f32 [heads, M]); `out`
    may supply the six."""
    where = "dq_linear_qkv_fp8_attn"
    if not isinstance(q, torch.Tensor) or q.dim() != 2 or not isinstance(qw, torch.Tensor) \
            or qw.dim() != 2:
        raise ValueError(f"{where}: q and qw must be 2-D tensors")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError(f"{where}: tensors must be on a GPU")
    M, K = q.shape
    heads = int(heads)
    N = 3 * heads * HEAD_DIM
    _need(q, "q", torch.uint8, (M, K), dev)
    _need(scale, "scale", torch.float32, (M,), dev)
    _need(qw, "qw", torch.uint8, (N, K), dev)
    _need(w_scale, "w_scale", torch.float32, (N,), dev)
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, (N,), dev)
    _need(norm_qk, "norm_qk", torch.bfloat16, (2, HEAD_DIM), dev)
    _need(rope_cos, "rope_cos", torch.float32, (M, HEAD_DIM // 2), dev)
    _need(rope_sin, "rope_sin", torch.float32, (M, HEAD_DIM // 2), dev)
    if out is None:
        out = (torch.empty((heads, M, HEAD_DIM), dtype=torch.uint8, device=dev),
               torch.empty((heads, M), dtype=torch.float32, device=dev),
               torch.empty((heads, M, HEAD_DIM), dtype=torch.uint8, device=dev),
               torch.empty((heads, M), dtype=torch.float32, device=dev),
               torch.empty((heads, HEAD_DIM, M), dtype=torch.uint8, device=dev),
               torch.empty((heads, M), dtype=torch.float32, device=dev))
    specs = ((torch.uint8, (heads, M, HEAD_DIM)), (torch.float32, (heads, M)),
             (torch.uint8, (heads, M, HEAD_DIM)), (torch.float32, (heads, M)),
             (torch.uint8, (heads, HEAD_DIM, M)), (torch.float32, (heads, M)))
    for t, name, (dt, shp) in zip(out, ("q8", "q_scale", "k8", "k_scale", "vt8", "v_scale"),
                                  specs):
        _need(t, name, dt, shp, dev)
    with torch.cuda.device(dev):
        st = stream if stream is not None else torch.cuda.current_stream(dev)
        workspace, ws_bytes = _resolve_workspace(workspace, dev, st, M, K, N)
        _check(lib().dq_linear_qkv_fp8_attn(
            _ptr(q), _ptr(scale), M, K, _ptr(qw), _ptr(w_scale), heads, _ptr(bias), _ptr(norm_qk),
            _ptr(rope_cos), _ptr(rope_sin), float(eps), *(_ptr(t) for t in out),
            _ptr(workspace), ws_bytes, ctypes.c_void_p(st.cuda_stream)), where)
    return tuple(out)


def dq_quantize_v_fp8(v, vt=None, v_scale=None, stream=None):
    """Per-(head, token) FP8 quantization of values bf16 [H, S, 128], codes written transposed:
    returns (vt uint8 [H, 128, S], v_scale float32 [H, S]). S must be a multiple of 16."""
    where = "dq_quantize_v_fp8"
    if not isinstance(v, torch.Tensor) or v.dim() != 3 or v.device.type != "cuda":
        raise ValueError(f"{where}: values must be a 3-D tensor on a GPU")
    H, S, D = v.shape
    dev = v.device
    _need(v, "v", torch.bfloat16, (H, S, HEAD_DIM), dev)
    vt = torch.empty((H, HEAD_DIM, S), dtype=torch.uint8, device=dev) if vt is None else vt
    v_scale = torch.empty((H, S), dtype=torch.float32, device=dev) if v_scale is None else v_scale
    _need(vt, "vt", torch.uint8, (H, HEAD_DIM, S), dev)
    _need(v_scale, "v_scale", torch.float32, (H, S), dev)
    with torch.cuda.device(dev):
        _check(lib().dq_quantize_v_fp8(_ptr(v), H, S, _ptr(vt), _ptr(v_scale),
                                       _stream(stream, dev)), where)
    return vt, v_scale


def quantize_qkv_heads_fp8(q, k, v, stream=None):
    """Codes and scales of head-major bf16 q, k, v [H, S, 128] for dq_attention_fp8:
    (q8, q_scale, k8, k_scale, vt8, v_scale)."""
    H, S, _ = q.shape
    q8, sq = dq_quantize_fp8(q.reshape(H * S, HEAD_DIM), stream=stream)
    k8, sk = dq_quantize_fp8(k.reshape(H * S, HEAD_DIM), stream=stream)
    vt, sv = dq_quantize_v_fp8(v, stream=stream)
    return (q8.view(H, S, HEAD_DIM), sq.view(H, S), k8.view(H, S, HEAD_DIM), sk.view(H, S), vt,
            sv)


def dq_attention_fp8_workspace_size(H, S):
    """Bytes of workspace dq_attention_fp8 may use for H heads of S tokens (0: invalid sizes)."""
    return int(lib().dq_attention_fp8_workspace_size(int(H), int(S)))


def dq_attention_fp8(q8, q_scale, k8, k_scale, vt8, v_scale, out=None, stream=None,
                     workspace="auto", max_workgroups=0):
    """Attention over FP8 queries, keys, values (codes [H, S, 128], values transposed
    [H, 128, S], scales [H, S]) -> bf16 [S, H, 128].

    workspace: "auto" (a zero-filled buffer cached per device and stream), None (whole tiles per
    workgroup) or a zero-initialized uint8 tensor of dq_attention_fp8_workspace_size(H, S) bytes.
    max_workgroups: 0 (one per compute unit) or a lower cap on the workgroups launched."""
    where = "dq_attention_fp8"
    if not isinstance(q8, torch.Tensor) or q8.dim() != 3 or q8.device.type != "cuda":
        raise ValueError(f"{where}: query codes must be a 3-D tensor on a GPU")
    H, S, _ = q8.shape
    dev = q8.device
    _need(q8, "q", torch.uint8, (H, S, HEAD_DIM), dev)
    _need(k8, "k", torch.uint8, (H, S, HEAD_DIM), dev)
    _need(vt8, "vt", torch.uint8, (H, HEAD_DIM, S), dev)
    for t, name in ((q_scale, "q_scale"), (k_scale, "k_scale"), (v_scale, "v_scale")):
        _need(t, name, torch.float32, (H, S), dev)
    out = torch.empty((S, H, HEAD_DIM), dtype=torch.bfloat16, device=dev) if out is None else out
    _need(out, "out", torch.bfloat16, (S, H, HEAD_DIM), dev)
    with torch.cuda.device(dev):
        st = torch.cuda.current_stream(dev) if stream is None else stream
        if isinstance(workspace, str):
            if workspace != "auto":
                raise ValueError(f"workspace must be 'auto', None or a tensor, not {workspace!r}")
            need = dq_attention_fp8_workspace_size(H, S)
            workspace = _cached_workspace(dev, st, need, "attention") if (need and H * S) else None
        if workspace is not None and (not isinstance(workspace, torch.Tensor)
                                      or workspace.dtype != torch.uint8 or workspace.device != dev
                                      or not workspace.is_contiguous()):
            raise ValueError("workspace must be a contiguous uint8 tensor on the device")
        ws_bytes = 0 if workspace is None else workspace.numel()
        _check(lib().dq_attention_fp8(_ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(vt8),
                                      _ptr(v_scale), H, S, _ptr(out),
                                      None if workspace is None else _ptr(workspace), ws_bytes,
                                      int(max_workgroups), _stream(st, dev)), where)
    return out


MX_BLOCK = 32


def dq_quantize_mx_fp8(x, q=None, scales=None, stream=None):
    """Block-scaled (MX) FP8 quantization of bf16 x [M, K] (K % 32 == 0): E4M3 codes [M, K] and
    one E8M0 scale byte per 32 values, [M, K / 32]."""
    where = "dq_quantize_mx_fp8"
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError(f"{where}: x must be a 2-D tensor")
    M, K = x.shape
    dev = x.device
    _need(x, "x", torch.bfloat16, (M, K), dev)
    q = torch.empty((M, K), dtype=torch.uint8, device=dev) if q is None else q
    scales = torch.empty((M, K // MX_BLOCK), dtype=torch.uint8, device=dev) if scales is None \
        else scales
    _need(q, "q", torch.uint8, (M, K), dev)
    _need(scales, "scales", torch.uint8, (M, K // MX_BLOCK), dev)
    with torch.cuda.device(dev):
        _check(lib().dq_quantize_mx_fp8(_ptr(x), M, K, _ptr(q), _ptr(scales),
                                        _stream(stream, dev)), where)
    return q, scales


def dq_linear_mx_fp8(qa, sa, qw, sw, bias=None, epilogue="bias", out=None, stream=None):
    """Block-scaled FP8 linear layer -> bf16 [M, N]: codes qa [M, K], qw [N, K] and their scale
    bytes sa [M, K / 32], sw [N, K / 32] (dq_quantize_mx_fp8); epilogue "bias" or "gelu_tanh"."""
    where = "dq_linear_mx_fp8"
    if not isinstance(qa, torch.Tensor) or qa.dim() != 2 or not isinstance(qw, torch.Tensor):
        raise ValueError(f"{where}: qa and qw must be 2-D tensors")
    M, K = qa.shape
    N = qw.shape[0]
    dev = qa.device
    _need(qa, "qa", torch.uint8, (M, K), dev)
    _need(qw, "qw", torch.uint8, (N, K), dev)
    _need(sa, "sa", torch.uint8, (M, K // MX_BLOCK), dev)
    _need(sw, "sw", torch.uint8, (N, K // MX_BLOCK), dev)
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, (N,), dev)
    if epilogue not in ("bias", "gelu_tanh"):
        raise ValueError(f"{where}: epilogue must be 'bias' or 'gelu_tanh'")
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if out is None else out
    _need(out, "out", torch.bfloat16, (M, N), dev)
    with torch.cuda.device(dev):
        _check(lib().dq_linear_mx_fp8(_ptr(qa), _ptr(sa), M, K, _ptr(qw), _ptr(sw), N,
                                      _ptr(bias), EPILOGUES[epilogue], _ptr(out),
                                      _stream(stream, dev)), where)
    return out


def dq_quantize_mxfp4(x, q=None, scales=None, stream=None):
    """Block-scaled FP4 (MXFP4) quantization of bf16 x [M, K] (K % 32 == 0): E2M1 codes, two per
    byte, [M, K / 2] (element 2j in the low nibble of byte j), and one E8M0 scale byte per 32
    values, [M, K / 32]."""
    where = "dq_quantize_mxfp4"
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError(f"{where}: x must be a 2-D tensor")
    M, K = x.shape
    dev = x.device
    _need(x, "x", torch.bfloat16, (M, K), dev)
    q = torch.empty((M, K // 2), dtype=torch.uint8, device=dev) if q is None else q
    scales = torch.empty((M, K // MX_BLOCK), dtype=torch.uint8, device=dev) if scales is None \
        else scales
    _need(q, "q", torch.uint8, (M, K // 2), dev)
    _need(scales, "scales", torch.uint8, (M, K // MX_BLOCK), dev)
    with torch.cuda.device(dev):
        _check(lib().dq_quantize_mxfp4(_ptr(x), M, K, _ptr(q), _ptr(scales),
                                       _stream(stream, dev)), where)
    return q, scales


def _mxfp4_args(qa, sa, qw, sw, bias, epilogue, gate, residual, out, where):
    """Checks of one MXFP4 weight's tensors against the shared ones; allocates out when None.
    Returns (device, M, K, N, out)."""
    if not isinstance(qa, torch.Tensor) or qa.dim() != 2 or not isinstance(qw, torch.Tensor):
        raise ValueError(f"{where}: qa and qw must be 2-D tensors")
    if epilogue not in EPILOGUES:
        raise ValueError(f"{where}: unknown epilogue {epilogue!r}")
    M, K = qa.shape[0], 2 * qa.shape[1]
    N = qw.shape[0]
    dev = qa.device
    _need(qa, "qa", torch.uint8, (M, K // 2), dev)
    _need(qw, "qw", torch.uint8, (N, K // 2), dev)
    _need(sa, "sa", torch.uint8, (M, K // MX_BLOCK), dev)
    _need(sw, "sw", torch.uint8, (N, K // MX_BLOCK), dev)
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, (N,), dev)
    if epilogue == "gated_residual":
        if gate is None or residual is None:
            raise ValueError(f"{where}: gated_residual needs gate and residual")
        _need(gate, "gate", torch.bfloat16, (N,), dev)
        _need(residual, "residual", torch.bfloat16, (M, N), dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if out is None else out
    _need(out, "out", torch.bfloat16, (M, N), dev)
    return dev, M, K, N, out


def dq_linear_mxfp4(qa, sa, qw, sw, bias=None, epilogue="bias", gate=None, residual=None,
                    out=None, stream=None):
    """MXFP4 linear layer -> bf16 [M, N]: packed codes qa [M, K / 2], qw [N, K / 2] and their
    scale bytes sa [M, K / 32], sw [N, K / 32] (dq_quantize_mxfp4); epilogue "bias",
    "gelu_tanh" or "gated_residual" (gate [N], residual [M, N]; out may be the residual)."""
    where = "dq_linear_mxfp4"
    dev, M, K, N, out = _mxfp4_args(qa, sa, qw, sw, bias, epilogue, gate, residual, out, where)
    gated = epilogue == "gated_residual"
    with torch.cuda.device(dev):
        _check(lib().dq_linear_mxfp4(_ptr(qa), _ptr(sa), M, K, _ptr(qw), _ptr(sw), N,
                                     _ptr(bias), EPILOGUES[epilogue],
                                     _ptr(gate) if gated else None,
                                     _ptr(residual) if gated else None, _ptr(out),
                                     _stream(stream, dev)), where)
    return out


def dq_linear_mxfp4_segmented(qa, sa, seg_rows, qws, sws, biases, epilogue="bias", gates=None,
                              residual=None, out=None, stream=None):
    """The MXFP4 linear over row segments with one weight each, in one launch -> bf16 [M, N].
    qa [M, K / 2] and sa [M, K / 32] for the whole sequence; seg_rows sums to M; qws / sws /
    biases (/ gates for "gated_residual"): one tensor per segment (a bias may be None)."""
    where = "dq_linear_mxfp4_segmented"
    nseg = len(seg_rows)
    if not (1 <= nseg <= 4) or len(qws) != nseg or len(sws) != nseg or len(biases) != nseg:
        raise ValueError(f"{where}: 1 to 4 segments, one weight, scale and bias each")
    gated = epilogue == "gated_residual"
    if gated and (gates is None or len(gates) != nseg):
        raise ValueError(f"{where}: gated_residual needs one gate per segment")
    M = sum(int(r) for r in seg_rows)
    if not isinstance(qa, torch.Tensor) or qa.dim() != 2 or qa.shape[0] != M:
        raise ValueError(f"{where}: qa must be [sum(seg_rows), K / 2]")
    for i in range(nseg):
        dev, _, K, N, out = _mxfp4_args(qa, sa, qws[i], sws[i], biases[i], epilogue,
                                        gates[i] if gated else None, residual, out, where)
    VP = ctypes.c_void_p * nseg
    rows = (ctypes.c_int64 * nseg)(*[int(r) for r in seg_rows])
    ptrs = [VP(*[t.data_ptr() if t is not None else None for t in ts])
            for ts in (qws, sws, biases)]
    gp = VP(*[t.data_ptr() for t in gates]) if gated else None
    with torch.cuda.device(dev):
        _check(lib().dq_linear_mxfp4_segmented(_ptr(qa), _ptr(sa), K, nseg, rows, ptrs[0],
                                               ptrs[1], N, ptrs[2], EPILOGUES[epilogue], gp,
                                               _ptr(residual) if gated else None, _ptr(out),
                                               _stream(stream, dev)), where)
    return out


__all__ = ["dq_quantize_fp8", "dq_quantize_weight_fp8", "dq_linear_fp8", "dq_linear_fp8_noalloc",
           "dq_linear_fp8_segmented", "dq_linear_fp8_segmented_workspace_size",
           "dq_layernorm_modulate_quantize_fp8", "dq_linear_qkv_fp8", "dq_linear_qkv_fp8_attn",
           "HEAD_DIM",
           "dq_quantize_v_fp8", "dq_attention_fp8", "dq_attention_fp8_workspace_size",
           "quantize_qkv_heads_fp8", "dq_quantize_mx_fp8", "dq_linear_mx_fp8", "MX_BLOCK",
           "dq_quantize_mxfp4", "dq_linear_mxfp4", "dq_linear_mxfp4_segmented",
           "dq_linear_fp8_workspace_size", "DQError", "EPILOGUES", "lib", "LIB_PATH"]
