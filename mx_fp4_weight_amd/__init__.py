"""Python binding of libmxfp4spec.so: MX-FP4 verify GEMM and speculative acceptance on gfx950.

Argument marshalling only. Every step runs in the HIP library; there is no
CPU or PyTorch fallback: the first call raises ImportError when the library
has not been built. PyTorch supplies device memory and the stream
(``torch.cuda.current_stream()``); the C functions keep their names:
``mxfp4_quantize``, ``mxfp4_verify_gemm``, ``spec_accept``.
"""
from __future__ import annotations

import ctypes
import os

import torch

# MXS_LIB: another build of the same library (the host-sanitizer build of the CPU checks)
LIB_PATH = os.environ.get("MXS_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmxfp4spec.so")

MXS_OK = 0
MXS_ERR_NULL = 1
MXS_ERR_SHAPE = 2
MXS_ERR_ALIGN = 3
MXS_ERR_WORKSPACE = 4
MXS_ERR_DEVICE = 5
MXS_ERR_LAUNCH = 6
MXS_ERR_VALUE = 7

FLAG_NONFINITE = 1
FLAG_TOKEN_RANGE = 2
FLAG_Q_ZERO = 4
FLAG_RESIDUAL_ZERO = 8

EXPORTS = ["mxs_status_string", "mxs_abi_version", "mxfp4_quantize", "mxfp4_verify_gemm",
           "mxfp4_verify_gemm_grouped", "spec_accept_workspace_bytes", "spec_accept",
           "spec_accept_sampled_workspace_bytes", "spec_accept_sampled",
           "spec_sampling_thresholds_workspace_bytes", "spec_sampling_thresholds", "nvfp4_quantize",
           "nvfp4_verify_gemm", "nvfp4_verify_gemm_grouped", "mx_quantize_act", "mx_verify_gemm_act",
           "mxfp4_tiled_bytes", "mxfp4_tile_codes", "mxfp4_tiled_scale_bytes", "mxfp4_tile_scales",
           "mx_verify_gemm_act_tiled", "mxfp4_verify_gemm_tiled", "mxfp4_verify_gemm_grouped_tiled",
           "nvfp4_verify_gemm_grouped_tiled", "spec_accept_noalloc", "mxs_stream_read", "mxfp4_kv_append",
           "spec_accept_tree_workspace_bytes", "spec_accept_tree", "mxfp4_kv_attention_workspace_bytes",
           "mxfp4_kv_attention"]

NOALLOC_SCRATCH_BYTES = 4 << 20  # MXS_NOALLOC_SCRATCH_BYTES


class GemmProblem(ctypes.Structure):
    """mxs_gemm_problem: one product of a grouped verify GEMM."""
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("x", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("n", ctypes.c_int64)]


class NvProblem(ctypes.Structure):
    """mxs_nvfp4_problem: one product of a grouped NVFP4 verify GEMM."""
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("global_scale", ctypes.c_void_p),
                ("x", ctypes.c_void_p), ("y", ctypes.c_void_p), ("n", ctypes.c_int64)]


class MxsError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m mx_fp4_weight_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    lib.mxs_status_string.argtypes = [ctypes.c_int]
    lib.mxs_status_string.restype = ctypes.c_char_p
    lib.mxs_abi_version.argtypes = []
    lib.mxs_abi_version.restype = ctypes.c_int
    lib.mxfp4_quantize.argtypes = [vp, i64, i64, vp, vp, vp, vp]
    lib.mxfp4_quantize.restype = ctypes.c_int
    lib.mxfp4_verify_gemm.argtypes = [vp, vp, i64, i64, vp, i64, vp, vp]
    lib.mxfp4_verify_gemm.restype = ctypes.c_int
    lib.mxfp4_verify_gemm_grouped.argtypes = [ctypes.POINTER(GemmProblem), i32, i64, i64, vp]
    lib.mxfp4_verify_gemm_grouped.restype = ctypes.c_int
    lib.spec_accept_workspace_bytes.argtypes = [i32, i32, i32]
    lib.spec_accept_workspace_bytes.restype = ctypes.c_size_t
    lib.spec_accept.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, ctypes.c_size_t, vp, vp]
    lib.spec_accept.restype = ctypes.c_int
    lib.spec_accept_tree_workspace_bytes.argtypes = [ctypes.POINTER(ctypes.c_int32), i32, i32, i32]
    lib.spec_accept_tree_workspace_bytes.restype = ctypes.c_size_t
    lib.spec_accept_tree.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_int32), i32, vp, vp, i32, i32, vp, vp, vp, vp,
                                     ctypes.c_size_t, vp, vp]
    lib.spec_accept_tree.restype = ctypes.c_int
    lib.mxfp4_kv_attention_workspace_bytes.argtypes = [i32, i32, i32, i32, i64]
    lib.mxfp4_kv_attention_workspace_bytes.restype = ctypes.c_size_t
    lib.mxfp4_kv_attention.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i64, i64,
                                       ctypes.POINTER(ctypes.c_uint64), f32, vp, vp, ctypes.c_size_t, vp, vp]
    lib.mxfp4_kv_attention.restype = ctypes.c_int
    lib.mxfp4_kv_append.argtypes = [vp, i64, i64, i64, vp, i64, vp, vp, vp, vp]
    lib.mxfp4_kv_append.restype = ctypes.c_int
    lib.mxs_stream_read.argtypes = [vp, ctypes.c_size_t, vp, vp]
    lib.mxs_stream_read.restype = ctypes.c_int
    lib.spec_accept_noalloc.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp]
    lib.spec_accept_noalloc.restype = ctypes.c_int
    lib.spec_accept_sampled_workspace_bytes.argtypes = [i32, i32, i32]
    lib.spec_accept_sampled_workspace_bytes.restype = ctypes.c_size_t
    lib.spec_accept_sampled.argtypes = [vp, vp, vp, vp, i32, i32, i32, f32, i32, f32, vp, vp, vp, vp,
                                        ctypes.c_size_t, vp, vp]
    lib.spec_accept_sampled.restype = ctypes.c_int
    lib.spec_sampling_thresholds_workspace_bytes.argtypes = [i32, i32]
    lib.spec_sampling_thresholds_workspace_bytes.restype = ctypes.c_size_t
    lib.spec_sampling_thresholds.argtypes = [vp, i32, i32, f32, i32, f32, vp, vp, vp, ctypes.c_size_t, vp]
    lib.spec_sampling_thresholds.restype = ctypes.c_int
    lib.nvfp4_quantize.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp]
    lib.nvfp4_quantize.restype = ctypes.c_int
    lib.nvfp4_verify_gemm.argtypes = [vp, vp, vp, i64, i64, vp, i64, vp, vp]
    lib.nvfp4_verify_gemm.restype = ctypes.c_int
    lib.nvfp4_verify_gemm_grouped.argtypes = [ctypes.POINTER(NvProblem), i32, i64, i64, vp]
    lib.nvfp4_verify_gemm_grouped.restype = ctypes.c_int
    lib.mx_quantize_act.argtypes = [vp, i64, i64, i32, vp, vp, vp, vp]
    lib.mx_quantize_act.restype = ctypes.c_int
    lib.mx_verify_gemm_act.argtypes = [vp, vp, i64, i64, vp, vp, i32, i64, vp, vp]
    lib.mx_verify_gemm_act.restype = ctypes.c_int
    lib.mxfp4_tiled_bytes.argtypes = [i64, i64]
    lib.mxfp4_tiled_bytes.restype = ctypes.c_size_t
    lib.mxfp4_tile_codes.argtypes = [vp, i64, i64, vp, vp]
    lib.mxfp4_tile_codes.restype = ctypes.c_int
    lib.mxfp4_tiled_scale_bytes.argtypes = [i64, i64]
    lib.mxfp4_tiled_scale_bytes.restype = ctypes.c_size_t
    lib.mxfp4_tile_scales.argtypes = [vp, i64, i64, vp, vp]
    lib.mxfp4_tile_scales.restype = ctypes.c_int
    lib.mx_verify_gemm_act_tiled.argtypes = [vp, vp, i64, i64, vp, vp, i32, i64, vp, vp]
    lib.mx_verify_gemm_act_tiled.restype = ctypes.c_int
    lib.mxfp4_verify_gemm_tiled.argtypes = [vp, vp, i64, i64, vp, i64, vp, vp]
    lib.mxfp4_verify_gemm_tiled.restype = ctypes.c_int
    lib.mxfp4_verify_gemm_grouped_tiled.argtypes = [ctypes.POINTER(GemmProblem), i32, i64, i64, vp]
    lib.mxfp4_verify_gemm_grouped_tiled.restype = ctypes.c_int
    lib.nvfp4_verify_gemm_grouped_tiled.argtypes = [ctypes.POINTER(NvProblem), i32, i64, i64, vp]
    lib.nvfp4_verify_gemm_grouped_tiled.restype = ctypes.c_int
    return lib


_LIB = None


def get_lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use; raises ImportError if it was never built)."""
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def status_string(status: int) -> str:
    return get_lib().mxs_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != MXS_OK:
        raise MxsError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _want(t, dtype, name, shape=None):
    """Type check of a tensor argument; with `shape`, also its exact shape (raised before any launch:
    the C ABI sees only pointers, so a short output buffer would otherwise be written past its end)."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous {dtype} CUDA/HIP tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _want_flags(dev_flags):
    _want(dev_flags, torch.int32, "dev_flags")
    if dev_flags is not None and dev_flags.numel() < 1:
        raise ValueError("dev_flags must hold at least one int32")


def mxfp4_quantize(w: torch.Tensor, codes: torch.Tensor | None = None,
                   scales: torch.Tensor | None = None, dev_flags: torch.Tensor | None = None,
                   stream=None):
    """fp32 W[n, k] -> (codes uint8 [n, k/2], scales uint8 [n, k/32]); flags OR-ed into dev_flags (int32[1])."""
    _want(w, torch.float32, "w")
    n, k = w.shape
    if codes is None:
        codes = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty((n, k // 32), dtype=torch.uint8, device=w.device)
    _want(codes, torch.uint8, "codes", (n, k // 2))
    _want(scales, torch.uint8, "scales", (n, k // 32))
    _want_flags(dev_flags)
    _check(get_lib().mxfp4_quantize(_ptr(w), n, k, _ptr(codes), _ptr(scales), _ptr(dev_flags),
                              _stream(stream)), "mxfp4_quantize")
    return codes, scales


def mxfp4_verify_gemm(codes: torch.Tensor, scales: torch.Tensor, x: torch.Tensor,
                      y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Y[m, n] fp32 = X[m, k] (bf16) · Ŵᵀ with Ŵ the MX-FP4 matrix (codes [n, k/2], scales [n, k/32])."""
    _want(codes, torch.uint8, "codes")
    _want(scales, torch.uint8, "scales")
    _want(x, torch.bfloat16, "x")
    n, kh = codes.shape
    k = kh * 2
    m = x.shape[0]
    if x.shape[1] != k or scales.shape != (n, k // 32):
        raise ValueError("shape mismatch between codes, scales and x")
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _want(y, torch.float32, "y", (m, n))
    _check(get_lib().mxfp4_verify_gemm(_ptr(codes), _ptr(scales), n, k, _ptr(x), m, _ptr(y),
                                 _stream(stream)), "mxfp4_verify_gemm")
    return y


def mxfp4_verify_gemm_grouped(items, ys=None, stream=None):
    """Several independent verify GEMMs with the same k and m in one launch.

    items: list of (codes [n_i, k/2] uint8, scales [n_i, k/32] uint8, x [m, k] bf16).
    Returns the list of outputs y_i [m, n_i] fp32 (or fills the given ys).
    """
    if not items:
        raise ValueError("no products")
    k = items[0][0].shape[1] * 2
    m = items[0][2].shape[0]
    arr = (GemmProblem * len(items))()
    out = []
    for i, (codes, scales, x) in enumerate(items):
        _want(codes, torch.uint8, "codes")
        _want(scales, torch.uint8, "scales")
        _want(x, torch.bfloat16, "x")
        n = codes.shape[0]
        if codes.shape[1] * 2 != k or x.shape != (m, k) or scales.shape != (n, k // 32):
            raise ValueError("all products must share k and m")
        y = ys[i] if ys is not None else torch.empty((m, n), dtype=torch.float32, device=x.device)
        _want(y, torch.float32, "y", (m, n))
        arr[i] = GemmProblem(codes.data_ptr(), scales.data_ptr(), x.data_ptr(), y.data_ptr(), n)
        out.append(y)
    _check(get_lib().mxfp4_verify_gemm_grouped(arr, len(items), k, m, _stream(stream)),
           "mxfp4_verify_gemm_grouped")
    return out


def tree_depth(parent) -> int:
    """Nodes on the longest root-to-leaf path of a tree given by its parent list."""
    d = []
    for i, p in enumerate(parent):
        d.append(1 if p < 0 else d[p] + 1)
    return max(d, default=0)


def _parent_array(parent):
    arr = (ctypes.c_int32 * max(1, len(parent)))(*[int(p) for p in parent])
    return arr


def spec_accept_tree_workspace_bytes(parent, b: int, v: int) -> int:
    return int(get_lib().spec_accept_tree_workspace_bytes(_parent_array(parent), len(parent), b, v))


def spec_accept_tree(parent, target: torch.Tensor, draft: torch.Tensor, tokens: torch.Tensor | None,
                     uniforms: torch.Tensor, out_tokens: torch.Tensor | None = None,
                     out_nodes: torch.Tensor | None = None, out_num: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None, dev_flags: torch.Tensor | None = None, stream=None):
    """One verification cycle over a tree of drafts for b sequences (see the C header).

    parent: list of N ints (-1 = root); target, draft fp32 [b, N+1, v]; tokens int32 [b, N];
    uniforms fp32 [b, N+1]. Returns (out_tokens [b, D+1], out_nodes [b, D], n [b]).
    """
    parent = [int(p) for p in parent]
    nn = len(parent)
    _want(target, torch.float32, "target")
    b, rows, v = target.shape
    if rows != nn + 1:
        raise ValueError("target must be [b, N+1, v]")
    _want(draft, torch.float32, "draft", (b, nn + 1, v))
    if nn:
        _want(tokens, torch.int32, "tokens", (b, nn))
    else:
        tokens = None
    _want(uniforms, torch.float32, "uniforms", (b, nn + 1))
    d = tree_depth(parent)
    dev = target.device
    if out_tokens is None:
        out_tokens = torch.empty((b, d + 1), dtype=torch.int32, device=dev)
    if out_nodes is None:
        out_nodes = torch.empty((b, max(d, 1)), dtype=torch.int32, device=dev)
    if out_num is None:
        out_num = torch.empty((b,), dtype=torch.int32, device=dev)
    _want(out_tokens, torch.int32, "out_tokens", (b, d + 1))
    if out_nodes.shape != (b, d) and not (d == 0 and out_nodes.shape == (b, 1)):
        raise ValueError(f"out_nodes must have shape {(b, d)}")
    _want(out_nodes, torch.int32, "out_nodes")
    _want(out_num, torch.int32, "out_num", (b,))
    need = spec_accept_tree_workspace_bytes(parent, b, v)
    if need == 0:
        raise ValueError("tree or sizes out of range")
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    _want(workspace, torch.uint8, "workspace")
    _want_flags(dev_flags)
    _check(get_lib().spec_accept_tree(_ptr(target), _ptr(draft), _parent_array(parent), nn, _ptr(tokens),
                                      _ptr(uniforms), b, v, _ptr(out_tokens), _ptr(out_nodes), _ptr(out_num),
                                      _ptr(workspace), workspace.numel(), _ptr(dev_flags), _stream(stream)),
           "spec_accept_tree")
    return out_tokens, out_nodes[:, :d], out_num


def mxfp4_kv_append(kv: torch.Tensor, slots: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                    dev_flags: torch.Tensor | None = None, stream=None):
    """Code kv bf16 [t, heads, d] into the MX-FP4 KV cache codes uint8 [capacity, heads, d/2] and
    scales uint8 [capacity, heads, d/32] at entries slots int32 [t] (in place)."""
    _want(kv, torch.bfloat16, "kv")
    if kv.dim() != 3:
        raise ValueError("kv must be [t, heads, d]")
    t, heads, d = kv.shape
    _want(slots, torch.int32, "slots", (t,))
    if codes is None or scales is None or codes.dim() != 3:
        raise ValueError("codes must be [capacity, heads, d/2]")
    cap = codes.shape[0]
    _want(codes, torch.uint8, "codes", (cap, heads, d // 2))
    _want(scales, torch.uint8, "scales", (cap, heads, d // 32))
    _want_flags(dev_flags)
    _check(get_lib().mxfp4_kv_append(_ptr(kv), t, heads, d, _ptr(slots), cap, _ptr(codes), _ptr(scales),
                                     _ptr(dev_flags), _stream(stream)), "mxfp4_kv_append")
    return codes, scales


def chain_masks(t: int) -> list[int]:
    """Attention masks of t positions of a chain: position i sees new positions 0..i."""
    return [(1 << (i + 1)) - 1 for i in range(t)]


def tree_masks(parent) -> list[int]:
    """Attention masks of the N + 1 positions of a tree's pass (position 0 = the root's input, i + 1 =
    node i): a position sees itself and its ancestors."""
    masks = [1]
    for i, p in enumerate(parent):
        masks.append(masks[int(p) + 1] | (1 << (i + 1)))
    return masks


def mxfp4_kv_attention_workspace_bytes(b: int, t: int, hq: int, hkv: int, max_len: int) -> int:
    return int(get_lib().mxfp4_kv_attention_workspace_bytes(b, t, hq, hkv, max_len))


def mxfp4_kv_attention(q: torch.Tensor, k_codes: torch.Tensor, k_scales: torch.Tensor, v_codes: torch.Tensor,
                       v_scales: torch.Tensor, ctx_len: torch.Tensor, masks, scale: float | None = None,
                       max_len: int | None = None, out: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None, dev_flags: torch.Tensor | None = None, stream=None):
    """Attention of q bf16 [b, t, hq, 128] over the MX-FP4 caches (codes uint8 [b, cap, hkv, 64],
    scales uint8 [b, cap, hkv, 4]) with ctx_len int32 [b] committed entries and masks (t ints).
    Returns out fp32 [b, t, hq, 128]."""
    _want(q, torch.bfloat16, "q")
    if q.dim() != 4:
        raise ValueError("q must be [b, t, hq, d]")
    b, t, hq, d = q.shape
    if k_codes is None or k_codes.dim() != 4:
        raise ValueError("k_codes must be [b, capacity, hkv, d/2]")
    cap, hkv = k_codes.shape[1], k_codes.shape[2]
    for nm, tt, shp in (("k_codes", k_codes, (b, cap, hkv, d // 2)), ("v_codes", v_codes, (b, cap, hkv, d // 2)),
                        ("k_scales", k_scales, (b, cap, hkv, d // 32)), ("v_scales", v_scales, (b, cap, hkv, d // 32))):
        _want(tt, torch.uint8, nm, shp)
    _want(ctx_len, torch.int32, "ctx_len", (b,))
    masks = [int(m) for m in masks]
    if len(masks) != t:
        raise ValueError("one mask per query position")
    scale = float(d) ** -0.5 if scale is None else float(scale)
    max_len = cap if max_len is None else int(max_len)
    if out is None:
        out = torch.empty((b, t, hq, d), dtype=torch.float32, device=q.device)
    _want(out, torch.float32, "out", (b, t, hq, d))
    need = mxfp4_kv_attention_workspace_bytes(b, t, hq, hkv, max_len)
    if need == 0:
        raise ValueError("sizes out of range")
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=q.device)
    _want(workspace, torch.uint8, "workspace")
    _want_flags(dev_flags)
    marr = (ctypes.c_uint64 * t)(*masks)
    _check(get_lib().mxfp4_kv_attention(_ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes), _ptr(v_scales),
                                        _ptr(ctx_len), b, t, hq, hkv, d, cap, max_len, marr, scale, _ptr(out),
                                        _ptr(workspace), workspace.numel(), _ptr(dev_flags), _stream(stream)),
           "mxfp4_kv_attention")
    return out


def stream_read(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """One plain read of a contiguous device tensor (its byte size a multiple of 16): the measured
    read ceiling against which the verify GEMM's bandwidth is read. sink: int32 [1] device word."""
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise TypeError("buf must be a contiguous CUDA/HIP tensor")
    _want(sink, torch.int32, "sink", (1,))
    _check(get_lib().mxs_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)),
           "mxs_stream_read")


def spec_accept_workspace_bytes(b: int, kd: int, v: int) -> int:
    return int(get_lib().spec_accept_workspace_bytes(b, kd, v))


def spec_accept(target: torch.Tensor, draft: torch.Tensor | None, tokens: torch.Tensor | None,
                uniforms: torch.Tensor, out_tokens: torch.Tensor | None = None,
                out_num: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                dev_flags: torch.Tensor | None = None, stream=None):
    """One verification cycle for b sequences.

    target [b, kd+1, v] fp32, draft [b, kd, v] fp32, tokens [b, kd] int32,
    uniforms [b, kd+1] fp32. Returns (out_tokens [b, kd+1] int32, n [b] int32).
    """
    _want(target, torch.float32, "target")
    b, kd1, v = target.shape
    kd = kd1 - 1
    if kd > 0:
        _want(draft, torch.float32, "draft")
        _want(tokens, torch.int32, "tokens")
        if draft.shape != (b, kd, v) or tokens.shape != (b, kd):
            raise ValueError("draft/tokens shape mismatch")
    else:
        draft = tokens = None
    _want(uniforms, torch.float32, "uniforms")
    if uniforms.shape != (b, kd + 1):
        raise ValueError("uniforms must be [b, kd+1]")
    dev = target.device
    if out_tokens is None:
        out_tokens = torch.empty((b, kd + 1), dtype=torch.int32, device=dev)
    if out_num is None:
        out_num = torch.empty((b,), dtype=torch.int32, device=dev)
    _want(out_tokens, torch.int32, "out_tokens", (b, kd + 1))
    _want(out_num, torch.int32, "out_num", (b,))
    need = spec_accept_workspace_bytes(b, kd, v)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    _want(workspace, torch.uint8, "workspace")
    _want_flags(dev_flags)
    _check(get_lib().spec_accept(_ptr(target), _ptr(draft), _ptr(tokens), _ptr(uniforms), b, kd, v,
                           _ptr(out_tokens), _ptr(out_num), _ptr(workspace), workspace.numel(),
                           _ptr(dev_flags), _stream(stream)), "spec_accept")
    return out_tokens, out_num


def spec_accept_noalloc(target: torch.Tensor, draft: torch.Tensor | None, tokens: torch.Tensor | None,
                        uniforms: torch.Tensor, out_tokens: torch.Tensor, out_num: torch.Tensor,
                        dev_flags: torch.Tensor | None = None, stream=None):
    """spec_accept with the library's built-in workspace (the C call allocates nothing).

    The caller supplies every output: out_tokens int32 [b, kd+1], out_num int32 [b]. Calls on
    one GPU share the built-in workspace, so they must not overlap (one stream, or ordered).
    Raises MxsError(MXS_ERR_WORKSPACE) when (b, kd, v) needs more than NOALLOC_SCRATCH_BYTES.
    """
    _want(target, torch.float32, "target")
    b, kd1, v = target.shape
    kd = kd1 - 1
    if kd > 0:
        _want(draft, torch.float32, "draft", (b, kd, v))
        _want(tokens, torch.int32, "tokens", (b, kd))
    else:
        draft = tokens = None
    _want(uniforms, torch.float32, "uniforms", (b, kd + 1))
    if out_tokens is None or out_num is None:
        raise ValueError("spec_accept_noalloc needs caller-supplied out_tokens and out_num")
    _want(out_tokens, torch.int32, "out_tokens", (b, kd + 1))
    _want(out_num, torch.int32, "out_num", (b,))
    _want_flags(dev_flags)
    _check(get_lib().spec_accept_noalloc(_ptr(target), _ptr(draft), _ptr(tokens), _ptr(uniforms), b, kd, v,
                                         _ptr(out_tokens), _ptr(out_num), _ptr(dev_flags), _stream(stream)),
           "spec_accept_noalloc")
    return out_tokens, out_num


def spec_accept_sampled_workspace_bytes(b: int, kd: int, v: int) -> int:
    return int(get_lib().spec_accept_sampled_workspace_bytes(b, kd, v))


def spec_accept_sampled(target: torch.Tensor, draft: torch.Tensor | None, tokens: torch.Tensor | None,
                        uniforms: torch.Tensor, temperature: float = 1.0, top_k: int = 0,
                        top_p: float = 1.0, mask: torch.Tensor | None = None,
                        out_tokens: torch.Tensor | None = None, out_num: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, dev_flags: torch.Tensor | None = None,
                        stream=None):
    """spec_accept on transformed laws: mask, temperature, top-k, top-p (see the C header).

    mask: int32 [b, kd+1, ceil(v/32)] holding the uint32 mask words (bit t % 32 of word
    t // 32 = token t allowed), or None.
    """
    _want(target, torch.float32, "target")
    b, kd1, v = target.shape
    kd = kd1 - 1
    if kd > 0:
        _want(draft, torch.float32, "draft")
        _want(tokens, torch.int32, "tokens")
        if draft.shape != (b, kd, v) or tokens.shape != (b, kd):
            raise ValueError("draft/tokens shape mismatch")
    else:
        draft = tokens = None
    _want(uniforms, torch.float32, "uniforms")
    if uniforms.shape != (b, kd + 1):
        raise ValueError("uniforms must be [b, kd+1]")
    if mask is not None:
        _want(mask, torch.int32, "mask")
        if mask.shape != (b, kd + 1, (v + 31) // 32):
            raise ValueError("mask must be [b, kd+1, ceil(v/32)]")
    dev = target.device
    if out_tokens is None:
        out_tokens = torch.empty((b, kd + 1), dtype=torch.int32, device=dev)
    if out_num is None:
        out_num = torch.empty((b,), dtype=torch.int32, device=dev)
    _want(out_tokens, torch.int32, "out_tokens", (b, kd + 1))
    _want(out_num, torch.int32, "out_num", (b,))
    need = spec_accept_sampled_workspace_bytes(b, kd, v)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    _want(workspace, torch.uint8, "workspace")
    _want_flags(dev_flags)
    _check(get_lib().spec_accept_sampled(_ptr(target), _ptr(draft), _ptr(tokens), _ptr(uniforms), b, kd, v,
                                         float(temperature), int(top_k), float(top_p), _ptr(mask),
                                         _ptr(out_tokens), _ptr(out_num), _ptr(workspace), workspace.numel(),
                                         _ptr(dev_flags), _stream(stream)), "spec_accept_sampled")
    return out_tokens, out_num


def spec_sampling_thresholds_workspace_bytes(rows: int, v: int) -> int:
    return int(get_lib().spec_sampling_thresholds_workspace_bytes(rows, v))


def spec_sampling_thresholds(logits: torch.Tensor, temperature: float = 1.0, top_k: int = 0,
                             top_p: float = 1.0, mask: torch.Tensor | None = None,
                             out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                             stream=None) -> torch.Tensor:
    """Top-k / top-p thresholds of fp32 logit rows [rows, v] (see the C header).

    Returns int32 [rows] holding the uint32 order-key thresholds (token t of a row is kept iff
    allowed, finite and key(z_t) >= threshold). mask: int32 [rows, ceil(v/32)] of uint32 words.
    """
    _want(logits, torch.float32, "logits")
    rows, v = logits.shape
    if mask is not None:
        _want(mask, torch.int32, "mask", (rows, (v + 31) // 32))
    dev = logits.device
    if out is None:
        out = torch.empty((rows,), dtype=torch.int32, device=dev)
    _want(out, torch.int32, "out", (rows,))
    need = spec_sampling_thresholds_workspace_bytes(rows, v)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    _want(workspace, torch.uint8, "workspace")
    _check(get_lib().spec_sampling_thresholds(_ptr(logits), rows, v, float(temperature), int(top_k),
                                              float(top_p), _ptr(mask), _ptr(out), _ptr(workspace),
                                              workspace.numel(), _stream(stream)), "spec_sampling_thresholds")
    return out


def nvfp4_quantize(w: torch.Tensor, codes: torch.Tensor | None = None, scales: torch.Tensor | None = None,
                   global_scale: torch.Tensor | None = None, dev_flags: torch.Tensor | None = None,
                   stream=None):
    """fp32 W[n, k] -> (codes uint8 [n, k/2], scales uint8 [n, k/16] E4M3, global_scale fp32 [1])."""
    _want(w, torch.float32, "w")
    n, k = w.shape
    dev = w.device
    if codes is None:
        codes = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((n, k // 16), dtype=torch.uint8, device=dev)
    if global_scale is None:
        global_scale = torch.empty((1,), dtype=torch.float32, device=dev)
    _want(codes, torch.uint8, "codes", (n, k // 2))
    _want(scales, torch.uint8, "scales", (n, k // 16))
    _want(global_scale, torch.float32, "global_scale", (1,))
    _want_flags(dev_flags)
    _check(get_lib().nvfp4_quantize(_ptr(w), n, k, _ptr(codes), _ptr(scales), _ptr(global_scale),
                                    _ptr(dev_flags), _stream(stream)), "nvfp4_quantize")
    return codes, scales, global_scale


def nvfp4_verify_gemm(codes: torch.Tensor, scales: torch.Tensor, global_scale: torch.Tensor,
                      x: torch.Tensor, y: torch.Tensor | None = None, stream=None):
    """Y[m, n] = X[m, k] · Ŵᵀ over NVFP4 weights (codes [n, k/2], E4M3 scales [n, k/16], fp32 g)."""
    _want(codes, torch.uint8, "codes")
    _want(scales, torch.uint8, "scales")
    _want(global_scale, torch.float32, "global_scale", (1,))
    _want(x, torch.bfloat16, "x")
    n = codes.shape[0]
    k = codes.shape[1] * 2
    m = x.shape[0]
    if x.shape != (m, k) or scales.shape != (n, k // 16):
        raise ValueError("shape mismatch")
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _want(y, torch.float32, "y", (m, n))
    _check(get_lib().nvfp4_verify_gemm(_ptr(codes), _ptr(scales), _ptr(global_scale), n, k, _ptr(x), m,
                                       _ptr(y), _stream(stream)), "nvfp4_verify_gemm")
    return y


def nvfp4_verify_gemm_grouped(items, ys=None, stream=None):
    """Several NVFP4 products with the same k and m in one launch.

    items: list of (codes [n_i, k/2], scales [n_i, k/16], global_scale fp32 [1], x [m, k] bf16).
    Returns the list of outputs y_i [m, n_i] fp32 (or fills the given ys).
    """
    if not items:
        raise ValueError("no products")
    k = items[0][0].shape[1] * 2
    m = items[0][3].shape[0]
    arr = (NvProblem * len(items))()
    out = []
    for i, (codes, scales, g, x) in enumerate(items):
        _want(codes, torch.uint8, "codes")
        _want(scales, torch.uint8, "scales")
        _want(g, torch.float32, "global_scale")
        _want(x, torch.bfloat16, "x")
        n = codes.shape[0]
        if codes.shape[1] * 2 != k or x.shape != (m, k) or scales.shape != (n, k // 16):
            raise ValueError("all products must share k and m")
        y = ys[i] if ys is not None else torch.empty((m, n), dtype=torch.float32, device=x.device)
        _want(y, torch.float32, "y", (m, n))
        arr[i] = NvProblem(codes.data_ptr(), scales.data_ptr(), g.data_ptr(), x.data_ptr(), y.data_ptr(), n)
        out.append(y)
    _check(get_lib().nvfp4_verify_gemm_grouped(arr, len(items), k, m, _stream(stream)),
           "nvfp4_verify_gemm_grouped")
    return out


ACT_FP8 = 0  # MXS_ACT_FP8: MX-FP8 (E4M3) activations
ACT_FP4 = 4  # MXS_ACT_FP4: MX-FP4 (E2M1) activations


def mx_quantize_act(x: torch.Tensor, fmt: int, codes: torch.Tensor | None = None,
                    scales: torch.Tensor | None = None, dev_flags: torch.Tensor | None = None, stream=None):
    """bf16 X[m, k] -> (codes, scales): MX-FP8 codes [m, k] or MX-FP4 codes [m, k/2]; scales [m, k/32]."""
    _want(x, torch.bfloat16, "x")
    m, k = x.shape
    if fmt not in (ACT_FP8, ACT_FP4):
        raise ValueError("fmt must be ACT_FP8 or ACT_FP4")
    if codes is None:
        codes = torch.empty((m, k if fmt == ACT_FP8 else k // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((m, k // 32), dtype=torch.uint8, device=x.device)
    _want(codes, torch.uint8, "codes", (m, k if fmt == ACT_FP8 else k // 2))
    _want(scales, torch.uint8, "scales", (m, k // 32))
    _want_flags(dev_flags)
    _check(get_lib().mx_quantize_act(_ptr(x), m, k, fmt, _ptr(codes), _ptr(scales), _ptr(dev_flags),
                                     _stream(stream)), "mx_quantize_act")
    return codes, scales


def mx_verify_gemm_act(codes: torch.Tensor, scales: torch.Tensor, act_codes: torch.Tensor,
                       act_scales: torch.Tensor, fmt: int, y: torch.Tensor | None = None, stream=None):
    """Y[m, n] = X^ · Ŵᵀ: MX-FP4 weights times MX-FP8 / MX-FP4 activations (fmt ACT_FP8 / ACT_FP4)."""
    for t, nm in ((codes, "codes"), (scales, "scales"), (act_codes, "act_codes"), (act_scales, "act_scales")):
        _want(t, torch.uint8, nm)
    n = codes.shape[0]
    k = codes.shape[1] * 2
    m = act_codes.shape[0]
    want_cols = k if fmt == ACT_FP8 else k // 2
    if act_codes.shape != (m, want_cols) or act_scales.shape != (m, k // 32) or scales.shape != (n, k // 32):
        raise ValueError("shape mismatch")
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=codes.device)
    _want(y, torch.float32, "y", (m, n))
    _check(get_lib().mx_verify_gemm_act(_ptr(codes), _ptr(scales), n, k, _ptr(act_codes), _ptr(act_scales), fmt,
                                        m, _ptr(y), _stream(stream)), "mx_verify_gemm_act")
    return y


def mxfp4_tiled_bytes(n: int, k: int) -> int:
    return int(get_lib().mxfp4_tiled_bytes(n, k))


def mxfp4_tile_codes(codes: torch.Tensor, tiled: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Row-layout MX-FP4 codes [n, k/2] -> the tiled layout (uint8, mxfp4_tiled_bytes(n, k) bytes)."""
    _want(codes, torch.uint8, "codes")
    n, k = codes.shape[0], codes.shape[1] * 2
    nb = mxfp4_tiled_bytes(n, k)
    if nb == 0:
        raise ValueError("k must be a multiple of 128")
    if tiled is None:
        tiled = torch.empty((nb,), dtype=torch.uint8, device=codes.device)
    _want(tiled, torch.uint8, "tiled")
    if tiled.numel() < nb:
        raise ValueError(f"tiled needs {nb} bytes")
    _check(get_lib().mxfp4_tile_codes(_ptr(codes), n, k, _ptr(tiled), _stream(stream)), "mxfp4_tile_codes")
    return tiled


def mxfp4_tiled_scale_bytes(n: int, k: int) -> int:
    return int(get_lib().mxfp4_tiled_scale_bytes(n, k))


def mxfp4_tile_scales(scales: torch.Tensor, tiled: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Row-layout E8M0 scales [n, k/32] -> the tiled scale layout (uint8, mxfp4_tiled_scale_bytes(n, k) bytes)."""
    _want(scales, torch.uint8, "scales")
    n, k = scales.shape[0], scales.shape[1] * 32
    nb = mxfp4_tiled_scale_bytes(n, k)
    if nb == 0:
        raise ValueError("k must be a multiple of 128")
    if tiled is None:
        tiled = torch.empty((nb,), dtype=torch.uint8, device=scales.device)
    _want(tiled, torch.uint8, "tiled")
    if tiled.numel() < nb:
        raise ValueError(f"tiled needs {nb} bytes")
    _check(get_lib().mxfp4_tile_scales(_ptr(scales), n, k, _ptr(tiled), _stream(stream)), "mxfp4_tile_scales")
    return tiled


def mx_verify_gemm_act_tiled(tiled_codes: torch.Tensor, tiled_scales: torch.Tensor, n: int, k: int,
                             act_codes: torch.Tensor, act_scales: torch.Tensor, fmt: int,
                             y: torch.Tensor | None = None, stream=None):
    """mx_verify_gemm_act on weights tiled by mxfp4_tile_codes / mxfp4_tile_scales (bit-identical result)."""
    for t, nm in ((tiled_codes, "tiled_codes"), (tiled_scales, "tiled_scales"), (act_codes, "act_codes"),
                  (act_scales, "act_scales")):
        _want(t, torch.uint8, nm)
    m = act_codes.shape[0]
    want_cols = k if fmt == ACT_FP8 else k // 2
    if act_codes.shape != (m, want_cols) or act_scales.shape != (m, k // 32) \
            or tiled_codes.numel() < mxfp4_tiled_bytes(n, k) or tiled_scales.numel() < mxfp4_tiled_scale_bytes(n, k):
        raise ValueError("shape mismatch")
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=act_codes.device)
    _want(y, torch.float32, "y", (m, n))
    _check(get_lib().mx_verify_gemm_act_tiled(_ptr(tiled_codes), _ptr(tiled_scales), n, k, _ptr(act_codes),
                                              _ptr(act_scales), fmt, m, _ptr(y), _stream(stream)),
           "mx_verify_gemm_act_tiled")
    return y


def mxfp4_verify_gemm_tiled(tiled_codes: torch.Tensor, tiled_scales: torch.Tensor, n: int, k: int,
                            x: torch.Tensor, y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """mxfp4_verify_gemm on weights tiled by mxfp4_tile_codes / mxfp4_tile_scales (bit-identical to
    mxfp4_verify_gemm wherever both run the same kernel)."""
    _want(tiled_codes, torch.uint8, "tiled_codes")
    _want(tiled_scales, torch.uint8, "tiled_scales")
    _want(x, torch.bfloat16, "x")
    m = x.shape[0]
    if x.shape[1] != k or tiled_codes.numel() < mxfp4_tiled_bytes(n, k) \
            or tiled_scales.numel() < mxfp4_tiled_scale_bytes(n, k):
        raise ValueError("shape mismatch")
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _want(y, torch.float32, "y", (m, n))
    _check(get_lib().mxfp4_verify_gemm_tiled(_ptr(tiled_codes), _ptr(tiled_scales), n, k, _ptr(x), m, _ptr(y),
                                             _stream(stream)), "mxfp4_verify_gemm_tiled")
    return y


def mxfp4_verify_gemm_grouped_tiled(items, ys=None, stream=None):
    """mxfp4_verify_gemm_grouped on tiled weights.

    items: list of (tiled_codes uint8, tiled_scales uint8, n, x [m, k] bf16), the tiled buffers
    as mxfp4_tile_codes / mxfp4_tile_scales return them. Returns the list of y_i [m, n_i] fp32
    (or fills the given ys).
    """
    if not items:
        raise ValueError("no products")
    m, k = items[0][3].shape
    arr = (GemmProblem * len(items))()
    out = []
    for i, (tc, ts, n, x) in enumerate(items):
        _want(tc, torch.uint8, "tiled_codes")
        _want(ts, torch.uint8, "tiled_scales")
        _want(x, torch.bfloat16, "x")
        if x.shape != (m, k) or tc.numel() < mxfp4_tiled_bytes(n, k) or ts.numel() < mxfp4_tiled_scale_bytes(n, k):
            raise ValueError("all products must share k and m, and tiled buffers must hold their weights")
        y = ys[i] if ys is not None else torch.empty((m, n), dtype=torch.float32, device=x.device)
        _want(y, torch.float32, "y", (m, n))
        arr[i] = GemmProblem(tc.data_ptr(), ts.data_ptr(), x.data_ptr(), y.data_ptr(), n)
        out.append(y)
    _check(get_lib().mxfp4_verify_gemm_grouped_tiled(arr, len(items), k, m, _stream(stream)),
           "mxfp4_verify_gemm_grouped_tiled")
    return out


def nvfp4_verify_gemm_grouped_tiled(items, ys=None, stream=None):
    """nvfp4_verify_gemm_grouped with the codes tiled by mxfp4_tile_codes (scales in the row layout).

    items: list of (tiled_codes uint8, scales [n_i, k/16], global_scale fp32 [1], n_i, x [m, k] bf16).
    """
    if not items:
        raise ValueError("no products")
    m, k = items[0][4].shape
    arr = (NvProblem * len(items))()
    out = []
    for i, (tc, scales, g, n, x) in enumerate(items):
        _want(tc, torch.uint8, "tiled_codes")
        _want(scales, torch.uint8, "scales")
        _want(g, torch.float32, "global_scale")
        _want(x, torch.bfloat16, "x")
        if x.shape != (m, k) or scales.shape != (n, k // 16) or tc.numel() < mxfp4_tiled_bytes(n, k):
            raise ValueError("all products must share k and m, and tiled codes must hold their weights")
        y = ys[i] if ys is not None else torch.empty((m, n), dtype=torch.float32, device=x.device)
        _want(y, torch.float32, "y", (m, n))
        arr[i] = NvProblem(tc.data_ptr(), scales.data_ptr(), g.data_ptr(), x.data_ptr(), y.data_ptr(), n)
        out.append(y)
    _check(get_lib().nvfp4_verify_gemm_grouped_tiled(arr, len(items), k, m, _stream(stream)),
           "nvfp4_verify_gemm_grouped_tiled")
    return out
