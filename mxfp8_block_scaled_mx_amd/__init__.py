"""Python binding of the MI355X MXFP8 grouped-MLP library (libmxfp8.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (include/mxfp8.h). PyTorch provides device memory
and the current stream. There is no CPU or PyTorch fallback: if the library
is missing, load() raises.

Entry points mirror the C ABI: quantize (mx_quantize), grouped_gemm
(mx_grouped_gemm), grouped_mlp_fwd / grouped_mlp_bwd, plus GroupedMLP, an
autograd Function over the fused forward/backward pair (GroupedLinear ->
ScaledSwiGLU -> GroupedLinear with routing-weight scaling: "Efficient MoE
training for biological foundation models", Key technical approaches item 3).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "load", "lib_path", "MXError", "MX_BF16", "MX_F32", "MX_GROUP_M", "MX_GROUP_K",
    "MAX_GROUPS", "padded_sizes", "quantize", "grouped_gemm", "mlp_sizes",
    "grouped_mlp_fwd", "grouped_mlp_bwd", "GroupedMLP", "MLPState", "MLPRunner",
    "set_stage_events", "FWD_STAGES", "BWD_STAGES", "mx_quantize_fp4", "mx_gemm_fp4", "mx_grouped_gemm_fp4",
]

FWD_STAGES = ("quantize_x", "quantize_w1", "quantize_w2", "gemm1_swiglu", "gemm2")
BWD_STAGES = ("quantize_dy", "dgrad2_swiglu_bwd", "dprobs_reduce", "wgrad2", "dgrad1", "wgrad1")

MX_BF16, MX_F32 = 0, 1
MX_GROUP_M, MX_GROUP_K = 0, 1
MAX_GROUPS = 128
STATUS = {0: "MX_OK", 1: "MX_EINVAL", 2: "MX_ESHAPE", 3: "MX_EALIGN",
          4: "MX_EWORKSPACE", 5: "MX_EHIP", 6: "MX_EUNSUPPORTED"}

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    """The built library: lib/libmxfp8.so in the package, or the file named by
    the MXFP8_AMD_LIB environment variable (another build of the same sources)."""
    return os.environ.get("MXFP8_AMD_LIB") or os.path.join(_HERE, "lib", "libmxfp8.so")


class MXError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class _Dims(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("rows", ctypes.c_int64),
                ("hidden", ctypes.c_int64), ("ffn", ctypes.c_int64)]


_lib = None


def load() -> ctypes.CDLL:
    """Load libmxfp8.so (build it with mxfp8_block_scaled_mx_amd.build first)."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path} is missing "
                           "(run python -m mxfp8_block_scaled_mx_amd.build)")
    L = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    p64 = ctypes.POINTER(ctypes.c_int64)
    L.mx_status_string.restype = ctypes.c_char_p
    L.mx_status_string.argtypes = [ctypes.c_int]
    L.mx_last_error.restype = ctypes.c_char_p
    L.mx_last_error.argtypes = []
    L.mx_version.restype = ctypes.c_int
    L.mx_quantize.restype = ctypes.c_int
    L.mx_quantize.argtypes = [vp, i32, i64, i64, p64, i32, vp, vp, vp, vp, vp]
    L.mx_grouped_gemm.restype = ctypes.c_int
    L.mx_grouped_gemm.argtypes = [i32, i32, p64, i64, i64, i64, vp, vp, i64, vp, vp, i64, i64,
                                  vp, i32, i64, i64, i32, vp]
    L.grouped_mlp_sizes.restype = ctypes.c_int
    L.grouped_mlp_sizes.argtypes = [ctypes.POINTER(_Dims), p64, ctypes.POINTER(sz),
                                    ctypes.POINTER(sz), ctypes.POINTER(sz)]
    L.grouped_mlp_intermediates.restype = ctypes.c_int
    L.grouped_mlp_intermediates.argtypes = [ctypes.POINTER(_Dims), p64, ctypes.c_void_p]
    L.grouped_mlp_fwd.restype = ctypes.c_int
    L.grouped_mlp_fwd.argtypes = [ctypes.POINTER(_Dims), p64, vp, vp, vp, vp, vp, vp, sz, vp, sz, vp]
    L.grouped_mlp_bwd.restype = ctypes.c_int
    L.grouped_mlp_bwd.argtypes = [ctypes.POINTER(_Dims), p64, vp, vp, vp, sz, vp, vp, vp, vp, i32,
                                  vp, sz, vp]
    L.grouped_mlp_weight_cache_bytes.restype = ctypes.c_int
    L.grouped_mlp_weight_cache_bytes.argtypes = [ctypes.POINTER(_Dims), ctypes.POINTER(sz)]
    L.grouped_mlp_quantize_weights.restype = ctypes.c_int
    L.grouped_mlp_quantize_weights.argtypes = [ctypes.POINTER(_Dims), vp, vp, vp, sz, vp]
    L.grouped_mlp_fwd_cached.restype = ctypes.c_int
    L.grouped_mlp_fwd_cached.argtypes = [ctypes.POINTER(_Dims), p64, vp, vp, vp, sz, vp, vp, sz, vp, sz, vp]
    L.grouped_mlp_bwd_cached.restype = ctypes.c_int
    L.grouped_mlp_bwd_cached.argtypes = [ctypes.POINTER(_Dims), p64, vp, vp, vp, sz, vp, sz, vp, vp, vp, vp,
                                         i32, vp, sz, vp]
    L.mx_moe_dispatch_workspace_bytes.restype = sz
    L.mx_moe_dispatch_workspace_bytes.argtypes = [i64, i32, i32]
    L.mx_moe_dispatch.restype = ctypes.c_int
    L.mx_moe_dispatch.argtypes = [vp, vp, vp, i64, i64, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    L.mx_moe_dispatch_noalloc.restype = ctypes.c_int
    L.mx_moe_dispatch_noalloc.argtypes = [vp, vp, vp, i64, i64, i32, i32, vp, vp, vp, vp, vp, vp]
    L.mx_moe_combine.restype = ctypes.c_int
    L.mx_moe_combine.argtypes = [vp, vp, i64, i64, i32, vp, vp]
    L.grouped_mlp_bwd_gather.restype = ctypes.c_int
    L.grouped_mlp_bwd_gather.argtypes = [ctypes.POINTER(_Dims), p64, vp, i64, vp, vp, vp, sz, vp, vp, vp, vp, i32,
                                         vp, sz, vp]
    L.grouped_mlp_fwd_gather.restype = ctypes.c_int
    L.grouped_mlp_fwd_gather.argtypes = [ctypes.POINTER(_Dims), p64, vp, i64, vp, vp, vp, vp, vp, vp, sz, vp, sz, vp]
    L.mx_quantize_fp4.restype = ctypes.c_int
    L.mx_quantize_fp4.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp]
    L.mx_gemm_fp4.restype = ctypes.c_int
    L.mx_gemm_fp4.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, i32, vp]
    L.mx_grouped_gemm_fp4.restype = ctypes.c_int
    L.mx_grouped_gemm_fp4.argtypes = [vp, vp, vp, vp, p64, i32, i64, i64, vp, i32, vp]
    L.grouped_mlp_sizes_device_split.restype = ctypes.c_int
    L.grouped_mlp_sizes_device_split.argtypes = [ctypes.POINTER(_Dims), ctypes.POINTER(sz), ctypes.POINTER(sz),
                                                 ctypes.POINTER(sz)]
    L.grouped_mlp_fwd_device_split.restype = ctypes.c_int
    L.grouped_mlp_fwd_device_split.argtypes = [ctypes.POINTER(_Dims), vp, vp, i64, vp, vp, vp, vp, vp, sz, vp, vp,
                                               sz, vp, sz, vp]
    L.grouped_mlp_bwd_device_split.restype = ctypes.c_int
    L.grouped_mlp_bwd_device_split.argtypes = [ctypes.POINTER(_Dims), vp, vp, i64, vp, vp, vp, sz, vp, sz, vp, vp,
                                               vp, vp, i32, vp, sz, vp]
    L.mx_quantize_fp4_colwise_grouped.restype = ctypes.c_int
    L.mx_quantize_fp4_colwise_grouped.argtypes = [vp, i64, i64, p64, i32, vp, vp, vp]
    L.mx_grouped_gemm_fp4_wgrad.restype = ctypes.c_int
    L.mx_grouped_gemm_fp4_wgrad.argtypes = [vp, vp, vp, vp, p64, i32, i64, i64, vp, i32, vp]
    L.grouped_mlp_fp4_sizes.restype = ctypes.c_int
    L.grouped_mlp_fp4_sizes.argtypes = [ctypes.POINTER(_Dims), p64, ctypes.POINTER(sz),
                                        ctypes.POINTER(sz), ctypes.POINTER(sz)]
    L.grouped_mlp_fwd_fp4.restype = ctypes.c_int
    L.grouped_mlp_fwd_fp4.argtypes = [ctypes.POINTER(_Dims), p64, vp, vp, vp, vp, vp, vp, sz, vp, sz, vp]
    L.grouped_mlp_fp4_weight_cache_bytes.restype = ctypes.c_int
    L.grouped_mlp_fp4_weight_cache_bytes.argtypes = [ctypes.POINTER(_Dims), ctypes.POINTER(sz)]
    L.grouped_mlp_fp4_quantize_weights.restype = ctypes.c_int
    L.grouped_mlp_fp4_quantize_weights.argtypes = [ctypes.POINTER(_Dims), vp, vp, vp, sz, vp]
    L.grouped_mlp_fwd_fp4_cached.restype = ctypes.c_int
    L.grouped_mlp_fwd_fp4_cached.argtypes = [ctypes.POINTER(_Dims), p64, vp, vp, vp, sz, vp, vp, sz, vp, sz, vp]
    L.grouped_mlp_bwd_fp4_cached.restype = ctypes.c_int
    L.grouped_mlp_bwd_fp4_cached.argtypes = [ctypes.POINTER(_Dims), p64, vp, vp, vp, sz, vp, sz, vp, vp, vp, vp,
                                             i32, vp, sz, vp]
    L.grouped_mlp_bwd_fp4.restype = ctypes.c_int
    L.grouped_mlp_bwd_fp4.argtypes = [ctypes.POINTER(_Dims), p64, vp, vp, vp, sz, vp, vp, vp, vp, i32,
                                      vp, sz, vp]
    L.mx_quantize_nvfp4.restype = ctypes.c_int
    L.mx_quantize_nvfp4.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp, vp]
    L.mx_gemm_nvfp4.restype = ctypes.c_int
    L.mx_gemm_nvfp4.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, vp, i32, vp]
    L.mx_grouped_gemm_nvfp4.restype = ctypes.c_int
    L.mx_grouped_gemm_nvfp4.argtypes = [vp, vp, vp, vp, vp, vp, p64, i32, i64, i64, vp, i32, vp]
    L.mx_device_copy.restype = ctypes.c_int
    L.mx_device_copy.argtypes = [vp, vp, i64, vp]
    L.mx_set_stage_events.restype = ctypes.c_int
    L.mx_set_stage_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), i32]
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise MXError(status, load().mx_last_error().decode())


def _i64_array(vals):
    vals = [int(v) for v in vals]
    return (ctypes.c_int64 * max(1, len(vals)))(*vals)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def padded_sizes(sizes):
    return [(int(m) + 31) // 32 * 32 for m in sizes]


def quantize(x: torch.Tensor, group_sizes=None, rowwise: bool = True, colwise: bool = True,
             stream=None):
    """MXFP8 of a 2-D bf16/fp32 CUDA tensor -> dict(q_row, s_row, q_col, s_col).

    Rowwise: codes [rows, cols], scales [rows, cols/32]. Columnwise (with
    optional row groups): codes [cols, sumP], scales [cols, sumP/32]."""
    if not (isinstance(x, torch.Tensor) and x.dtype in (torch.bfloat16, torch.float32) and x.dim() == 2
            and x.is_contiguous() and x.is_cuda):
        raise ValueError("quantize: x must be a contiguous 2-D bfloat16 or float32 CUDA tensor")
    L = load()
    dt = {torch.bfloat16: MX_BF16, torch.float32: MX_F32}[x.dtype]
    rows, cols = x.shape
    dev = x.device
    out = {"q_row": None, "s_row": None, "q_col": None, "s_col": None}
    if rowwise:
        out["q_row"] = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        out["s_row"] = torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)
    if colwise:
        P = sum(padded_sizes(group_sizes if group_sizes is not None else [rows]))
        out["q_col"] = torch.empty((cols, P), dtype=torch.uint8, device=dev)
        out["s_col"] = torch.empty((cols, P // 32), dtype=torch.uint8, device=dev)
    gs = None if group_sizes is None else _i64_array(group_sizes)
    ng = 0 if group_sizes is None else len(group_sizes)
    _check(L.mx_quantize(_ptr(x), dt, rows, cols, gs, ng, _ptr(out["q_row"]), _ptr(out["s_row"]),
                         _ptr(out["q_col"]), _ptr(out["s_col"]), _stream(stream)))
    return out


def grouped_gemm(mode: int, sizes, a_q, a_s, b_q, b_s, *, N: int, K: int, M: int | None = None,
                 lda: int | None = None, ldb: int | None = None, b_group_stride: int = 0,
                 out: torch.Tensor | None = None, out_dtype=torch.float32, accumulate: bool = False,
                 c_group_stride: int | None = None, stream=None):
    """Grouped block-scaled GEMM C = A . B^T (mx_grouped_gemm).

    MX_GROUP_M: A [M, lda] rows split by sizes, B_g = b_q + g*b_group_stride
    ([N, ldb]); C [M, N]. MX_GROUP_K: K = sum of padded sizes, C [G, M, N]."""
    L = load()
    G = len(sizes)
    if M is None:
        M = sum(int(s) for s in sizes) if mode == MX_GROUP_M else a_q.shape[0]
    lda = a_q.shape[1] if lda is None else lda
    ldb = b_q.shape[-1] if ldb is None else ldb
    if out is None:
        shape = (M, N) if mode == MX_GROUP_M else (G, M, N)
        out = torch.empty(shape, dtype=out_dtype, device=a_q.device)
    cdt = {torch.bfloat16: MX_BF16, torch.float32: MX_F32}[out.dtype]
    if c_group_stride is None:
        c_group_stride = M * N if mode == MX_GROUP_K else 0
    # the extents the kernel reads and writes must lie inside the tensors
    for t, nm in ((a_q, "a_q"), (a_s, "a_s"), (b_q, "b_q"), (b_s, "b_s")):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous() or t.dtype != torch.uint8:
            raise ValueError(f"grouped_gemm: {nm} must be a contiguous uint8 CUDA tensor")
    if not out.is_cuda or not out.is_contiguous():
        raise ValueError("grouped_gemm: out must be a contiguous CUDA tensor")
    ldc = out.shape[-1]
    # (row r of a [rows, ld] operand spans [r * ld, r * ld + K); scales 1/32 of that)
    b_end = (G - 1) * b_group_stride + (N - 1) * ldb + K if mode == MX_GROUP_M else (N - 1) * ldb + K
    need = {"a_q": (M - 1) * lda + K, "a_s": ((M - 1) * lda + K) // 32, "b_q": b_end, "b_s": b_end // 32,
            "out": (M - 1) * ldc + N if mode == MX_GROUP_M else (G - 1) * c_group_stride + (M - 1) * ldc + N}
    if M == 0:
        need.update(a_q=0, a_s=0, out=0)
    for t, nm in ((a_q, "a_q"), (a_s, "a_s"), (b_q, "b_q"), (b_s, "b_s"), (out, "out")):
        if t.numel() < need[nm]:
            raise ValueError(f"grouped_gemm: {nm} has {t.numel()} elements, the call addresses {need[nm]}")
    _check(L.mx_grouped_gemm(mode, G, _i64_array(sizes), M, N, K, _ptr(a_q), _ptr(a_s), lda,
                             _ptr(b_q), _ptr(b_s), ldb, b_group_stride, _ptr(out), cdt,
                             out.shape[-1], c_group_stride, int(accumulate), _stream(stream)))
    return out


def _dims(E, R, H, F):
    return _Dims(int(E), int(R), int(H), int(F))


def mlp_sizes(E: int, R: int, H: int, F: int, split_sizes):
    """(fwd workspace, saved, bwd workspace) byte sizes for one call."""
    L = load()
    f, s, b = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(L.grouped_mlp_sizes(ctypes.byref(_dims(E, R, H, F)), _i64_array(split_sizes),
                               ctypes.byref(f), ctypes.byref(s), ctypes.byref(b)))
    return f.value, s.value, b.value


class _Intermediates(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "a_row_codes", "a_row_scales", "h1", "a_col_codes", "a_col_scales",
        "dh1_row_codes", "dh1_row_scales", "dh1_col_codes", "dh1_col_scales")] + [("nq_col", ctypes.c_int64)]


def mlp_intermediates(E: int, R: int, H: int, F: int, split_sizes) -> dict:
    """Byte offsets of the requantized intermediates (A, dH1) and of H1 inside
    the forward workspace, saved and backward workspace buffers, plus nq_col
    (grouped_mlp_intermediates)."""
    L = load()
    out = _Intermediates()
    _check(L.grouped_mlp_intermediates(ctypes.byref(_dims(E, R, H, F)), _i64_array(split_sizes),
                                       ctypes.byref(out)))
    return {n: int(getattr(out, n)) for n, _ in _Intermediates._fields_}


class MLPState:
    """What the fused forward keeps for the backward (a caller-owned buffer);
    fmt is the block format of the forward that filled it, cache the weight
    cache it read (None: it cast the weights itself and saved their
    columnwise copies, which a cached forward does not)."""

    def __init__(self, saved: torch.Tensor, dims, split_sizes, fmt: str = "mxfp8", cache=None):
        self.saved = saved
        self.dims = dims
        self.split_sizes = list(int(s) for s in split_sizes)
        self.fmt = fmt
        self.cache = cache


def _check_state(state: MLPState, fmt: str, cache, who: str):
    """The backward `who` takes the state of a forward of block format fmt
    that used the weight cache `cache` (None: the uncached forward)."""
    if state.fmt != fmt:
        raise ValueError(f"{who} needs the state of an {fmt.upper()} forward, not {state.fmt.upper()}")
    if cache is None and state.cache is not None:
        raise ValueError(f"{who}: the state comes from a cached forward; use the *_cached backward with its cache")
    if cache is not None and state.cache is not cache:
        raise ValueError(f"{who}: the state was not made by the cached forward with this weight cache")


def _expect_all(items):
    """items: (tensor or None, shape, dtype, name, optional). Raise ValueError
    unless every given tensor has its shape and dtype (checked for all first)
    and is a contiguous CUDA tensor. The C ABI takes plain pointers and trusts
    the sizes it is given, so a tensor smaller than the dims would be read or
    written past its end; the bindings check every buffer first."""
    for t, shape, dtype, name, optional in items:
        if t is None:
            if not optional:
                raise ValueError(f"{name} is required")
            continue
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a tensor")
        want = tuple(int(v) for v in shape)
        if tuple(t.shape) != want or t.dtype != dtype:
            raise ValueError(f"{name}: expected {dtype} {want}, got {t.dtype} {tuple(t.shape)}")
    for t, _, _, name, _ in items:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous CUDA tensor")


def _expect(t, shape, dtype, name, optional=False):
    _expect_all([(t, shape, dtype, name, optional)])


def _mlp_items(E, R, H, F, x=None, w1=None, w2=None, probs=None, x_rows=None):
    items = [(probs, (R,), torch.float32, "probs", True)]
    if x is not None:
        items.append((x, (R if x_rows is None else x_rows, H), torch.bfloat16, "x", False))
    if w1 is not None:
        items.append((w1, (E, 2 * F, H), torch.bfloat16, "w1", False))
    if w2 is not None:
        items.append((w2, (E, H, F), torch.bfloat16, "w2", False))
    return items


def _check_split(E, R, split_sizes):
    if len(split_sizes) != E or sum(int(m) for m in split_sizes) != R:
        raise ValueError(f"split_sizes {list(split_sizes)} must have {E} entries summing to {R}")


def _mlp_inputs(E, R, H, F, split_sizes, x=None, w1=None, w2=None, probs=None, x_rows=None, extra=()):
    _check_split(E, R, split_sizes)
    _expect_all(_mlp_items(E, R, H, F, x, w1, w2, probs, x_rows) + list(extra))


def _mlp_grads(E, R, H, F, dw1=None, dw2=None):
    return [(dw1, (E, 2 * F, H), torch.float32, "dw1", True), (dw2, (E, H, F), torch.float32, "dw2", True)]


def _byte_buffer(nbytes: int, device):
    # 256-byte aligned (the caching allocator aligns to at least 512 bytes)
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def grouped_mlp_fwd(x, probs, w1, w2, split_sizes, *, training: bool = True, workspace=None,
                    out=None, stream=None):
    """Fused grouped MLP forward. x [R,H] bf16, w1 [E,2F,H] bf16, w2 [E,H,F] bf16,
    probs [R] fp32 or None. Returns (y [R,H] bf16, MLPState or None)."""
    L = load()
    if x.dim() != 2 or w1.dim() != 3:
        raise ValueError("grouped_mlp_fwd: x must be [R, H] and w1 [E, 2F, H]")
    R, H = x.shape
    E, F2, _ = w1.shape
    F = F2 // 2
    _mlp_inputs(E, R, H, F, split_sizes, x, w1, w2, probs, extra=[(out, (R, H), torch.bfloat16, "out", True)])
    fws, sv, _ = mlp_sizes(E, R, H, F, split_sizes)
    if workspace is None or workspace.numel() < fws:
        workspace = _byte_buffer(fws, x.device)
    y = torch.empty((R, H), dtype=torch.bfloat16, device=x.device) if out is None else out
    saved = _byte_buffer(sv, x.device) if training else None
    _check(L.grouped_mlp_fwd(ctypes.byref(_dims(E, R, H, F)), _i64_array(split_sizes), _ptr(x),
                             _ptr(probs), _ptr(w1), _ptr(w2), _ptr(y), _ptr(saved),
                             0 if saved is None else saved.numel(), _ptr(workspace),
                             workspace.numel(), _stream(stream)))
    state = MLPState(saved, (E, R, H, F), split_sizes) if training else None
    return y, state


def grouped_mlp_fwd_gather(x_tokens, row_token, probs, w1, w2, split_sizes, *, training: bool = True,
                           workspace=None, out=None, stream=None):
    """grouped_mlp_fwd on the routed rows x_tokens[row_token] (row_token as
    mx_moe_dispatch returns it; split_sizes its counts), gathered by the X
    cast itself. Returns (y [R,H] bf16, MLPState or None)."""
    L = load()
    if x_tokens.dim() != 2 or w1.dim() != 3:
        raise ValueError("grouped_mlp_fwd_gather: x_tokens must be [T, H] and w1 [E, 2F, H]")
    T, H = x_tokens.shape
    E, F2, _ = w1.shape
    F = F2 // 2
    R = int(sum(int(m) for m in split_sizes))
    _mlp_inputs(E, R, H, F, split_sizes, x_tokens, w1, w2, probs, x_rows=T,
                extra=[(row_token, (R,), torch.int32, "row_token", R == 0),
                       (out, (R, H), torch.bfloat16, "out", True)])
    fws, sv, _ = mlp_sizes(E, R, H, F, split_sizes)
    if workspace is None or workspace.numel() < fws:
        workspace = _byte_buffer(fws, x_tokens.device)
    y = torch.empty((R, H), dtype=torch.bfloat16, device=x_tokens.device) if out is None else out
    saved = _byte_buffer(sv, x_tokens.device) if training else None
    _check(L.grouped_mlp_fwd_gather(ctypes.byref(_dims(E, R, H, F)), _i64_array(split_sizes), _ptr(x_tokens), T,
                                    _ptr(row_token), _ptr(probs), _ptr(w1), _ptr(w2), _ptr(y), _ptr(saved),
                                    0 if saved is None else saved.numel(), _ptr(workspace), workspace.numel(),
                                    _stream(stream)))
    state = MLPState(saved, (E, R, H, F), split_sizes) if training else None
    return y, state


def grouped_mlp_bwd_gather(dy_tokens, row_token, probs, state: MLPState, *, dw1=None, dw2=None,
                           accumulate: bool = False, want_dprobs: bool = True, workspace=None, stream=None):
    """grouped_mlp_bwd with dY gathered from dy_tokens [T, H] through row_token
    by its cast. Returns (dx [R, H] bf16 per routed row, dprobs, dw1, dw2)."""
    L = load()
    _check_state(state, "mxfp8", None, "grouped_mlp_bwd_gather")
    E, R, H, F = state.dims
    if dy_tokens.dim() != 2:
        raise ValueError("grouped_mlp_bwd_gather: dy_tokens must be [T, H]")
    T = dy_tokens.shape[0]
    _expect_all([(dy_tokens, (T, H), torch.bfloat16, "dy_tokens", False),
                 (row_token, (R,), torch.int32, "row_token", R == 0),
                 (probs, (R,), torch.float32, "probs", True)] + _mlp_grads(E, R, H, F, dw1, dw2))
    _, _, bws = mlp_sizes(E, R, H, F, state.split_sizes)
    if workspace is None or workspace.numel() < bws:
        workspace = _byte_buffer(bws, dy_tokens.device)
    dev = dy_tokens.device
    dx = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
    dprobs = torch.empty((R,), dtype=torch.float32, device=dev) if want_dprobs else None
    if dw1 is None:
        dw1 = torch.empty((E, 2 * F, H), dtype=torch.float32, device=dev)
        accumulate = False if dw2 is None else accumulate
    if dw2 is None:
        dw2 = torch.empty((E, H, F), dtype=torch.float32, device=dev)
    _check(L.grouped_mlp_bwd_gather(ctypes.byref(_dims(E, R, H, F)), _i64_array(state.split_sizes), _ptr(dy_tokens),
                                    T, _ptr(row_token), _ptr(probs), _ptr(state.saved), state.saved.numel(),
                                    _ptr(dx), _ptr(dprobs), _ptr(dw1), _ptr(dw2), int(accumulate), _ptr(workspace),
                                    workspace.numel(), _stream(stream)))
    return dx, dprobs, dw1, dw2


def grouped_mlp_bwd(dy, probs, state: MLPState, *, dw1=None, dw2=None, accumulate: bool = False,
                    want_dprobs: bool = True, workspace=None, stream=None):
    """Fused grouped MLP backward. Returns (dx bf16, dprobs fp32 or None, dw1 fp32, dw2 fp32).
    With accumulate=True, dw1/dw2 (fp32 main grads) are added into."""
    L = load()
    _check_state(state, "mxfp8", None, "grouped_mlp_bwd")
    E, R, H, F = state.dims
    _expect_all([(dy, (R, H), torch.bfloat16, "dy", False), (probs, (R,), torch.float32, "probs", True)]
                + _mlp_grads(E, R, H, F, dw1, dw2))
    _, _, bws = mlp_sizes(E, R, H, F, state.split_sizes)
    if workspace is None or workspace.numel() < bws:
        workspace = _byte_buffer(bws, dy.device)
    dev = dy.device
    dx = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
    dprobs = torch.empty((R,), dtype=torch.float32, device=dev) if want_dprobs else None
    if dw1 is None:
        dw1 = torch.empty((E, 2 * F, H), dtype=torch.float32, device=dev)
        accumulate = False if dw2 is None else accumulate
    if dw2 is None:
        dw2 = torch.empty((E, H, F), dtype=torch.float32, device=dev)
    _check(L.grouped_mlp_bwd(ctypes.byref(_dims(E, R, H, F)), _i64_array(state.split_sizes),
                             _ptr(dy), _ptr(probs), _ptr(state.saved), state.saved.numel(),
                             _ptr(dx), _ptr(dprobs), _ptr(dw1), _ptr(dw2), int(accumulate),
                             _ptr(workspace), workspace.numel(), _stream(stream)))
    return dx, dprobs, dw1, dw2


def mlp_fp4_sizes(E: int, R: int, H: int, F: int, split_sizes):
    """(fwd workspace, saved, bwd workspace) byte sizes of the MXFP4 MLP."""
    L = load()
    f, s, b = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(L.grouped_mlp_fp4_sizes(ctypes.byref(_dims(E, R, H, F)), _i64_array(split_sizes),
                                   ctypes.byref(f), ctypes.byref(s), ctypes.byref(b)))
    return f.value, s.value, b.value


def grouped_mlp_fwd_fp4(x, probs, w1, w2, split_sizes, *, training: bool = True, workspace=None,
                        out=None, stream=None):
    """Grouped MLP forward with every GEMM on MXFP4 copies
    (grouped_mlp_fwd_fp4). Same arguments and shapes as grouped_mlp_fwd;
    returns (y [R,H] bf16, MLPState or None)."""
    L = load()
    if x.dim() != 2 or w1.dim() != 3:
        raise ValueError("grouped_mlp_fwd_fp4: x must be [R, H] and w1 [E, 2F, H]")
    R, H = x.shape
    E, F2, _ = w1.shape
    F = F2 // 2
    _mlp_inputs(E, R, H, F, split_sizes, x, w1, w2, probs, extra=[(out, (R, H), torch.bfloat16, "out", True)])
    fws, sv, _ = mlp_fp4_sizes(E, R, H, F, split_sizes)
    if workspace is None or workspace.numel() < fws:
        workspace = _byte_buffer(fws, x.device)
    y = torch.empty((R, H), dtype=torch.bfloat16, device=x.device) if out is None else out
    saved = _byte_buffer(sv, x.device) if training else None
    _check(L.grouped_mlp_fwd_fp4(ctypes.byref(_dims(E, R, H, F)), _i64_array(split_sizes), _ptr(x),
                                 _ptr(probs), _ptr(w1), _ptr(w2), _ptr(y), _ptr(saved),
                                 0 if saved is None else saved.numel(), _ptr(workspace),
                                 workspace.numel(), _stream(stream)))
    state = MLPState(saved, (E, R, H, F), split_sizes, fmt="mxfp4") if training else None
    return y, state


def grouped_mlp_bwd_fp4(dy, probs, state: MLPState, *, dw1=None, dw2=None, accumulate: bool = False,
                        want_dprobs: bool = True, workspace=None, stream=None):
    """Backward of grouped_mlp_fwd_fp4 (grouped_mlp_bwd_fp4). Returns
    (dx bf16, dprobs fp32 or None, dw1 fp32, dw2 fp32)."""
    L = load()
    _check_state(state, "mxfp4", None, "grouped_mlp_bwd_fp4")
    E, R, H, F = state.dims
    _expect_all([(dy, (R, H), torch.bfloat16, "dy", False), (probs, (R,), torch.float32, "probs", True)]
                + _mlp_grads(E, R, H, F, dw1, dw2))
    _, _, bws = mlp_fp4_sizes(E, R, H, F, state.split_sizes)
    if workspace is None or workspace.numel() < bws:
        workspace = _byte_buffer(bws, dy.device)
    dev = dy.device
    dx = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
    dprobs = torch.empty((R,), dtype=torch.float32, device=dev) if want_dprobs else None
    if dw1 is None:
        dw1 = torch.empty((E, 2 * F, H), dtype=torch.float32, device=dev)
        accumulate = False if dw2 is None else accumulate
    if dw2 is None:
        dw2 = torch.empty((E, H, F), dtype=torch.float32, device=dev)
    _check(L.grouped_mlp_bwd_fp4(ctypes.byref(_dims(E, R, H, F)), _i64_array(state.split_sizes),
                                 _ptr(dy), _ptr(probs), _ptr(state.saved), state.saved.numel(),
                                 _ptr(dx), _ptr(dprobs), _ptr(dw1), _ptr(dw2), int(accumulate),
                                 _ptr(workspace), workspace.numel(), _stream(stream)))
    return dx, dprobs, dw1, dw2


def grouped_mlp_weight_cache_bytes(E: int, H: int, F: int) -> int:
    """Bytes of the MXFP8 weight cache for E experts, hidden H, ffn F."""
    L = load()
    n = ctypes.c_size_t()
    _check(L.grouped_mlp_weight_cache_bytes(ctypes.byref(_dims(E, 0, H, F)), ctypes.byref(n)))
    return n.value


class WeightCache:
    """MXFP8 (fmt "mxfp8") or MXFP4 ("mxfp4") copies of w1 [E,2F,H] and w2
    [E,H,F] in both layouts (a caller-owned device buffer filled by
    grouped_mlp_quantize_weights, resp. grouped_mlp_fp4_quantize_weights)."""

    def __init__(self, E: int, H: int, F: int, device="cuda", fmt: str = "mxfp8"):
        if fmt not in ("mxfp8", "mxfp4"):
            raise ValueError(f"WeightCache: unknown format {fmt!r}")
        self.ehf = (int(E), int(H), int(F))
        self.fmt = fmt
        n = grouped_mlp_weight_cache_bytes(E, H, F) if fmt == "mxfp8" else grouped_mlp_fp4_weight_cache_bytes(E, H, F)
        self.buf = _byte_buffer(n, device)


def grouped_mlp_quantize_weights(w1, w2, cache: WeightCache | None = None, stream=None) -> WeightCache:
    """Cast the bf16 master weights into `cache` (allocated when None); run
    once after each optimizer update, then use the *_cached calls."""
    L = load()
    if w1.dim() != 3:
        raise ValueError("grouped_mlp_quantize_weights: w1 must be [E, 2F, H]")
    E, F2, H = w1.shape
    F = F2 // 2
    _expect_all([(w1, (E, 2 * F, H), torch.bfloat16, "w1", False), (w2, (E, H, F), torch.bfloat16, "w2", False)])
    if cache is None:
        cache = WeightCache(E, H, F, device=w1.device)
    if cache.ehf != (E, H, F) or cache.fmt != "mxfp8":
        raise ValueError(f"weight cache is {cache.fmt} for (E, H, F) = {cache.ehf}, weights are MXFP8 {(E, H, F)}")
    _check(L.grouped_mlp_quantize_weights(ctypes.byref(_dims(E, 0, H, F)), _ptr(w1), _ptr(w2),
                                          _ptr(cache.buf), cache.buf.numel(), _stream(stream)))
    return cache


def grouped_mlp_fwd_cached(x, probs, cache: WeightCache, split_sizes, *, training: bool = True,
                           workspace=None, out=None, stream=None):
    """grouped_mlp_fwd on the cached MXFP8 weights. Returns (y, MLPState or None)."""
    L = load()
    if x.dim() != 2:
        raise ValueError("grouped_mlp_fwd_cached: x must be [R, H]")
    R, H = x.shape
    E, Hc, F = cache.ehf
    if Hc != H or cache.fmt != "mxfp8":
        raise ValueError(f"x has hidden {H}; the weight cache is {cache.fmt} with hidden {Hc}")
    _mlp_inputs(E, R, H, F, split_sizes, x, probs=probs, extra=[(out, (R, H), torch.bfloat16, "out", True)])
    fws, sv, _ = mlp_sizes(E, R, H, F, split_sizes)
    if workspace is None or workspace.numel() < fws:
        workspace = _byte_buffer(fws, x.device)
    y = torch.empty((R, H), dtype=torch.bfloat16, device=x.device) if out is None else out
    saved = _byte_buffer(sv, x.device) if training else None
    _check(L.grouped_mlp_fwd_cached(ctypes.byref(_dims(E, R, H, F)), _i64_array(split_sizes), _ptr(x),
                                    _ptr(probs), _ptr(cache.buf), cache.buf.numel(), _ptr(y), _ptr(saved),
                                    0 if saved is None else saved.numel(), _ptr(workspace),
                                    workspace.numel(), _stream(stream)))
    state = MLPState(saved, (E, R, H, F), split_sizes, cache=cache) if training else None
    return y, state


def grouped_mlp_bwd_cached(dy, probs, state: MLPState, cache: WeightCache, *, dw1=None, dw2=None,
                           accumulate: bool = False, want_dprobs: bool = True, workspace=None, stream=None):
    """grouped_mlp_bwd after grouped_mlp_fwd_cached (same cache).
    Returns (dx bf16, dprobs fp32 or None, dw1 fp32, dw2 fp32)."""
    L = load()
    if cache.fmt != "mxfp8":
        raise ValueError("grouped_mlp_bwd_cached needs an MXFP8 weight cache")
    _check_state(state, "mxfp8", cache, "grouped_mlp_bwd_cached")
    E, R, H, F = state.dims
    _expect_all([(dy, (R, H), torch.bfloat16, "dy", False), (probs, (R,), torch.float32, "probs", True)]
                + _mlp_grads(E, R, H, F, dw1, dw2))
    _, _, bws = mlp_sizes(E, R, H, F, state.split_sizes)
    if workspace is None or workspace.numel() < bws:
        workspace = _byte_buffer(bws, dy.device)
    dev = dy.device
    dx = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
    dprobs = torch.empty((R,), dtype=torch.float32, device=dev) if want_dprobs else None
    if dw1 is None:
        dw1 = torch.empty((E, 2 * F, H), dtype=torch.float32, device=dev)
        accumulate = False if dw2 is None else accumulate
    if dw2 is None:
        dw2 = torch.empty((E, H, F), dtype=torch.float32, device=dev)
    _check(L.grouped_mlp_bwd_cached(ctypes.byref(_dims(E, R, H, F)), _i64_array(state.split_sizes),
                                    _ptr(dy), _ptr(probs), _ptr(cache.buf), cache.buf.numel(),
                                    _ptr(state.saved), state.saved.numel(), _ptr(dx), _ptr(dprobs),
                                    _ptr(dw1), _ptr(dw2), int(accumulate), _ptr(workspace),
                                    workspace.numel(), _stream(stream)))
    return dx, dprobs, dw1, dw2


def grouped_mlp_fp4_weight_cache_bytes(E: int, H: int, F: int) -> int:
    """Bytes of the MXFP4 weight cache for E experts, hidden H, ffn F."""
    L = load()
    n = ctypes.c_size_t()
    _check(L.grouped_mlp_fp4_weight_cache_bytes(ctypes.byref(_dims(E, 0, H, F)), ctypes.byref(n)))
    return n.value


def grouped_mlp_fp4_quantize_weights(w1, w2, cache: WeightCache | None = None, stream=None) -> WeightCache:
    """Cast the bf16 master weights into an MXFP4 weight cache (allocated
    when None); run once after each optimizer update, then use the
    grouped_mlp_*_fp4_cached calls."""
    L = load()
    if w1.dim() != 3:
        raise ValueError("grouped_mlp_fp4_quantize_weights: w1 must be [E, 2F, H]")
    E, F2, H = w1.shape
    F = F2 // 2
    _expect_all([(w1, (E, 2 * F, H), torch.bfloat16, "w1", False), (w2, (E, H, F), torch.bfloat16, "w2", False)])
    if cache is None:
        cache = WeightCache(E, H, F, device=w1.device, fmt="mxfp4")
    if cache.ehf != (E, H, F) or cache.fmt != "mxfp4":
        raise ValueError(f"weight cache is {cache.fmt} for (E, H, F) = {cache.ehf}, weights are MXFP4 {(E, H, F)}")
    _check(L.grouped_mlp_fp4_quantize_weights(ctypes.byref(_dims(E, 0, H, F)), _ptr(w1), _ptr(w2),
                                              _ptr(cache.buf), cache.buf.numel(), _stream(stream)))
    return cache


def grouped_mlp_fwd_fp4_cached(x, probs, cache: WeightCache, split_sizes, *, training: bool = True,
                               workspace=None, out=None, stream=None):
    """grouped_mlp_fwd_fp4 on the cached MXFP4 weights. Returns (y, MLPState or None)."""
    L = load()
    if x.dim() != 2:
        raise ValueError("grouped_mlp_fwd_fp4_cached: x must be [R, H]")
    R, H = x.shape
    E, Hc, F = cache.ehf
    if Hc != H or cache.fmt != "mxfp4":
        raise ValueError(f"x has hidden {H}; the weight cache is {cache.fmt} with hidden {Hc}")
    _mlp_inputs(E, R, H, F, split_sizes, x, probs=probs, extra=[(out, (R, H), torch.bfloat16, "out", True)])
    fws, sv, _ = mlp_fp4_sizes(E, R, H, F, split_sizes)
    if workspace is None or workspace.numel() < fws:
        workspace = _byte_buffer(fws, x.device)
    y = torch.empty((R, H), dtype=torch.bfloat16, device=x.device) if out is None else out
    saved = _byte_buffer(sv, x.device) if training else None
    _check(L.grouped_mlp_fwd_fp4_cached(ctypes.byref(_dims(E, R, H, F)), _i64_array(split_sizes), _ptr(x),
                                        _ptr(probs), _ptr(cache.buf), cache.buf.numel(), _ptr(y), _ptr(saved),
                                        0 if saved is None else saved.numel(), _ptr(workspace),
                                        workspace.numel(), _stream(stream)))
    state = MLPState(saved, (E, R, H, F), split_sizes, fmt="mxfp4", cache=cache) if training else None
    return y, state


def grouped_mlp_bwd_fp4_cached(dy, probs, state: MLPState, cache: WeightCache, *, dw1=None, dw2=None,
                               accumulate: bool = False, want_dprobs: bool = True, workspace=None, stream=None):
    """grouped_mlp_bwd_fp4 after grouped_mlp_fwd_fp4_cached (same cache).
    Returns (dx bf16, dprobs fp32 or None, dw1 fp32, dw2 fp32)."""
    L = load()
    if cache.fmt != "mxfp4":
        raise ValueError("grouped_mlp_bwd_fp4_cached needs an MXFP4 weight cache")
    _check_state(state, "mxfp4", cache, "grouped_mlp_bwd_fp4_cached")
    E, R, H, F = state.dims
    _expect_all([(dy, (R, H), torch.bfloat16, "dy", False), (probs, (R,), torch.float32, "probs", True)]
                + _mlp_grads(E, R, H, F, dw1, dw2))
    _, _, bws = mlp_fp4_sizes(E, R, H, F, state.split_sizes)
    if workspace is None or workspace.numel() < bws:
        workspace = _byte_buffer(bws, dy.device)
    dev = dy.device
    dx = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
    dprobs = torch.empty((R,), dtype=torch.float32, device=dev) if want_dprobs else None
    if dw1 is None:
        dw1 = torch.empty((E, 2 * F, H), dtype=torch.float32, device=dev)
        accumulate = False if dw2 is None else accumulate
    if dw2 is None:
        dw2 = torch.empty((E, H, F), dtype=torch.float32, device=dev)
    _check(L.grouped_mlp_bwd_fp4_cached(ctypes.byref(_dims(E, R, H, F)), _i64_array(state.split_sizes),
                                        _ptr(dy), _ptr(probs), _ptr(cache.buf), cache.buf.numel(),
                                        _ptr(state.saved), state.saved.numel(), _ptr(dx), _ptr(dprobs),
                                        _ptr(dw1), _ptr(dw2), int(accumulate), _ptr(workspace),
                                        workspace.numel(), _stream(stream)))
    return dx, dprobs, dw1, dw2


def mx_quantize_fp4(x: torch.Tensor, colwise: bool = False, stream=None):
    """MXFP4 of bf16 x [rows, cols]: (q [rows, cols/2], s [rows, cols/32]) rowwise
    (two codes per byte, element 2i in the low nibble), plus (q_col [cols,
    rows/2], s_col [cols, rows/32]) when colwise."""
    if not (isinstance(x, torch.Tensor) and x.dtype == torch.bfloat16 and x.dim() == 2 and x.is_contiguous()
            and x.is_cuda):
        raise ValueError("mx_quantize_fp4: x must be a contiguous 2-D bfloat16 CUDA tensor")
    L = load()
    rows, cols = x.shape
    q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
    s = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    qc = torch.empty((cols, rows // 2), dtype=torch.uint8, device=x.device) if colwise else None
    sc = torch.empty((cols, rows // 32), dtype=torch.uint8, device=x.device) if colwise else None
    _check(L.mx_quantize_fp4(_ptr(x), rows, cols, _ptr(q), _ptr(s), _ptr(qc), _ptr(sc), _stream(stream)))
    return (q, s, qc, sc) if colwise else (q, s)


def mx_gemm_fp4(a_q, a_s, b_q, b_s, out_dtype=torch.bfloat16, out=None, stream=None):
    """C [m, n] = A . B^T on rowwise MXFP4 operands (a_q [m, k/2], a_s [m, k/32],
    b_q [n, k/2], b_s [n, k/32]: the layout of mx_quantize_fp4), bf16 or fp32."""
    L = load()
    m, n, k = a_q.shape[0], b_q.shape[0], a_q.shape[1] * 2
    for t in (a_q, a_s, b_q, b_s):
        if t.dtype != torch.uint8 or not t.is_contiguous() or t.dim() != 2:
            raise ValueError("mx_gemm_fp4: codes and scales must be contiguous 2-D uint8 tensors")
    if b_q.shape[1] != a_q.shape[1] or tuple(a_s.shape) != (m, k // 32) or tuple(b_s.shape) != (n, k // 32):
        raise ValueError(f"mx_gemm_fp4: operand shapes {tuple(a_q.shape)}, {tuple(a_s.shape)}, "
                         f"{tuple(b_q.shape)}, {tuple(b_s.shape)} do not describe A [m, k] and B [n, k]")
    if out is not None and (tuple(out.shape) != (m, n) or not out.is_contiguous()
                            or out.dtype not in (torch.bfloat16, torch.float32)):
        raise ValueError("mx_gemm_fp4: out must be a contiguous bf16 or fp32 [m, n] tensor")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=a_q.device)
    dt = MX_F32 if out.dtype == torch.float32 else MX_BF16
    _check(L.mx_gemm_fp4(_ptr(a_q), _ptr(a_s), _ptr(b_q), _ptr(b_s), m, n, k, _ptr(out), dt, _stream(stream)))
    return out


def mx_grouped_gemm_fp4(a_q, a_s, b_q, b_s, group_sizes, out_dtype=torch.bfloat16, out=None, stream=None):
    """Grouped MXFP4 GEMM over split_sizes: rows of group g of A (a_q [M, k/2],
    a_s [M, k/32], M = sum(group_sizes)) times B_g^T with b_q [G, n, k/2],
    b_s [G, n, k/32]; returns C [M, n] (bf16 or fp32)."""
    L = load()
    sizes = [int(v) for v in group_sizes]
    G, n, k = len(sizes), b_q.shape[1], a_q.shape[1] * 2
    m = a_q.shape[0]
    for t in (a_q, a_s, b_q, b_s):
        if t.dtype != torch.uint8 or not t.is_contiguous():
            raise ValueError("mx_grouped_gemm_fp4: codes and scales must be contiguous uint8 tensors")
    if (sum(sizes) != m or tuple(a_s.shape) != (m, k // 32) or tuple(b_q.shape) != (G, n, k // 2)
            or tuple(b_s.shape) != (G, n, k // 32)):
        raise ValueError("mx_grouped_gemm_fp4: operand shapes do not match the group sizes")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=a_q.device)
    if tuple(out.shape) != (m, n) or not out.is_contiguous() or out.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("mx_grouped_gemm_fp4: out must be a contiguous bf16 or fp32 [M, n] tensor")
    dt = MX_F32 if out.dtype == torch.float32 else MX_BF16
    arr = (ctypes.c_int64 * max(G, 1))(*sizes)
    _check(L.mx_grouped_gemm_fp4(_ptr(a_q), _ptr(a_s), _ptr(b_q), _ptr(b_s), arr, G, n, k, _ptr(out), dt,
                                 _stream(stream)))
    return out


def mx_quantize_nvfp4(x: torch.Tensor, colwise: bool = False, rowwise: bool = True, stream=None):
    """NVFP4 of bf16 x [rows, cols] (mx_quantize_nvfp4): returns (q [rows,
    cols/2], s [rows, cols/16] E4M3 codes, amax [1] fp32) rowwise, and with
    colwise also (q_col [cols, rows/2], s_col [cols, rows/16]); None for a
    layout not asked for."""
    if not (isinstance(x, torch.Tensor) and x.dtype == torch.bfloat16 and x.dim() == 2 and x.is_contiguous()
            and x.is_cuda):
        raise ValueError("mx_quantize_nvfp4: x must be a contiguous 2-D bfloat16 CUDA tensor")
    L = load()
    rows, cols = x.shape
    dev = x.device
    q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev) if rowwise else None
    s = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev) if rowwise else None
    qc = torch.empty((cols, rows // 2), dtype=torch.uint8, device=dev) if colwise else None
    sc = torch.empty((cols, rows // 16), dtype=torch.uint8, device=dev) if colwise else None
    amax = torch.empty((1,), dtype=torch.float32, device=dev)
    _check(L.mx_quantize_nvfp4(_ptr(x), rows, cols, _ptr(q), _ptr(s), _ptr(qc), _ptr(sc), _ptr(amax),
                               _stream(stream)))
    return (q, s, amax, qc, sc) if colwise else (q, s, amax)


def mx_grouped_gemm_nvfp4(a_q, a_s, a_amax, b_q, b_s, b_amax, group_sizes, out_dtype=torch.bfloat16, out=None,
                          stream=None):
    """Grouped NVFP4 GEMM (mx_grouped_gemm_nvfp4): rows of group g of A (a_q
    [M, k/2], a_s [M, k/16], a_amax [1]) times B_g^T (b_q [G, n, k/2], b_s
    [G, n, k/16], b_amax [G]); returns C [M, n] (bf16 or fp32)."""
    L = load()
    sizes = [int(v) for v in group_sizes]
    G, n, k = len(sizes), b_q.shape[1], a_q.shape[1] * 2
    m = a_q.shape[0]
    for t in (a_q, a_s, b_q, b_s):
        if t.dtype != torch.uint8 or not t.is_contiguous():
            raise ValueError("mx_grouped_gemm_nvfp4: codes and scales must be contiguous uint8 tensors")
    for t, want in ((a_amax, 1), (b_amax, G)):
        if t.dtype != torch.float32 or t.numel() != want or not t.is_contiguous():
            raise ValueError("mx_grouped_gemm_nvfp4: a_amax must be 1 and b_amax G fp32 values")
    if (sum(sizes) != m or tuple(a_s.shape) != (m, k // 16) or tuple(b_q.shape) != (G, n, k // 2)
            or tuple(b_s.shape) != (G, n, k // 16)):
        raise ValueError("mx_grouped_gemm_nvfp4: operand shapes do not match the group sizes")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=a_q.device)
    if tuple(out.shape) != (m, n) or not out.is_contiguous() or out.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("mx_grouped_gemm_nvfp4: out must be a contiguous bf16 or fp32 [M, n] tensor")
    dt = MX_F32 if out.dtype == torch.float32 else MX_BF16
    arr = (ctypes.c_int64 * max(G, 1))(*sizes)
    _check(L.mx_grouped_gemm_nvfp4(_ptr(a_q), _ptr(a_s), _ptr(a_amax), _ptr(b_q), _ptr(b_s), _ptr(b_amax), arr, G,
                                   n, k, _ptr(out), dt, _stream(stream)))
    return out


def mx_gemm_nvfp4(a_q, a_s, a_amax, b_q, b_s, b_amax, out_dtype=torch.bfloat16, out=None, stream=None):
    """C [m, n] = A . B^T on rowwise NVFP4 operands (mx_gemm_nvfp4): the grouped
    call with one group."""
    if b_q.dim() != 2 or b_s.dim() != 2:
        raise ValueError("mx_gemm_nvfp4: b_q and b_s must be 2-D")
    return mx_grouped_gemm_nvfp4(a_q, a_s, a_amax, b_q.unsqueeze(0), b_s.unsqueeze(0), b_amax.reshape(1),
                                 [a_q.shape[0]], out_dtype=out_dtype, out=out, stream=stream)


def mx_quantize_fp4_colwise_grouped(x, group_sizes, stream=None):
    """Columnwise MXFP4 of bf16 x [rows, cols] with per-group padding to 32
    rows: (q_col [cols, sum P / 2], s_col [cols, sum P / 32])."""
    if not (isinstance(x, torch.Tensor) and x.dtype == torch.bfloat16 and x.dim() == 2 and x.is_contiguous()
            and x.is_cuda):
        raise ValueError("mx_quantize_fp4_colwise_grouped: x must be a contiguous 2-D bfloat16 CUDA tensor")
    sizes = [int(v) for v in group_sizes]
    rows, cols = x.shape
    if not sizes or sum(sizes) != rows or min(sizes) < 0:
        raise ValueError(f"mx_quantize_fp4_colwise_grouped: group sizes {sizes} must be >= 0 and sum to {rows}")
    P = sum(padded_sizes(sizes))
    L = load()
    qc = torch.empty((cols, P // 2), dtype=torch.uint8, device=x.device)
    sc = torch.empty((cols, P // 32), dtype=torch.uint8, device=x.device)
    _check(L.mx_quantize_fp4_colwise_grouped(_ptr(x), rows, cols, _i64_array(sizes), len(sizes), _ptr(qc), _ptr(sc),
                                             _stream(stream)))
    return qc, sc


def mx_grouped_gemm_fp4_wgrad(a_q, a_s, b_q, b_s, group_sizes, out=None, accumulate=False, stream=None):
    """Weight-gradient GEMM at MXFP4: C_g (+)= A[:, K_g] . B[:, K_g]^T per
    group, A (a_q [m, K/2], a_s [m, K/32]) and B [n, K] in the grouped
    columnwise layout, K = sum of the padded group sizes; returns fp32
    C [G, m, n] (out, accumulated into when accumulate)."""
    sizes = [int(v) for v in group_sizes]
    G = len(sizes)
    K = sum(padded_sizes(sizes))
    m, n = a_q.shape[0], b_q.shape[0]
    _expect_all([(a_q, (m, K // 2), torch.uint8, "a_q", False), (a_s, (m, K // 32), torch.uint8, "a_s", False),
                 (b_q, (n, K // 2), torch.uint8, "b_q", False), (b_s, (n, K // 32), torch.uint8, "b_s", False),
                 (out, (G, m, n), torch.float32, "out", True)])
    if accumulate and out is None:
        raise ValueError("mx_grouped_gemm_fp4_wgrad: accumulate needs out")
    if out is None:
        out = torch.empty((G, m, n), dtype=torch.float32, device=a_q.device)
    L = load()
    _check(L.mx_grouped_gemm_fp4_wgrad(_ptr(a_q), _ptr(a_s), _ptr(b_q), _ptr(b_s), _i64_array(sizes), G, m, n,
                                       _ptr(out), int(bool(accumulate)), _stream(stream)))
    return out


def mx_moe_dispatch(x, topk_idx, topk_w, num_experts: int, stream=None, gather: bool = True):
    """Token dispatch (mx_moe_dispatch): x bf16 [T, H], topk_idx int32 [T, k],
    topk_w fp32 [T, k] or None. Returns (x_perm bf16 [T*k, H] or None,
    probs_perm fp32 [T*k] or None, perm int32 [T, k], row_token int32 [T*k],
    counts int64 [E]); the first counts.sum() routed rows are valid.
    gather=False: routing only (no row copy; x_perm is None)."""
    L = load()
    if x.dim() != 2 or topk_idx.dim() != 2:
        raise ValueError("mx_moe_dispatch: x must be [T, H] and topk_idx [T, k]")
    T, H = x.shape
    k = topk_idx.shape[1]
    _expect_all([(x, (T, H), torch.bfloat16, "x", False), (topk_idx, (T, k), torch.int32, "topk_idx", False),
                 (topk_w, (T, k), torch.float32, "topk_w", True)])
    dev = x.device
    x_perm = torch.empty((T * k, H), dtype=x.dtype, device=dev) if gather else None
    probs_perm = torch.empty((T * k,), dtype=torch.float32, device=dev) if topk_w is not None else None
    perm = torch.empty((T, k), dtype=torch.int32, device=dev)
    row_token = torch.empty((T * k,), dtype=torch.int32, device=dev)
    counts = torch.empty((num_experts,), dtype=torch.int64, device=dev)
    ws = _byte_buffer(L.mx_moe_dispatch_workspace_bytes(T, k, num_experts), dev)
    _check(L.mx_moe_dispatch(_ptr(x) if gather else None, _ptr(topk_idx), _ptr(topk_w), T, H, k, num_experts,
                             _ptr(x_perm),
                             _ptr(probs_perm), _ptr(perm), _ptr(row_token), _ptr(counts), _ptr(ws), ws.numel(),
                             _stream(stream)))
    return x_perm, probs_perm, perm, row_token, counts


def mx_moe_combine(y_perm, perm, out=None, stream=None):
    """Token combine (mx_moe_combine): y [T, H] bf16, the fp32 sum of each
    token's routed rows, rounded once to bf16."""
    L = load()
    if perm.dim() != 2 or y_perm.dim() != 2:
        raise ValueError("mx_moe_combine: perm must be [T, k] and y_perm [rows, H]")
    T, k = perm.shape
    H = y_perm.shape[1]
    # y_perm holds the routed rows: at most T * k (the rows perm points at)
    if not 1 <= y_perm.shape[0] <= max(T * k, 1):
        raise ValueError(f"mx_moe_combine: y_perm has {y_perm.shape[0]} rows, expected 1 .. {max(T * k, 1)}")
    _expect_all([(perm, (T, k), torch.int32, "perm", False),
                 (y_perm, (y_perm.shape[0], H), torch.bfloat16, "y_perm", False),
                 (out, (T, H), torch.bfloat16, "out", True)])
    y = torch.empty((T, H), dtype=y_perm.dtype, device=y_perm.device) if out is None else out
    _check(L.mx_moe_combine(_ptr(y_perm), _ptr(perm), T, H, k, _ptr(y), _stream(stream)))
    return y


_event_arrays = []   # keeps the handle arrays alive while the library holds them


def set_stage_events(events):
    """Record torch.cuda.Event objects at the stage boundaries of the next fused
    MLP calls on this thread (events[i] before stage i and after the last);
    None switches stage timing off."""
    L = load()
    if not events:
        _check(L.mx_set_stage_events(None, 0))
        _event_arrays.clear()
        return
    handles = [e.cuda_event for e in events]
    if not all(handles):
        raise ValueError("record each event once before handing it to set_stage_events "
                         "(torch creates the HIP event on first record)")
    arr = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(h) for h in handles])
    _event_arrays.append(arr)
    if len(_event_arrays) > 4:
        del _event_arrays[0]
    _check(L.mx_set_stage_events(arr, len(events)))


class MLPRunner:
    """Preallocated fused-MLP training step (no allocation per call): owns the
    workspaces, the saved buffer and the outputs for one shape and split."""

    def __init__(self, E: int, R: int, H: int, F: int, split_sizes, device="cuda"):
        self.dims = (int(E), int(R), int(H), int(F))
        self.split = [int(s) for s in split_sizes]
        fws, sv, bws = mlp_sizes(E, R, H, F, self.split)
        self.fwd_ws = _byte_buffer(fws, device)
        self.saved = _byte_buffer(sv, device)
        self.bwd_ws = _byte_buffer(bws, device)
        self.y = torch.empty((R, H), dtype=torch.bfloat16, device=device)
        self.dx = torch.empty((R, H), dtype=torch.bfloat16, device=device)
        self.dprobs = torch.empty((R,), dtype=torch.float32, device=device)
        self._c_dims = _dims(E, R, H, F)
        self._c_split = _i64_array(self.split)

    def _inputs(self, x, probs, w1=None, w2=None):
        E, R, H, F = self.dims
        _mlp_inputs(E, R, H, F, self.split, x, w1, w2, probs)

    def _grads(self, dy, probs, dw1, dw2):
        E, R, H, F = self.dims
        _expect_all([(dy, (R, H), torch.bfloat16, "dy", False), (probs, (R,), torch.float32, "probs", True),
                     (dw1, (E, 2 * F, H), torch.float32, "dw1", False), (dw2, (E, H, F), torch.float32, "dw2", False)])

    def forward(self, x, probs, w1, w2, training=True, stream=None):
        L = load()
        self._inputs(x, probs, w1, w2)
        saved = self.saved if training else None
        _check(L.grouped_mlp_fwd(ctypes.byref(self._c_dims), self._c_split, _ptr(x), _ptr(probs),
                                 _ptr(w1), _ptr(w2), _ptr(self.y), _ptr(saved),
                                 0 if saved is None else saved.numel(), _ptr(self.fwd_ws),
                                 self.fwd_ws.numel(), _stream(stream)))
        return self.y

    def quantize_weights(self, w1, w2, stream=None):
        """Fill this runner's weight cache (allocated on first use) from w1, w2."""
        E, _, H, F = self.dims
        if getattr(self, "cache", None) is None:
            self.cache = WeightCache(E, H, F, device=self.y.device)
        grouped_mlp_quantize_weights(w1, w2, self.cache, stream=stream)
        return self.cache

    def forward_cached(self, x, probs, training=True, stream=None):
        L = load()
        self._inputs(x, probs)
        saved = self.saved if training else None
        _check(L.grouped_mlp_fwd_cached(ctypes.byref(self._c_dims), self._c_split, _ptr(x), _ptr(probs),
                                        _ptr(self.cache.buf), self.cache.buf.numel(), _ptr(self.y),
                                        _ptr(saved), 0 if saved is None else saved.numel(),
                                        _ptr(self.fwd_ws), self.fwd_ws.numel(), _stream(stream)))
        return self.y

    def backward_cached(self, dy, probs, dw1, dw2, accumulate=True, want_dprobs=True, stream=None):
        L = load()
        self._grads(dy, probs, dw1, dw2)
        _check(L.grouped_mlp_bwd_cached(ctypes.byref(self._c_dims), self._c_split, _ptr(dy), _ptr(probs),
                                        _ptr(self.cache.buf), self.cache.buf.numel(), _ptr(self.saved),
                                        self.saved.numel(), _ptr(self.dx),
                                        _ptr(self.dprobs) if want_dprobs else None, _ptr(dw1), _ptr(dw2),
                                        int(accumulate), _ptr(self.bwd_ws), self.bwd_ws.numel(),
                                        _stream(stream)))
        return self.dx, (self.dprobs if want_dprobs else None)

    def backward(self, dy, probs, dw1, dw2, accumulate=True, want_dprobs=True, stream=None):
        L = load()
        self._grads(dy, probs, dw1, dw2)
        _check(L.grouped_mlp_bwd(ctypes.byref(self._c_dims), self._c_split, _ptr(dy), _ptr(probs),
                                 _ptr(self.saved), self.saved.numel(), _ptr(self.dx),
                                 _ptr(self.dprobs) if want_dprobs else None, _ptr(dw1), _ptr(dw2),
                                 int(accumulate), _ptr(self.bwd_ws), self.bwd_ws.numel(),
                                 _stream(stream)))
        return self.dx, (self.dprobs if want_dprobs else None)


def mlp_sizes_device_split(E: int, R: int, H: int, F: int):
    """(fwd workspace, saved, bwd workspace) byte sizes of the device-split
    calls: valid for every split of R routed rows over E experts."""
    L = load()
    f, s, b = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(L.grouped_mlp_sizes_device_split(ctypes.byref(_dims(E, R, H, F)), ctypes.byref(f), ctypes.byref(s),
                                            ctypes.byref(b)))
    return f.value, s.value, b.value


class DeviceSplitMLPRunner:
    """Fused-MLP training step whose per-expert row counts stay on the device
    (e.g. mx_moe_dispatch's counts): no host round trip, no wait. Owns the
    workspaces (sized for every split of R rows), the saved buffer and the
    outputs. Rows past the sum of the (clamped) counts are not read; y and dx
    are not written there and dprobs is 0 there."""

    def __init__(self, E: int, R: int, H: int, F: int, device="cuda"):
        self.dims = (int(E), int(R), int(H), int(F))
        fws, sv, bws = mlp_sizes_device_split(E, R, H, F)
        self.fwd_ws = _byte_buffer(fws, device)
        self.saved = _byte_buffer(sv, device)
        self.bwd_ws = _byte_buffer(bws, device)
        self.y = torch.empty((R, H), dtype=torch.bfloat16, device=device)
        self.dx = torch.empty((R, H), dtype=torch.bfloat16, device=device)
        self.dprobs = torch.empty((R,), dtype=torch.float32, device=device)
        self._c_dims = _dims(E, R, H, F)

    def _rows(self, x, row_token, name):
        """Rows x must have: R without a gather, else its own (tokens)."""
        E, R, H, F = self.dims
        if row_token is None:
            return R, []
        if not isinstance(x, torch.Tensor) or x.dim() != 2:
            raise ValueError(f"{name} must be a 2-D tensor")
        return int(x.shape[0]), [(row_token, (R,), torch.int32, "row_token", False)]

    def _cache(self, cache):
        E, _, H, F = self.dims
        if cache is None:
            return None, 0
        if not isinstance(cache, WeightCache) or cache.ehf != (E, H, F):
            raise ValueError("cache must be a WeightCache of this runner's E, H, F")
        return _ptr(cache.buf), cache.buf.numel()

    def forward(self, counts, x, probs, w1=None, w2=None, *, cache=None, row_token=None, training=True,
                stream=None):
        L = load()
        E, R, H, F = self.dims
        rows, extra = self._rows(x, row_token, "x")
        items = [(counts, (E,), torch.int64, "counts", False)] + extra
        items += _mlp_items(E, R, H, F, x, None if cache is not None else w1,
                            None if cache is not None else w2, probs, x_rows=rows)
        if cache is None and (w1 is None or w2 is None):
            raise ValueError("w1 and w2 (or a weight cache) are required")
        _expect_all(items)
        cp, cb = self._cache(cache)
        saved = self.saved if training else None
        _check(L.grouped_mlp_fwd_device_split(
            ctypes.byref(self._c_dims), _ptr(counts), _ptr(x), rows if row_token is not None else 0,
            _ptr(row_token), _ptr(probs), None if cache is not None else _ptr(w1),
            None if cache is not None else _ptr(w2), cp, cb, _ptr(self.y), _ptr(saved),
            0 if saved is None else saved.numel(), _ptr(self.fwd_ws), self.fwd_ws.numel(), _stream(stream)))
        return self.y

    def backward(self, counts, dy, probs, dw1, dw2, *, accumulate=True, want_dprobs=True, cache=None,
                 row_token=None, stream=None):
        L = load()
        E, R, H, F = self.dims
        rows, extra = self._rows(dy, row_token, "dy")
        _expect_all([(counts, (E,), torch.int64, "counts", False), (dy, (rows, H), torch.bfloat16, "dy", False),
                     (probs, (R,), torch.float32, "probs", True),
                     (dw1, (E, 2 * F, H), torch.float32, "dw1", False),
                     (dw2, (E, H, F), torch.float32, "dw2", False)] + extra)
        cp, cb = self._cache(cache)
        _check(L.grouped_mlp_bwd_device_split(
            ctypes.byref(self._c_dims), _ptr(counts), _ptr(dy), rows if row_token is not None else 0,
            _ptr(row_token), _ptr(probs), cp, cb, _ptr(self.saved), self.saved.numel(), _ptr(self.dx),
            _ptr(self.dprobs) if want_dprobs else None, _ptr(dw1), _ptr(dw2), int(accumulate),
            _ptr(self.bwd_ws), self.bwd_ws.numel(), _stream(stream)))
        return self.dx, (self.dprobs if want_dprobs else None)


class GroupedMLP(torch.autograd.Function):
    """y = GroupedMLP.apply(x, probs, w1, w2, split_sizes): the fused MXFP8
    grouped MLP with a fused backward (gradients for x, probs, w1, w2)."""

    @staticmethod
    def forward(ctx, x, probs, w1, w2, split_sizes):
        y, state = grouped_mlp_fwd(x.contiguous(), probs, w1.contiguous(), w2.contiguous(),
                                   list(split_sizes), training=True)
        ctx.state = state
        ctx.save_for_backward(probs)
        return y

    @staticmethod
    def backward(ctx, dy):
        (probs,) = ctx.saved_tensors
        dx, dprobs, dw1, dw2 = grouped_mlp_bwd(dy.contiguous(), probs, ctx.state,
                                               want_dprobs=probs is not None)
        return dx, dprobs, dw1, dw2, None
