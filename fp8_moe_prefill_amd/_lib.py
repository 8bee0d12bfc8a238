"""ctypes binding of ``libfp8moe.so`` (argument marshalling only).

Every function here takes torch tensors that live on a HIP device, checks their dtypes,
shapes and contiguity, allocates outputs with torch when the caller passes none, and calls
the C ABI on torch's current stream. All computation happens in the library's HIP kernels;
there is no CPU path. If the library is missing this module raises at import.
"""

from __future__ import annotations

import ctypes
import functools
import inspect
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp8moe.so")

GROUP = 128
QUANT_ROW = -1  # fp8_quant_act group: one scale per row
DTYPE_F32, DTYPE_BF16 = 0, 1
EPI_STORE, EPI_SWIGLU_QUANT = 0, 1
OP_QUANT_ACT, OP_ROUTE_PERMUTE, OP_ATTENTION = 0, 1, 2

_c_void_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t

SIGNATURES = {
    "fp8moe_abi_version": (_i32, []),
    "fp8moe_status_str": (ctypes.c_char_p, [_i32]),
    "fp8moe_workspace_bytes": (_sz, [_i32, _i64, _i64, _i64]),
    "fp8_quant_act": (_i32, [_c_void_p, _i64, _i64, _i32, _c_void_p, _c_void_p, _c_void_p,
                             _c_void_p, _sz, _c_void_p]),
    "moe_route_permute": (_i32, [_c_void_p, _i64, _i32, _i32, _c_void_p, _c_void_p, _c_void_p,
                                 _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _c_void_p,
                                 _c_void_p, _c_void_p, _c_void_p, _c_void_p, _sz, _c_void_p]),
    "moe_route_permute_noalloc": (_i32, [_c_void_p, _i64, _i32, _i32, _c_void_p, _c_void_p,
                                         _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                         _i64, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                         _c_void_p]),
    "fp8moe_quant_route": (_i32, [_c_void_p, _i64, _i64, _c_void_p, _c_void_p, _c_void_p,
                                  _c_void_p, _i32, _i32, _c_void_p, _c_void_p, _c_void_p,
                                  _c_void_p, _c_void_p, _c_void_p, _sz, _c_void_p]),
    "fp8moe_pack_expert_bank": (_i32, [_c_void_p, _c_void_p, _i64, _i64, _i64, _c_void_p,
                                       _c_void_p, _c_void_p]),
    "fp8_grouped_expert_gemm": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32,
                                       _c_void_p, _c_void_p, _c_void_p, _i64, _i32, _i64, _i64,
                                       _i32, _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "fp8_dense_gemm": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64, _i32,
                              _c_void_p, _c_void_p]),
    "fp8_dense_gemm_rowwise": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64,
                                      _i32, _c_void_p, _c_void_p]),
    "fp8_block_gemm": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64, _i32,
                              _c_void_p, _c_void_p]),
    "fp8_quant_weight_block128": (_i32, [_c_void_p, _i64, _i64, _c_void_p, _c_void_p,
                                         _c_void_p]),
    "mxfp4_quant_act": (_i32, [_c_void_p, _i64, _i64, _c_void_p, _c_void_p, _c_void_p]),
    "fp8moe_pack_expert_bank_mxfp4": (_i32, [_c_void_p, _c_void_p, _i64, _i64, _i64, _c_void_p,
                                             _c_void_p, _c_void_p]),
    "mxfp4_grouped_expert_gemm": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i32, _c_void_p,
                                         _c_void_p, _c_void_p, _i64, _i32, _i64, _i64, _i32,
                                         _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "moe_unpermute_combine": (_i32, [_c_void_p, _i32, _c_void_p, _c_void_p, _i64, _i32, _i64,
                                     _i32, _c_void_p, _c_void_p]),
    "fp8moe_rmsnorm": (_i32, [_c_void_p, _c_void_p, _i64, _i64, ctypes.c_double, _c_void_p,
                              _c_void_p, _c_void_p]),
    "fp8moe_bf16_gemm": (_i32, [_c_void_p, _c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p]),
    "fp8moe_causal_attention": (_i32, [_c_void_p, _i64, _i32, _i32, _i32, _c_void_p, _c_void_p,
                                       _sz, _c_void_p]),
}


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python fp8_moe_prefill_amd/build.py`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = load_library()


class Fp8MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: status {status} "
                         f"({_lib.fp8moe_status_str(status).decode()})")


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise Fp8MoeError(fn, status)


def _on_stream(fn):
    """Run a wrapper with ``stream`` as torch's current stream, so that the outputs and
    workspaces it allocates belong to that stream in the caching allocator: a temporary
    freed when the wrapper returns is then reused only by work ordered after the kernels
    that still read it (torch's rule for memory used on one stream)."""
    pos = list(inspect.signature(fn).parameters).index("stream")

    @functools.wraps(fn)
    def wrapped(*args, **kw):
        stream = args[pos] if len(args) > pos else kw.get("stream")
        if stream is None:
            return fn(*args, **kw)
        with torch.cuda.stream(stream):
            return fn(*args, **kw)

    return wrapped


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _dt(dtype) -> int:
    return {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}[dtype]


def workspace_bytes(op: int, a: int, b: int, c: int) -> int:
    n = _lib.fp8moe_workspace_bytes(op, a, b, c)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid workspace query")
    return n


def _workspace(nbytes: int, device, ws=None):
    if nbytes == 0:
        return None
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def abi_version() -> int:
    return _lib.fp8moe_abi_version()


# ------------------------------------------------------------------------------------
# The entry points
# ------------------------------------------------------------------------------------


@_on_stream
def fp8_quant_act(x: torch.Tensor, group: int = GROUP, q=None, scales=None, ws=None,
                  stream=None, sums=None, with_sums: bool = False):
    """bf16 [M, K] -> (e4m3 codes uint8 [M, K], fp32 scales: [M, K/128] for group=128,
    block[4] for group=0, [M] for group=QUANT_ROW). With ``with_sums`` (group=128) also the
    code sums fp32 [M, K/128]: (q, scales, sums)."""
    _dev(x, "x", torch.bfloat16)
    M, K = x.shape
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if scales is None:
        shape = (M, K // GROUP) if group == GROUP else (M,) if group == QUANT_ROW else (4,)
        scales = torch.empty(shape, dtype=torch.float32, device=x.device)
    if with_sums and sums is None:
        sums = torch.empty((M, K // GROUP), dtype=torch.float32, device=x.device)
    nbytes = workspace_bytes(OP_QUANT_ACT, M, K, group)
    wsb = _workspace(nbytes, x.device, ws)
    _check("fp8_quant_act", _lib.fp8_quant_act(_ptr(x), M, K, group, _ptr(q), _ptr(scales),
                                               _ptr(sums), _ptr(wsb), nbytes, _stream(stream)))
    return (q, scales, sums) if sums is not None else (q, scales)


def _route_buffers(logits, k, xq, xs, xsum, out):
    _dev(logits, "logits", torch.float32)
    T, E = logits.shape
    dev = logits.device
    o = out if out is not None else {}

    def buf(name, shape, dtype):
        return o[name] if name in o else torch.empty(shape, dtype=dtype, device=dev)

    r = dict(ids=buf("ids", (T, k), torch.int32), weights=buf("weights", (T, k), torch.float32),
             offsets=buf("offsets", (E + 1,), torch.int32),
             sorted=buf("sorted", (T * k,), torch.int32), pos=buf("pos", (T * k,), torch.int32))
    H = 0
    if xq is not None:
        _dev(xq, "xq", torch.uint8)
        H = xq.shape[1]
        r["xq_perm"] = buf("xq_perm", (T * k, H), torch.uint8)
    if xs is not None:
        _dev(xs, "xs", torch.float32)
        H = xs.shape[1] * GROUP
        r["xs_perm"] = buf("xs_perm", (H // GROUP, T * k), torch.float32)
    if xsum is not None:
        _dev(xsum, "xsum", torch.float32)
        r["xsum_perm"] = buf("xsum_perm", (H // GROUP, T * k), torch.float32)
    head = (_ptr(logits), T, E, k, _ptr(r["ids"]), _ptr(r["weights"]), _ptr(r["offsets"]),
            _ptr(r["sorted"]), _ptr(r["pos"]), _ptr(xq), _ptr(xs), H, _ptr(r.get("xq_perm")),
            _ptr(r.get("xs_perm")), _ptr(xsum), _ptr(r.get("xsum_perm")))
    return r, head


@_on_stream
def moe_route_permute(logits: torch.Tensor, k: int, xq=None, xs=None, out=None, ws=None,
                      stream=None, xsum=None) -> dict:
    """fp32 logits [T, E] -> dict(ids, weights, offsets, sorted, pos[, xq_perm][, xs_perm]
    [, xsum_perm]).

    ``xq`` (e4m3 [T, H]) is gathered into xq_perm [T*k, H]; ``xs`` (fp32 [T, H/128]) into
    xs_perm [H/128, T*k], group-major; ``xsum`` (the code sums, fp32 [T, H/128], only with
    ``xs``) into xsum_perm of the same layout as xs_perm. xq and xs may be given alone."""
    r, head = _route_buffers(logits, k, xq, xs, xsum, out)
    T, E = logits.shape
    nbytes = workspace_bytes(OP_ROUTE_PERMUTE, T, E, k)
    wsb = _workspace(nbytes, logits.device, ws)
    _check("moe_route_permute", _lib.moe_route_permute(*head, _ptr(wsb), nbytes,
                                                       _stream(stream)))
    return r


@_on_stream
def moe_route_permute_noalloc(logits: torch.Tensor, k: int, xq=None, xs=None, out=None,
                              stream=None, xsum=None) -> dict:
    """moe_route_permute with the library's static per-GPU workspace instead of a caller
    one: the C call allocates nothing (outputs missing from ``out`` are still allocated
    here, by torch). Calls that overlap in time on one GPU race on that workspace."""
    r, head = _route_buffers(logits, k, xq, xs, xsum, out)
    _check("moe_route_permute_noalloc", _lib.moe_route_permute_noalloc(*head, _stream(stream)))
    return r


@_on_stream
def quant_route(x: torch.Tensor, logits: torch.Tensor, k: int, q=None, scales=None, sums=None,
                out=None, ws=None, stream=None, with_sums: bool = True):
    """fp8_quant_act(x, GROUP) and moe_route_permute(logits, k) (no gathers) in one call:
    returns (q, scales, sums or None, route dict), the same bytes as the two calls."""
    _dev(x, "x", torch.bfloat16)
    T, H = x.shape
    if logits.shape[0] != T:
        raise ValueError("x and logits must have the same number of rows")
    if q is None:
        q = torch.empty((T, H), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((T, H // GROUP), dtype=torch.float32, device=x.device)
    if with_sums and sums is None:
        sums = torch.empty((T, H // GROUP), dtype=torch.float32, device=x.device)
    r, head = _route_buffers(logits, k, None, None, None, out)
    E = logits.shape[1]
    nbytes = workspace_bytes(OP_ROUTE_PERMUTE, T, E, k)
    wsb = _workspace(nbytes, x.device, ws)
    _check("fp8moe_quant_route", _lib.fp8moe_quant_route(
        _ptr(x), T, H, _ptr(q), _ptr(scales), _ptr(sums), _ptr(logits), E, k,
        _ptr(r["ids"]), _ptr(r["weights"]), _ptr(r["offsets"]), _ptr(r["sorted"]),
        _ptr(r["pos"]), _ptr(wsb), nbytes, _stream(stream)))
    return q, scales, sums, r


@_on_stream
def pack_expert_bank(w: torch.Tensor, w_scales: torch.Tensor, out=None, stream=None,
                     mxfp4: bool = False):
    """Canonical bank (packed int4 [E, N, K/2], low nibble = even k; fp32 scales
    [E, N, K/128]) -> the grouped GEMM's layout: (bank bytes, kept as a [E, N, K/2] uint8
    tensor, and scales [E, K/128, N]). ``mxfp4``: the K order of the MXFP4-activation
    GEMM (``mxfp4_grouped_expert_gemm``)."""
    _dev(w, "w", torch.uint8)
    _dev(w_scales, "w_scales", torch.float32)
    E, N, Kh = w.shape
    K = Kh * 2
    if out is None:
        out = (torch.empty_like(w),
               torch.empty((E, K // GROUP, N), dtype=torch.float32, device=w.device))
    wp, sp = out
    name = "fp8moe_pack_expert_bank_mxfp4" if mxfp4 else "fp8moe_pack_expert_bank"
    _check(name, getattr(_lib, name)(_ptr(w), _ptr(w_scales), E, N, K, _ptr(wp), _ptr(sp),
                                     _stream(stream)))
    return wp, sp


@_on_stream
def fp8_grouped_expert_gemm(a, a_scales, w, w_scales, offsets, R: int, epilogue=EPI_STORE,
                            out_dtype=torch.float32, sorted_=None, k_route: int = 1, out=None,
                            out_scales=None, stream=None, a_sums=None, out_sums=None,
                            with_sums: bool = False):
    """Grouped expert GEMM on a bank from ``pack_expert_bank`` (w [E, N, K/2] bytes,
    w_scales [E, K/128, N]). Without ``sorted_`` the rows are in grouped order and a_scales
    (and a_sums) are group-major [K/128, R]; with it the rows are gathered from token order
    (a = [T, K] with T = R / k_route) and a_scales (and a_sums) are the per-token
    [T, K/128] arrays the quantiser writes. STORE -> out [R, N];
    SWIGLU_QUANT -> (codes [R, N/2], scales [N/256, R], group-major), plus the code sums
    [N/256, R] of the quantised output when ``out_sums`` or ``with_sums`` is given.
    ``a_sums`` (optional, group-major [K/128, R]) are the per-(row, K group) sums of the
    decoded activation codes; without them the kernel forms them itself."""
    return _grouped(a, a_scales, w, w_scales, offsets, R, epilogue, out_dtype, sorted_, k_route,
                    out, out_scales, stream, False, a_sums, out_sums, with_sums)


@_on_stream
def mxfp4_grouped_expert_gemm(a, a_scales, w, w_scales, offsets, R: int, epilogue=EPI_STORE,
                              out_dtype=torch.float32, sorted_=None, k_route: int = 1,
                              out=None, out_scales=None, stream=None, out_sums=None,
                              with_sums: bool = False):
    """The grouped expert GEMM with MXFP4 activations: a = codes [rows, K/2] from
    ``mxfp4_quant_act``, a_scales = 32-bit words of four E8M0 bytes each: the quantiser's
    scales viewed as [rows, K/128] words when gathering through ``sorted_``, else
    group-major [K/128, R]; the bank from ``pack_expert_bank(..., mxfp4=True)``."""
    return _grouped(a, a_scales, w, w_scales, offsets, R, epilogue, out_dtype, sorted_, k_route,
                    out, out_scales, stream, True, None, out_sums, with_sums)


def _grouped(a, a_scales, w, w_scales, offsets, R, epilogue, out_dtype, sorted_, k_route, out,
             out_scales, stream, a_fp4, a_sums, out_sums, with_sums):
    _dev(a, "a", torch.uint8)
    _dev(a_scales, "a_scales")
    if a_scales.element_size() != 4:
        raise ValueError("a_scales must hold 32-bit elements")
    _dev(w, "w", torch.uint8)
    _dev(w_scales, "w_scales", torch.float32)
    _dev(offsets, "offsets", torch.int32)
    E, N, Kh = w.shape
    K = Kh * 2
    if a.shape[1] != (K // 2 if a_fp4 else K):
        raise ValueError(f"a has {a.shape[1]} bytes per row, expected {K // 2 if a_fp4 else K}")
    # rows gathered through `sorted`: per-token scales (and sums) [T, K/128], as the
    # quantiser writes them; otherwise group-major [K/128, R] in grouped row order
    s_shape = (R // k_route, K // GROUP) if sorted_ is not None else (K // GROUP, R)
    if tuple(a_scales.shape) != s_shape:
        raise ValueError(f"a_scales must be {s_shape}, got {tuple(a_scales.shape)}")
    if tuple(w_scales.shape) != (E, K // GROUP, N):
        raise ValueError(f"w_scales must be [E, K/128, N] = {(E, K // GROUP, N)}, "
                         f"got {tuple(w_scales.shape)}")
    dev = a.device
    if sorted_ is not None:
        _dev(sorted_, "sorted", torch.int32)
    if epilogue == EPI_SWIGLU_QUANT:
        I = N // 2
        if out is None:
            out = torch.empty((R, I), dtype=torch.uint8, device=dev)
        if out_scales is None:
            out_scales = torch.empty((I // GROUP, R), dtype=torch.float32, device=dev)
        if with_sums and out_sums is None:
            out_sums = torch.empty((I // GROUP, R), dtype=torch.float32, device=dev)
        dt = DTYPE_F32
    else:
        if out_sums is not None or with_sums:
            raise ValueError("output code sums come only with the SwiGLU epilogue")
        if out is None:
            out = torch.empty((R, N), dtype=out_dtype, device=dev)
        dt = _dt(out.dtype)
    if a_sums is not None:
        _dev(a_sums, "a_sums", torch.float32)
        if tuple(a_sums.shape) != s_shape:
            raise ValueError(f"a_sums must be {s_shape}, got {tuple(a_sums.shape)}")
    if a_fp4:
        _check("mxfp4_grouped_expert_gemm", _lib.mxfp4_grouped_expert_gemm(
            _ptr(a), _ptr(a_scales), _ptr(sorted_), k_route, _ptr(w), _ptr(w_scales),
            _ptr(offsets), R, E, N, K, epilogue, dt, _ptr(out), _ptr(out_scales),
            _ptr(out_sums), _stream(stream)))
    else:
        _check("fp8_grouped_expert_gemm", _lib.fp8_grouped_expert_gemm(
            _ptr(a), _ptr(a_scales), _ptr(a_sums), _ptr(sorted_), k_route, _ptr(w),
            _ptr(w_scales), _ptr(offsets), R, E, N, K, epilogue, dt, _ptr(out),
            _ptr(out_scales), _ptr(out_sums), _stream(stream)))
    if epilogue != EPI_SWIGLU_QUANT:
        return out
    return (out, out_scales, out_sums) if out_sums is not None else (out, out_scales)


@_on_stream
def mxfp4_quant_act(x: torch.Tensor, q=None, scales=None, stream=None):
    """bf16 [M, K] -> (MXFP4 codes uint8 [M, K/2], E8M0 scale bytes uint8 [M, K/32])."""
    _dev(x, "x", torch.bfloat16)
    M, K = x.shape
    if q is None:
        q = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((M, K // 32), dtype=torch.uint8, device=x.device)
    _check("mxfp4_quant_act", _lib.mxfp4_quant_act(_ptr(x), M, K, _ptr(q), _ptr(scales),
                                                   _stream(stream)))
    return q, scales


@_on_stream
def fp8_dense_gemm(a, a_scale_blk, w, w_scale, out_dtype=torch.bfloat16, out=None, stream=None):
    """e4m3 [M, K] x e4m3 [N, K]^T with scales s_a = a_scale_blk[2], s_w = w_scale[0]."""
    _dev(a, "a", torch.uint8)
    _dev(w, "w", torch.uint8)
    _dev(a_scale_blk, "a_scale_blk", torch.float32)
    _dev(w_scale, "w_scale", torch.float32)
    M, K = a.shape
    N = w.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    _check("fp8_dense_gemm", _lib.fp8_dense_gemm(_ptr(a), _ptr(a_scale_blk), _ptr(w),
                                                 _ptr(w_scale), M, N, K, _dt(out.dtype),
                                                 _ptr(out), _stream(stream)))
    return out


@_on_stream
def fp8_dense_gemm_rowwise(a, a_scales, w, w_scale, out_dtype=torch.bfloat16, out=None,
                           stream=None):
    """e4m3 [M, K] x e4m3 [N, K]^T with one activation scale per row (a_scales fp32 [M])
    and s_w = w_scale[0]."""
    _dev(a, "a", torch.uint8)
    _dev(w, "w", torch.uint8)
    _dev(a_scales, "a_scales", torch.float32)
    _dev(w_scale, "w_scale", torch.float32)
    M, K = a.shape
    N = w.shape[0]
    if a_scales.numel() != M:
        raise ValueError(f"a_scales has {a_scales.numel()} elements, expected {M}")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    _check("fp8_dense_gemm_rowwise",
           _lib.fp8_dense_gemm_rowwise(_ptr(a), _ptr(a_scales), _ptr(w), _ptr(w_scale), M, N, K,
                                       _dt(out.dtype), _ptr(out), _stream(stream)))
    return out


@_on_stream
def fp8_quant_weight_block128(w, q=None, scales=None, stream=None):
    """bf16 weight [N, K] -> (e4m3 codes [N, K], fp32 block scales [ceil(N/128), K/128])."""
    _dev(w, "w", torch.bfloat16)
    N, K = w.shape
    if q is None:
        q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty(((N + 127) // 128, K // GROUP), dtype=torch.float32, device=w.device)
    _check("fp8_quant_weight_block128",
           _lib.fp8_quant_weight_block128(_ptr(w), N, K, _ptr(q), _ptr(scales), _stream(stream)))
    return q, scales


@_on_stream
def fp8_block_gemm(a, a_scales, w, w_scales, out_dtype=torch.bfloat16, out=None, stream=None):
    """e4m3 [M, K] (scales fp32 [M, K/128]) x block-128 e4m3 [N, K] (scales fp32
    [ceil(N/128), K/128])."""
    _dev(a, "a", torch.uint8)
    _dev(w, "w", torch.uint8)
    _dev(a_scales, "a_scales", torch.float32)
    _dev(w_scales, "w_scales", torch.float32)
    M, K = a.shape
    N = w.shape[0]
    if a_scales.shape != (M, K // GROUP):
        raise ValueError(f"a_scales has shape {tuple(a_scales.shape)}, expected {(M, K // GROUP)}")
    if w_scales.shape != ((N + 127) // 128, K // GROUP):
        raise ValueError(f"w_scales has shape {tuple(w_scales.shape)}, expected "
                         f"{((N + 127) // 128, K // GROUP)}")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    _check("fp8_block_gemm", _lib.fp8_block_gemm(_ptr(a), _ptr(a_scales), _ptr(w), _ptr(w_scales),
                                                 M, N, K, _dt(out.dtype), _ptr(out),
                                                 _stream(stream)))
    return out


@_on_stream
def moe_unpermute_combine(y, pos, weights, out_dtype=torch.bfloat16, out=None, stream=None):
    """out[t] = sum_j weights[t, j] * y[pos[t*k + j]]."""
    _dev(y, "y")
    _dev(pos, "pos", torch.int32)
    _dev(weights, "weights", torch.float32)
    T, k = weights.shape
    H = y.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=y.device)
    _check("moe_unpermute_combine", _lib.moe_unpermute_combine(
        _ptr(y), _dt(y.dtype), _ptr(pos), _ptr(weights), T, k, H, _dt(out.dtype), _ptr(out),
        _stream(stream)))
    return out


# ------------------------------------------------------------------------------------
# Depth-stack support: residual + RMSNorm, bf16 GEMM, causal GQA attention
# ------------------------------------------------------------------------------------

RMSNORM_EPS = 1e-6


@_on_stream
def rmsnorm(x: torch.Tensor, delta=None, eps: float = RMSNORM_EPS, x_out=None, y=None,
            stream=None):
    """y = bf16(RMSNorm(x)) or, with ``delta``, x_out = bf16(x + delta) and
    y = bf16(RMSNorm(x_out)). ``x_out`` may be ``x`` (in-place). Returns y, or
    (x_out, y) when ``delta`` is given."""
    _dev(x, "x", torch.bfloat16)
    T, H = x.shape
    if delta is not None:
        _dev(delta, "delta", torch.bfloat16)
        if delta.shape != x.shape:
            raise ValueError("delta must have the shape of x")
        if x_out is None:
            x_out = torch.empty_like(x)
        _dev(x_out, "x_out", torch.bfloat16)
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y", torch.bfloat16)
    _check("fp8moe_rmsnorm", _lib.fp8moe_rmsnorm(_ptr(x), _ptr(delta), T, H, float(eps),
                                                 _ptr(x_out), _ptr(y), _stream(stream)))
    return (x_out, y) if delta is not None else y


@_on_stream
def bf16_gemm(a: torch.Tensor, w: torch.Tensor, out=None, stream=None):
    """fp32 [M, N] = a [M, K] . w [N, K]^T, bf16 operands."""
    _dev(a, "a", torch.bfloat16)
    _dev(w, "w", torch.bfloat16)
    M, K = a.shape
    N, K2 = w.shape
    if K2 != K:
        raise ValueError("a and w must share K")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a.device)
    _dev(out, "out", torch.float32)
    _check("fp8moe_bf16_gemm", _lib.fp8moe_bf16_gemm(_ptr(a), _ptr(w), M, N, K, _ptr(out),
                                                     _stream(stream)))
    return out


@_on_stream
def causal_attention(qkv: torch.Tensor, n_q: int, n_kv: int, head_dim: int = 128, out=None,
                     ws=None, stream=None):
    """bf16 [T, (n_q + 2 n_kv) * d] fused q|k|v -> bf16 [T, n_q * d]."""
    _dev(qkv, "qkv", torch.bfloat16)
    T, W = qkv.shape
    if W != (n_q + 2 * n_kv) * head_dim:
        raise ValueError("qkv width must be (n_q + 2 n_kv) * head_dim")
    if out is None:
        out = torch.empty((T, n_q * head_dim), dtype=torch.bfloat16, device=qkv.device)
    _dev(out, "out", torch.bfloat16)
    nbytes = workspace_bytes(OP_ATTENTION, T, n_kv, head_dim)
    wsb = _workspace(nbytes, qkv.device, ws)
    _check("fp8moe_causal_attention",
           _lib.fp8moe_causal_attention(_ptr(qkv), T, n_q, n_kv, head_dim, _ptr(out), _ptr(wsb),
                                        nbytes, _stream(stream)))
    return out

