"""The C-ABI library on the CPU: it loads, exports every function ``include/fp8moe.h``
declares, and rejects bad arguments on the host before touching the GPU.

No call here reaches a kernel launch: each one fails a host-side check first (the
pointers passed are never dereferenced).
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8moe.h")
LIB = os.path.join(ROOT, "fp8_moe_prefill_amd", "libfp8moe.so")

OK, NULL, SHAPE, ALIGN, WS, UNSUP = 0, -1, -2, -3, -4, -5


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int32_t|size_t|const char\*)\s+(\w+)\s*\(", text,
                                 flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} not built (python fp8_moe_prefill_amd/build.py)")
    from fp8_moe_prefill_amd._lib import load_library
    return load_library(LIB)


def test_header_declares_the_five_entry_points():
    fns = declared_functions()
    for name in ["fp8_quant_act", "moe_route_permute", "fp8_grouped_expert_gemm",
                 "fp8_dense_gemm", "moe_unpermute_combine"]:
        assert name in fns
    assert "fp8moe_workspace_bytes" in fns and "fp8moe_status_str" in fns
    for name in ["fp8moe_rmsnorm", "fp8moe_bf16_gemm", "fp8moe_causal_attention",
                 "fp8_dense_gemm_rowwise", "fp8_block_gemm", "fp8_quant_weight_block128",
                 "mxfp4_quant_act", "fp8moe_pack_expert_bank_mxfp4", "mxfp4_grouped_expert_gemm",
                 "moe_route_permute_noalloc", "fp8moe_quant_route"]:
        assert name in fns


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(LIB)
    for name in declared_functions():
        assert hasattr(raw, name), name
    assert lib.fp8moe_abi_version() == 9


def test_status_strings(lib):
    for s in range(-6, 1):
        assert lib.fp8moe_status_str(s)
    assert lib.fp8moe_status_str(-99) == b"unknown status"


def test_workspace_queries(lib):
    assert lib.fp8moe_workspace_bytes(0, 64, 256, 128) == 0
    assert lib.fp8moe_workspace_bytes(0, 2048, 4096, 0) == 4096
    assert lib.fp8moe_workspace_bytes(0, 8, 8, 0) == 0  # fused single-workgroup path
    assert lib.fp8moe_workspace_bytes(0, 2048, 4096, -1) == 0  # row mode needs none
    n = lib.fp8moe_workspace_bytes(1, 4096, 64, 8)
    assert n >= (4096 // 16) * 64 * 4 and n % 256 == 0
    bad = ctypes.c_size_t(-1).value
    assert lib.fp8moe_workspace_bytes(1, 16, 2000, 8) == bad  # E > 1024
    assert lib.fp8moe_workspace_bytes(1, 16, 8, 9) == bad  # k > E
    assert lib.fp8moe_workspace_bytes(0, 16, 100, 64) == bad
    assert lib.fp8moe_workspace_bytes(7, 1, 1, 1) == bad


P = 0x1000  # aligned dummy device address, never dereferenced
U = 0x1004  # misaligned


def test_quant_act_validation(lib):
    f = lib.fp8_quant_act
    assert f(None, 4, 128, 128, P, P, None, None, 0, None) == NULL
    assert f(P, 4, 128, 64, P, P, None, None, 0, None) == UNSUP
    assert f(P, 0, 128, 128, P, P, None, None, 0, None) == SHAPE
    assert f(P, 4, 100, 128, P, P, None, None, 0, None) == SHAPE
    assert f(P, 3, 3, 0, P, P, None, None, 0, None) == SHAPE  # M*K % 8
    assert f(U, 4, 128, 128, P, P, None, None, 0, None) == ALIGN
    assert f(P, 2048, 4096, 0, P, P, None, None, 0, None) == WS
    assert f(P, 2048, 4096, 0, P, P, None, P, 100, None) == WS
    assert f(P, 4, 100, -1, P, P, None, None, 0, None) == SHAPE  # row mode: K % 8
    assert f(P, 4, 96, -1, U, P, None, None, 0, None) == ALIGN
    assert f(P, 4, 96, -2, P, P, None, None, 0, None) == UNSUP
    # code sums come only with the per-(token, 128) mode
    assert f(P, 4, 128, 0, P, P, P, None, 0, None) == UNSUP
    assert f(P, 4, 128, -1, P, P, P, None, 0, None) == UNSUP
    assert f(P, 4, 128, 128, P, P, U, None, 0, None) == ALIGN


def _route(lib, logits=P, T=16, E=8, k=2, ws=P, ws_bytes=1 << 20, xq=None, xs=None, H=0,
           xqp=None, xsp=None, ids=P, xsum=None, xsump=None):
    return lib.moe_route_permute(logits, T, E, k, ids, P, P, P, P, xq, xs, H, xqp, xsp, xsum,
                                 xsump, ws, ws_bytes, None)


def test_route_validation(lib):
    assert _route(lib, logits=None) == NULL
    assert _route(lib, ws=None) == NULL
    assert _route(lib, xq=P) == NULL  # each gather pair must come together
    assert _route(lib, xs=P) == NULL
    assert _route(lib, xqp=P) == NULL
    assert _route(lib, T=0) == SHAPE
    assert _route(lib, E=0) == SHAPE
    assert _route(lib, E=1025, k=2) == SHAPE
    assert _route(lib, k=0) == SHAPE
    assert _route(lib, E=4, k=5) == SHAPE
    assert _route(lib, E=64, k=33) == SHAPE
    assert _route(lib, T=1 << 28, k=8) == SHAPE  # T*k >= 2^31
    assert _route(lib, xq=P, xs=P, xqp=P, xsp=P, H=100) == SHAPE
    assert _route(lib, xs=P, xsp=P, H=100) == SHAPE  # scales-only gather
    assert _route(lib, xs=P, xsp=U, H=256) == ALIGN
    assert _route(lib, ids=U) == ALIGN
    assert _route(lib, ws_bytes=16) == WS
    assert _route(lib, xs=P, xsp=P, H=256, xsum=P) == NULL  # the sum pair comes together
    assert _route(lib, xsum=P, xsump=P) == NULL  # and only with the scale gather
    assert _route(lib, xs=P, xsp=P, H=256, xsum=P, xsump=U) == ALIGN


def _route_na(lib, logits=P, T=64, E=8, k=2, ids=P, xq=None, xs=None, H=0, xqp=None, xsp=None,
              xsum=None, xsump=None):
    return lib.moe_route_permute_noalloc(logits, T, E, k, ids, P, P, P, P, xq, xs, H, xqp, xsp,
                                         xsum, xsump, None)


def test_route_noalloc_validation(lib):
    # the same argument checks as moe_route_permute, all on the host before any launch
    assert _route_na(lib, logits=None) == NULL
    assert _route_na(lib, xq=P) == NULL
    assert _route_na(lib, xs=P, xsp=P, H=256, xsum=P) == NULL
    assert _route_na(lib, T=0) == SHAPE
    assert _route_na(lib, E=4, k=5) == SHAPE
    assert _route_na(lib, xs=P, xsp=P, H=100) == SHAPE
    assert _route_na(lib, ids=U) == ALIGN
    # past the 4 MiB static workspace: 2^20 tokens x 64 experts need 16 MiB of counts
    assert lib.fp8moe_workspace_bytes(1, 1 << 20, 64, 8) > 4 << 20
    assert _route_na(lib, T=1 << 20, E=64, k=8) == WS


def _qr(lib, x=P, T=64, H=256, q=P, scales=P, sums=P, logits=P, E=8, k=2, ids=P, ws=P,
        ws_bytes=1 << 20):
    return lib.fp8moe_quant_route(x, T, H, q, scales, sums, logits, E, k, ids, P, P, P, P, ws,
                                  ws_bytes, None)


def test_quant_route_validation(lib):
    # the checks of fp8_quant_act (group mode) and of moe_route_permute, on the host
    for kw in ("x", "q", "scales", "logits", "ids", "ws"):
        assert _qr(lib, **{kw: None}) == NULL, kw
    assert _qr(lib, sums=None, ws_bytes=16) == WS  # sums are optional
    assert _qr(lib, T=0) == SHAPE
    assert _qr(lib, H=100) == SHAPE
    assert _qr(lib, H=64) == SHAPE
    assert _qr(lib, T=1 << 40, H=128) == SHAPE  # T*H >= 2^40
    assert _qr(lib, E=0) == SHAPE
    assert _qr(lib, E=4, k=5) == SHAPE
    assert _qr(lib, E=1025, k=2) == SHAPE
    assert _qr(lib, T=1 << 28, H=128, k=8) == SHAPE  # T*k >= 2^31
    for kw in ("x", "q", "scales", "sums", "ids", "ws"):
        assert _qr(lib, **{kw: U}) == ALIGN, kw
    assert _qr(lib, ws_bytes=16) == WS


def _gg(lib, a=P, R=256, E=8, N=512, K=256, epi=0, dt=0, out_scales=P, sorted_=None, kr=1,
        out=P, a_sums=None, out_sums=None):
    return lib.fp8_grouped_expert_gemm(a, P, a_sums, sorted_, kr, P, P, P, R, E, N, K, epi, dt,
                                       out, out_scales, out_sums, None)


def test_grouped_gemm_validation(lib):
    assert _gg(lib, epi=2) == UNSUP
    assert _gg(lib, dt=3) == UNSUP
    assert _gg(lib, a=None) == NULL
    assert _gg(lib, epi=1, out_scales=None) == NULL
    assert _gg(lib, R=-1) == SHAPE
    assert _gg(lib, E=0) == SHAPE
    assert _gg(lib, E=1025) == SHAPE
    assert _gg(lib, K=100) == SHAPE
    assert _gg(lib, K=0) == SHAPE
    assert _gg(lib, K=32768) == SHAPE
    assert _gg(lib, R=1 << 22, K=2048) == SHAPE  # R*K >= 2^32
    assert _gg(lib, N=24) == SHAPE
    assert _gg(lib, N=80) == SHAPE  # STORE needs N % 64 == 0
    assert _gg(lib, epi=1, N=384) == SHAPE  # SwiGLU needs N % 256 == 0
    assert _gg(lib, sorted_=P, kr=0) == SHAPE
    assert _gg(lib, sorted_=P, kr=3) == SHAPE  # gathered rows: R = T * k_route
    assert _gg(lib, out=U) == ALIGN
    assert _gg(lib, R=0) == OK  # empty input is a no-op; nothing is launched
    # with no rows the row-sized buffers may be NULL (torch's empty tensors), the bank not
    f = lib.fp8_grouped_expert_gemm
    assert f(None, None, None, None, 1, P, P, P, 0, 8, 512, 256, 1, 0, None, None, None,
             None) == OK
    assert f(None, None, None, None, 1, None, P, P, 0, 8, 512, 256, 0, 0, None, None, None,
             None) == NULL
    assert _gg(lib, a=None, R=1) == NULL
    assert _gg(lib, R=64, N=1 << 20, K=16384) == SHAPE  # N*K/2 >= 2^32
    # (ceil(R/128) + E) * ceil(N/256) >= 2^28: tile indices would not fit 32 bits
    assert _gg(lib, R=(1 << 25) - 128, N=(1 << 24) - 256, K=128) == SHAPE
    assert _gg(lib, out_sums=P) == UNSUP  # output code sums only with SwiGLU
    assert _gg(lib, a_sums=U) == ALIGN
    assert _gg(lib, epi=1, out_sums=U) == ALIGN


def _pack(lib, w=P, s=P, E=4, N=64, K=256, wp=P, sp=P):
    return lib.fp8moe_pack_expert_bank(w, s, E, N, K, wp, sp, None)


def test_pack_bank_validation(lib):
    assert _pack(lib, w=None) == NULL
    assert _pack(lib, sp=None) == NULL
    assert _pack(lib, E=0) == SHAPE
    assert _pack(lib, E=1025) == SHAPE
    assert _pack(lib, N=24) == SHAPE
    assert _pack(lib, N=80) == SHAPE
    assert _pack(lib, K=200) == SHAPE
    assert _pack(lib, K=32768) == SHAPE
    assert _pack(lib, N=1 << 20, K=16384) == SHAPE
    assert _pack(lib, wp=U) == ALIGN


def test_dense_gemm_validation(lib):
    f = lib.fp8_dense_gemm
    assert f(P, P, P, P, 16, 64, 128, 5, P, None) == UNSUP
    assert f(None, P, P, P, 16, 64, 128, 0, P, None) == NULL
    assert f(P, P, P, P, 0, 64, 128, 0, P, None) == SHAPE
    assert f(P, P, P, P, 16, 24, 128, 0, P, None) == SHAPE
    assert f(P, P, P, P, 16, 64, 96, 0, P, None) == SHAPE
    assert f(P, P, U, P, 16, 64, 128, 0, P, None) == ALIGN


def test_dense_gemm_rowwise_validation(lib):
    f = lib.fp8_dense_gemm_rowwise
    assert f(P, P, P, P, 16, 64, 128, 5, P, None) == UNSUP
    assert f(P, None, P, P, 16, 64, 128, 0, P, None) == NULL
    assert f(P, P, P, P, 0, 64, 128, 0, P, None) == SHAPE
    assert f(P, P, P, P, 16, 24, 128, 0, P, None) == SHAPE
    assert f(P, P, P, P, 16, 64, 96, 0, P, None) == SHAPE
    assert f(P, P, P, P, 1 << 21, 64, 4096, 0, P, None) == SHAPE  # M*K >= 2^32
    assert f(P, U, P, P, 16, 64, 128, 0, P, None) == ALIGN


def test_block_gemm_validation(lib):
    f = lib.fp8_block_gemm
    assert f(P, P, P, P, 16, 64, 128, 5, P, None) == UNSUP
    assert f(P, P, P, None, 16, 64, 128, 0, P, None) == NULL
    assert f(P, P, P, P, 0, 64, 128, 0, P, None) == SHAPE
    assert f(P, P, P, P, 16, 24, 128, 0, P, None) == SHAPE
    assert f(P, P, P, P, 16, 64, 200, 0, P, None) == SHAPE
    assert f(P, P, P, U, 16, 64, 128, 0, P, None) == ALIGN
    assert f(P, P, P, P, 16, 64, 16384 + 128, 0, P, None) == SHAPE


def test_quant_weight_block128_validation(lib):
    f = lib.fp8_quant_weight_block128
    assert f(None, 64, 128, P, P, None) == NULL
    assert f(P, 0, 128, P, P, None) == SHAPE
    assert f(P, 64, 100, P, P, None) == SHAPE
    assert f(P, 128 * 65536, 128, P, P, None) == SHAPE  # row-block grid limit
    assert f(P, 64, 128, P, U, None) == ALIGN


def test_mxfp4_validation(lib):
    q = lib.mxfp4_quant_act
    assert q(None, 4, 64, P, P, None) == NULL
    assert q(P, 0, 64, P, P, None) == SHAPE
    assert q(P, 4, 48, P, P, None) == SHAPE  # K % 32
    assert q(P, 4, 64, P, U, None) == ALIGN
    pk = lib.fp8moe_pack_expert_bank_mxfp4
    assert pk(None, P, 4, 64, 256, P, P, None) == NULL
    assert pk(P, P, 4, 24, 256, P, P, None) == SHAPE
    assert pk(P, P, 4, 64, 100, P, P, None) == SHAPE
    g = lib.mxfp4_grouped_expert_gemm
    assert g(P, P, None, 1, P, P, P, 256, 8, 512, 256, 2, 0, P, P, None, None) == UNSUP
    assert g(None, P, None, 1, P, P, P, 256, 8, 512, 256, 0, 0, P, P, None, None) == NULL
    assert g(P, P, None, 1, P, P, P, 256, 8, 512, 100, 0, 0, P, P, None, None) == SHAPE
    assert g(P, P, None, 1, P, P, P, 256, 8, 512, 256, 0, 0, U, P, None, None) == ALIGN
    assert g(P, P, None, 1, P, P, P, 0, 8, 512, 256, 0, 0, P, P, None, None) == OK
    assert g(P, P, None, 1, P, P, P, 256, 8, 512, 256, 0, 0, P, P, P, None) == UNSUP


def test_combine_validation(lib):
    f = lib.moe_unpermute_combine
    assert f(P, 2, P, P, 4, 2, 64, 1, P, None) == UNSUP
    assert f(None, 1, P, P, 4, 2, 64, 1, P, None) == NULL
    assert f(P, 1, P, P, 0, 2, 64, 1, P, None) == SHAPE
    assert f(P, 1, P, P, 4, 33, 64, 1, P, None) == SHAPE
    assert f(P, 1, P, P, 4, 2, 60, 1, P, None) == SHAPE
    assert f(P, 1, U, P, 4, 2, 64, 1, P, None) == ALIGN


def test_binding_refuses_host_tensors():
    import torch

    import fp8_moe_prefill_amd as f
    with pytest.raises(ValueError):
        f.fp8_quant_act(torch.zeros((4, 128), dtype=torch.bfloat16))


def test_attention_workspace_query(lib):
    bad = ctypes.c_size_t(-1).value
    assert lib.fp8moe_workspace_bytes(2, 2048, 4, 128) == 4 * 128 * 2048 * 2
    assert lib.fp8moe_workspace_bytes(2, 100, 2, 128) == 2 * 128 * 128 * 2  # T padded to 64
    assert lib.fp8moe_workspace_bytes(2, 100, 2, 64) == bad  # head_dim must be 128
    assert lib.fp8moe_workspace_bytes(2, 0, 2, 128) == bad


def test_rmsnorm_validation(lib):
    f = lib.fp8moe_rmsnorm
    assert f(None, None, 4, 64, 1e-6, None, P, None) == NULL
    assert f(P, P, 4, 64, 1e-6, None, P, None) == NULL  # delta without x_out
    assert f(P, None, 0, 64, 1e-6, None, P, None) == SHAPE
    assert f(P, None, 4, 60, 1e-6, None, P, None) == SHAPE  # H % 8
    assert f(P, None, 4, 64, -1.0, None, P, None) == SHAPE
    assert f(P, None, 4, 64, float("nan"), None, P, None) == SHAPE
    assert f(U, None, 4, 64, 1e-6, None, P, None) == ALIGN
    assert f(P, U, 4, 64, 1e-6, P, P, None) == ALIGN


def test_bf16_gemm_validation(lib):
    f = lib.fp8moe_bf16_gemm
    assert f(None, P, 4, 4, 64, P, None) == NULL
    assert f(P, P, 0, 4, 64, P, None) == SHAPE
    assert f(P, P, 4, 0, 64, P, None) == SHAPE
    assert f(P, P, 4, 4, 96, P, None) == SHAPE  # K % 64
    assert f(P, P, 4, 4, 64, U, None) == ALIGN


def test_attention_validation(lib):
    f = lib.fp8moe_causal_attention
    n = 4 * 128 * 64 * 2
    assert f(None, 64, 16, 4, 128, P, P, n, None) == NULL
    assert f(P, 64, 16, 4, 64, P, P, n, None) == SHAPE   # head_dim
    assert f(P, 64, 16, 3, 128, P, P, n, None) == SHAPE  # n_q % n_kv
    assert f(P, 0, 16, 4, 128, P, P, n, None) == SHAPE
    assert f(P, 64, 16, 4, 128, U, P, n, None) == ALIGN
    assert f(P, 64, 16, 4, 128, P, P, n - 1, None) == WS

