"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/i8h.h declares, and rejects invalid arguments on the host
with the documented status codes before anything is launched. The invalid
calls pass dummy non-null addresses that are never dereferenced."""

import ctypes
import os
import re

import pytest

import int8_hadamard_domain_amd as i8h

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "i8h.h")

EINVAL, EUNSUP, OK = i8h.I8H_EINVAL, i8h.I8H_EUNSUPPORTED, i8h.I8H_OK
A = ctypes.c_void_p(0x10000)     # a 256-byte aligned dummy address, never touched
ODD = ctypes.c_void_p(0x10002)   # misaligned for 4/16-byte data


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z][a-z0-9_]*)\s*\(", src)) - {"defined"})


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(i8h.LIB_PATH):
        pytest.skip("libi8h.so not built")
    return i8h.lib()


def test_every_declared_function_is_exported(L):
    names = declared_functions()
    assert len(names) == 27, names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    assert L.i8h_status_string(0) == b"ok"
    assert L.i8h_status_string(-1) == b"invalid argument"
    assert L.i8h_status_string(-2) == b"unsupported size"
    assert L.i8h_status_string(-3) == b"HIP launch error"
    assert L.i8h_status_string(7) == b"unknown status"


def test_workspace_sizes(L):
    assert L.moe_route_permute_workspace_size(1, 128, 8) == 0          # single-block path
    assert L.moe_route_permute_workspace_size(2048, 128, 8) == 64 * 128 * 4
    assert L.moe_route_permute_workspace_size(0, 128, 8) == 0
    assert L.moe_gateup_fp8blk_workspace_size(128, 2048) == 128 * 2048 + 128 * 16 * 4 + 128 * 2048 * 2
    assert L.moe_gateup_fp8blk_workspace_size(3, 128) == 512 + 256 + 768   # each part rounded to 256 B
    assert L.moe_gateup_i8h_fused_workspace_size(1, 2048) == 0          # rotation inside the decode kernel
    assert L.moe_gateup_i8h_fused_workspace_size(128, 2048) == 128 * 2048 * 2
    # bf16 act rows, then y, each rounded to 256 B
    assert L.moe_down_bf16_workspace_size(2048, 768, 2048, 8) == 16384 * 768 * 2 + 16384 * 2048 * 4
    assert L.moe_down_bf16_workspace_size(1, 8, 8, 1) == 256 + 256
    assert L.moe_down_bf16_workspace_size(0, 768, 2048, 8) == 0
    # W8A8: int8 activations, then their float32 scales, each rounded to 256 B
    assert L.moe_gateup_i8g_workspace_size(2048, 2048) == 2048 * 2048 + 2048 * 16 * 4
    assert L.moe_gateup_i8g_workspace_size(3, 128) == 512 + 256
    assert L.moe_gateup_i8g_workspace_size(0, 2048) == 0
    assert L.moe_gateup_i8g_workspace_size(4, 100) == 0


def route(L, T=8, E=16, k=2, ptr=A, ws=A, wsb=1 << 20):
    return L.moe_route_permute(ptr, T, E, k, A, A, A, A, A, ws, wsb, None)


def test_route_validation(L):
    assert route(L, T=-1) == EINVAL
    assert route(L, E=0) == EINVAL
    assert route(L, k=0) == EINVAL
    assert route(L, E=1025) == EUNSUP
    assert route(L, E=64, k=33) == EUNSUP
    assert route(L, E=4, k=5) == EUNSUP
    assert route(L, T=0) == OK                       # no-op
    assert route(L, ptr=None) == EINVAL
    assert route(L, ptr=ODD) == EINVAL
    assert route(L, T=100, ws=None) == EINVAL        # workspace needed
    assert route(L, T=100, wsb=16) == EINVAL         # too small
    assert route(L, T=1 << 27, k=16, E=64) == EUNSUP  # P overflows int32
    # P fits in int32, but ceil(P / 256) * E (the chunk histograms' index) does not
    assert route(L, T=1 << 24, k=32, E=1024) == EUNSUP
    assert route(L, T=(1 << 24) - 8, k=32, E=1024, ptr=None) == EINVAL   # just below: other checks apply


def test_route_rotate_validation(L):
    f = lambda T=8, E=16, k=2, K=256, lg=A, x=A, xr=ctypes.c_void_p(0x90000), ws=A, wsb=1 << 20: \
        L.moe_route_permute_rotate(lg, x, T, E, k, K, A, A, A, A, A, xr, ws, wsb, None)
    assert f(K=100) == EINVAL                        # K % 128
    assert f(K=0) == EINVAL
    assert f(E=1025) == EUNSUP
    assert f(E=4, k=5) == EUNSUP
    assert f(T=0) == OK
    assert f(x=None) == EINVAL
    assert f(xr=None) == EINVAL
    assert f(x=ctypes.c_void_p(0x10008)) == EINVAL   # 16-B alignment
    assert f(xr=ctypes.c_void_p(0x10100)) == EINVAL  # partial overlap of x and x_rot
    assert f(T=100, ws=None) == EINVAL               # workspace needed
    assert f(T=1 << 20, K=4096) == EUNSUP            # T*K offsets are 32-bit
    # the chunk histograms: chunks of max(1, min(floor(256 / topk), ceil(T / 32))) whole tokens
    assert L.moe_route_permute_workspace_size(100, 16, 3) == 25 * 16 * 4    # 4 tokens a chunk
    assert L.moe_route_permute_workspace_size(3000, 16, 3) == 36 * 16 * 4   # 85 tokens a chunk
    assert L.moe_route_permute_workspace_size(100, 16, 32) == 25 * 16 * 4   # 4 tokens a chunk
    assert L.moe_route_permute_workspace_size(1000, 16, 32) == 125 * 16 * 4  # 8 tokens a chunk
    assert L.moe_route_permute_workspace_size(300, 16, 1) == 30 * 16 * 4    # 10 tokens a chunk
    assert L.moe_route_permute_workspace_size(128, 128, 8) == 32 * 128 * 4  # verify: 4 tokens a chunk


def test_route_noalloc_validation(L):
    f = lambda T=8, E=16, k=2, ptr=A: L.moe_route_permute_noalloc(ptr, T, E, k, A, A, A, A, A, None)
    assert f(T=-1) == EINVAL
    assert f(E=0) == EINVAL
    assert f(E=1025) == EUNSUP
    assert f(E=4, k=5) == EUNSUP
    assert f(T=0) == OK
    # the fixed 1 MiB scratch holds ceil(P / 256) * E counts: P = 524288 pairs at E = 128 is the
    # largest admitted, one chunk more is refused (both before any HIP call)
    assert L.moe_route_permute_workspace_size(65536, 128, 8) == 1 << 20
    assert f(T=65536 + 32, E=128, k=8) == EUNSUP
    assert f(T=65536, E=128, k=8, ptr=None) == EINVAL     # within the limit: the other checks apply
    assert f(T=1 << 20, E=1024, k=1) == EUNSUP
    assert f(ptr=ODD) == EINVAL


def rot(L, x=A, ldx=256, y=A, ldy=256, T=4, K=256):
    return L.hadamard128_rotate(x, ldx, y, ldy, T, K, None)


def test_rotate_validation(L):
    assert rot(L, K=200) == EINVAL
    assert rot(L, K=0) == EINVAL
    assert rot(L, ldx=128) == EINVAL                 # ldx < K
    assert rot(L, ldy=260) == EINVAL                 # not a multiple of 8
    assert rot(L, x=None) == EINVAL
    assert rot(L, x=ctypes.c_void_p(0x10008)) == EINVAL
    assert rot(L, T=0) == OK
    # partial overlap of distinct x and y
    assert rot(L, x=ctypes.c_void_p(0x10000), y=ctypes.c_void_p(0x10100)) == EINVAL
    # in place with different strides
    assert rot(L, ldy=264) == EINVAL


def gemm(L, x=A, T=4, K=256, codes=A, scales=A, E=8, N=256, k=2, off=A, sp=A, gu=A, act=A, path=0):
    return L.moe_gateup_i8h_grouped_path(x, T, K, codes, scales, E, N, k, off, sp, gu, act, path, None)


def test_gateup_i8h_validation(L):
    assert gemm(L, K=100) == EINVAL
    assert gemm(L, N=97) == EINVAL                   # odd N: no gate/up halves
    assert gemm(L, N=96) == EUNSUP                   # even, but not whole 32-row gate/up tiles
    assert gemm(L, N=160, path=1) == EUNSUP          # (every path)
    assert gemm(L, N=2, path=4) == EUNSUP
    assert gemm(L, E=2000) == EUNSUP
    assert gemm(L, k=3, E=2) == EUNSUP
    assert gemm(L, path=7) == EINVAL
    assert gemm(L, T=0) == OK
    assert gemm(L, x=None) == EINVAL
    assert gemm(L, codes=ODD) == EINVAL
    assert gemm(L, gu=ODD) == EINVAL
    assert gemm(L, gu=None, act=None) == OK          # nothing requested
    assert gemm(L, K=8192, path=1) == EUNSUP         # decode kernel keeps K <= 4096
    assert L.moe_gateup_i8h_grouped(None, 4, 256, A, A, 8, 256, 2, A, A, A, A, None) == EINVAL


def test_fused_validation(L):
    f = L.moe_gateup_i8h_grouped_fused
    assert f(A, 4, 100, A, A, 8, 256, 2, A, A, A, A, None, 0, None) == EINVAL
    assert f(A, 4, 256, A, A, 8, 255, 2, A, A, A, A, None, 0, None) == EINVAL    # odd N
    assert f(A, 4, 256, A, A, 8, 160, 2, A, A, A, A, None, 0, None) == EUNSUP    # even N, not N % 64
    assert f(A, 100, 256, A, A, 8, 256, 2, A, A, A, A, None, 0, None) == EINVAL     # workspace needed
    assert f(A, 100, 256, A, A, 8, 256, 2, A, A, A, A, A, 16, None) == EINVAL       # too small
    assert f(A, 0, 256, A, A, 8, 256, 2, A, A, A, A, None, 0, None) == OK
    assert f(A, 1 << 20, 4096, A, A, 8, 256, 2, A, A, A, A, A, 1 << 40, None) == EUNSUP  # T*K overflows


def test_fp8_validation(L):
    f = L.moe_gateup_fp8blk_grouped
    assert f(A, 4, 256, A, A, 8, 192, 2, A, A, A, A, A, 1 << 20, None) == EINVAL    # N % 128
    assert f(A, 4, 256, A, A, 8, 256, 2, A, A, A, A, None, 1 << 20, None) == EINVAL  # no workspace
    assert f(A, 4, 256, A, A, 8, 256, 2, A, A, A, A, A, 16, None) == EINVAL         # too small
    assert f(A, 4, 256, A, A, 8, 256, 2, A, A, A, A, ctypes.c_void_p(0x10010), 1 << 20, None) == EINVAL
    assert f(A, 0, 256, A, A, 8, 256, 2, A, A, A, A, None, 0, None) == OK
    fp = L.moe_gateup_fp8blk_grouped_path
    assert fp(A, 4, 256, A, A, 8, 256, 2, A, A, A, A, A, 1 << 20, 5, None) == EINVAL    # no such path
    assert fp(A, 4, 256, A, A, 8, 256, 2, A, A, A, A, A, 1 << 20, -1, None) == EINVAL
    assert fp(A, 4, 256, A, A, 8, 256, 2, A, A, A, A, A, 1 << 20, 1, None) == EUNSUP    # GEMV: no E4M3 form
    assert fp(A, 4, 256, A, A, 8, 256, 2, A, A, A, A, A, 1 << 20, 3, None) == EUNSUP    # TALL: no E4M3 form
    assert fp(A, 4, 256, A, A, 8, 192, 2, A, A, A, A, A, 1 << 20, 4, None) == EINVAL    # N % 128
    assert fp(A, 0, 256, A, A, 8, 256, 2, A, A, A, A, None, 0, 4, None) == OK
    q = L.fp8_quantize_activations
    assert q(A, 4, 100, A, A, None) == EINVAL
    assert q(ODD, 4, 128, A, A, None) == EINVAL
    assert q(A, 0, 128, A, A, None) == OK


def dec(L, lg=A, x=A, T=1, K=2048, codes=A, scales=A, E=128, N=1536, k=8, gu=A, act=A, ids=A):
    return L.moe_route_gateup_i8h_decode(lg, x, T, K, codes, scales, E, N, k, ids, A, A, A, A, gu, act, None)


def test_decode_validation(L):
    assert dec(L, K=100) == EINVAL
    assert dec(L, N=95) == EINVAL                    # odd N
    assert dec(L, N=96) == EUNSUP                    # even N outside the 32-row tiles
    assert dec(L, T=9) == EUNSUP                     # 72 pairs > 64
    assert dec(L, E=257, k=8) == EUNSUP              # more than 4 logits per lane
    assert dec(L, K=8192) == EUNSUP
    assert dec(L, T=0) == OK
    assert dec(L, lg=None) == EINVAL
    assert dec(L, ids=None) == EINVAL                # routing outputs are required
    assert dec(L, gu=None, act=None) == EINVAL       # nothing to compute
    assert dec(L, x=ODD) == EINVAL
    assert dec(L, lg=ODD) == EINVAL


def down(L, act=A, T=4, I=256, w=A, E=8, H=512, k=2, ids=A, tw=A, off=A, pos=A, out=A, ws=A, wsb=1 << 30,
         path=0):
    return L.moe_down_bf16_combine_path(act, T, I, w, E, H, k, ids, tw, off, pos, out, ws, wsb, path, None)


def test_down_validation(L):
    assert down(L, I=100) == EINVAL                   # I % 8
    assert down(L, H=12) == EINVAL                    # H % 8
    assert down(L, E=2000) == EUNSUP
    assert down(L, k=3, E=2) == EUNSUP
    assert down(L, path=5) == EINVAL
    assert down(L, T=0) == OK
    assert down(L, act=None) == EINVAL
    assert down(L, pos=None) == EINVAL
    assert down(L, act=ODD) == EINVAL
    assert down(L, out=ODD) == EINVAL
    assert down(L, I=2048, path=1) == EUNSUP          # the one-launch form keeps I <= 1024
    assert down(L, I=200, path=2) == EUNSUP           # the GEMM form needs I % 32 == 0
    assert down(L, H=520, path=2) == EUNSUP           # ... and H % 256 == 0
    assert down(L, T=100, ws=None) == EINVAL          # AUTO takes the GEMM form: workspace needed
    assert down(L, T=100, wsb=16) == EINVAL           # too small
    assert down(L, T=100, ws=ctypes.c_void_p(0x10010)) == EINVAL   # not 256-B aligned
    assert down(L, I=2048, H=520, T=100) == EUNSUP    # neither form applies
    assert L.moe_down_bf16_combine(None, 4, 256, A, 8, 512, 2, A, A, A, A, A, A, 1 << 30, None) == EINVAL


def test_act_bf16_entries_validation(L):
    # the bf16 act forms: act 2-B aligned for the gate_up calls, 16-B for the down call, whose GEMM form
    # needs a workspace for y only; the other checks as in the float32 forms
    B1 = ctypes.c_void_p(0x10001)    # misaligned even for bf16
    g = lambda act=A, gu=A, path=0, N=256, T=4, K=256: L.moe_gateup_i8h_grouped_act_bf16(
        A, T, K, A, A, 8, N, 2, A, A, gu, act, path, None)
    assert g(K=100) == EINVAL
    assert g(N=97) == EINVAL
    assert g(N=96) == EUNSUP
    assert g(act=B1) == EINVAL
    assert g(gu=ODD) == EINVAL
    assert g(path=7) == EINVAL
    assert g(T=0) == OK
    assert g(gu=None, act=None) == OK
    assert g(K=8192, path=1) == EUNSUP
    f = L.moe_gateup_fp8blk_grouped_act_bf16
    assert f(A, 4, 256, A, A, 8, 256, 2, A, A, A, B1, A, 1 << 20, 0, None) == EINVAL
    assert f(A, 4, 256, A, A, 8, 192, 2, A, A, A, A, A, 1 << 20, 0, None) == EINVAL    # N % 128
    assert f(A, 4, 256, A, A, 8, 256, 2, A, A, A, A, A, 1 << 20, 1, None) == EUNSUP    # GEMV: no E4M3 form
    assert f(A, 4, 256, A, A, 8, 256, 2, A, A, A, A, None, 0, 0, None) == EINVAL       # no workspace
    assert f(A, 0, 256, A, A, 8, 256, 2, A, A, A, A, None, 0, 0, None) == OK
    w = L.moe_gateup_i8g_grouped_act_bf16
    assert w(A, 4, 256, A, A, 8, 256, 2, A, A, A, B1, A, 1 << 20, None) == EINVAL
    assert w(A, 4, 256, A, A, 8, 224, 2, A, A, A, A, A, 1 << 20, None) == EUNSUP
    assert w(A, 4, 256, A, A, 8, 256, 2, A, A, A, A, None, 0, None) == EINVAL        # no workspace
    assert w(A, 0, 256, A, A, 8, 256, 2, A, A, A, A, None, 0, None) == OK
    # y only, rounded to 256 B
    assert L.moe_down_bf16_act_bf16_workspace_size(2048, 768, 2048, 8) == 16384 * 2048 * 4
    assert L.moe_down_bf16_act_bf16_workspace_size(1, 8, 8, 1) == 256
    assert L.moe_down_bf16_act_bf16_workspace_size(0, 768, 2048, 8) == 0
    need = L.moe_down_bf16_act_bf16_workspace_size(100, 256, 512, 2)
    d = lambda act=A, T=100, I=256, H=512, ws=A, wsb=need, path=0: L.moe_down_bf16_combine_act_bf16(
        act, T, I, A, 8, H, 2, A, A, A, A, A, ws, wsb, path, None)
    assert d(I=100) == EINVAL
    assert d(act=ctypes.c_void_p(0x10008)) == EINVAL          # 16-B alignment
    assert d(act=None) == EINVAL
    assert d(path=5) == EINVAL
    assert d(T=0) == OK
    assert d(ws=None) == EINVAL                               # AUTO takes the GEMM form: workspace needed
    assert d(wsb=need - 1) == EINVAL                          # too small
    assert d(I=2048, path=1) == EUNSUP


def test_linear_validation(L):
    f = L.linear_i8f16
    assert f(A, 4, 100, A, A, 64, A, None) == EINVAL          # K % 128
    assert f(A, 4, 256, A, A, 24, A, None) == EINVAL          # N % 16
    assert f(A, 0, 256, A, A, 64, A, None) == OK
    assert f(None, 4, 256, A, A, 64, A, None) == EINVAL
    assert f(ODD, 4, 256, A, A, 64, A, None) == EINVAL
    assert f(A, 4, 256, A, ctypes.c_void_p(0x10001), 64, A, None) == EINVAL   # scales 2-B aligned
    assert f(A, 1 << 20, 4096, A, A, 64, A, None) == EUNSUP   # T*K offsets are 32-bit


def test_i8g_validation(L):
    f = L.moe_gateup_i8g_grouped
    assert f(A, 4, 256, A, A, 8, 225, 2, A, A, A, A, A, 1 << 20, None) == EINVAL    # odd N
    assert f(A, 4, 256, A, A, 8, 224, 2, A, A, A, A, A, 1 << 20, None) == EUNSUP    # even N, not N % 64
    assert f(A, 4, 200, A, A, 8, 256, 2, A, A, A, A, A, 1 << 20, None) == EINVAL    # K % 128
    assert f(A, 4, 256, A, A, 8, 256, 2, A, A, A, A, None, 1 << 20, None) == EINVAL  # no workspace
    assert f(A, 4, 256, A, A, 8, 256, 2, A, A, A, A, A, 16, None) == EINVAL         # too small
    assert f(A, 4, 256, A, A, 8, 256, 2, A, A, A, A, ctypes.c_void_p(0x10010), 1 << 20, None) == EINVAL
    assert f(ODD, 4, 256, A, A, 8, 256, 2, A, A, A, A, A, 1 << 20, None) == EINVAL
    assert f(A, 4, 256, A, ODD, 8, 256, 2, A, A, A, A, A, 1 << 20, None) == EINVAL
    assert f(A, 4, 1 << 16, A, A, 8, 1 << 15, 2, A, A, A, A, A, 1 << 30, None) == EUNSUP   # N*K >= 2^31
    assert f(A, 0, 256, A, A, 8, 256, 2, A, A, A, A, None, 0, None) == OK
    assert f(A, 4, 256, A, A, 8, 256, 9, A, A, A, A, A, 1 << 20, None) == EUNSUP    # topk > E
    q = L.i8_quantize_activations
    assert q(A, 4, 100, A, A, None) == EINVAL
    assert q(ODD, 4, 128, A, A, None) == EINVAL
    assert q(A, 4, 128, ctypes.c_void_p(0x10004), A, None) == EINVAL            # qx needs 8-B alignment
    assert q(A, 1 << 20, 4096, A, A, None) == EUNSUP
    assert q(A, 0, 128, A, A, None) == OK


PROBE_HEADER = os.path.join(os.path.dirname(HEADER), "i8h_probe.h")
PROBE_LIB = os.path.join(os.path.dirname(i8h.LIB_PATH), "libi8h_probe.so")


def test_probe_library_exports_and_validation():
    if not os.path.exists(PROBE_LIB):
        pytest.skip("libi8h_probe.so not built")
    P = ctypes.CDLL(PROBE_LIB)
    src = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b([a-z][a-z0-9_]*)\s*\(", src)) - {"defined"})
    assert names == ["i8h_fp8_mfma_probe", "i8h_overlap_probe", "i8h_read_probe"], names
    for n in names:
        assert hasattr(P, n), n
    f = P.i8h_fp8_mfma_probe
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p]
    assert f(3, A, A, A, 1, 1, None) == -1                           # no such form
    assert f(0, A, A, A, 0, 1, None) == -1                           # no tiles
    assert f(0, A, A, A, 1, 0, None) == -1                           # no steps
    assert f(0, ctypes.c_void_p(0x10010), A, A, 1, 1, None) == -1    # form 0 needs 32-B operands
    assert f(2, A, ctypes.c_void_p(0x10008), A, 1, 1, None) == -1    # form 2 needs 16-B operands
    assert f(1, A, A, ODD, 1, 1, None) == -1                         # c 4-B aligned
    assert f(1, None, A, A, 1, 1, None) == -1
    r = P.i8h_read_probe
    r.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    assert r(A, 0, 1, 0, A, None) == -1
    assert r(A, 24, 1, 0, A, None) == -1
    assert r(A, 32, 0, 0, A, None) == -1
    assert r(ODD, 32, 1, 0, A, None) == -1
    o = P.i8h_overlap_probe
    o.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert o(5, 256, 1, 1, A, None) == -1                            # no such VALU count
    assert o(4, 128, 1, 1, A, None) == -1                            # 256 or 512 threads
    assert o(4, 256, 0, 1, A, None) == -1
    assert o(4, 256, 1, 0, A, None) == -1
    assert o(4, 256, 1, 1, None, None) == -1
    assert o(4, 256, 1, 1, ODD, None) == -1
