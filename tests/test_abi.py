"""The C ABI library loads, exports every entry point its header declares, and
rejects invalid arguments on the host, before anything touches a device.

Runs without a GPU: every call below fails validation, so no HIP API call is
made.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8bs.h")

import fp8_block_scaled_x1_amd as fb  # noqa: E402


def _declared_functions():
    text = open(HEADER).read()
    return re.findall(r"FP8BS_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fb.LIB_PATH):
        pytest.skip("libfp8bs.so not built")
    return fb.lib()


def test_header_declares_the_entry_points():
    names = set(_declared_functions())
    assert {"fp8_quant_act_1x128", "fp8_quant_w_128x128", "fp8_quant_act_128x1_T",
            "fp8_quant_act_128x1_T_grouped", "fp8_quant_act_1x128_128x1_T", "fp8_quant_act_1x128_128x1_T_grouped",
            "fp8_gemm_blockscaled", "fp8_gemm_blockscaled_q1x128",
            "fp8_gemm_blockscaled_q1x128_q128x1T", "fp8_gemm_blockscaled_tile",
            "fp8_grouped_gemm_blockscaled", "fp8_grouped_gemm_wgrad", "fp8_moe_dispatch",
            "fp8_moe_dispatch_workspace_bytes", "fp8_moe_dispatch_noalloc", "fp8_moe_combine", "fp8_quant_act_1x128_pow2",
            "fp8_quant_w_128x128_pow2", "fp8_quant_act_128x1_T_pow2", "fp8_gemm_blockscaled_pow2",
            "fp8bs_status_string", "fp8bs_abi_version"} == names


def test_library_exports_every_declared_symbol(L):
    raw = ctypes.CDLL(fb.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(raw, name), name


def test_version_and_status_strings(L):
    assert L.fp8bs_abi_version() == fb.ABI_VERSION == 11
    for code in range(-8, 1):
        assert fb.status_string(code) not in ("", "unknown status")
    assert fb.status_string(-99) == "unknown status"


NULL = None
P = 4096   # a fake, 16-byte aligned, non-null address: never dereferenced by a failing call
MIS = 4100


def test_quant_act_validation(L):
    f = L.fp8_quant_act_1x128
    assert f(P, 2, 4, 128, P, P, NULL) == -4          # dtype
    assert f(P, 1, 4, 100, P, P, NULL) == -2          # K not a multiple of 128
    assert f(P, 1, -1, 128, P, P, NULL) == -2
    assert f(NULL, 1, 4, 128, P, P, NULL) == -1
    assert f(P, 1, 4, 128, NULL, P, NULL) == -1
    assert f(MIS, 1, 4, 128, P, P, NULL) == -3
    assert f(P, 1, 4, 128, P, MIS, NULL) == -3
    assert f(NULL, 1, 0, 128, NULL, NULL, NULL) == 0  # empty: no-op
    assert f(NULL, 0, 7, 0, NULL, NULL, NULL) == 0


def test_quant_w_validation(L):
    f = L.fp8_quant_w_128x128
    assert f(P, 1, 128, 128, P, P, P, NULL, NULL) == -5   # one-sided transposed outputs
    assert f(P, 1, 100, 128, P, P, NULL, NULL, NULL) == -2
    assert f(P, 1, 128, 200, P, P, NULL, NULL, NULL) == -2
    assert f(P, 5, 128, 128, P, P, NULL, NULL, NULL) == -4
    assert f(NULL, 1, 128, 128, P, P, NULL, NULL, NULL) == -1
    assert f(P, 1, 128, 128, P, P, MIS, P, NULL) == -3
    assert f(NULL, 1, 0, 128, NULL, NULL, NULL, NULL, NULL) == 0


def test_quant_128x1_validation(L):
    f = L.fp8_quant_act_128x1_T
    assert f(P, 1, 100, 64, P, P, NULL) == -2         # M not a multiple of 128
    assert f(P, 1, 128, -3, P, P, NULL) == -2
    assert f(P, 1, 128, 64, NULL, P, NULL) == -1
    assert f(P, 1, 128, 64, P, MIS, NULL) == -3
    assert f(NULL, 1, 128, 0, NULL, NULL, NULL) == 0


def test_gemm_validation(L):
    f = L.fp8_gemm_blockscaled
    assert f(P, P, P, P, 2, P, 4, 128, 128, NULL) == -5
    assert f(P, P, P, P, 0, P, 4, 100, 128, NULL) == -2   # N not a multiple of 128
    assert f(P, P, P, P, 0, P, 4, 128, 0, NULL) == -2     # K must be positive
    assert f(P, P, P, P, 0, P, 4, 128, 130, NULL) == -2
    assert f(P, P, NULL, P, 0, P, 4, 128, 128, NULL) == -1
    assert f(P, P, P, P, 0, MIS, 4, 128, 128, NULL) == -3
    assert f(P, P, P, P, 0, P, 1 << 20, 1 << 12, 1 << 12, NULL) == -7   # M*N >= 2^31
    assert f(NULL, NULL, NULL, NULL, 1, NULL, 0, 128, 128, NULL) == 0  # M == 0: no-op


def test_grouped_validation(L):
    f = L.fp8_grouped_gemm_blockscaled
    assert f(P, P, P, P, P, P, -1, 4, 128, 128, NULL) == -2
    assert f(P, P, P, P, P, P, 0, 4, 128, 128, NULL) == -2      # rows but no experts
    assert f(P, P, P, P, P, NULL, 2, 4, 128, 128, NULL) == -1   # offsets missing
    assert f(P, P, P, P, P, P, 2, 4, 128, 100, NULL) == -2
    assert f(MIS, P, P, P, P, P, 2, 4, 128, 128, NULL) == -3
    assert f(P, P, P, P, P, P + 2, 2, 4, 128, 128, NULL) == -3  # offsets not 4-byte aligned
    assert f(NULL, NULL, NULL, NULL, NULL, NULL, 3, 0, 128, 128, NULL) == 0


def test_pow2_entry_points_validate_like_their_counterparts(L):
    assert L.fp8_quant_act_1x128_pow2(P, 2, 4, 128, P, P, NULL) == -4
    assert L.fp8_quant_act_1x128_pow2(P, 1, 4, 100, P, P, NULL) == -2
    assert L.fp8_quant_w_128x128_pow2(P, 1, 128, 128, P, P, P, NULL, NULL) == -5
    assert L.fp8_quant_act_128x1_T_pow2(P, 1, 100, 64, P, P, NULL) == -2
    assert L.fp8_gemm_blockscaled_pow2(P, P, P, P, 2, P, 4, 128, 128, NULL) == -5
    assert L.fp8_gemm_blockscaled_pow2(P, P, P, P, 0, MIS, 4, 128, 128, NULL) == -3
    assert L.fp8_gemm_blockscaled_pow2(NULL, NULL, NULL, NULL, 0, NULL, 0, 128, 128, NULL) == 0


def test_fused_epilogue_validation(L):
    f = L.fp8_gemm_blockscaled_q1x128
    assert f(P, P, P, P, 3, P, P, 4, 128, 128, NULL) == -5
    assert f(P, P, P, P, 0, P, P, 4, 100, 128, NULL) == -2
    assert f(P, P, P, P, 0, NULL, P, 4, 128, 128, NULL) == -1
    assert f(P, P, P, P, 0, P, MIS, 4, 128, 128, NULL) == -3
    g = L.fp8_gemm_blockscaled_q1x128_q128x1T
    assert g(P, P, P, P, 0, P, P, P, P, 100, 128, 128, NULL) == -2     # M not a multiple of 128
    assert g(P, P, P, P, 0, P, P, NULL, P, 128, 128, 128, NULL) == -1
    assert g(P, P, P, P, 0, P, P, P, MIS, 128, 128, 128, NULL) == -3
    assert g(NULL, NULL, NULL, NULL, 0, NULL, NULL, NULL, NULL, 0, 128, 128, NULL) == 0


def test_dual_layout_quantizer_validation(L):
    f = L.fp8_quant_act_1x128_128x1_T
    assert f(P, 3, 128, 128, P, P, P, P, NULL) == -4                # unknown dtype
    assert f(P, 1, 100, 128, P, P, P, P, NULL) == -2                # M not a multiple of 128
    assert f(P, 1, 128, 100, P, P, P, P, NULL) == -2                # C not a multiple of 128
    assert f(P, 1, 128, 128, P, P, NULL, P, NULL) == -1
    assert f(P, 1, 128, 128, P, MIS, P, P, NULL) == -3
    assert f(P, 1, 1 << 24, 128, P, P, P, P, NULL) == -7            # M / 128 beyond the grid
    assert f(NULL, 1, 0, 128, NULL, NULL, NULL, NULL, NULL) == 0    # no rows: no-op
    g = L.fp8_quant_act_1x128_128x1_T_grouped
    ld = fb.grouped_ld(300, 2)
    assert g(P, 1, 300, 128, P, 2, ld - 128, P, P, P, P, NULL) == -2  # ld too small for the padding
    assert g(P, 1, 300, 100, P, 2, ld, P, P, P, P, NULL) == -2        # C not a multiple of 128
    assert g(P, 1, 300, 128, P, 0, ld, P, P, P, P, NULL) == -2        # rows but no experts
    assert g(P, 1, 300, 128, NULL, 2, ld, P, P, P, P, NULL) == -1
    assert g(P, 1, 300, 128, P, 2, ld, P, NULL, P, P, NULL) == -1
    assert g(P, 1, 300, 128, P + 2, 2, ld, P, P, P, P, NULL) == -3    # offsets not 4-byte aligned
    assert g(P, 1, 300, 128, P, 2, ld, P, P, MIS, P, NULL) == -3
    assert g(NULL, 1, 0, 128, NULL, 2, fb.grouped_ld(0, 2), NULL, NULL, NULL, NULL, NULL) == 0


def test_grouped_backward_validation(L):
    q = L.fp8_quant_act_128x1_T_grouped
    ld = fb.grouped_ld(300, 2)
    assert q(P, 1, 300, 128, P, 2, ld - 128, P, P, NULL) == -2      # ld too small for the padding
    assert q(P, 1, 300, 100, P, 2, ld, P, P, NULL) == -2            # C not a multiple of 128
    assert q(P, 1, 300, 128, P, 0, ld, P, P, NULL) == -2            # rows but no experts
    assert q(P, 3, 300, 128, P, 2, ld, P, P, NULL) == -4
    assert q(P, 1, 300, 128, NULL, 2, ld, P, P, NULL) == -1
    assert q(MIS, 1, 300, 128, P, 2, ld, P, P, NULL) == -3
    assert q(P, 1, 300, 128, P + 2, 2, ld, P, P, NULL) == -3       # offsets not 4-byte aligned
    assert q(NULL, 1, 0, 128, NULL, 2, fb.grouped_ld(0, 2), NULL, NULL, NULL) == 0   # no rows: no-op
    w = L.fp8_grouped_gemm_wgrad
    assert w(P, P, P, P, P, P, 2, 300, 128, 128, ld - 128, NULL) == -2
    assert w(P, P, P, P, P, P, 2, 300, 100, 128, ld, NULL) == -2
    assert w(P, P, P, P, NULL, P, 2, 300, 128, 128, ld, NULL) == -1
    assert w(P, P, P, P, P, P + 2, 2, 300, 128, 128, ld, NULL) == -3  # offsets not 4-byte aligned
    assert w(P, P, P, P, P, P, 2, 300, 1 << 20, 128, 1 << 12, NULL) == -7
    assert w(NULL, NULL, NULL, NULL, NULL, NULL, 0, 0, 128, 128, 0, NULL) == 0
    assert fb.grouped_ld(300, 2) == 640 and fb.grouped_ld(0, 0) == 0


def test_dispatch_validation(L):
    ws = L.fp8_moe_dispatch_workspace_bytes
    assert ws(8192, 8, 32) == 4 * 32 * 64
    assert ws(0, 8, 32) == 0
    assert ws(10, 0, 4) < 0 and ws(10, 65, 4) < 0 and ws(10, 8, 0) < 0 and ws(10, 8, 1025) < 0
    d = L.fp8_moe_dispatch
    assert d(P, 1, 10, 100, P, 2, 4, P, P, P, P, P, P, NULL) == -2  # K not a multiple of 128
    assert d(P, 7, 10, 128, P, 2, 4, P, P, P, P, P, P, NULL) == -4
    assert d(P, 1, 10, 128, P, 2, 4, P, P, NULL, P, P, P, NULL) == -1
    assert d(P, 1, 10, 128, P, 2, 4, P, P, P, P, P, NULL, NULL) == -1
    assert d(MIS, 1, 10, 128, P, 2, 4, P, P, P, P, P, P, NULL) == -3
    assert d(P, 1, 10, 128, P + 2, 2, 4, P, P, P, P, P, P, NULL) == -3   # int32 buffers 4-byte aligned
    c = L.fp8_moe_combine
    assert c(P, P, P, 10, 2, 12, P, NULL) == -2                      # N not a multiple of 8
    assert c(P, P, P, 10, 0, 16, P, NULL) == -2
    assert c(MIS, P, P, 10, 2, 16, P, NULL) == -3
    assert c(P, NULL, P, 10, 2, 16, P, NULL) == -1
    assert c(NULL, NULL, NULL, 0, 2, 16, NULL, NULL) == 0


def test_binding_requires_gpu_tensors(L):
    import torch
    x = torch.zeros(4, 128)
    with pytest.raises(ValueError):
        fb.fp8_quant_act_1x128(x)


def test_binding_rejects_wrong_output_shapes(L):
    # the output's shape is checked before anything else touches it, so a
    # caller-supplied buffer too small for the result is never written
    import torch
    u8, f32, bf16 = torch.uint8, torch.float32, torch.bfloat16
    A = torch.zeros((300, 256), dtype=u8)
    sA = torch.ones((2, 300), dtype=f32)
    B = torch.zeros((4, 384, 256), dtype=u8)
    sB = torch.ones((4, 3, 2), dtype=f32)
    off = torch.tensor([0, 100, 100, 250, 300], dtype=torch.int32)
    for bad in ((299, 384), (300, 256), (384, 300)):
        with pytest.raises(ValueError, match="out has the wrong shape"):
            fb.fp8_grouped_gemm_blockscaled(A, sA, B, sB, off, out=torch.empty(bad, dtype=bf16))
    with pytest.raises(ValueError, match="out has the wrong shape"):
        fb.fp8_gemm_blockscaled(A, sA, B[0], sB[0], out=torch.empty((300, 256), dtype=bf16))
    qa, sqa = torch.zeros((384, 512), dtype=u8), torch.ones((4, 384), dtype=f32)
    qb, sqb = torch.zeros((256, 512), dtype=u8), torch.ones((4, 256), dtype=f32)
    with pytest.raises(ValueError, match="out has the wrong shape"):
        fb.fp8_grouped_gemm_wgrad(qa, sqa, qb, sqb, off, 300, out=torch.empty((4, 384, 128), dtype=bf16))


def test_tile_query_validation(L):
    import ctypes
    bm, bn, d, t = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    q = L.fp8_gemm_blockscaled_tile
    outs = (ctypes.byref(bm), ctypes.byref(bn), ctypes.byref(d), ctypes.byref(t))
    assert q(4096, 7168, 7168, 2, *outs) == -5
    assert q(4096, 7100, 7168, 0, *outs) == -2
    assert q(4096, 7168, 7100, 1, *outs) == -2
    assert q(4096, 7168, 7168, 0, None, ctypes.byref(bn), ctypes.byref(d), ctypes.byref(t)) == -1
    assert q(4096, 7168, 7168, 0, ctypes.byref(bm), ctypes.byref(bn), None, None) == 0   # depth, tail optional
    assert (bm.value, bn.value) == (256, 224)


def test_noalloc_dispatch_validation(L):
    # rejected on the host, before any device call: invalid sizes, and a
    # routing workspace beyond the library's 1 MiB scratch array
    d = L.fp8_moe_dispatch_noalloc
    assert d(P, 1, 16, 128, P, 0, 8, P, P, P, P, P, NULL) == -2                  # topk < 1
    assert d(P, 1, 16, 100, P, 2, 8, P, P, P, P, P, NULL) == -2                  # K % 128
    assert d(P, 3, 16, 128, P, 2, 8, P, P, P, P, P, NULL) == -4
    assert d(P, 1, 16, 128, P, 2, 8, P, P, NULL, P, P, NULL) == -1
    assert d(MIS, 1, 16, 128, P, 2, 8, P, P, P, P, P, NULL) == -3
    # E * ceil(T*topk/1024) * 4 bytes: 1024 experts x 257 blocks > 2^20
    assert d(P, 1, 257 * 128, 128, P, 8, 1024, P, P, P, P, P, NULL) == -8
    assert fb.status_string(-8).startswith("the problem needs more scratch memory")


def test_tile_query_follows_the_shape(L):
    # host-side choice, no device needed (a 256-CU MI355X is assumed when no
    # device answers): skinny problems take the small tiles that spread them
    # over every CU, full-size layers the large ones
    import ctypes
    bm, bn, d, t = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()

    def tile(M, N, K):
        assert L.fp8_gemm_blockscaled_tile(M, N, K, 0, ctypes.byref(bm), ctypes.byref(bn), ctypes.byref(d),
                                           ctypes.byref(t)) == 0
        return bm.value, bn.value, d.value, t.value

    # a few tokens: 112 tiles of 256 rows would idle 144 CUs; one small tile
    # per CU, alone there, with its loads two chunks ahead
    assert tile(64, 7168, 7168) == (64, 64, 4, 0)
    assert tile(512, 7168, 7168) == (128, 128, 4, 0)
    assert tile(1024, 7168, 7168) == (128, 256, 2, 0)
    assert tile(4096, 2048, 7168) == (128, 256, 2, 0)
    assert tile(4096, 7168, 7168) == (256, 224, 3, 0)     # 512 tiles: two full rounds
    assert tile(4096, 4096, 4096) == (256, 256, 2, 0)
    assert tile(7168, 4096, 4096) == (224, 256, 3, 0)
    assert tile(1, 128, 128) == (64, 64, 4, 0)
    # 784 tiles of 256x256: three rounds, and the 16 left as 256 subtiles of 64x64
    assert tile(7168, 7168, 4096) == (256, 256, 2, 16)
    assert tile(5120, 7168, 7168) == (256, 256, 2, 48)
