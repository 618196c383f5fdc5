"""ctypes binding of libfp8bs.so: argument marshalling only.

Every function here has the name of the C entry point it calls. It checks the
torch tensors it is given (device, dtype, contiguity), allocates the outputs
with torch on the input's device, and calls the library on the current torch
stream. All arithmetic happens in the HIP kernels; there is no fallback: if the
library is missing or a call fails, an exception is raised.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8bs.so")

F32, BF16 = 0, 1
SCALE_BLOCK128, SCALE_ROW = 0, 1
ABI_VERSION = 11

_c_int64 = ctypes.c_int64
_vp = ctypes.c_void_p

_SIGNATURES = {
    "fp8_quant_act_1x128": [_vp, ctypes.c_int, _c_int64, _c_int64, _vp, _vp, _vp],
    "fp8_quant_w_128x128": [_vp, ctypes.c_int, _c_int64, _c_int64, _vp, _vp, _vp, _vp, _vp],
    "fp8_quant_act_128x1_T": [_vp, ctypes.c_int, _c_int64, _c_int64, _vp, _vp, _vp],
    "fp8_gemm_blockscaled": [_vp, _vp, _vp, _vp, ctypes.c_int, _vp, _c_int64, _c_int64, _c_int64, _vp],
    "fp8_gemm_blockscaled_tile": [_c_int64, _c_int64, _c_int64, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                  ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                  ctypes.POINTER(ctypes.c_int)],
    "fp8_quant_act_1x128_pow2": [_vp, ctypes.c_int, _c_int64, _c_int64, _vp, _vp, _vp],
    "fp8_quant_w_128x128_pow2": [_vp, ctypes.c_int, _c_int64, _c_int64, _vp, _vp, _vp, _vp, _vp],
    "fp8_quant_act_128x1_T_pow2": [_vp, ctypes.c_int, _c_int64, _c_int64, _vp, _vp, _vp],
    "fp8_gemm_blockscaled_pow2": [_vp, _vp, _vp, _vp, ctypes.c_int, _vp, _c_int64, _c_int64, _c_int64, _vp],
    "fp8_gemm_blockscaled_q1x128": [_vp, _vp, _vp, _vp, ctypes.c_int, _vp, _vp, _c_int64, _c_int64,
                                    _c_int64, _vp],
    "fp8_gemm_blockscaled_q1x128_q128x1T": [_vp, _vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, _vp, _c_int64,
                                            _c_int64, _c_int64, _vp],
    "fp8_grouped_gemm_blockscaled": [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _c_int64, _c_int64,
                                     _c_int64, _vp],
    "fp8_quant_act_128x1_T_grouped": [_vp, ctypes.c_int, _c_int64, _c_int64, _vp, ctypes.c_int, _c_int64, _vp,
                                      _vp, _vp],
    "fp8_quant_act_1x128_128x1_T": [_vp, ctypes.c_int, _c_int64, _c_int64, _vp, _vp, _vp, _vp, _vp],
    "fp8_quant_act_1x128_128x1_T_grouped": [_vp, ctypes.c_int, _c_int64, _c_int64, _vp, ctypes.c_int, _c_int64,
                                            _vp, _vp, _vp, _vp, _vp],
    "fp8_grouped_gemm_wgrad": [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _c_int64, _c_int64, _c_int64,
                               _c_int64, _vp],
    "fp8_moe_dispatch": [_vp, ctypes.c_int, _c_int64, _c_int64, _vp, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp,
                         _vp, _vp, _vp, _vp],
    "fp8_moe_dispatch_workspace_bytes": [_c_int64, ctypes.c_int, ctypes.c_int],
    "fp8_moe_dispatch_noalloc": [_vp, ctypes.c_int, _c_int64, _c_int64, _vp, ctypes.c_int, ctypes.c_int, _vp, _vp,
                                 _vp, _vp, _vp, _vp],
    "fp8_moe_combine": [_vp, _vp, _vp, _c_int64, ctypes.c_int, _c_int64, _vp, _vp],
    "fp8bs_status_string": [ctypes.c_int],
    "fp8bs_abi_version": [],
}

_lib = None


class Fp8bsError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")
        self.status = status


def lib():
    """The loaded library (loaded on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m fp8_block_scaled_x1_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = {"fp8bs_status_string": ctypes.c_char_p,
                          "fp8_moe_dispatch_workspace_bytes": ctypes.c_int64}.get(name, ctypes.c_int)
        if handle.fp8bs_abi_version() != ABI_VERSION:
            raise ImportError(f"libfp8bs ABI {handle.fp8bs_abi_version()} != {ABI_VERSION}")
        _lib = handle
    return _lib


def status_string(status):
    return lib().fp8bs_status_string(int(status)).decode()


def _check(fn, status):
    if status != 0:
        raise Fp8bsError(fn, status)


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t, name, dtypes):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _in_dtype(x):
    return {torch.float32: F32, torch.bfloat16: BF16}[x.dtype]


def fp8_quant_act_1x128(x, pow2=False):
    """x[M][K] f32|bf16 -> (q uint8 [M][K], s float32 [K/128][M]).

    pow2: power-of-two scales (the E8M0-compatible variant)."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    M, K = x.shape
    px = _dev(x, "x", (torch.float32, torch.bfloat16))
    q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    s = torch.empty((K // 128 if K % 128 == 0 else 0, M), dtype=torch.float32, device=x.device)
    fn = "fp8_quant_act_1x128_pow2" if pow2 else "fp8_quant_act_1x128"
    _check(fn, getattr(lib(), fn)(px, _in_dtype(x), M, K, q.data_ptr(), s.data_ptr(), _stream(x)))
    return q, s


def fp8_quant_w_128x128(w, transposed=False, pow2=False):
    """w[N][K] -> (q[N][K], s[N/128][K/128]) and, if transposed, (qT[K][N], sT[K/128][N/128])."""
    if w.dim() != 2:
        raise ValueError("w must be 2-D")
    N, K = w.shape
    pw = _dev(w, "w", (torch.float32, torch.bfloat16))
    q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    s = torch.empty((N // 128, K // 128), dtype=torch.float32, device=w.device)
    qT = sT = None
    if transposed:
        qT = torch.empty((K, N), dtype=torch.uint8, device=w.device)
        sT = torch.empty((K // 128, N // 128), dtype=torch.float32, device=w.device)
    fn = "fp8_quant_w_128x128_pow2" if pow2 else "fp8_quant_w_128x128"
    _check(fn, getattr(lib(), fn)(pw, _in_dtype(w), N, K, q.data_ptr(), s.data_ptr(),
                                  qT.data_ptr() if qT is not None else None,
                                  sT.data_ptr() if sT is not None else None, _stream(w)))
    return (q, s, qT, sT) if transposed else (q, s)


def fp8_quant_act_128x1_T(x, pow2=False):
    """x[M][C] -> (qT uint8 [C][M], sT float32 [M/128][C]); M a multiple of 128."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    M, C = x.shape
    px = _dev(x, "x", (torch.float32, torch.bfloat16))
    qT = torch.empty((C, M), dtype=torch.uint8, device=x.device)
    sT = torch.empty((M // 128, C), dtype=torch.float32, device=x.device)
    fn = "fp8_quant_act_128x1_T_pow2" if pow2 else "fp8_quant_act_128x1_T"
    _check(fn, getattr(lib(), fn)(px, _in_dtype(x), M, C, qT.data_ptr(), sT.data_ptr(), _stream(x)))
    return qT, sT


def fp8_quant_act_1x128_128x1_T(x):
    """x[M][C] -> (q [M][C], s [C/128][M], qT [C][M], sT [M/128][C]): the 1x128
    and the transposed 128x1 quantization in one pass; M, C multiples of 128."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    M, C = x.shape
    px = _dev(x, "x", (torch.float32, torch.bfloat16))
    dev = x.device
    q = torch.empty((M, C), dtype=torch.uint8, device=dev)
    s = torch.empty((C // 128, M), dtype=torch.float32, device=dev)
    qT = torch.empty((C, M), dtype=torch.uint8, device=dev)
    sT = torch.empty((M // 128, C), dtype=torch.float32, device=dev)
    _check("fp8_quant_act_1x128_128x1_T",
           lib().fp8_quant_act_1x128_128x1_T(px, _in_dtype(x), M, C, q.data_ptr(), s.data_ptr(), qT.data_ptr(),
                                             sT.data_ptr(), _stream(x)))
    return q, s, qT, sT


def _gemm_operands(A, sA, B, sB, b_scale_mode):
    """(M, N, K, pointers) of a dense GEMM's operands after the shape checks."""
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError("A and B disagree on K")
    if b_scale_mode == SCALE_BLOCK128:
        exp_sb = (N // 128, K // 128)
    elif b_scale_mode == SCALE_ROW:
        exp_sb = (K // 128, N)
    else:
        raise ValueError("unknown b_scale_mode")
    if tuple(sA.shape) != (K // 128, M) or tuple(sB.shape) != exp_sb:
        raise ValueError(f"scale grids {tuple(sA.shape)}, {tuple(sB.shape)} do not match the operands")
    ptrs = (_dev(A, "A", (torch.uint8,)), _dev(sA, "sA", (torch.float32,)),
            _dev(B, "B", (torch.uint8,)), _dev(sB, "sB", (torch.float32,)))
    return M, N, K, ptrs


def fp8_gemm_blockscaled(A, sA, B, sB, b_scale_mode=SCALE_BLOCK128, out=None, pow2=False):
    """C[M][N] (bf16) = block-scaled FP8 GEMM of A[M][K] and B[N][K] (both K-contiguous).

    pow2: the scales are powers of two and the MFMA applies them (E8M0)."""
    if out is not None and tuple(out.shape) != (A.shape[0], B.shape[0]):
        raise ValueError("out has the wrong shape")
    M, N, K, (pa, psa, pb, psb) = _gemm_operands(A, sA, B, sB, b_scale_mode)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    pc = _dev(out, "out", (torch.bfloat16,))
    fn = "fp8_gemm_blockscaled_pow2" if pow2 else "fp8_gemm_blockscaled"
    _check(fn, getattr(lib(), fn)(pa, psa, pb, psb, int(b_scale_mode), pc, M, N, K, _stream(A)))
    return out


def fp8_gemm_blockscaled_tile(M, N, K, b_scale_mode=SCALE_BLOCK128):
    """(rows, columns, ring depth, tail tiles) of the kernel fp8_gemm_blockscaled uses for this shape."""
    bm, bn, depth, tail = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check("fp8_gemm_blockscaled_tile",
           lib().fp8_gemm_blockscaled_tile(M, N, K, int(b_scale_mode), ctypes.byref(bm), ctypes.byref(bn),
                                           ctypes.byref(depth), ctypes.byref(tail)))
    return bm.value, bn.value, depth.value, tail.value


def fp8_gemm_blockscaled_q1x128(A, sA, B, sB, b_scale_mode=SCALE_BLOCK128):
    """The GEMM's BF16 result quantized 1x128: (Q uint8 [M][N], sQ float32 [N/128][M])."""
    M, N, K, (pa, psa, pb, psb) = _gemm_operands(A, sA, B, sB, b_scale_mode)
    Q = torch.empty((M, N), dtype=torch.uint8, device=A.device)
    sQ = torch.empty((N // 128, M), dtype=torch.float32, device=A.device)
    _check("fp8_gemm_blockscaled_q1x128",
           lib().fp8_gemm_blockscaled_q1x128(pa, psa, pb, psb, int(b_scale_mode), Q.data_ptr(),
                                             sQ.data_ptr(), M, N, K, _stream(A)))
    return Q, sQ


def fp8_gemm_blockscaled_q1x128_q128x1T(A, sA, B, sB, b_scale_mode=SCALE_BLOCK128):
    """The GEMM's BF16 result quantized both ways: (Q [M][N], sQ [N/128][M]) 1x128 and
    (QT [N][M], sQT [M/128][N]) 128x1 transposed; M a multiple of 128."""
    M, N, K, (pa, psa, pb, psb) = _gemm_operands(A, sA, B, sB, b_scale_mode)
    dev = A.device
    Q = torch.empty((M, N), dtype=torch.uint8, device=dev)
    sQ = torch.empty((N // 128, M), dtype=torch.float32, device=dev)
    QT = torch.empty((N, M), dtype=torch.uint8, device=dev)
    sQT = torch.empty((M // 128, N), dtype=torch.float32, device=dev)
    _check("fp8_gemm_blockscaled_q1x128_q128x1T",
           lib().fp8_gemm_blockscaled_q1x128_q128x1T(pa, psa, pb, psb, int(b_scale_mode), Q.data_ptr(),
                                                     sQ.data_ptr(), QT.data_ptr(), sQT.data_ptr(), M, N, K,
                                                     _stream(A)))
    return Q, sQ, QT, sQT


def fp8_grouped_gemm_blockscaled(A, sA, B, sB, group_offsets, out=None):
    """Per-expert GEMM: rows [off[e], off[e+1]) of A times B[e]; offsets int32 on the GPU."""
    M_total, K = A.shape
    E, N, Kb = B.shape
    if Kb != K:
        raise ValueError("A and B disagree on K")
    if tuple(sA.shape) != (K // 128, M_total) or tuple(sB.shape) != (E, N // 128, K // 128):
        raise ValueError("scale grids do not match the operands")
    if tuple(group_offsets.shape) != (E + 1,):
        raise ValueError("group_offsets must have E+1 entries")
    if out is not None and tuple(out.shape) != (M_total, N):
        raise ValueError("out has the wrong shape")
    pa = _dev(A, "A", (torch.uint8,))
    psa = _dev(sA, "sA", (torch.float32,))
    pb = _dev(B, "B", (torch.uint8,))
    psb = _dev(sB, "sB", (torch.float32,))
    po = _dev(group_offsets, "group_offsets", (torch.int32,))
    if out is None:
        out = torch.empty((M_total, N), dtype=torch.bfloat16, device=A.device)
    pc = _dev(out, "out", (torch.bfloat16,))
    _check("fp8_grouped_gemm_blockscaled",
           lib().fp8_grouped_gemm_blockscaled(pa, psa, pb, psb, pc, po, E, M_total, N, K, _stream(A)))
    return out


def grouped_ld(M_total, E):
    """Smallest valid row length of the grouped 128x1 transposed codes:
    room for M_total tokens plus every expert's padding, in whole groups."""
    return 128 * ((M_total + 127 * E + 127) // 128)


def fp8_quant_act_128x1_T_grouped(x, group_offsets, ld=None):
    """x[M_total][C] rows grouped by expert -> (qT uint8 [C][ld], sT float32 [ld/128][C]).

    Expert e's tokens are cut into groups of 128 from its first row (the last
    one zero-padded); groups are numbered expert-major. Columns and scale rows
    past the last group are left as allocated (uninitialized).
    """
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    M, C = x.shape
    E = group_offsets.shape[0] - 1
    if E < 0:
        raise ValueError("group_offsets must have E+1 entries")
    ld = grouped_ld(M, E) if ld is None else int(ld)
    px = _dev(x, "x", (torch.float32, torch.bfloat16))
    po = _dev(group_offsets, "group_offsets", (torch.int32,))
    qT = torch.empty((C, ld), dtype=torch.uint8, device=x.device)
    sT = torch.empty((ld // 128, C), dtype=torch.float32, device=x.device)
    _check("fp8_quant_act_128x1_T_grouped",
           lib().fp8_quant_act_128x1_T_grouped(px, _in_dtype(x), M, C, po, E, ld, qT.data_ptr(), sT.data_ptr(),
                                               _stream(x)))
    return qT, sT


def fp8_quant_act_1x128_128x1_T_grouped(x, group_offsets, ld=None):
    """x[M_total][C] rows grouped by expert -> (q [M_total][C], s [C/128][M_total],
    qT [C][ld], sT [ld/128][C]): fp8_quant_act_1x128 and
    fp8_quant_act_128x1_T_grouped in one pass."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    M, C = x.shape
    E = group_offsets.shape[0] - 1
    if E < 0:
        raise ValueError("group_offsets must have E+1 entries")
    ld = grouped_ld(M, E) if ld is None else int(ld)
    px = _dev(x, "x", (torch.float32, torch.bfloat16))
    po = _dev(group_offsets, "group_offsets", (torch.int32,))
    dev = x.device
    q = torch.empty((M, C), dtype=torch.uint8, device=dev)
    s = torch.empty((C // 128, M), dtype=torch.float32, device=dev)
    qT = torch.empty((C, ld), dtype=torch.uint8, device=dev)
    sT = torch.empty((ld // 128, C), dtype=torch.float32, device=dev)
    _check("fp8_quant_act_1x128_128x1_T_grouped",
           lib().fp8_quant_act_1x128_128x1_T_grouped(px, _in_dtype(x), M, C, po, E, ld, q.data_ptr(), s.data_ptr(),
                                                     qT.data_ptr(), sT.data_ptr(), _stream(x)))
    return q, s, qT, sT


def fp8_grouped_gemm_wgrad(A, sA, B, sB, group_offsets, M_total, out=None):
    """Per-expert Wgrad: C[e] = dY_e^T X_e from the grouped 128x1 transposed
    quantizations A = qT(dY) [N][ld], B = qT(X) [K][ld]; returns bf16 [E][N][K]."""
    N, ld = A.shape
    K, ldb = B.shape
    E = group_offsets.shape[0] - 1
    if ldb != ld:
        raise ValueError("A and B disagree on the token length")
    if tuple(sA.shape) != (ld // 128, N) or tuple(sB.shape) != (ld // 128, K):
        raise ValueError("scale grids do not match the operands")
    if out is not None and tuple(out.shape) != (E, N, K):
        raise ValueError("out has the wrong shape")
    pa = _dev(A, "A", (torch.uint8,))
    psa = _dev(sA, "sA", (torch.float32,))
    pb = _dev(B, "B", (torch.uint8,))
    psb = _dev(sB, "sB", (torch.float32,))
    po = _dev(group_offsets, "group_offsets", (torch.int32,))
    if out is None:
        out = torch.empty((E, N, K), dtype=torch.bfloat16, device=A.device)
    pc = _dev(out, "out", (torch.bfloat16,))
    _check("fp8_grouped_gemm_wgrad",
           lib().fp8_grouped_gemm_wgrad(pa, psa, pb, psb, pc, po, E, int(M_total), N, K, ld, _stream(A)))
    return out


def fp8_moe_dispatch(x, topk_ids, E):
    """Route token copies to experts and quantize the payload 1x128.

    x[T][K] f32|bf16, topk_ids[T][topk] int32 (GPU) -> (q uint8 [T*topk][K],
    s float32 [K/128][T*topk], offsets int32 [E+1], pos int32 [T][topk],
    src_row int32 [T*topk]); rows sorted by expert, then token, then slot.
    """
    if x.dim() != 2 or topk_ids.dim() != 2 or topk_ids.shape[0] != x.shape[0]:
        raise ValueError("x must be [T][K] and topk_ids [T][topk]")
    T, K = x.shape
    topk = topk_ids.shape[1]
    px = _dev(x, "x", (torch.float32, torch.bfloat16))
    pid = _dev(topk_ids, "topk_ids", (torch.int32,))
    L = lib()
    ws_bytes = L.fp8_moe_dispatch_workspace_bytes(T, topk, E)
    _check("fp8_moe_dispatch_workspace_bytes", min(0, ws_bytes))
    dev = x.device
    ws = torch.empty(max(ws_bytes // 4, 1), dtype=torch.int32, device=dev)
    q = torch.empty((T * topk, K), dtype=torch.uint8, device=dev)
    s = torch.empty((K // 128 if K % 128 == 0 else 0, T * topk), dtype=torch.float32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    pos = torch.empty((T, topk), dtype=torch.int32, device=dev)
    src = torch.empty(T * topk, dtype=torch.int32, device=dev)
    _check("fp8_moe_dispatch",
           L.fp8_moe_dispatch(px, _in_dtype(x), T, K, pid, topk, E, q.data_ptr(), s.data_ptr(), offsets.data_ptr(),
                              pos.data_ptr(), src.data_ptr(), ws.data_ptr(), _stream(x)))
    return q, s, offsets, pos, src


def fp8_moe_dispatch_noalloc(x, topk_ids, E, q, s, offsets, pos, src_row):
    """fp8_moe_dispatch into caller-provided outputs, with no allocation at all:
    the routing workspace is the library's own device array (1 MiB per GPU).
    Shapes as fp8_moe_dispatch returns them; returns the outputs."""
    if x.dim() != 2 or topk_ids.dim() != 2 or topk_ids.shape[0] != x.shape[0]:
        raise ValueError("x must be [T][K] and topk_ids [T][topk]")
    T, K = x.shape
    topk = topk_ids.shape[1]
    P = T * topk
    want = {"q": (P, K), "s": (K // 128 if K % 128 == 0 else 0, P), "offsets": (E + 1,), "pos": (T, topk),
            "src_row": (P,)}
    for name, t in (("q", q), ("s", s), ("offsets", offsets), ("pos", pos), ("src_row", src_row)):
        if tuple(t.shape) != want[name]:
            raise ValueError(f"{name} has the wrong shape")
    args = (_dev(x, "x", (torch.float32, torch.bfloat16)), _in_dtype(x), T, K, _dev(topk_ids, "topk_ids", (torch.int32,)),
            topk, E, _dev(q, "q", (torch.uint8,)), _dev(s, "s", (torch.float32,)),
            _dev(offsets, "offsets", (torch.int32,)), _dev(pos, "pos", (torch.int32,)),
            _dev(src_row, "src_row", (torch.int32,)), _stream(x))
    _check("fp8_moe_dispatch_noalloc", lib().fp8_moe_dispatch_noalloc(*args))
    return q, s, offsets, pos, src_row


def fp8_moe_combine(Y, pos, w):
    """out[T][N] bf16 = sum over slots j of w[t][j] * Y[pos[t][j]] (FP32 sums in slot order)."""
    T, topk = pos.shape
    N = Y.shape[1]
    if tuple(w.shape) != (T, topk) or Y.shape[0] != T * topk:
        raise ValueError("Y, pos and w disagree")
    py = _dev(Y, "Y", (torch.bfloat16,))
    pp = _dev(pos, "pos", (torch.int32,))
    pw = _dev(w, "w", (torch.float32,))
    out = torch.empty((T, N), dtype=torch.bfloat16, device=Y.device)
    _check("fp8_moe_combine", lib().fp8_moe_combine(py, pp, pw, T, topk, N, out.data_ptr(), _stream(Y)))
    return out
