"""MI355X (gfx950) FP8 GEMM with fine-grained block scaling: Python binding of libfp8gemm.so.

Argument marshalling only -- every step of the computation runs in the HIP kernels behind the
C ABI declared in include/fp8gemm.h.  torch supplies device memory and the current stream.

    D = gemm_nt(A, sa, B, sb)                              # dense NT, bf16 out
    D = gemm_nt_specialized(A, sa, B, sb)                  # the same, kernel built at run time for N, K
    D = grouped_contiguous(A, sa, B, sb, m_indices)        # MoE, groups concatenated along M
    D = grouped_masked(A, sa, B, sb, masked_m, expected_m) # MoE, fixed per-group capacity
    D = fp8fp4_grouped_masked(A, sa, B4, sb4, masked_m, expected_m)  # the same, B in E2M1 + E8M0
    A, sa = quantize_1x128(X)                              # bf16 activations -> codes + scales
    A, sa = quantize_1x128_masked(X, masked_m)             # the same, masked layout
    H, sh = swiglu_quantize_1x128(Y)                       # silu(gate) * up -> codes + scales
    out = moe_expert_masked(A, sa, W1, s1, W2, s2, masked_m, expected_m)  # one MoE expert layer

A and B are E4M3 codes (torch.float8_e4m3fn or uint8), sa one fp32 scale per 1x128 block of a
row of A stored K-block-major (sa[kb, m], shape [K/128, M]), sb one per 128x128 block of B (page "DeepSeek開源第三彈：V3/R1訓練推理關鍵秘籍，核心代碼僅
300行", sections 深入了解DeepGEMM and 如何使用？).  There is no CPU fallback: without the built
library every call raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["gemm_nt", "gemm_nt_noalloc", "gemm_nt_specialized", "specialize_nt", "specialized_code_object", "specialized_count",
           "grouped_contiguous", "grouped_masked", "quantize_1x128",
           "quantize_1x128_masked", "fp8fp4_grouped_masked", "swiglu_quantize_1x128", "swiglu_quantize_1x128_masked",
           "moe_expert_masked", "init", "prepare_stream", "set_num_cus",
           "last_config", "read_device_error", "status_string", "lib", "library_path",
           "Fp8GemmError", "STATUS", "DEVERR_BAD_INDEX", "DEVERR_BAD_COUNT"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libfp8gemm.so")
_lib = None

STATUS = {0: "FP8GEMM_OK", 1: "FP8GEMM_ERR_NULL_PTR", 2: "FP8GEMM_ERR_BAD_SHAPE",
          3: "FP8GEMM_ERR_MISALIGNED", 4: "FP8GEMM_ERR_UNSUPPORTED", 5: "FP8GEMM_ERR_LAUNCH",
          6: "FP8GEMM_ERR_HIP"}
DEVERR_BAD_INDEX = 1
DEVERR_BAD_COUNT = 2

#: exported C symbols and their ctypes signatures (restype, argtypes)
_P, _I64, _I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
SIGNATURES = {
    "fp8gemm_nt": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P]),
    "fp8gemm_nt_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P]),
    "fp8gemm_nt_specialized": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P]),
    "fp8gemm_specialize_nt": (ctypes.c_int, [_I64, _I64, _I64, ctypes.POINTER(ctypes.c_double)]),
    "fp8gemm_specialized_code_object": (ctypes.c_int, [ctypes.c_int] * 6 + [_I64, _I64, _P,
                                                       ctypes.POINTER(ctypes.c_size_t), ctypes.c_char_p,
                                                       ctypes.c_int]),
    "fp8gemm_specialized_count": (ctypes.c_int, []),
    "fp8gemm_grouped_contiguous": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _P]),
    "fp8gemm_grouped_masked": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _I64, _P]),
    "fp8gemm_quantize_1x128": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P]),
    "fp8gemm_quantize_1x128_masked": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I64, _I64, _P]),
    "fp8gemm_fp8fp4_grouped_masked": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _I64, _P]),
    "fp8gemm_swiglu_quantize_1x128": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P]),
    "fp8gemm_swiglu_quantize_1x128_masked": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I64, _I64, _P]),
    "fp8gemm_moe_expert_masked": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                                 _I32, _I64, _I64, _I64, _I64, _P]),
    "fp8gemm_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fp8gemm_init": (ctypes.c_int, []),
    "fp8gemm_prepare_stream": (ctypes.c_int, [_P]),
    "fp8gemm_set_num_cus": (ctypes.c_int, [ctypes.c_int]),
    "fp8gemm_last_config": (ctypes.c_int, [ctypes.c_char_p, ctypes.c_int]),
    "fp8gemm_read_device_error": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_int32)]),
}


class Fp8GemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (%s)" % (where, status_string(status), STATUS.get(status, status)))


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libfp8gemm.so is not built (python -m fp8_block_scaled_x128_amd.build)")
        l = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def status_string(status: int) -> str:
    return lib().fp8gemm_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise Fp8GemmError(status, where)


def init() -> None:
    _check(lib().fp8gemm_init(), "fp8gemm_init")


def prepare_stream(stream=None) -> None:
    """Create the split-K workspace of `stream` (default: torch's current stream) now, so that
    later calls on it -- HIP graph capture included -- allocate nothing."""
    torch = _torch()
    _check(lib().fp8gemm_prepare_stream(_stream(stream, torch.cuda.current_device())), "fp8gemm_prepare_stream")


def set_num_cus(n: int) -> None:
    _check(lib().fp8gemm_set_num_cus(int(n)), "fp8gemm_set_num_cus")


def last_config() -> str:
    buf = ctypes.create_string_buffer(256)
    _check(lib().fp8gemm_last_config(buf, 256), "fp8gemm_last_config")
    return buf.value.decode()


# ---- tensor front end -------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def read_device_error(stream=None) -> int:
    """Synchronise the stream and return (and clear) the device error word."""
    torch = _torch()
    dev = torch.cuda.current_device()
    v = ctypes.c_int32(0)
    _check(lib().fp8gemm_read_device_error(_stream(stream, dev), ctypes.byref(v)),
           "fp8gemm_read_device_error")
    return v.value


def _codes(t, name):
    torch = _torch()
    if t.dtype not in (torch.float8_e4m3fn, torch.uint8):
        raise TypeError("%s must be float8_e4m3fn or uint8 codes, got %s" % (name, t.dtype))
    return _dev_contig(t, name)


def _dev_contig(t, name):
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _f32(t, name):
    torch = _torch()
    if t.dtype != torch.float32:
        raise TypeError("%s must be float32, got %s" % (name, t.dtype))
    return _dev_contig(t, name)


def _i32(t, name):
    torch = _torch()
    if t.dtype != torch.int32:
        raise TypeError("%s must be int32, got %s" % (name, t.dtype))
    return _dev_contig(t, name)


def _out(out, shape, device):
    torch = _torch()
    if out is None:
        return torch.empty(shape, dtype=torch.bfloat16, device=device)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != tuple(shape):
        raise ValueError("out must be bfloat16 of shape %s" % (tuple(shape),))
    return _dev_contig(out, "out")


def _shape_check(cond, msg):
    if not cond:
        raise ValueError(msg)


def gemm_nt(A, sa, B, sb, out=None, stream=None):
    """D[M,N] (bf16) = A[M,K] . B[N,K]^T with sa [K/128, M] and sb [ceil(N/128), K/128]."""
    return _dense("fp8gemm_nt", A, sa, B, sb, out, stream)


def gemm_nt_noalloc(A, sa, B, sb, out=None, stream=None):
    """gemm_nt with its split-K partials in the library's static device scratch: the library
    allocates nothing (pass `out`, so that this wrapper does not allocate either).  Calls that
    overlap in time on one GPU race on the scratch."""
    return _dense("fp8gemm_nt_noalloc", A, sa, B, sb, out, stream)


def gemm_nt_specialized(A, sa, B, sb, out=None, stream=None):
    """gemm_nt with the tiled kernel compiled at run time for this N and K (cached per device);
    the same results, bit for bit."""
    return _dense("fp8gemm_nt_specialized", A, sa, B, sb, out, stream)


def specialize_nt(M: int, N: int, K: int) -> float:
    """Build (or find cached) the kernel gemm_nt_specialized runs for (M, N, K) on the current
    device; returns the compile + load time in ms (0.0 when it was cached)."""
    ms = ctypes.c_double(0.0)
    _check(lib().fp8gemm_specialize_nt(int(M), int(N), int(K), ctypes.byref(ms)), "fp8gemm_specialize_nt")
    return ms.value


def specialized_code_object(layout: int, bm: int, bn: int, waves_m: int, waves_n: int, stages: int,
                            N: int, K: int):
    """(code object bytes, kernel symbol) of a tiled table entry specialised to (N, K); no GPU."""
    size = ctypes.c_size_t(0)
    log = ctypes.create_string_buffer(65536)
    args = [int(layout), int(bm), int(bn), int(waves_m), int(waves_n), int(stages), int(N), int(K)]
    _check(lib().fp8gemm_specialized_code_object(*args, None, ctypes.byref(size), log, len(log)),
           "fp8gemm_specialized_code_object: " + log.value.decode(errors="replace")[:2000])
    buf = ctypes.create_string_buffer(size.value)
    _check(lib().fp8gemm_specialized_code_object(*args, buf, ctypes.byref(size), log, len(log)),
           "fp8gemm_specialized_code_object")
    return buf.raw[:size.value], log.value.decode()


def specialized_count() -> int:
    """Number of run-time specialised kernels cached in this process."""
    return int(lib().fp8gemm_specialized_count())


def _dense(fn, A, sa, B, sb, out, stream):
    torch = _torch()
    A, B = _codes(A, "A"), _codes(B, "B")
    sa, sb = _f32(sa, "sa"), _f32(sb, "sb")
    _shape_check(A.dim() == 2 and B.dim() == 2 and A.shape[1] == B.shape[1], "A [M,K] and B [N,K]")
    M, K = A.shape
    N = B.shape[0]
    _shape_check(tuple(sa.shape) == (K // 128, M) and tuple(sb.shape) == ((N + 127) // 128, K // 128),
                 "sa [K/128,M], sb [ceil(N/128),K/128]")
    D = _out(out, (M, N), A.device)
    with torch.cuda.device(A.device):
        st = getattr(lib(), fn)(A.data_ptr(), sa.data_ptr(), B.data_ptr(), sb.data_ptr(), D.data_ptr(),
                                M, N, K, _stream(stream, A.device))
    _check(st, fn)
    return D


def grouped_contiguous(A, sa, B, sb, m_indices, out=None, stream=None):
    """MoE contiguous layout: A [M_total,K], sa [K/128,M_total], B [G,N,K], m_indices int32 [M_total]
    (-1 = padding).
    Padding rows of ``out`` are left untouched (zeros when ``out`` is allocated here)."""
    torch = _torch()
    A, B = _codes(A, "A"), _codes(B, "B")
    sa, sb = _f32(sa, "sa"), _f32(sb, "sb")
    m_indices = _i32(m_indices, "m_indices")
    _shape_check(A.dim() == 2 and B.dim() == 3 and A.shape[1] == B.shape[2], "A [M,K] and B [G,N,K]")
    M, K = A.shape
    G, N = B.shape[0], B.shape[1]
    _shape_check(tuple(sa.shape) == (K // 128, M) and tuple(sb.shape) == (G, (N + 127) // 128, K // 128)
                 and tuple(m_indices.shape) == (M,), "sa [K/128,M], sb [G,ceil(N/128),K/128], m_indices [M]")
    if out is None:
        out = torch.zeros((M, N), dtype=torch.bfloat16, device=A.device)
    D = _out(out, (M, N), A.device)
    with torch.cuda.device(A.device):
        st = lib().fp8gemm_grouped_contiguous(A.data_ptr(), sa.data_ptr(), B.data_ptr(), sb.data_ptr(),
                                              m_indices.data_ptr(), D.data_ptr(), M, N, K, G,
                                              _stream(stream, A.device))
    _check(st, "fp8gemm_grouped_contiguous")
    return D


def grouped_masked(A, sa, B, sb, masked_m, expected_m: int, out=None, stream=None):
    """MoE masked layout: A [G,M_max,K], sa [G,K/128,M_max], B [G,N,K], masked_m int32 [G]; rows past masked_m[g] of
    ``out`` are left untouched (zeros when ``out`` is allocated here)."""
    torch = _torch()
    A, B = _codes(A, "A"), _codes(B, "B")
    sa, sb = _f32(sa, "sa"), _f32(sb, "sb")
    masked_m = _i32(masked_m, "masked_m")
    _shape_check(A.dim() == 3 and B.dim() == 3 and A.shape[0] == B.shape[0] and A.shape[2] == B.shape[2],
                 "A [G,M_max,K] and B [G,N,K]")
    G, M_max, K = A.shape
    N = B.shape[1]
    _shape_check(tuple(sa.shape) == (G, K // 128, M_max) and tuple(sb.shape) == (G, (N + 127) // 128, K // 128)
                 and tuple(masked_m.shape) == (G,), "sa [G,K/128,M_max], sb [G,ceil(N/128),K/128], masked_m [G]")
    if out is None:
        out = torch.zeros((G, M_max, N), dtype=torch.bfloat16, device=A.device)
    D = _out(out, (G, M_max, N), A.device)
    with torch.cuda.device(A.device):
        st = lib().fp8gemm_grouped_masked(A.data_ptr(), sa.data_ptr(), B.data_ptr(), sb.data_ptr(),
                                          masked_m.data_ptr(), D.data_ptr(), G, M_max, N, K,
                                          int(expected_m), _stream(stream, A.device))
    _check(st, "fp8gemm_grouped_masked")
    return D


def _u8(t, name):
    torch = _torch()
    if t.dtype != torch.uint8:
        raise TypeError("%s must be uint8, got %s" % (name, t.dtype))
    return _dev_contig(t, name)


def fp8fp4_grouped_masked(A, sa, B, sb, masked_m, expected_m: int, out=None, stream=None):
    """Masked layout with B in E2M1: A [G,M_max,K] e4m3 codes, sa [G,K/128,M_max], B uint8
    [G,N,K/2] (two E2M1 codes per byte, even element in the low nibble), sb uint8 [G,N,K/32]
    (E8M0 scales per 32 K), masked_m int32 [G].  Rows past masked_m[g] of ``out`` are left
    untouched (zeros when ``out`` is allocated here)."""
    torch = _torch()
    A = _codes(A, "A")
    B, sb = _u8(B, "B"), _u8(sb, "sb")
    sa = _f32(sa, "sa")
    masked_m = _i32(masked_m, "masked_m")
    _shape_check(A.dim() == 3 and B.dim() == 3 and A.shape[0] == B.shape[0] and 2 * B.shape[2] == A.shape[2],
                 "A [G,M_max,K] and B [G,N,K/2]")
    G, M_max, K = A.shape
    N = B.shape[1]
    _shape_check(tuple(sa.shape) == (G, K // 128, M_max) and tuple(sb.shape) == (G, N, K // 32)
                 and tuple(masked_m.shape) == (G,), "sa [G,K/128,M_max], sb [G,N,K/32], masked_m [G]")
    if out is None:
        out = torch.zeros((G, M_max, N), dtype=torch.bfloat16, device=A.device)
    D = _out(out, (G, M_max, N), A.device)
    with torch.cuda.device(A.device):
        st = lib().fp8gemm_fp8fp4_grouped_masked(A.data_ptr(), sa.data_ptr(), B.data_ptr(), sb.data_ptr(),
                                                 masked_m.data_ptr(), D.data_ptr(), G, M_max, N, K,
                                                 int(expected_m), _stream(stream, A.device))
    _check(st, "fp8gemm_fp8fp4_grouped_masked")
    return D


def _bf16(t, name):
    torch = _torch()
    if t.dtype != torch.bfloat16:
        raise TypeError("%s must be bfloat16, got %s" % (name, t.dtype))
    return _dev_contig(t, name)


def _quant_outputs(codes, scales, codes_shape, scales_shape, device):
    torch = _torch()
    if codes is None:
        codes = torch.empty(codes_shape, dtype=torch.float8_e4m3fn, device=device)
    if scales is None:
        scales = torch.empty(scales_shape, dtype=torch.float32, device=device)
    codes, scales = _codes(codes, "codes"), _f32(scales, "scales")
    _shape_check(tuple(codes.shape) == tuple(codes_shape) and tuple(scales.shape) == tuple(scales_shape),
                 "codes %s, scales %s" % (tuple(codes_shape), tuple(scales_shape)))
    return codes, scales


def quantize_1x128(X, codes=None, scales=None, stream=None):
    """Activations X bf16 [M,K] -> (E4M3 codes [M,K], scales fp32 [K/128,M]), one scale per 1x128
    block of a row, in the layout gemm_nt and grouped_contiguous take as A and sa."""
    torch = _torch()
    X = _bf16(X, "X")
    _shape_check(X.dim() == 2, "X [M,K]")
    M, K = X.shape
    codes, scales = _quant_outputs(codes, scales, (M, K), (K // 128, M), X.device)
    with torch.cuda.device(X.device):
        st = lib().fp8gemm_quantize_1x128(X.data_ptr(), codes.data_ptr(), scales.data_ptr(), M, K,
                                          _stream(stream, X.device))
    _check(st, "fp8gemm_quantize_1x128")
    return codes, scales


def quantize_1x128_masked(X, masked_m, codes=None, scales=None, stream=None):
    """Masked layout: X bf16 [G,M_max,K] -> (codes [G,M_max,K], scales [G,K/128,M_max]); rows at or
    past masked_m[g] are not written (zeros when the outputs are allocated here)."""
    torch = _torch()
    X = _bf16(X, "X")
    masked_m = _i32(masked_m, "masked_m")
    _shape_check(X.dim() == 3 and tuple(masked_m.shape) == (X.shape[0],), "X [G,M_max,K], masked_m [G]")
    G, M_max, K = X.shape
    if codes is None:
        codes = torch.zeros((G, M_max, K), dtype=torch.uint8, device=X.device).view(torch.float8_e4m3fn)
    if scales is None:
        scales = torch.zeros((G, K // 128, M_max), dtype=torch.float32, device=X.device)
    codes, scales = _quant_outputs(codes, scales, (G, M_max, K), (G, K // 128, M_max), X.device)
    with torch.cuda.device(X.device):
        st = lib().fp8gemm_quantize_1x128_masked(X.data_ptr(), codes.data_ptr(), scales.data_ptr(),
                                                 masked_m.data_ptr(), G, M_max, K,
                                                 _stream(stream, X.device))
    _check(st, "fp8gemm_quantize_1x128_masked")
    return codes, scales


def swiglu_quantize_1x128(Y, codes=None, scales=None, stream=None):
    """SwiGLU + requantisation: Y bf16 [M,2I] (gate | up) -> (codes [M,I], scales fp32 [I/128,M]) of
    h = silu(gate) * up, one scale per 1x128 block (the second expert layer's A and sa)."""
    torch = _torch()
    Y = _bf16(Y, "Y")
    _shape_check(Y.dim() == 2 and Y.shape[1] % 2 == 0, "Y [M,2I]")
    M, I = Y.shape[0], Y.shape[1] // 2
    codes, scales = _quant_outputs(codes, scales, (M, I), (I // 128, M), Y.device)
    with torch.cuda.device(Y.device):
        st = lib().fp8gemm_swiglu_quantize_1x128(Y.data_ptr(), codes.data_ptr(), scales.data_ptr(), M, I,
                                                 _stream(stream, Y.device))
    _check(st, "fp8gemm_swiglu_quantize_1x128")
    return codes, scales


def swiglu_quantize_1x128_masked(Y, masked_m, codes=None, scales=None, stream=None):
    """Masked layout: Y bf16 [G,M_max,2I] -> (codes [G,M_max,I], scales [G,I/128,M_max]); rows at or
    past masked_m[g] are not written (zeros when the outputs are allocated here)."""
    torch = _torch()
    Y = _bf16(Y, "Y")
    masked_m = _i32(masked_m, "masked_m")
    _shape_check(Y.dim() == 3 and Y.shape[2] % 2 == 0 and tuple(masked_m.shape) == (Y.shape[0],),
                 "Y [G,M_max,2I], masked_m [G]")
    G, M_max, I = Y.shape[0], Y.shape[1], Y.shape[2] // 2
    if codes is None:
        codes = torch.zeros((G, M_max, I), dtype=torch.uint8, device=Y.device).view(torch.float8_e4m3fn)
    if scales is None:
        scales = torch.zeros((G, I // 128, M_max), dtype=torch.float32, device=Y.device)
    codes, scales = _quant_outputs(codes, scales, (G, M_max, I), (G, I // 128, M_max), Y.device)
    with torch.cuda.device(Y.device):
        st = lib().fp8gemm_swiglu_quantize_1x128_masked(Y.data_ptr(), codes.data_ptr(), scales.data_ptr(),
                                                        masked_m.data_ptr(), G, M_max, I,
                                                        _stream(stream, Y.device))
    _check(st, "fp8gemm_swiglu_quantize_1x128_masked")
    return codes, scales


def moe_expert_masked(A, sa, W1, s1, W2, s2, masked_m, expected_m: int, out=None, workspace=None,
                      stream=None):
    """One MoE expert layer per group, masked layout: out = (swiglu(A . W1^T) requantised) . W2^T.
    A [G,M_max,H] codes, sa [G,H/128,M_max], W1 [G,2I,H], s1 [G,2I/128,H/128], W2 [G,H,I],
    s2 [G,H/128,I/128], masked_m int32 [G].  ``workspace``: optional (Y1 bf16 [G,M_max,2I],
    Hq codes [G,M_max,I], sh fp32 [G,I/128,M_max]), allocated here when None.  Returns out bf16
    [G,M_max,H] (rows past masked_m[g] untouched: zeros when allocated here)."""
    torch = _torch()
    A, W1, W2 = _codes(A, "A"), _codes(W1, "W1"), _codes(W2, "W2")
    sa, s1, s2 = _f32(sa, "sa"), _f32(s1, "s1"), _f32(s2, "s2")
    masked_m = _i32(masked_m, "masked_m")
    _shape_check(A.dim() == 3 and W1.dim() == 3 and W2.dim() == 3, "A [G,M_max,H], W1 [G,2I,H], W2 [G,H,I]")
    G, M_max, H = A.shape
    I = W2.shape[2]
    _shape_check(tuple(W1.shape) == (G, 2 * I, H) and tuple(W2.shape) == (G, H, I)
                 and tuple(sa.shape) == (G, H // 128, M_max)
                 and tuple(s1.shape) == (G, (2 * I + 127) // 128, H // 128)
                 and tuple(s2.shape) == (G, (H + 127) // 128, I // 128) and tuple(masked_m.shape) == (G,),
                 "A [G,M_max,H], sa [G,H/128,M_max], W1 [G,2I,H], s1 [G,2I/128,H/128], W2 [G,H,I], "
                 "s2 [G,H/128,I/128], masked_m [G]")
    if workspace is None:
        workspace = (torch.empty((G, M_max, 2 * I), dtype=torch.bfloat16, device=A.device),
                     torch.empty((G, M_max, I), dtype=torch.float8_e4m3fn, device=A.device),
                     torch.empty((G, I // 128, M_max), dtype=torch.float32, device=A.device))
    Y1, Hq, sh = workspace
    Y1, Hq, sh = _bf16(Y1, "Y1"), _codes(Hq, "Hq"), _f32(sh, "sh")
    _shape_check(tuple(Y1.shape) == (G, M_max, 2 * I) and tuple(Hq.shape) == (G, M_max, I)
                 and tuple(sh.shape) == (G, I // 128, M_max), "workspace shapes")
    if out is None:
        out = torch.zeros((G, M_max, H), dtype=torch.bfloat16, device=A.device)
    D = _out(out, (G, M_max, H), A.device)
    with torch.cuda.device(A.device):
        st = lib().fp8gemm_moe_expert_masked(A.data_ptr(), sa.data_ptr(), W1.data_ptr(), s1.data_ptr(),
                                             W2.data_ptr(), s2.data_ptr(), masked_m.data_ptr(),
                                             Y1.data_ptr(), Hq.data_ptr(), sh.data_ptr(), D.data_ptr(),
                                             G, M_max, H, I, int(expected_m), _stream(stream, A.device))
    _check(st, "fp8gemm_moe_expert_masked")
    return D
