"""Thin ctypes binding of libqgemm.so (C ABI in include/qgemm.h).

Argument marshalling only: every step of the computation runs in the HIP
library.  Functions take torch tensors on the GPU, pass their device pointers
and torch's current HIP stream, and raise QGemmError on a non-zero status.
There is no fallback: if libqgemm.so is missing, importing this module raises.

bf16 data travels as torch.bfloat16 (or int16 / uint16 bit patterns) tensors;
e4m3 codes as torch.uint8 (or torch.float8_e4m3fn) tensors.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqgemm.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python -m weight_only_quantized_w4a16_amd.build` "
        "(hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

_SIGS = {
    "qg_status_string": (ctypes.c_char_p, [_I]),
    "qg_version": (ctypes.c_char_p, []),
    "qg_int4_g128_packed_bytes": (_SZ, [_I64, _I64]),
    "qg_int4_g128_scale_bytes": (_SZ, [_I64, _I64]),
    "qg_w4a16_kernel_for": (ctypes.c_char_p, [_I64, _I64, _I64]),
    "qg_w8a8_kernel_for": (ctypes.c_char_p, [_I64, _I64, _I64]),
    "qg_w4a16_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "qg_w8a8_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "pack_int4_g128": (_I, [_P, _I, _I, _P, _P, _P]),
    "pack_int4_g128_mse": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "dequant_int4_g128": (_I, [_P, _P, _I, _I, _P, _P, _P]),
    "qgemm_w4a16": (_I, [_P, _P, _P, _P, _I, _I, _I, _P, _SZ, _P]),
    "qgemm_w4a16_noalloc": (_I, [_P, _P, _P, _P, _I, _I, _I, _P]),
    "qg_w4a16_grouped_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64]),
    "qgemm_w4a16_grouped": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _SZ, _P]),
    "quant_act_per_token": (_I, [_P, _I, _I, _P, _P, _P]),
    "quant_weight_fp8_per_channel": (_I, [_P, _I, _I, _P, _P, _P]),
    "qgemm_w8a8_fp8": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _P, _SZ, _P]),
    "qgemm_w4a8_fp8": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _P]),
    "qgemm_w4a8_fp8_grouped": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _SZ, _P]),
    "qg_w8a8_int8_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "quant_act_per_token_int8": (_I, [_P, _I, _I, _P, _P, _P]),
    "quant_weight_int8_per_channel": (_I, [_P, _I, _I, _P, _P, _P]),
    "qgemm_w8a8_int8": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _P, _SZ, _P]),
    "qg_w8a8_dynamic_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "qg_w8a8_dynamic_kernel_for": (ctypes.c_char_p, [_I64, _I64, _I64]),
    "qgemm_w8a8_fp8_dynamic": (_I, [_P, _P, _P, _P, _I, _I, _I, _P, _SZ, _P]),
    "qgemm_w8a8_int8_dynamic": (_I, [_P, _P, _P, _P, _I, _I, _I, _P, _SZ, _P]),
    "qg_w4a8_grouped_dynamic_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64]),
    "qg_w4a8_grouped_dynamic_kernel_for": (ctypes.c_char_p, [_I64, _I64, _I64, _I64]),
    "qgemm_w4a8_fp8_grouped_dynamic": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _SZ, _P]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_SIGS)


class QGemmError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: status {status} ({status_string(status)})")


def status_string(status):
    return _lib.qg_status_string(int(status)).decode()


def version():
    return _lib.qg_version().decode()


def packed_bytes(K, N):
    return _lib.qg_int4_g128_packed_bytes(K, N)


def scale_bytes(K, N):
    return _lib.qg_int4_g128_scale_bytes(K, N)


def w4a16_kernel_for(M, N, K):
    return _lib.qg_w4a16_kernel_for(M, N, K).decode()


def w8a8_kernel_for(M, N, K):
    return _lib.qg_w8a8_kernel_for(M, N, K).decode()


def w8a8_dynamic_kernel_for(M, N, K):
    return _lib.qg_w8a8_dynamic_kernel_for(M, N, K).decode()


def w8a8_dynamic_workspace_bytes(M, N, K):
    return _lib.qg_w8a8_dynamic_workspace_bytes(M, N, K)


def w4a16_workspace_bytes(M, N, K):
    return _lib.qg_w4a16_workspace_bytes(M, N, K)


def w8a8_workspace_bytes(M, N, K):
    return _lib.qg_w8a8_workspace_bytes(M, N, K)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(fn, status):
    if status != 0:
        raise QGemmError(fn, status)


# ---- raw entry points (same names and argument order as the C ABI) ----------

def pack_int4_g128(w_bf16, K, N, packed, scales, stream=None):
    _check("pack_int4_g128", _lib.pack_int4_g128(_ptr(w_bf16), K, N, _ptr(packed), _ptr(scales),
                                                 _stream(stream)))


def pack_int4_g128_mse(w_bf16, K, N, n_alpha, packed, scales, stream=None):
    _check("pack_int4_g128_mse", _lib.pack_int4_g128_mse(_ptr(w_bf16), K, N, n_alpha, _ptr(packed),
                                                         _ptr(scales), _stream(stream)))


def dequant_int4_g128(packed, scales, K, N, w_bf16_out, codes_out=None, stream=None):
    _check("dequant_int4_g128", _lib.dequant_int4_g128(_ptr(packed), _ptr(scales), K, N,
                                                       _ptr(w_bf16_out), _ptr(codes_out),
                                                       _stream(stream)))


def qgemm_w4a16(a_bf16, packed, scales, y_bf16, M, N, K, workspace=None, workspace_bytes=0,
                stream=None):
    _check("qgemm_w4a16", _lib.qgemm_w4a16(_ptr(a_bf16), _ptr(packed), _ptr(scales), _ptr(y_bf16),
                                           M, N, K, _ptr(workspace), workspace_bytes,
                                           _stream(stream)))


def qgemm_w4a16_noalloc(a_bf16, packed, scales, y_bf16, M, N, K, stream=None):
    _check("qgemm_w4a16_noalloc", _lib.qgemm_w4a16_noalloc(_ptr(a_bf16), _ptr(packed), _ptr(scales),
                                                           _ptr(y_bf16), M, N, K, _stream(stream)))


NOALLOC_SCRATCH_BYTES = 32 << 20    # QG_NOALLOC_SCRATCH_BYTES of include/qgemm.h


def quant_act_per_token(a_bf16, M, K, a_e4m3, a_scale, stream=None):
    _check("quant_act_per_token", _lib.quant_act_per_token(_ptr(a_bf16), M, K, _ptr(a_e4m3),
                                                           _ptr(a_scale), _stream(stream)))


def quant_weight_fp8_per_channel(w_bf16, K, N, w_e4m3, w_scale, stream=None):
    _check("quant_weight_fp8_per_channel",
           _lib.quant_weight_fp8_per_channel(_ptr(w_bf16), K, N, _ptr(w_e4m3), _ptr(w_scale),
                                             _stream(stream)))


def qgemm_w8a8_fp8(a_e4m3, a_scale, w_e4m3, w_scale, y_bf16, M, N, K, workspace=None,
                   workspace_bytes=0, stream=None):
    _check("qgemm_w8a8_fp8", _lib.qgemm_w8a8_fp8(_ptr(a_e4m3), _ptr(a_scale), _ptr(w_e4m3),
                                                 _ptr(w_scale), _ptr(y_bf16), M, N, K,
                                                 _ptr(workspace), workspace_bytes,
                                                 _stream(stream)))


def qgemm_w4a8_fp8(a_e4m3, a_scale, packed, scales, y_bf16, M, N, K, stream=None):
    _check("qgemm_w4a8_fp8", _lib.qgemm_w4a8_fp8(_ptr(a_e4m3), _ptr(a_scale), _ptr(packed), _ptr(scales),
                                                 _ptr(y_bf16), M, N, K, _stream(stream)))


def qgemm_w4a8_fp8_grouped(a_e4m3, a_scale, offsets_i32, packed, scales, y_bf16, E, T, N, K, workspace,
                           workspace_bytes, stream=None):
    _check("qgemm_w4a8_fp8_grouped",
           _lib.qgemm_w4a8_fp8_grouped(_ptr(a_e4m3), _ptr(a_scale), _ptr(offsets_i32), _ptr(packed),
                                       _ptr(scales), _ptr(y_bf16), E, T, N, K, _ptr(workspace),
                                       workspace_bytes, _stream(stream)))


def w8a8_int8_workspace_bytes(M, N, K):
    return _lib.qg_w8a8_int8_workspace_bytes(M, N, K)


def quant_act_per_token_int8(a_bf16, M, K, a_i8, a_scale, stream=None):
    _check("quant_act_per_token_int8",
           _lib.quant_act_per_token_int8(_ptr(a_bf16), M, K, _ptr(a_i8), _ptr(a_scale), _stream(stream)))


def quant_weight_int8_per_channel(w_bf16, K, N, w_i8, w_scale, stream=None):
    _check("quant_weight_int8_per_channel",
           _lib.quant_weight_int8_per_channel(_ptr(w_bf16), K, N, _ptr(w_i8), _ptr(w_scale),
                                              _stream(stream)))


def qgemm_w8a8_int8(a_i8, a_scale, w_i8, w_scale, y_bf16, M, N, K, workspace=None,
                    workspace_bytes=0, stream=None):
    _check("qgemm_w8a8_int8", _lib.qgemm_w8a8_int8(_ptr(a_i8), _ptr(a_scale), _ptr(w_i8),
                                                   _ptr(w_scale), _ptr(y_bf16), M, N, K,
                                                   _ptr(workspace), workspace_bytes,
                                                   _stream(stream)))


def qgemm_w8a8_fp8_dynamic(a_bf16, w_e4m3, w_scale, y_bf16, M, N, K, workspace=None,
                           workspace_bytes=0, stream=None):
    _check("qgemm_w8a8_fp8_dynamic",
           _lib.qgemm_w8a8_fp8_dynamic(_ptr(a_bf16), _ptr(w_e4m3), _ptr(w_scale), _ptr(y_bf16), M, N, K,
                                       _ptr(workspace), workspace_bytes, _stream(stream)))


def qgemm_w8a8_int8_dynamic(a_bf16, w_i8, w_scale, y_bf16, M, N, K, workspace=None,
                            workspace_bytes=0, stream=None):
    _check("qgemm_w8a8_int8_dynamic",
           _lib.qgemm_w8a8_int8_dynamic(_ptr(a_bf16), _ptr(w_i8), _ptr(w_scale), _ptr(y_bf16), M, N, K,
                                        _ptr(workspace), workspace_bytes, _stream(stream)))


def w4a8_grouped_dynamic_workspace_bytes(E, T, N, K):
    return _lib.qg_w4a8_grouped_dynamic_workspace_bytes(E, T, N, K)


def w4a8_grouped_dynamic_kernel_for(E, T, N, K):
    return _lib.qg_w4a8_grouped_dynamic_kernel_for(E, T, N, K).decode()


def qgemm_w4a8_fp8_grouped_dynamic(a_bf16, offsets_i32, packed, scales, y_bf16, E, T, N, K, workspace,
                                   workspace_bytes, stream=None):
    _check("qgemm_w4a8_fp8_grouped_dynamic",
           _lib.qgemm_w4a8_fp8_grouped_dynamic(_ptr(a_bf16), _ptr(offsets_i32), _ptr(packed), _ptr(scales),
                                               _ptr(y_bf16), E, T, N, K, _ptr(workspace), workspace_bytes,
                                               _stream(stream)))


# ---- tensor-level helpers (allocate outputs with torch, then call the above) --

def _bf16(t):
    if t.dtype in (torch.int16, torch.uint16):
        return t
    if t.dtype != torch.bfloat16:
        raise TypeError(f"expected bf16 data, got {t.dtype}")
    return t


class Int4G128Weight:
    """A [K, N] weight in native INT4 g128 form (device buffers owned by torch)."""

    def __init__(self, packed, scales, K, N):
        self.packed, self.scales, self.K, self.N = packed, scales, K, N

    @classmethod
    def from_bf16(cls, w, stream=None, mse_grid=0):
        """Abs-max scales, or with mse_grid > 0 the MSE-optimal clipping
        threshold searched over alpha = i / mse_grid, i = 1 .. mse_grid."""
        K, N = w.shape
        packed = torch.empty(max(packed_bytes(K, N) // 4, 1), dtype=torch.int32, device=w.device)
        scales = torch.empty(max(scale_bytes(K, N) // 2, 1), dtype=torch.int16, device=w.device)
        if mse_grid:
            pack_int4_g128_mse(_bf16(w.contiguous()), K, N, mse_grid, packed, scales, stream)
        else:
            pack_int4_g128(_bf16(w.contiguous()), K, N, packed, scales, stream)
        return cls(packed, scales, K, N)

    def dequant(self, with_codes=False, stream=None):
        w = torch.empty((self.K, self.N), dtype=torch.bfloat16, device=self.packed.device)
        codes = torch.empty((self.K, self.N), dtype=torch.uint8, device=self.packed.device) \
            if with_codes else None
        dequant_int4_g128(self.packed, self.scales, self.K, self.N, w, codes, stream)
        return (w, codes) if with_codes else w


class W4A16Linear:
    """y = a @ w_hat for a packed INT4 g128 weight; owns a reusable workspace."""

    def __init__(self, weight: Int4G128Weight):
        self.w = weight
        self._ws = None

    def workspace(self, M):
        need = w4a16_workspace_bytes(M, self.w.N, self.w.K)
        if need and (self._ws is None or self._ws.numel() < need):
            # zero-filled once; every call resets the counters it uses
            self._ws = torch.zeros(need, dtype=torch.uint8, device=self.w.packed.device)
        return (self._ws, need) if need else (None, 0)

    def __call__(self, a, out=None, stream=None):
        M, K = a.shape
        if K != self.w.K:
            raise ValueError(f"activation K={K} != weight K={self.w.K}")
        y = out if out is not None else torch.empty((M, self.w.N), dtype=torch.bfloat16,
                                                    device=a.device)
        ws, nbytes = self.workspace(M)
        qgemm_w4a16(_bf16(a), self.w.packed, self.w.scales, y, M, self.w.N, K, ws, nbytes, stream)
        return y


class Fp8Weight:
    """A [K, N] weight as native per-channel e4m3 codes plus fp32 channel scales."""

    def __init__(self, codes, scales, K, N):
        self.codes, self.scales, self.K, self.N = codes, scales, K, N

    @classmethod
    def from_bf16(cls, w, stream=None):
        K, N = w.shape
        codes = torch.empty(K * N, dtype=torch.uint8, device=w.device)
        scales = torch.empty(N, dtype=torch.float32, device=w.device)
        quant_weight_fp8_per_channel(_bf16(w.contiguous()), K, N, codes, scales, stream)
        return cls(codes, scales, K, N)


def w4a16_grouped_workspace_bytes(E, T, N, K):
    return _lib.qg_w4a16_grouped_workspace_bytes(E, T, N, K)


def qgemm_w4a16_grouped(a_bf16, offsets_i32, packed, scales, y_bf16, E, T, N, K, workspace,
                        workspace_bytes, stream=None):
    _check("qgemm_w4a16_grouped",
           _lib.qgemm_w4a16_grouped(_ptr(a_bf16), _ptr(offsets_i32), _ptr(packed), _ptr(scales),
                                    _ptr(y_bf16), E, T, N, K, _ptr(workspace), workspace_bytes,
                                    _stream(stream)))


class GroupedInt4Weight:
    """E experts' [K, N] weights packed back to back (device buffers owned by torch)."""

    def __init__(self, packed, scales, E, K, N):
        self.packed, self.scales, self.E, self.K, self.N = packed, scales, E, K, N
        self._ws = None

    @classmethod
    def from_bf16(cls, w, stream=None):
        """w: [E, K, N] bf16 on the device."""
        E, K, N = w.shape
        words, nsc = packed_bytes(K, N) // 4, scale_bytes(K, N) // 2
        packed = torch.empty(E * words, dtype=torch.int32, device=w.device)
        scales = torch.empty(E * nsc, dtype=torch.int16, device=w.device)
        for e in range(E):
            pack_int4_g128(_bf16(w[e].contiguous()), K, N, packed[e * words:(e + 1) * words],
                           scales[e * nsc:(e + 1) * nsc], stream)
        return cls(packed, scales, E, K, N)

    def __call__(self, a, offsets, out=None, stream=None):
        """a: [T, K] bf16 rows grouped by expert; offsets: int32 [E + 1] on the device."""
        T, K = a.shape
        if K != self.K or offsets.numel() != self.E + 1 or offsets.dtype != torch.int32:
            raise ValueError("grouped GEMM: activation K or offsets do not match the weights")
        y = out if out is not None else torch.empty((T, self.N), dtype=torch.bfloat16, device=a.device)
        need = w4a16_grouped_workspace_bytes(self.E, T, self.N, K)
        if need and (self._ws is None or self._ws.numel() * 4 < need):
            self._ws = torch.empty((need + 3) // 4, dtype=torch.int32, device=a.device)
        qgemm_w4a16_grouped(_bf16(a), offsets, self.packed, self.scales, y, self.E, T, self.N, K,
                            self._ws if need else None, need, stream)
        return y

    def w4a8(self, qa, sa, offsets, out=None, stream=None):
        """The W4A8-FP8 product: qa [T, K] e4m3 codes and sa [T] from quant_act_per_token."""
        T, K = qa.shape
        if K != self.K or offsets.numel() != self.E + 1 or offsets.dtype != torch.int32:
            raise ValueError("grouped GEMM: activation K or offsets do not match the weights")
        y = out if out is not None else torch.empty((T, self.N), dtype=torch.bfloat16, device=qa.device)
        need = w4a16_grouped_workspace_bytes(self.E, T, self.N, K)
        if need and (self._ws is None or self._ws.numel() * 4 < need):
            self._ws = torch.empty((need + 3) // 4, dtype=torch.int32, device=qa.device)
        qgemm_w4a8_fp8_grouped(qa, sa, offsets, self.packed, self.scales, y, self.E, T, self.N, K,
                               self._ws if need else None, need, stream)
        return y

    def w4a8_dynamic(self, a, offsets, out=None, stream=None):
        """The W4A8-FP8 product on bf16 rows, quantized per token inside the call."""
        T, K = a.shape
        if K != self.K or offsets.numel() != self.E + 1 or offsets.dtype != torch.int32:
            raise ValueError("grouped GEMM: activation K or offsets do not match the weights")
        y = out if out is not None else torch.empty((T, self.N), dtype=torch.bfloat16, device=a.device)
        need = w4a8_grouped_dynamic_workspace_bytes(self.E, T, self.N, K)
        if need and (self._ws is None or self._ws.numel() * 4 < need):
            self._ws = torch.empty((need + 3) // 4, dtype=torch.int32, device=a.device)
        qgemm_w4a8_fp8_grouped_dynamic(_bf16(a), offsets, self.packed, self.scales, y, self.E, T, self.N, K,
                                       self._ws if need else None, need, stream)
        return y


def quantize_activations(a, stream=None):
    M, K = a.shape
    q = torch.empty((M, K), dtype=torch.uint8, device=a.device)
    s = torch.empty(M, dtype=torch.float32, device=a.device)
    quant_act_per_token(_bf16(a), M, K, q, s, stream)
    return q, s


class W8A8Fp8Linear:
    """y = bf16(s_a s_w (qa @ qw)) with per-token quantization of a on every call."""

    def __init__(self, weight: Fp8Weight):
        self.w = weight
        self._ws = None

    def workspace(self, M, dynamic=False):
        need = (w8a8_dynamic_workspace_bytes if dynamic else w8a8_workspace_bytes)(M, self.w.N, self.w.K)
        if need and (self._ws is None or self._ws.numel() < need):
            # zero-filled once; every call resets the counters it uses
            self._ws = torch.zeros(need, dtype=torch.uint8, device=self.w.codes.device)
        return (self._ws, need) if need else (None, 0)

    def __call__(self, a, out=None, stream=None, qa=None, sa=None):
        """Without qa / sa the activations are quantized inside the call
        (qgemm_w8a8_fp8_dynamic); with them the GEMM runs on the given codes."""
        M, K = a.shape
        if K != self.w.K:
            raise ValueError(f"activation K={K} != weight K={self.w.K}")
        y = out if out is not None else torch.empty((M, self.w.N), dtype=torch.bfloat16,
                                                    device=a.device)
        ws, need = self.workspace(M, dynamic=qa is None)
        if qa is None:
            qgemm_w8a8_fp8_dynamic(_bf16(a), self.w.codes, self.w.scales, y, M, self.w.N, K, ws, need,
                                   stream)
        else:
            qgemm_w8a8_fp8(qa, sa, self.w.codes, self.w.scales, y, M, self.w.N, K, ws, need, stream)
        return y


class W4A8Linear:
    """y = bf16(s_a (qa @ w_hat)) for a packed INT4 g128 weight and e4m3 per-token activations."""

    def __init__(self, weight: "Int4G128Weight"):
        self.w = weight

    def __call__(self, a, out=None, stream=None, qa=None, sa=None):
        M, K = a.shape
        if K != self.w.K:
            raise ValueError(f"activation K={K} != weight K={self.w.K}")
        if qa is None:
            qa, sa = quantize_activations(a, stream)
        y = out if out is not None else torch.empty((M, self.w.N), dtype=torch.bfloat16, device=a.device)
        qgemm_w4a8_fp8(qa, sa, self.w.packed, self.w.scales, y, M, self.w.N, K, stream)
        return y


class Int8Weight:
    """A [K, N] weight as native per-channel int8 codes plus fp32 channel scales."""

    def __init__(self, codes, scales, K, N):
        self.codes, self.scales, self.K, self.N = codes, scales, K, N

    @classmethod
    def from_bf16(cls, w, stream=None):
        K, N = w.shape
        codes = torch.empty(K * N, dtype=torch.int8, device=w.device)
        scales = torch.empty(N, dtype=torch.float32, device=w.device)
        quant_weight_int8_per_channel(_bf16(w.contiguous()), K, N, codes, scales, stream)
        return cls(codes, scales, K, N)


def quantize_activations_int8(a, stream=None):
    M, K = a.shape
    q = torch.empty((M, K), dtype=torch.int8, device=a.device)
    s = torch.empty(M, dtype=torch.float32, device=a.device)
    quant_act_per_token_int8(_bf16(a), M, K, q, s, stream)
    return q, s


class W8A8Int8Linear:
    """y = bf16(s_a s_w (qa @ qw)) with int8 codes, per-token quantization of a on every call."""

    def __init__(self, weight: Int8Weight):
        self.w = weight
        self._ws = None

    def workspace(self, M, dynamic=False):
        need = (w8a8_dynamic_workspace_bytes if dynamic else w8a8_int8_workspace_bytes)(
            M, self.w.N, self.w.K)
        if need and (self._ws is None or self._ws.numel() < need):
            self._ws = torch.zeros(need, dtype=torch.uint8, device=self.w.codes.device)
        return (self._ws, need) if need else (None, 0)

    def __call__(self, a, out=None, stream=None, qa=None, sa=None):
        """Without qa / sa the activations are quantized inside the call
        (qgemm_w8a8_int8_dynamic); with them the GEMM runs on the given codes."""
        M, K = a.shape
        if K != self.w.K:
            raise ValueError(f"activation K={K} != weight K={self.w.K}")
        y = out if out is not None else torch.empty((M, self.w.N), dtype=torch.bfloat16,
                                                    device=a.device)
        ws, need = self.workspace(M, dynamic=qa is None)
        if qa is None:
            qgemm_w8a8_int8_dynamic(_bf16(a), self.w.codes, self.w.scales, y, M, self.w.N, K, ws, need,
                                    stream)
        else:
            qgemm_w8a8_int8(qa, sa, self.w.codes, self.w.scales, y, M, self.w.N, K, ws, need, stream)
        return y
