"""Python access to the fp64 CPU oracle (``rq_oracle.c``) through ctypes.

TEST INFRASTRUCTURE ONLY.  The tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module; the library package
never does.  It does nothing but marshal numpy arrays into the C routines and
shares no code with the GPU path.

Logical slice arrays (one K or V slice of one batch row, layer and kv head;
L loops, N tokens, head_dim d, group g, ng = d // g):
    x      uint16 [L, N, d]    BF16 bit patterns
    codes  uint8  [L, N, d]    one code per element
    s8/z8  uint8  [L, N, ng]   FP8 e4m3fn scale / offset bit patterns
    alpha  uint16 [L, N]       BF16 residual coefficient (0 where none)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SAN_LIB_PATH = os.path.join(_HERE, "liboracle_san.so")

MODE_RESIDUAL = 0
MODE_DIRECT = 1
MODE_CHAINED = 2
ALPHA_LS = 0
ALPHA_NORM_RATIO = 1
ALPHA_ONE = 2


def build(force: bool = False) -> str:
    """Compile rq_oracle.c with gcc (no contraction, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
            "-Wall", "-Wextra", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def build_sanitized() -> str:
    """liboracle_san.so: the same source under ASan + UBSan, built with the
    ROCm clang so that one ASan runtime serves it and librq_san.so (load it
    with ORACLE_LIB=<path>; see decode_attention_int4_amd/build.py)."""
    clang = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang")
    tmp = _SAN_LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.check_call([
        clang, "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-Wall",
        "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
        "-fno-omit-frame-pointer", "-shared-libasan", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _SAN_LIB_PATH)
    return _SAN_LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB") or build()
        _lib = ctypes.CDLL(path)
        _declare(_lib)
    return _lib


class _Params(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "d", "g", "P", "anchor_bits", "residual_bits", "mode", "alpha_mode", "rotate")]


@dataclass(frozen=True)
class Params:
    d: int
    g: int = 16
    P: int = 4
    anchor_bits: int = 4
    residual_bits: int = 2
    mode: int = MODE_RESIDUAL
    alpha_mode: int = ALPHA_LS
    rotate: int = 1

    def c(self) -> _Params:
        return _Params(self.d, self.g, self.P, self.anchor_bits, self.residual_bits,
                       self.mode, self.alpha_mode, self.rotate)

    @property
    def ng(self) -> int:
        return self.d // self.g


_P = ctypes.POINTER
_u8 = _P(ctypes.c_uint8)
_u16 = _P(ctypes.c_uint16)
_i8 = _P(ctypes.c_int8)
_f64 = _P(ctypes.c_double)


def _declare(L):
    L.rqo_fp8_decode_n.argtypes = [_u8, ctypes.c_long, _f64]
    L.rqo_fp8_encode_n.argtypes = [_f64, ctypes.c_long, _u8]
    L.rqo_bf16_decode_n.argtypes = [_u16, ctypes.c_long, _f64]
    L.rqo_bf16_encode_n.argtypes = [_f64, ctypes.c_long, _u16]
    L.rqo_rotation_matrix.argtypes = [ctypes.c_int, _i8, _f64]
    L.rqo_rotation_matrix.restype = ctypes.c_int
    L.rqo_rotate.argtypes = [ctypes.c_int, _i8, _f64, _f64]
    L.rqo_rotate.restype = ctypes.c_int
    L.rqo_rotate_t.argtypes = [ctypes.c_int, _i8, _f64, _f64]
    L.rqo_rotate_t.restype = ctypes.c_int
    L.rqo_quant_group.argtypes = [_f64, ctypes.c_int, ctypes.c_int, _u8, _u8, _u8]
    L.rqo_quant_vector.argtypes = [_f64, ctypes.c_int, ctypes.c_int, ctypes.c_int, _u8, _u8, _u8]
    L.rqo_dequant_vector.argtypes = [_u8, _u8, _u8, ctypes.c_int, ctypes.c_int, _f64]
    L.rqo_encode_group.argtypes = [_P(_Params), _f64, _i8, _u8, _u8, _u8, _u16]
    L.rqo_encode_group.restype = ctypes.c_int
    L.rqo_reconstruct_group.argtypes = [_P(_Params), _u8, _u8, _u8, _u16, _i8, ctypes.c_int, _f64]
    L.rqo_reconstruct_group.restype = ctypes.c_int
    L.rqo_encode_slice.argtypes = [_P(_Params), ctypes.c_int, ctypes.c_int, _u16, _i8,
                                   _u8, _u8, _u8, _u16]
    L.rqo_encode_slice.restype = ctypes.c_int
    L.rqo_reconstruct_slice.argtypes = [_P(_Params), ctypes.c_int, ctypes.c_int, _u8, _u8, _u8,
                                        _u16, _i8, ctypes.c_int, ctypes.c_int, ctypes.c_int, _f64]
    L.rqo_reconstruct_slice.restype = ctypes.c_int
    L.rqo_attention_dense.argtypes = [ctypes.c_int, ctypes.c_int, _f64, _f64, _f64,
                                      ctypes.c_double, _f64]
    L.rqo_attention_dense.restype = ctypes.c_int
    L.rqo_attention_slice.argtypes = [_P(_Params), ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, _u16, _i8, _i8,
                                      _u8, _u8, _u8, _u16, _u8, _u8, _u8, _u16,
                                      ctypes.c_double, ctypes.c_int, _f64]
    L.rqo_attention_slice.restype = ctypes.c_int
    L.rqo_bits_per_element.argtypes = [ctypes.c_int] * 5 + [ctypes.c_int]
    L.rqo_bits_per_element.restype = ctypes.c_double


def _ptr(a: np.ndarray, ctype):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(_P(ctype))


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


# ---------------------------------------------------------------- formats
def fp8_decode(codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().rqo_fp8_decode_n(_ptr(c, ctypes.c_uint8), c.size, _ptr(out, ctypes.c_double))
    return out


def fp8_encode(x) -> np.ndarray:
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(a.shape, np.uint8)
    lib().rqo_fp8_encode_n(_ptr(a, ctypes.c_double), a.size, _ptr(out, ctypes.c_uint8))
    return out


def bf16_decode(codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint16)
    out = np.empty(c.shape, np.float64)
    lib().rqo_bf16_decode_n(_ptr(c, ctypes.c_uint16), c.size, _ptr(out, ctypes.c_double))
    return out


def bf16_encode(x) -> np.ndarray:
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(a.shape, np.uint16)
    lib().rqo_bf16_encode_n(_ptr(a, ctypes.c_double), a.size, _ptr(out, ctypes.c_uint16))
    return out


# ---------------------------------------------------------------- rotation
def _signs_ptr(signs, d):
    """(array kept alive, pointer) for an optional int8 [d] sign vector."""
    if signs is None:
        return None, None
    a = np.ascontiguousarray(signs, dtype=np.int8)
    assert a.shape == (d,), f"signs must have shape ({d},)"
    return a, _ptr(a, ctypes.c_int8)


def rotation_matrix(d: int, signs) -> np.ndarray:
    s = np.ascontiguousarray(signs, dtype=np.int8)
    assert s.shape == (d,)
    H = np.empty((d, d), np.float64)
    _check(lib().rqo_rotation_matrix(d, _ptr(s, ctypes.c_int8), _ptr(H, ctypes.c_double)),
           "rotation_matrix")
    return H


def rotate(d: int, signs, r) -> np.ndarray:
    """y = H r, as exact +-1 sums followed by the 1/sqrt(n) scale."""
    s, sp = _signs_ptr(signs, d)
    v = np.ascontiguousarray(r, np.float64)
    out = np.empty(d, np.float64)
    _check(lib().rqo_rotate(d, sp, _ptr(v, ctypes.c_double), _ptr(out, ctypes.c_double)), "rotate")
    return out


def rotate_t(d: int, signs, y) -> np.ndarray:
    """r = H^T y."""
    s, sp = _signs_ptr(signs, d)
    v = np.ascontiguousarray(y, np.float64)
    out = np.empty(d, np.float64)
    _check(lib().rqo_rotate_t(d, sp, _ptr(v, ctypes.c_double), _ptr(out, ctypes.c_double)),
           "rotate_t")
    return out


# ---------------------------------------------------------------- quantizer
def quant_group(x, bits: int):
    a = np.ascontiguousarray(x, dtype=np.float64)
    s8 = np.zeros(1, np.uint8)
    z8 = np.zeros(1, np.uint8)
    codes = np.zeros(a.size, np.uint8)
    lib().rqo_quant_group(_ptr(a, ctypes.c_double), a.size, bits, _ptr(s8, ctypes.c_uint8),
                          _ptr(z8, ctypes.c_uint8), _ptr(codes, ctypes.c_uint8))
    return int(s8[0]), int(z8[0]), codes


def dequant_vector(codes, s8, z8, g: int) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    s = np.ascontiguousarray(s8, dtype=np.uint8)
    z = np.ascontiguousarray(z8, dtype=np.uint8)
    out = np.empty(c.size, np.float64)
    lib().rqo_dequant_vector(_ptr(c, ctypes.c_uint8), _ptr(s, ctypes.c_uint8),
                             _ptr(z, ctypes.c_uint8), c.size, g, _ptr(out, ctypes.c_double))
    return out


def encode_group(p: Params, x, signs=None):
    """x: float64 [P, d] -> (codes [P,d], s8 [P,ng], z8 [P,ng], alpha [P])."""
    a = np.ascontiguousarray(x, dtype=np.float64)
    assert a.shape == (p.P, p.d)
    s, sp = _signs_ptr(signs, p.d)
    codes = np.zeros((p.P, p.d), np.uint8)
    s8 = np.zeros((p.P, p.ng), np.uint8)
    z8 = np.zeros((p.P, p.ng), np.uint8)
    alpha = np.zeros(p.P, np.uint16)
    cp = p.c()
    _check(lib().rqo_encode_group(ctypes.byref(cp), _ptr(a, ctypes.c_double), sp,
                                  _ptr(codes, ctypes.c_uint8), _ptr(s8, ctypes.c_uint8),
                                  _ptr(z8, ctypes.c_uint8), _ptr(alpha, ctypes.c_uint16)),
           "encode_group")
    return codes, s8, z8, alpha


def reconstruct_group(p: Params, codes, s8, z8, alpha, signs, j: int) -> np.ndarray:
    args = [np.ascontiguousarray(codes, np.uint8), np.ascontiguousarray(s8, np.uint8),
            np.ascontiguousarray(z8, np.uint8), np.ascontiguousarray(alpha, np.uint16)]
    s, sp = _signs_ptr(signs, p.d)
    out = np.empty(p.d, np.float64)
    cp = p.c()
    _check(lib().rqo_reconstruct_group(
        ctypes.byref(cp), _ptr(args[0], ctypes.c_uint8), _ptr(args[1], ctypes.c_uint8),
        _ptr(args[2], ctypes.c_uint8), _ptr(args[3], ctypes.c_uint16), sp, j,
        _ptr(out, ctypes.c_double)), "reconstruct_group")
    return out


# ---------------------------------------------------------------- slices
@dataclass
class Encoded:
    codes: np.ndarray   # uint8 [L, N, d]
    s8: np.ndarray      # uint8 [L, N, ng]
    z8: np.ndarray      # uint8 [L, N, ng]
    alpha: np.ndarray   # uint16 [L, N]


def encode_slice(p: Params, x_bf16, signs=None) -> Encoded:
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    L, N, d = x.shape
    assert d == p.d
    s, sp = _signs_ptr(signs, d)
    e = Encoded(np.zeros((L, N, d), np.uint8), np.zeros((L, N, p.ng), np.uint8),
                np.zeros((L, N, p.ng), np.uint8), np.zeros((L, N), np.uint16))
    cp = p.c()
    _check(lib().rqo_encode_slice(ctypes.byref(cp), L, N, _ptr(x, ctypes.c_uint16), sp,
                                  _ptr(e.codes, ctypes.c_uint8), _ptr(e.s8, ctypes.c_uint8),
                                  _ptr(e.z8, ctypes.c_uint8), _ptr(e.alpha, ctypes.c_uint16)),
           "encode_slice")
    return e


def reconstruct_slice(p: Params, e: Encoded, signs, loop: int, t0: int = 0, t1=None) -> np.ndarray:
    L, N, d = e.codes.shape
    t1 = N if t1 is None else t1
    s, sp = _signs_ptr(signs, d)
    out = np.empty((t1 - t0, d), np.float64)
    cp = p.c()
    _check(lib().rqo_reconstruct_slice(
        ctypes.byref(cp), L, N, _ptr(e.codes, ctypes.c_uint8), _ptr(e.s8, ctypes.c_uint8),
        _ptr(e.z8, ctypes.c_uint8), _ptr(e.alpha, ctypes.c_uint16), sp,
        loop, t0, t1, _ptr(out, ctypes.c_double)), "reconstruct_slice")
    return out


def attention_dense(q, K, V, scale: float) -> np.ndarray:
    qq = np.ascontiguousarray(q, np.float64)
    KK = np.ascontiguousarray(K, np.float64)
    VV = np.ascontiguousarray(V, np.float64)
    n, d = KK.shape
    out = np.empty(d, np.float64)
    _check(lib().rqo_attention_dense(n, d, _ptr(qq, ctypes.c_double), _ptr(KK, ctypes.c_double),
                                     _ptr(VV, ctypes.c_double), scale,
                                     _ptr(out, ctypes.c_double)), "attention_dense")
    return out


def attention_slice(p: Params, ek: Encoded, ev: Encoded, signs_k, signs_v, q_bf16, loop: int,
                    n: int, scale: float, fused: bool = False) -> np.ndarray:
    L, N, d = ek.codes.shape
    q = np.ascontiguousarray(q_bf16, np.uint16)
    assert q.shape == (d,)
    sk, skp = _signs_ptr(signs_k, d)
    sv, svp = _signs_ptr(signs_v, d)
    out = np.empty(d, np.float64)
    cp = p.c()
    _check(lib().rqo_attention_slice(
        ctypes.byref(cp), L, N, n, loop, _ptr(q, ctypes.c_uint16), skp, svp,
        _ptr(ek.codes, ctypes.c_uint8), _ptr(ek.s8, ctypes.c_uint8), _ptr(ek.z8, ctypes.c_uint8),
        _ptr(ek.alpha, ctypes.c_uint16),
        _ptr(ev.codes, ctypes.c_uint8), _ptr(ev.s8, ctypes.c_uint8), _ptr(ev.z8, ctypes.c_uint8),
        _ptr(ev.alpha, ctypes.c_uint16), scale, 1 if fused else 0,
        _ptr(out, ctypes.c_double)), "attention_slice")
    return out


def bits_per_element(anchor_bits: int, residual_bits: int, g: int, d: int, P: int,
                     with_alpha: bool = True) -> float:
    return float(lib().rqo_bits_per_element(anchor_bits, residual_bits, g, d, P,
                                            1 if with_alpha else 0))
