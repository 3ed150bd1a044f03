"""ctypes front end of the CPU oracle (oracle/kivi_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use this module; the GPU library never imports it.

Arrays cross the boundary as numpy arrays; fp16 / bf16 tensors are passed as
their uint16 bit patterns.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kivi_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (IEEE fp32, no contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(
            os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "kivi_oracle.h"))):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        l = ctypes.CDLL(build())
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int, ctypes.c_int64
        l.or_half_to_float.restype = ctypes.c_float
        l.or_half_to_float.argtypes = [ctypes.c_uint16]
        l.or_bf16_to_float.restype = ctypes.c_float
        l.or_bf16_to_float.argtypes = [ctypes.c_uint16]
        l.or_half_to_float_array.argtypes = [P, P, i64]
        l.or_quant_group.argtypes = [P, i32, i32, P, P, P]
        l.or_pack_row.argtypes = [P, i32, i32, P]
        l.or_unpack_row.argtypes = [P, i32, i32, P]
        l.or_pack_rows.argtypes = [P, i64, i32, i32, P]
        l.or_cache_new.restype = P
        l.or_cache_new.argtypes = [i32] * 9
        l.or_cache_free.argtypes = [P]
        l.or_append.restype = i32
        l.or_append.argtypes = [P, P, P, i32]
        l.or_flush.restype = i64
        l.or_flush.argtypes = [P]
        l.or_state.argtypes = [P, P, P]
        l.or_unit_quantized.argtypes = [P, i32, P, P, P, P, P, P]
        l.or_unit_residual.argtypes = [P, i32, P, P]
        l.or_attend.restype = i32
        l.or_attend.argtypes = [P, P, i32, P]
        l.or_num_threads.restype = i32
        l.or_set_num_threads.argtypes = [i32]
        l.or_squat_token.argtypes = [P, P, P, P, i32, i32, P]
        l.or_squat_replay.argtypes = [P, P, P, P, i32, i32, P, P, P]
        l.or_cache_set_squat.argtypes = [P, P]
        _lib = l
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _bits16(a) -> np.ndarray:
    """fp16/bf16 tensor or array -> contiguous uint16 bit patterns."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().contiguous().view(torch.int16).numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    return np.ascontiguousarray(a.view(np.uint16))


def half_to_float(h) -> np.ndarray:
    h = _bits16(h)
    out = np.empty(h.shape, np.float32)
    lib().or_half_to_float_array(_ptr(h), _ptr(out), h.size)
    return out


def bf16_to_float(b: int) -> float:
    return float(lib().or_bf16_to_float(int(b)))


def quant_group(x, bits: int):
    """One group -> (codes uint8[n], s float32, z float32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.empty(x.size, np.uint8)
    s = np.empty(1, np.float32)
    z = np.empty(1, np.float32)
    lib().or_quant_group(_ptr(x), x.size, bits, _ptr(codes), _ptr(s), _ptr(z))
    return codes, s[0], z[0]


def pack_row(codes, bits: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    d = codes.size
    words = np.empty(d * bits // 32, np.uint32)
    lib().or_pack_row(_ptr(codes), d, bits, _ptr(words))
    return words


def pack_rows(codes, bits: int) -> np.ndarray:
    """[rows, d] codes -> [rows, d*bits/32] words."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    rows, d = codes.shape
    words = np.empty((rows, d * bits // 32), np.uint32)
    lib().or_pack_rows(_ptr(codes), rows, d, bits, _ptr(words))
    return words


def unpack_row(words, d: int, bits: int) -> np.ndarray:
    words = np.ascontiguousarray(words, dtype=np.uint32)
    codes = np.empty(d, np.uint8)
    lib().or_unpack_row(_ptr(words), d, bits, _ptr(codes))
    return codes


def num_threads() -> int:
    return int(lib().or_num_threads())


def set_num_threads(n: int) -> None:
    """OpenMP threads of the oracle's later calls."""
    lib().or_set_num_threads(int(n))


def squat_token(k, s, z, g, bits: int) -> np.ndarray:
    """SQuat-style codes of one key: k [d] fp32 (a widened fp16 key), s, z [d]
    fp32 (its block's per-channel statistics), g [d, d] fp32 update coefficients."""
    k, s, z = (np.ascontiguousarray(a, dtype=np.float32) for a in (k, s, z))
    g = np.ascontiguousarray(g, dtype=np.float32)
    codes = np.empty(k.size, np.uint8)
    lib().or_squat_token(_ptr(k), _ptr(s), _ptr(z), _ptr(g), k.size, bits, _ptr(codes))
    return codes


def squat_replay(k, s, z, g, bits: int, given):
    """The oracle's walk along the codes `given`: (own decisions uint8 [d],
    quotients (x - z) / s of its own trajectory, fp64 [d])."""
    k, s, z = (np.ascontiguousarray(a, dtype=np.float32) for a in (k, s, z))
    g = np.ascontiguousarray(g, dtype=np.float32)
    given = np.ascontiguousarray(given, dtype=np.uint8)
    own = np.empty(k.size, np.uint8)
    q = np.empty(k.size, np.float64)
    lib().or_squat_replay(_ptr(k), _ptr(s), _ptr(z), _ptr(g), k.size, bits, _ptr(given), _ptr(own), _ptr(q))
    return own, q


class OracleCache:
    """The oracle's cache: full fp16 history per (batch, KV head) unit,
    quantized token by token as the residual ring overflows or is flushed."""

    def __init__(self, batch, n_kv_heads, n_q_heads, head_dim, bits, max_tokens,
                 k_block=32, v_group=32, residual=128):
        self.batch, self.n_kv_heads, self.n_q_heads = batch, n_kv_heads, n_q_heads
        self.head_dim, self.bits, self.max_tokens = head_dim, bits, max_tokens
        self.k_block, self.v_group, self.residual = k_block, v_group, residual
        self._h = lib().or_cache_new(batch, n_kv_heads, n_q_heads, head_dim, bits,
                                     k_block, v_group, residual, max_tokens)
        if not self._h:
            raise MemoryError("oracle cache allocation failed")

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            lib().or_cache_free(h)
            self._h = None

    def append(self, k, v):
        k, v = _bits16(k), _bits16(v)
        assert k.shape == v.shape and k.ndim == 4
        assert k.shape[0] == self.batch and k.shape[1] == self.n_kv_heads and k.shape[3] == self.head_dim
        rc = lib().or_append(self._h, _ptr(k), _ptr(v), k.shape[2])
        if rc != 0:
            raise ValueError("oracle append beyond capacity")

    def flush(self) -> int:
        return int(lib().or_flush(self._h))

    def set_squat(self, g):
        """Key blocks quantized from now on take SQuat-style codes with the
        per-unit update coefficients g [units, d, d] (fp32)."""
        g = np.ascontiguousarray(g, dtype=np.float32)
        assert g.shape == (self.batch * self.n_kv_heads, self.head_dim, self.head_dim)
        lib().or_cache_set_squat(self._h, _ptr(g))

    def state(self):
        nt = ctypes.c_int64()
        nq = ctypes.c_int64()
        lib().or_state(self._h, ctypes.byref(nt), ctypes.byref(nq))
        return nt.value, nq.value

    def unit_quantized(self, unit: int):
        """(kcodes [n_q,d] u8, ks [n_q/G,d], kz, vcodes [n_q,d] u8, vs [n_q,d/vg], vz)."""
        _, nq = self.state()
        d, G, ng = self.head_dim, self.k_block, self.head_dim // self.v_group
        kc = np.zeros((nq, d), np.uint8)
        vc = np.zeros((nq, d), np.uint8)
        ks = np.zeros((nq // G, d), np.float32)
        kz = np.zeros((nq // G, d), np.float32)
        vs = np.zeros((nq, ng), np.float32)
        vz = np.zeros((nq, ng), np.float32)
        lib().or_unit_quantized(self._h, unit, _ptr(kc), _ptr(ks), _ptr(kz), _ptr(vc), _ptr(vs), _ptr(vz))
        return kc, ks, kz, vc, vs, vz

    def unit_residual(self, unit: int):
        """(kres, vres): fp16 bit patterns [n_res, d] in token order."""
        nt, nq = self.state()
        kr = np.zeros((nt - nq, self.head_dim), np.uint16)
        vr = np.zeros((nt - nq, self.head_dim), np.uint16)
        lib().or_unit_residual(self._h, unit, _ptr(kr), _ptr(vr))
        return kr, vr

    def attend(self, q, q_is_bf16: bool = False) -> np.ndarray:
        q = _bits16(q)
        assert q.shape == (self.batch, self.n_q_heads, self.head_dim)
        out = np.zeros(q.shape, np.float64)
        rc = lib().or_attend(self._h, _ptr(q), int(bool(q_is_bf16)), _ptr(out))
        if rc != 0:
            raise ValueError("oracle attend on an empty cache")
        return out
