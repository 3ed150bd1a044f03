"""ctypes binding of libkivi.so (include/kivi.h), argument marshalling only."""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkivi.so")
# KIVI_ABI_VERSION of include/kivi.h that the structures below mirror
ABI_VERSION = 5

KIVI_F16 = 0
KIVI_BF16 = 1

STATUS = {
    0: "KIVI_OK", -1: "KIVI_E_INVAL", -2: "KIVI_E_UNSUPPORTED", -3: "KIVI_E_NOMEM",
    -4: "KIVI_E_CAPACITY", -5: "KIVI_E_EMPTY", -6: "KIVI_E_DEVICE", -7: "KIVI_E_STATE", -8: "KIVI_E_RAGGED",
}


class KiviError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{STATUS.get(code, code)}: {message}")
        self.code = code
        self.status = STATUS.get(code, str(code))


class kivi_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_kv_heads", "n_q_heads", "head_dim", "bits", "k_block", "v_group",
        "residual", "max_tokens", "max_splits", "n_pages", "squat_rank")]


class kivi_layout(ctypes.Structure):
    _fields_ = [
        ("total_bytes", ctypes.c_size_t),
        ("off_blocks", ctypes.c_size_t), ("unit_stride", ctypes.c_size_t), ("block_bytes", ctypes.c_size_t),
        ("rec_kcode", ctypes.c_size_t), ("rec_vcode", ctypes.c_size_t),
        ("rec_ksz", ctypes.c_size_t), ("rec_vsz", ctypes.c_size_t),
        ("max_blocks", ctypes.c_int64),
        ("off_ring", ctypes.c_size_t), ("ring_unit_stride", ctypes.c_size_t),
        ("ring_slots", ctypes.c_int64),
        ("off_partial", ctypes.c_size_t), ("partial_stride", ctypes.c_size_t),
        ("max_splits", ctypes.c_int32),
        ("n_pages", ctypes.c_int32), ("page_bytes", ctypes.c_size_t),
        ("off_squat", ctypes.c_size_t), ("squat_r8", ctypes.c_int32), ("squat_unit_bytes", ctypes.c_size_t),
    ]


class kivi_state(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int64), ("n_quant", ctypes.c_int64), ("n_resid", ctypes.c_int64)]


_lib = None

# name -> (restype, argtypes)
_P = ctypes.c_void_p
_SIGS = {
    "kivi_abi_version": (ctypes.c_int, []),
    "kivi_last_error": (ctypes.c_char_p, []),
    "kivi_cache_bytes": (ctypes.c_int, [ctypes.POINTER(kivi_config), ctypes.POINTER(ctypes.c_size_t)]),
    "kivi_cache_layout": (ctypes.c_int, [ctypes.POINTER(kivi_config), ctypes.POINTER(kivi_layout)]),
    "kivi_cache_create": (ctypes.c_int, [ctypes.POINTER(kivi_config), _P, ctypes.c_size_t, ctypes.POINTER(_P)]),
    "kivi_cache_destroy": (ctypes.c_int, [_P]),
    "kivi_cache_reset": (ctypes.c_int, [_P]),
    "kivi_append": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, _P]),
    "kivi_flush": (ctypes.c_int, [_P, _P, ctypes.POINTER(ctypes.c_int32)]),
    "kivi_attend_decode": (ctypes.c_int, [_P, _P, ctypes.c_int32, _P, _P]),
    "kivi_attend_decode_noalloc": (ctypes.c_int, [_P, _P, ctypes.c_int32, _P, _P]),
    "kivi_squat_build": (ctypes.c_int, [_P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, _P]),
    "kivi_cache_query": (ctypes.c_int, [_P, ctypes.POINTER(kivi_state)]),
    "kivi_plan_append": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.POINTER(kivi_state)]),
    "kivi_plan_attend": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]),
    "kivi_set_attend_splits": (ctypes.c_int, [_P, ctypes.c_int32]),
    "kivi_decode_step": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int32, _P, _P, ctypes.POINTER(ctypes.c_int32)]),
    "kivi_append_rows": (ctypes.c_int, [_P, _P, _P, ctypes.POINTER(ctypes.c_int32), ctypes.c_int32, _P]),
    "kivi_reset_row": (ctypes.c_int, [_P, ctypes.c_int32]),
    "kivi_set_block_table": (ctypes.c_int, [_P, _P, ctypes.c_int32]),
    "kivi_query_row": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.POINTER(kivi_state)]),
}

EXPORTED = tuple(_SIGS)


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libkivi.so; fails loudly when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with kv_cache_compression_kivi_amd/build.py "
                               "(or __graft_entry__.build()) before using the library")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if lib.kivi_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{_LIB_PATH} has ABI version {lib.kivi_abi_version()}, the binding expects "
                               f"{ABI_VERSION}: rebuild it")
        _lib = lib
    return _lib


def _check(rc: int):
    if rc != 0:
        raise KiviError(rc, kivi_last_error())


def kivi_abi_version() -> int:
    return int(load_library().kivi_abi_version())


def kivi_last_error() -> str:
    msg = load_library().kivi_last_error()
    return msg.decode() if msg else ""


def kivi_cache_bytes(cfg: kivi_config) -> int:
    n = ctypes.c_size_t()
    _check(load_library().kivi_cache_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def kivi_cache_layout(cfg: kivi_config) -> kivi_layout:
    L = kivi_layout()
    _check(load_library().kivi_cache_layout(ctypes.byref(cfg), ctypes.byref(L)))
    return L


def kivi_cache_create(cfg: kivi_config, dev_ptr: int, nbytes: int) -> int:
    h = ctypes.c_void_p()
    _check(load_library().kivi_cache_create(ctypes.byref(cfg), ctypes.c_void_p(dev_ptr), nbytes, ctypes.byref(h)))
    return h.value


def kivi_cache_destroy(h: int) -> None:
    _check(load_library().kivi_cache_destroy(ctypes.c_void_p(h)))


def kivi_cache_reset(h: int) -> None:
    _check(load_library().kivi_cache_reset(ctypes.c_void_p(h)))


def kivi_append(h: int, k_ptr: int, v_ptr: int, ntok: int, stream: int = 0) -> None:
    _check(load_library().kivi_append(ctypes.c_void_p(h), ctypes.c_void_p(k_ptr), ctypes.c_void_p(v_ptr),
                                      ntok, ctypes.c_void_p(stream)))


def kivi_append_rows(h: int, k_ptr: int, v_ptr: int, ntok, max_ntok: int, stream: int = 0) -> None:
    arr = (ctypes.c_int32 * len(ntok))(*[int(x) for x in ntok])
    _check(load_library().kivi_append_rows(ctypes.c_void_p(h), ctypes.c_void_p(k_ptr), ctypes.c_void_p(v_ptr),
                                           arr, max_ntok, ctypes.c_void_p(stream)))


def kivi_set_block_table(h: int, table_ptr: int, stride: int) -> None:
    _check(load_library().kivi_set_block_table(ctypes.c_void_p(h), ctypes.c_void_p(table_ptr), stride))


def kivi_reset_row(h: int, row: int) -> None:
    _check(load_library().kivi_reset_row(ctypes.c_void_p(h), row))


def kivi_query_row(h: int, row: int) -> kivi_state:
    st = kivi_state()
    _check(load_library().kivi_query_row(ctypes.c_void_p(h), row, ctypes.byref(st)))
    return st


def kivi_flush(h: int, stream: int = 0) -> int:
    n = ctypes.c_int32()
    _check(load_library().kivi_flush(ctypes.c_void_p(h), ctypes.c_void_p(stream), ctypes.byref(n)))
    return n.value


def kivi_attend_decode(h: int, q_ptr: int, q_dtype: int, out_ptr: int, stream: int = 0) -> None:
    _check(load_library().kivi_attend_decode(ctypes.c_void_p(h), ctypes.c_void_p(q_ptr), q_dtype,
                                             ctypes.c_void_p(out_ptr), ctypes.c_void_p(stream)))


def kivi_attend_decode_noalloc(h: int, q_ptr: int, q_dtype: int, out_ptr: int, stream: int = 0) -> None:
    _check(load_library().kivi_attend_decode_noalloc(ctypes.c_void_p(h), ctypes.c_void_p(q_ptr), q_dtype,
                                                     ctypes.c_void_p(out_ptr), ctypes.c_void_p(stream)))


def kivi_decode_step(h: int, k_ptr: int, v_ptr: int, q_ptr: int, q_dtype: int, out_ptr: int,
                     stream: int = 0) -> int:
    n = ctypes.c_int32()
    _check(load_library().kivi_decode_step(ctypes.c_void_p(h), ctypes.c_void_p(k_ptr), ctypes.c_void_p(v_ptr),
                                           ctypes.c_void_p(q_ptr), q_dtype, ctypes.c_void_p(out_ptr),
                                           ctypes.c_void_p(stream), ctypes.byref(n)))
    return n.value


def kivi_cache_query(h: int) -> kivi_state:
    st = kivi_state()
    _check(load_library().kivi_cache_query(ctypes.c_void_p(h), ctypes.byref(st)))
    return st


def kivi_plan_append(h: int, ntok: int) -> kivi_state:
    st = kivi_state()
    _check(load_library().kivi_plan_append(ctypes.c_void_p(h), ntok, ctypes.byref(st)))
    return st


def kivi_plan_attend(h: int):
    n = ctypes.c_int32()
    bps = ctypes.c_int32()
    _check(load_library().kivi_plan_attend(ctypes.c_void_p(h), ctypes.byref(n), ctypes.byref(bps)))
    return n.value, bps.value


def kivi_set_attend_splits(h: int, n_key_splits: int) -> None:
    _check(load_library().kivi_set_attend_splits(ctypes.c_void_p(h), n_key_splits))


def kivi_squat_build(h: int, q_ptr: int, q_dtype: int, n_q: int, lam: float, stream: int = 0) -> None:
    _check(load_library().kivi_squat_build(ctypes.c_void_p(h), ctypes.c_void_p(q_ptr), q_dtype, n_q, lam,
                                           ctypes.c_void_p(stream)))


def make_config(batch, n_kv_heads, n_q_heads, head_dim, bits, max_tokens, residual=128, k_block=32,
                v_group=32, max_splits=0, n_pages=0, squat_rank=0) -> kivi_config:
    return kivi_config(batch, n_kv_heads, n_q_heads, head_dim, bits, k_block, v_group, residual, max_tokens,
                       max_splits, n_pages, squat_rank)


class KiviCache:
    """Owns one cache: its device memory (a torch uint8 tensor) and the handle.

    Tensors are passed by device pointer on torch's current stream, or on the
    stream given as `stream=` (a torch.cuda.Stream or a raw hipStream_t int).
    """

    def __init__(self, batch, n_kv_heads, n_q_heads, head_dim, bits, max_tokens, residual=128,
                 k_block=32, v_group=32, max_splits=0, device="cuda", memory=None, n_pages=0, squat_rank=0):
        import torch
        self.cfg = make_config(batch, n_kv_heads, n_q_heads, head_dim, bits, max_tokens, residual,
                               k_block, v_group, max_splits, n_pages, squat_rank)
        self.block_table = None
        self.nbytes = kivi_cache_bytes(self.cfg)
        self.layout = kivi_cache_layout(self.cfg)
        if memory is None:
            memory = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        assert memory.dtype == torch.uint8 and memory.numel() >= self.nbytes and memory.is_contiguous()
        self.memory = memory
        self.handle = kivi_cache_create(self.cfg, memory.data_ptr(), memory.numel())

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            try:
                kivi_cache_destroy(h)
            except Exception:
                pass
            self.handle = None

    @staticmethod
    def _stream(stream):
        import torch
        if stream is None:
            return torch.cuda.current_stream().cuda_stream
        if isinstance(stream, int):
            return stream
        return stream.cuda_stream

    def _check_kv(self, k, v):
        import torch
        c = self.cfg
        for t in (k, v):
            if t.dtype != torch.float16 or not t.is_cuda or not t.is_contiguous():
                raise ValueError("k and v must be contiguous fp16 device tensors")
            if t.dim() != 4 or t.shape[0] != c.batch or t.shape[1] != c.n_kv_heads or t.shape[3] != c.head_dim:
                raise ValueError(f"k and v must be [batch, n_kv_heads, ntok, head_dim], got {tuple(t.shape)}")
        if k.shape != v.shape:
            raise ValueError("k and v shapes differ")

    def append(self, k, v, stream=None):
        self._check_kv(k, v)
        kivi_append(self.handle, k.data_ptr(), v.data_ptr(), int(k.shape[2]), self._stream(stream))

    def append_rows(self, k, v, ntok, stream=None):
        """Append ntok[b] tokens to sequence b: k, v are [batch, n_kv_heads, max_ntok,
        head_dim] fp16 and row b's tokens are its first ntok[b] slots."""
        self._check_kv(k, v)
        ntok = [int(x) for x in ntok]
        if len(ntok) != self.cfg.batch:
            raise ValueError(f"ntok must have {self.cfg.batch} entries, got {len(ntok)}")
        kivi_append_rows(self.handle, k.data_ptr(), v.data_ptr(), ntok, int(k.shape[2]), self._stream(stream))

    def set_block_table(self, table):
        """Paged caches: `table` is a device int32 [batch, stride] tensor (stride >=
        max_blocks) mapping (row, block) to a page; it is kept referenced here."""
        import torch
        if table.dtype != torch.int32 or not table.is_cuda or not table.is_contiguous() or table.dim() != 2 \
                or table.shape[0] != self.cfg.batch:
            raise ValueError("the block table must be a contiguous int32 [batch, stride] device tensor")
        kivi_set_block_table(self.handle, table.data_ptr(), int(table.shape[1]))
        self.block_table = table

    def reset_row(self, row):
        kivi_reset_row(self.handle, row)

    def row_state(self, row):
        st = kivi_query_row(self.handle, row)
        return st.n_tokens, st.n_quant, st.n_resid

    def flush(self, stream=None) -> int:
        return kivi_flush(self.handle, self._stream(stream))

    def attend(self, q, out=None, stream=None):
        import torch
        c = self.cfg
        if q.dtype not in (torch.float16, torch.bfloat16) or not q.is_cuda or not q.is_contiguous():
            raise ValueError("q must be a contiguous fp16 or bf16 device tensor")
        if tuple(q.shape) != (c.batch, c.n_q_heads, c.head_dim):
            raise ValueError(f"q must be [batch, n_q_heads, head_dim], got {tuple(q.shape)}")
        if out is None:
            out = torch.empty((c.batch, c.n_q_heads, c.head_dim), dtype=torch.float32, device=q.device)
        elif out.dtype != torch.float32 or not out.is_contiguous() or tuple(out.shape) != tuple(q.shape):
            raise ValueError("out must be a contiguous float32 tensor shaped like q")
        kivi_attend_decode(self.handle, q.data_ptr(), KIVI_BF16 if q.dtype == torch.bfloat16 else KIVI_F16,
                           out.data_ptr(), self._stream(stream))
        return out

    def decode_step(self, k, v, q, out=None, stream=None) -> int:
        """append(1) + flush when a full group is past the residual + attend, in one
        call; returns the output (the tokens flushed are in self.last_flushed)."""
        import torch
        self._check_kv(k, v)
        c = self.cfg
        if k.shape[2] != 1:
            raise ValueError("decode_step appends exactly one token per sequence")
        if q.dtype not in (torch.float16, torch.bfloat16) or not q.is_contiguous() or \
                tuple(q.shape) != (c.batch, c.n_q_heads, c.head_dim):
            raise ValueError("q must be a contiguous fp16/bf16 [batch, n_q_heads, head_dim] tensor")
        if out is None:
            out = torch.empty((c.batch, c.n_q_heads, c.head_dim), dtype=torch.float32, device=q.device)
        n = kivi_decode_step(self.handle, k.data_ptr(), v.data_ptr(), q.data_ptr(),
                             KIVI_BF16 if q.dtype == torch.bfloat16 else KIVI_F16, out.data_ptr(),
                             self._stream(stream))
        self.last_flushed = n
        return out

    def state(self):
        st = kivi_cache_query(self.handle)
        return st.n_tokens, st.n_quant, st.n_resid

    def plan_append(self, ntok):
        st = kivi_plan_append(self.handle, ntok)
        return st.n_tokens, st.n_quant, st.n_resid

    def plan_attend(self):
        return kivi_plan_attend(self.handle)

    def set_attend_splits(self, n):
        kivi_set_attend_splits(self.handle, n)

    def squat_build(self, q_hist, lam=0.1, stream=None):
        """Update coefficients of the SQuat-style key coder from past queries
        q_hist [batch, n_q_heads, n_q, head_dim] (fp16 or bf16, on the device)."""
        import torch
        c = self.cfg
        if q_hist.dtype not in (torch.float16, torch.bfloat16) or not q_hist.is_cuda or \
                not q_hist.is_contiguous() or q_hist.dim() != 4 or \
                tuple(q_hist.shape[:2]) != (c.batch, c.n_q_heads) or q_hist.shape[3] != c.head_dim:
            raise ValueError("q_hist must be a contiguous fp16/bf16 [batch, n_q_heads, n_q, head_dim] device tensor")
        kivi_squat_build(self.handle, q_hist.data_ptr(), KIVI_BF16 if q_hist.dtype == torch.bfloat16 else KIVI_F16,
                         q_hist.shape[2], float(lam), self._stream(stream))

    def squat_factors(self, unit):
        """Unit's coder coefficients as the device holds them: (U, W), each
        [head_dim, squat_r8] fp32 (row c: u_c, w_c)."""
        import torch
        d, r8 = self.cfg.head_dim, self.layout.squat_r8
        start = self.layout.off_squat + unit * self.layout.squat_unit_bytes
        f = self.memory[start:start + self.layout.squat_unit_bytes].view(torch.float32).reshape(2, d, r8)
        return f[0], f[1]

    def reset(self):
        kivi_cache_reset(self.handle)
