"""CPU oracle for batched paged-attention decode (TEST INFRASTRUCTURE ONLY).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product library never links, loads or calls it.

The arithmetic lives in ``photon_oracle.c`` (plain C, fp64, optional OpenMP
over independent (sequence, head) pairs); this module builds it with gcc and
wraps it with ctypes, marshalling numpy arrays only.

Rotary embedding (``rope``, ``rope_kv_cache_write``) is pinned against
transformers' GPT-J and Llama rotary routines and against the rotation
group's identities (see ``tests/test_oracle_rope.py``).

Parity pins (all in ``tests/test_oracle_*.py``): hand-derived golden cases,
dense attention through ``torch.nn.functional.scaled_dot_product_attention``,
closed forms (one token, constant V, zero query, dominant key), invariance
under a permutation of physical blocks, GQA equal to MHA with repeated KV
heads, softmax rows summing to one, the binary16 and bfloat16 decoders over
all 65536 bit patterns each, brute-force cache writes and the precondition error codes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "photon_oracle.c")
_LIB = os.path.join(_HERE, "libphoton_oracle.so")

OK = 0
ERR_ARG = 1
ERR_SLOT_RANGE = 2
ERR_SLOT_DUP = 3
ERR_BLOCK_RANGE = 4
ERR_CTX = 5
ERR_HEADS = 6

# Storage types: float32, float16, and bfloat16 held as a one-field record of
# its 16 bits (the input module's ``BF16``; any uint16 record dtype is read as
# bfloat16 bits).
_BF16 = np.dtype([("bf16", "<u2")])
_DTYPE_CODE = {np.dtype(np.float32): 0, np.dtype(np.float16): 1, _BF16: 2}


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: oracle error code {code}")
        self.code = code


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _configure(lib):
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_half_to_double.restype = ctypes.c_double
    lib.oracle_bfloat16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bfloat16_to_double.restype = ctypes.c_double
    lib.oracle_kv_cache_write.argtypes = [vp, vp, vp, i64, vp, vp, i64, i64, i64, i64, i64]
    lib.oracle_kv_cache_write.restype = ctypes.c_int
    lib.oracle_paged_attn_decode.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                             i64, ctypes.c_int, ctypes.c_double, vp, vp,
                                             ctypes.c_int]
    lib.oracle_paged_attn_decode.restype = ctypes.c_int
    lib.oracle_paged_attn_multi_query.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                                  i64, i64, ctypes.c_int, ctypes.c_double, vp,
                                                  ctypes.c_int]
    lib.oracle_paged_attn_multi_query.restype = ctypes.c_int
    lib.oracle_rope.argtypes = [vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_double, ctypes.c_int,
                                vp]
    lib.oracle_rope.restype = ctypes.c_int
    lib.oracle_widen.argtypes = [vp, i64, ctypes.c_int, vp]
    lib.oracle_widen.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        _lib = _configure(ctypes.CDLL(build()))
    return _lib


class use_library:
    """Context manager that points this module at another build of the oracle.

    Used by the mutation test, which compiles copies of the oracle with a
    planted mistake and checks that the pins reject each of them.
    """

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self._saved = _lib
        _lib = _configure(ctypes.CDLL(self.path))
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self._saved
        return False


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def half_to_double(bits: int) -> float:
    return _load().oracle_half_to_double(int(bits) & 0xFFFF)


def bfloat16_to_double(bits: int) -> float:
    return _load().oracle_bfloat16_to_double(int(bits) & 0xFFFF)


def max_threads() -> int:
    return _load().oracle_max_threads()


def kv_cache_write(k: np.ndarray, v: np.ndarray, slot_mapping: np.ndarray,
                   k_cache: np.ndarray, v_cache: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """New (k_cache, v_cache) after writing token i's rows to ``slot_mapping[i]``.

    k, v: [T, Hkv, D]; pools: [NB, Hkv, bs, D], same dtype.  Inputs are not
    modified.  Raises OracleError on a slot out of range or a repeated slot.
    """
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int32)
    kc = np.array(k_cache, copy=True, order="C")
    vc = np.array(v_cache, copy=True, order="C")
    if k.dtype != kc.dtype or v.dtype != kc.dtype or vc.dtype != kc.dtype:
        raise OracleError(ERR_ARG, "dtype mismatch")
    nb, hkv, bs, d = kc.shape
    if k.shape != (len(slots), hkv, d) or v.shape != k.shape or vc.shape != kc.shape:
        raise OracleError(ERR_ARG, "shape mismatch")
    rc = _load().oracle_kv_cache_write(_ptr(k), _ptr(v), _ptr(slots), len(slots), _ptr(kc),
                                       _ptr(vc), nb, hkv, bs, d, kc.dtype.itemsize)
    if rc != OK:
        raise OracleError(rc, "kv_cache_write")
    return kc, vc


def paged_attn_decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                      block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
                      return_probs: bool = False, num_threads: int = 0):
    """fp64 decode attention; returns out [B, Hq, D] (and probs [B, Hq, max_blocks*bs])."""
    q = np.ascontiguousarray(q)
    kc = np.ascontiguousarray(k_cache)
    vc = np.ascontiguousarray(v_cache)
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    if q.dtype not in _DTYPE_CODE or kc.dtype != q.dtype or vc.dtype != q.dtype:
        raise OracleError(ERR_ARG, "dtype")
    b, hq, d = q.shape
    nb, hkv, bs, d2 = kc.shape
    if d2 != d or vc.shape != kc.shape or tables.ndim != 2 or tables.shape[0] != b \
            or lens.shape != (b,):
        raise OracleError(ERR_ARG, "shape mismatch")
    mb = tables.shape[1]
    # NaN-filled so that any output row the C code fails to write shows up.
    out = np.full((b, hq, d), np.nan, dtype=np.float64)
    probs = np.zeros((b, hq, mb * bs), dtype=np.float64) if return_probs else None
    rc = _load().oracle_paged_attn_decode(_ptr(q), _ptr(kc), _ptr(vc), _ptr(tables), _ptr(lens),
                                          b, hq, hkv, d, bs, nb, mb, _DTYPE_CODE[q.dtype],
                                          float(scale), _ptr(out), _ptr(probs), int(num_threads))
    if rc != OK:
        raise OracleError(rc, "paged_attn_decode")
    return (out, probs) if return_probs else out


def _code(a: np.ndarray) -> int:
    if a.dtype not in _DTYPE_CODE:
        raise OracleError(ERR_ARG, f"dtype {a.dtype}")
    return _DTYPE_CODE[a.dtype]


def widen(a: np.ndarray) -> np.ndarray:
    """Exact float64 values of a float32 / float16 / bfloat16 storage array."""
    a = np.ascontiguousarray(a)
    out = np.empty(a.shape, dtype=np.float64)
    rc = _load().oracle_widen(_ptr(a), a.size, _code(a), _ptr(out))
    if rc != OK:
        raise OracleError(rc, "widen")
    return out


def rope(x: np.ndarray, positions: np.ndarray, base: float, interleaved: bool = False) -> np.ndarray:
    """fp64 rotary embedding of x [T, H, D] at ``positions`` [T] (see photon_oracle.c)."""
    x = np.ascontiguousarray(x)
    pos = np.ascontiguousarray(positions, dtype=np.int32)
    t, h, d = x.shape
    if pos.shape != (t,):
        raise OracleError(ERR_ARG, "positions shape")
    out = np.full(x.shape, np.nan, dtype=np.float64)
    rc = _load().oracle_rope(_ptr(x), _ptr(pos), t, h, d, _code(x), float(base), int(interleaved),
                             _ptr(out))
    if rc != OK:
        raise OracleError(rc, "rope")
    return out


def rope_kv_cache_write(q, k, v, positions, slot_mapping, k_cache, v_cache, base: float,
                        interleaved: bool = False):
    """Rotary embedding of q and k, then the slot-mapped write of rotated k and raw v.

    Returns (q_out [T, Hq, D] float64, k_cache as float64 with the rotated rows
    of written slots in place, v_cache in the pool dtype after a raw-byte
    write).  Slot checks are those of :func:`kv_cache_write`.
    """
    q_out = rope(q, positions, base, interleaved)
    k_rot = rope(k, positions, base, interleaved)
    _, v_new = kv_cache_write(k, v, slot_mapping, k_cache, v_cache)
    k_new = widen(k_cache)
    bs = k_cache.shape[2]
    for i, s in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if s >= 0:
            k_new[s // bs, :, s % bs, :] = k_rot[i]
    return q_out, k_new, v_new


def paged_attn_multi_query(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                           block_tables: np.ndarray, context_lens: np.ndarray,
                           query_start: np.ndarray, scale: float, num_threads: int = 0) -> np.ndarray:
    """fp64 multi-query attention with a causal tail; returns out [T, Hq, D].

    Sequence b owns q rows query_start[b] .. query_start[b+1]-1, the last
    n_b of its context_lens[b] tokens; row j attends to positions
    <= context_lens[b] - n_b + j.
    """
    q = np.ascontiguousarray(q)
    kc = np.ascontiguousarray(k_cache)
    vc = np.ascontiguousarray(v_cache)
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    qs = np.ascontiguousarray(query_start, dtype=np.int32)
    if q.dtype not in _DTYPE_CODE or kc.dtype != q.dtype or vc.dtype != q.dtype:
        raise OracleError(ERR_ARG, "dtype")
    t, hq, d = q.shape
    nb, hkv, bs, d2 = kc.shape
    b = len(lens)
    if d2 != d or vc.shape != kc.shape or tables.ndim != 2 or tables.shape[0] != b \
            or qs.shape != (b + 1,) or (b and qs[-1] != t):
        raise OracleError(ERR_ARG, "shape mismatch")
    out = np.full((t, hq, d), np.nan, dtype=np.float64)
    rc = _load().oracle_paged_attn_multi_query(_ptr(q), _ptr(kc), _ptr(vc), _ptr(tables), _ptr(lens),
                                               _ptr(qs), b, hq, hkv, d, bs, nb, tables.shape[1],
                                               _code(q), float(scale), _ptr(out), int(num_threads))
    if rc != OK:
        raise OracleError(rc, "paged_attn_multi_query")
    return out
