"""Python binding of the host block manager and two-phase scheduler.

Argument marshalling only: the rules run in the C++ code of
``libphoton_decode.so`` (csrc/scheduler.cpp), declared in
``include/photon_sched.h``.  :meth:`Scheduler.schedule` returns numpy arrays
ready to upload as the decode path's inputs.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import ERR_INVALID_ARG, PhotonError, check, lib

_i32, _i64 = ctypes.c_int32, ctypes.c_int64
_P32, _P64 = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)


class SchedConfig(ctypes.Structure):
    _fields_ = [("num_blocks", _i32), ("block_size", _i32), ("max_seqs", _i32),
                ("max_tokens_per_step", _i32), ("max_blocks_per_seq", _i32)]


class SchedBatch(ctypes.Structure):
    _fields_ = [("num_seqs", _i32), ("num_tokens", _i32), ("num_preempted", _i32),
                ("reserved", _i32), ("request_ids", _P64), ("query_start", _P32),
                ("context_lens", _P32), ("block_tables", _P32), ("slot_mapping", _P32),
                ("positions", _P32), ("preempted_ids", _P64)]


class SchedRequestInfo(ctypes.Structure):
    _fields_ = [("state", _i32), ("num_computed", _i32), ("num_known", _i32),
                ("num_generated", _i32), ("num_blocks", _i32), ("num_preemptions", _i32)]


_vp = ctypes.c_void_p
lib.photon_sched_create.argtypes = [ctypes.POINTER(SchedConfig), ctypes.POINTER(_vp)]
lib.photon_sched_create.restype = ctypes.c_int
lib.photon_sched_destroy.argtypes = [_vp]
lib.photon_sched_destroy.restype = None
lib.photon_sched_add_request.argtypes = [_vp, _i64, _i32, _i32]
lib.photon_sched_add_request.restype = ctypes.c_int
lib.photon_sched_schedule.argtypes = [_vp, ctypes.POINTER(SchedBatch)]
lib.photon_sched_schedule.restype = ctypes.c_int
lib.photon_sched_update.argtypes = [_vp, _P32, _P64]
lib.photon_sched_update.restype = ctypes.c_int
lib.photon_sched_counts.argtypes = [_vp, _P32, _P32, _P32, _P32]
lib.photon_sched_counts.restype = ctypes.c_int
lib.photon_sched_request.argtypes = [_vp, _i64, ctypes.POINTER(SchedRequestInfo)]
lib.photon_sched_request.restype = ctypes.c_int


def _p(a, kind):
    return a.ctypes.data_as(kind)


class Scheduler:
    """Owner of one native scheduler; arrays returned by schedule() are fresh copies."""

    def __init__(self, num_blocks: int, block_size: int, max_seqs: int, max_tokens_per_step: int,
                 max_blocks_per_seq: int):
        self.config = SchedConfig(num_blocks, block_size, max_seqs, max_tokens_per_step,
                                  max_blocks_per_seq)
        h = _vp()
        self._h = None
        self._destroy = lib.photon_sched_destroy  # kept for close() at interpreter exit
        check(lib.photon_sched_create(ctypes.byref(self.config), ctypes.byref(h)))
        self._h = h
        ms, mt, mb = max_seqs, max_tokens_per_step, max_blocks_per_seq
        self._ids = np.zeros(ms, np.int64)
        self._qs = np.zeros(ms + 1, np.int32)
        self._ctx = np.zeros(ms, np.int32)
        self._tables = np.zeros((ms, mb), np.int32)
        self._slots = np.zeros(mt, np.int32)
        self._pos = np.zeros(mt, np.int32)
        self._pre = np.zeros(ms, np.int64)
        self._fin = np.zeros(ms, np.int64)
        # the arrays never move, so one batch descriptor serves every step
        self._batch = SchedBatch(0, 0, 0, 0, _p(self._ids, _P64), _p(self._qs, _P32),
                                 _p(self._ctx, _P32), _p(self._tables, _P32), _p(self._slots, _P32),
                                 _p(self._pos, _P32), _p(self._pre, _P64))
        self._nfin = _i32(0)
        self._fin_p = _p(self._fin, _P64)

    def close(self) -> None:
        if getattr(self, "_h", None):
            self._destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def add_request(self, request_id: int, prompt_len: int, max_new_tokens: int) -> None:
        check(lib.photon_sched_add_request(self._h, int(request_id), int(prompt_len),
                                           int(max_new_tokens)))

    def schedule(self) -> dict:
        b = self._batch
        check(lib.photon_sched_schedule(self._h, ctypes.byref(b)))
        n, t = b.num_seqs, b.num_tokens
        return {"request_ids": self._ids[:n].copy(), "query_start": self._qs[:n + 1].copy(),
                "context_lens": self._ctx[:n].copy(), "block_tables": self._tables[:n].copy(),
                "slot_mapping": self._slots[:t].copy(), "positions": self._pos[:t].copy(),
                "preempted": self._pre[:b.num_preempted].copy()}

    def update(self) -> np.ndarray:
        check(lib.photon_sched_update(self._h, ctypes.byref(self._nfin), self._fin_p))
        return self._fin[:self._nfin.value].copy()

    def counts(self) -> dict:
        v = [_i32(0) for _ in range(4)]
        check(lib.photon_sched_counts(self._h, *[ctypes.byref(x) for x in v]))
        return dict(zip(("waiting", "running", "finished", "free_blocks"), (x.value for x in v)))

    def request(self, request_id: int) -> dict:
        info = SchedRequestInfo()
        check(lib.photon_sched_request(self._h, int(request_id), ctypes.byref(info)))
        return {f: getattr(info, f) for f, _ in SchedRequestInfo._fields_}


__all__ = ["Scheduler", "SchedConfig", "SchedBatch", "SchedRequestInfo", "PhotonError",
           "ERR_INVALID_ARG"]
