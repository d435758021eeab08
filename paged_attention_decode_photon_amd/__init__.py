"""Python binding of the MI355X paged-attention decode library.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libphoton_decode.so`` (built from ``csrc/`` by ``build.py``).
Functions take torch tensors on a ROCm device, pass their data pointers and
the current HIP stream through the C ABI declared in
``include/photon_decode.h``, and raise :class:`PhotonError` on a non-OK
status.  There is no fallback: the library is loaded on the first call
that needs it (or the first access to ``lib``), and that call raises
ImportError if the library is missing.  Importing the package itself loads
nothing, so ``python -m paged_attention_decode_photon_amd.build`` works on a
fresh checkout.

The library must run inside the same HIP runtime as PyTorch (it uses torch's
streams and allocations), so torch is imported before the library is loaded:
the dynamic loader then binds the library's ``libamdhip64.so.7`` dependency
to the copy torch already mapped.  Loading fails if two runtimes end up
mapped.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libphoton_decode.so")

OK = 0
ERR_INVALID_ARG = 1
ERR_UNSUPPORTED = 2
ERR_WORKSPACE = 3
ERR_HIP = 4

F32 = 0
F16 = 1
BF16 = 2

DECODE_OUT_F32 = 1  # photon_decode_desc.flags: fp32 output for 16-bit storage

BLOCK_SIZE = 16

NOALLOC_SCRATCH_BYTES = 32 << 20  # PHOTON_NOALLOC_SCRATCH_BYTES


class PhotonError(RuntimeError):
    """A photon_* call returned a non-OK status."""

    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: {detail}" if detail else name)
        self.status = status
        self.name = name
        self.detail = detail


class KvDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class DecodeDesc(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("max_context_len", ctypes.c_int32),
                ("partition_tokens", ctypes.c_int32), ("kv", KvDesc), ("flags", ctypes.c_int32)]


class MultiQueryDesc(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_tokens", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("max_query_len", ctypes.c_int32), ("max_context_len", ctypes.c_int32),
                ("split_tokens", ctypes.c_int32), ("flags", ctypes.c_int32), ("kv", KvDesc)]


class RopeDesc(ctypes.Structure):
    _fields_ = [("base", ctypes.c_double), ("adjacent_pairs", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


def _hip_runtimes_mapped() -> set[str]:
    try:
        with open("/proc/self/maps") as f:
            return {ln.split()[-1] for ln in f if "libamdhip64" in ln}
    except OSError:
        return set()


def _load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    import torch  # noqa: F401  (maps torch's HIP runtime first; see module docstring)

    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m paged_attention_decode_photon_amd.build`")
    lib = ctypes.CDLL(path)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise ImportError(f"two HIP runtimes are mapped ({sorted(runtimes)}); the decode library "
                          "must share PyTorch's")
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    st = ctypes.c_int
    lib.photon_kv_cache_write.argtypes = [vp, vp, vp, i32, vp, vp, ctypes.POINTER(KvDesc), vp]
    lib.photon_kv_cache_write.restype = st
    lib.photon_paged_attn_multi_query.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_float,
                                                  ctypes.POINTER(MultiQueryDesc), vp, vp, sz, vp]
    lib.photon_paged_attn_multi_query_workspace_bytes.argtypes = [ctypes.POINTER(MultiQueryDesc),
                                                                  ctypes.POINTER(sz)]
    lib.photon_paged_attn_multi_query_workspace_bytes.restype = st
    lib.photon_paged_attn_multi_query.restype = st
    lib.photon_rope_kv_cache_write.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, vp, vp,
                                               ctypes.POINTER(KvDesc), ctypes.POINTER(RopeDesc), vp]
    lib.photon_rope_kv_cache_write.restype = st
    lib.photon_paged_attn_partition_quantum.argtypes = [ctypes.POINTER(DecodeDesc)]
    lib.photon_paged_attn_partition_quantum.restype = i32
    lib.photon_paged_attn_partition_tokens.argtypes = [ctypes.POINTER(DecodeDesc)]
    lib.photon_paged_attn_partition_tokens.restype = i32
    lib.photon_paged_attn_workspace_bytes.argtypes = [ctypes.POINTER(DecodeDesc),
                                                      ctypes.POINTER(sz)]
    lib.photon_paged_attn_workspace_bytes.restype = st
    lib.photon_paged_attn_decode.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float,
                                             ctypes.POINTER(DecodeDesc), vp, vp, sz, vp]
    lib.photon_paged_attn_decode.restype = st
    lib.photon_paged_attn_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_float,
                                                  ctypes.POINTER(DecodeDesc), vp, vp, sz, vp]
    lib.photon_paged_attn_decode_step.restype = st
    lib.photon_paged_attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float,
                                                     ctypes.POINTER(DecodeDesc), vp, vp]
    lib.photon_paged_attn_decode_noalloc.restype = st
    lib.photon_probe_stream_read.argtypes = [vp, sz, i32, vp, vp]
    lib.photon_probe_stream_read.restype = st
    lib.photon_probe_gather.argtypes = [vp, vp, vp, vp, ctypes.POINTER(DecodeDesc), i32, vp, vp]
    lib.photon_probe_gather.restype = st
    lib.photon_probe_gather_staged.argtypes = [vp, vp, vp, vp, ctypes.POINTER(DecodeDesc), i32, i32,
                                               vp, vp]
    lib.photon_probe_gather_staged.restype = st
    lib.photon_probe_gather_queue.argtypes = [vp, vp, vp, vp, ctypes.POINTER(DecodeDesc), i32, i32,
                                              i32, vp, vp, vp]
    lib.photon_probe_gather_queue.restype = st
    lib.photon_status_str.argtypes = [st]
    lib.photon_status_str.restype = ctypes.c_char_p
    lib.photon_last_error_detail.argtypes = []
    lib.photon_last_error_detail.restype = ctypes.c_char_p
    lib.photon_abi_version.argtypes = []
    lib.photon_abi_version.restype = i32
    return lib


_lib = None
_lib_lock = threading.Lock()


def get_lib() -> ctypes.CDLL:
    """The loaded ``libphoton_decode.so`` (loaded on first use)."""
    global _lib
    if _lib is None:
        with _lib_lock:
            if _lib is None:
                _lib = _load_library()
    return _lib


def __getattr__(name: str):
    # ``lib`` is loaded lazily (PEP 562 module attribute)
    if name == "lib":
        return get_lib()
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")


def check(status: int) -> None:
    if status != OK:
        lib = get_lib()
        raise PhotonError(status, lib.photon_status_str(status).decode(),
                          lib.photon_last_error_detail().decode())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.bfloat16:
        return BF16
    raise PhotonError(ERR_INVALID_ARG, "PHOTON_ERR_INVALID_ARG", f"dtype {t.dtype} not supported")


def _stream_ptr(t) -> int:
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _contig(name: str, t) -> None:
    if not t.is_contiguous():
        raise PhotonError(ERR_INVALID_ARG, "PHOTON_ERR_INVALID_ARG", f"{name} is not contiguous")


def _args_ok(device, **tensors) -> None:
    """Every tensor is contiguous and lives on ``device``, a GPU.

    The kernels dereference every pointer they get on the GPU, so a host
    tensor (or one on another GPU) is refused here rather than handed over.
    """
    if device.type != "cuda":
        raise PhotonError(ERR_INVALID_ARG, "PHOTON_ERR_INVALID_ARG",
                          f"tensors must be on a ROCm GPU, not {device}")
    for name, t in tensors.items():
        _contig(name, t)
        if t.device != device:
            raise PhotonError(ERR_INVALID_ARG, "PHOTON_ERR_INVALID_ARG",
                              f"{name} is on {t.device}, the pools on {device}")


def _int32(**tensors) -> None:
    import torch
    for name, t in tensors.items():
        if t.dtype != torch.int32:
            raise PhotonError(ERR_INVALID_ARG, "PHOTON_ERR_INVALID_ARG",
                              f"{name} must be int32, not {t.dtype}")


def kv_desc(k_cache) -> KvDesc:
    nb, hkv, bs, d = k_cache.shape
    return KvDesc(nb, hkv, bs, d, _dtype_code(k_cache))


def decode_desc(q, k_cache, block_tables, max_context_len: int,
                partition_tokens: int = 0, flags: int = 0) -> DecodeDesc:
    b, hq, _ = q.shape
    return DecodeDesc(b, hq, block_tables.shape[1], int(max_context_len), int(partition_tokens),
                      kv_desc(k_cache), int(flags))


def kv_cache_write(k, v, slot_mapping, k_cache, v_cache) -> None:
    """Write k[i], v[i] ([T, Hkv, D]) into pool slot ``slot_mapping[i]`` (in place)."""
    _int32(slot_mapping=slot_mapping)
    _args_ok(k_cache.device, k=k, v=v, slot_mapping=slot_mapping, k_cache=k_cache,
             v_cache=v_cache)
    if k.dtype != k_cache.dtype or v.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
        raise PhotonError(ERR_INVALID_ARG, "PHOTON_ERR_INVALID_ARG", "k, v and pools differ in dtype")
    _, hkv, _, d = k_cache.shape
    if tuple(k.shape) != (slot_mapping.shape[0], hkv, d) or k.shape != v.shape \
            or v_cache.shape != k_cache.shape:
        raise PhotonError(ERR_INVALID_ARG, "PHOTON_ERR_INVALID_ARG", "shape mismatch")
    desc = kv_desc(k_cache)
    check(get_lib().photon_kv_cache_write(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(),
                                    slot_mapping.shape[0], k_cache.data_ptr(), v_cache.data_ptr(),
                                    ctypes.byref(desc), _stream_ptr(k_cache)))


def rope_kv_cache_write(q, k, v, positions, slot_mapping, k_cache, v_cache, base: float,
                        adjacent_pairs: bool = False, q_out=None):
    """Rotate q and k by their tokens' positions, then write rotated k and v to their slots.

    q: [T, Hq, D]; k, v: [T, Hkv, D]; positions, slot_mapping: [T] int32;
    pools [NB, Hkv, 16, D] are updated in place.  Returns q_out (a new
    tensor unless given; passing q itself rotates q in place).
    """
    import torch
    _int32(positions=positions, slot_mapping=slot_mapping)
    _args_ok(k_cache.device, q=q, k=k, v=v, positions=positions, slot_mapping=slot_mapping,
             k_cache=k_cache, v_cache=v_cache)
    if any(t.dtype != k_cache.dtype for t in (q, k, v, v_cache)):
        raise PhotonError(ERR_INVALID_ARG, "PHOTON_ERR_INVALID_ARG", "q, k, v and pools differ in dtype")
    t_, hq, d = q.shape
    _, hkv, _, d2 = k_cache.shape
    if d != d2 or tuple(k.shape) != (t_, hkv, d) or v.shape != k.shape \
            or tuple(positions.shape) != (t_,) or tuple(slot_mapping.shape) != (t_,) \
            or v_cache.shape != k_cache.shape:
        raise PhotonError(ERR_INVALID_ARG, "PHOTON_ERR_INVALID_ARG", "shape mismatch")
    if q_out is None:
        q_out = torch.empty_like(q)
    else:
        _args_ok(k_cache.device, q_out=q_out)
        if q_out.shape != q.shape or q_out.dtype != q.dtype:
            raise PhotonError(ERR_INVALID_ARG, "PHOTON_ERR_INVALID_ARG", "q_out shape or dtype")
    desc = kv_desc(k_cache)
    rope = RopeDesc(float(base), int(bool(adjacent_pairs)), 0)
    check(get_lib().photon_rope_kv_cache_write(q.data_ptr(), q_out.data_ptr(), k.data_ptr(), v.data_ptr(),
                                         positions.data_ptr(), slot_mapping.data_ptr(), t_, hq,
                                         k_cache.data_ptr(), v_cache.data_ptr(), ctypes.byref(desc),
                                         ctypes.byref(rope), _stream_ptr(k_cache)))
    return q_out


def partition_quantum(desc: DecodeDesc) -> int:
    n = get_lib().photon_paged_attn_partition_quantum(ctypes.byref(desc))
    if n == 0:
        raise PhotonError(ERR_INVALID_ARG, "PHOTON_ERR_INVALID_ARG",
                          get_lib().photon_last_error_detail().decode())
    return n


def partition_tokens(desc: DecodeDesc) -> int:
    n = get_lib().photon_paged_attn_partition_tokens(ctypes.byref(desc))
    if n == 0:
        raise PhotonError(ERR_INVALID_ARG, "PHOTON_ERR_INVALID_ARG",
                          get_lib().photon_last_error_detail().decode())
    return n


def workspace_bytes(desc: DecodeDesc) -> int:
    n = ctypes.c_size_t(0)
    check(get_lib().photon_paged_attn_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def new_workspace(nbytes: int, device):
    """Workspace tensor of at least ``nbytes`` (its contents do not matter:
    the arrival counters in it are tagged with each call's number)."""
    import torch
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def paged_attn_decode(q, k_cache, v_cache, block_tables, context_lens, scale: float,
                      max_context_len: int | None = None, out=None, workspace=None,
                      partition_tokens: int = 0, out_dtype=None):
    """GQA paged decode: out[b, h] = softmax(scale q K^T) V over context_lens[b] tokens.

    q, out: [B, Hq, D]; pools: [NB, Hkv, 16, D]; block_tables: [B, max_blocks]
    int32; context_lens: [B] int32.  ``max_context_len`` must bound every
    context length (if None it is read back from the device, which
    synchronises).  ``workspace`` (uint8 device tensor from
    :func:`new_workspace`) is allocated through torch when not given and needed.
    ``out`` (or ``out_dtype`` when ``out`` is None) is q's dtype or float32;
    float32 with 16-bit storage selects the fp32-output kernels.
    """
    import torch
    _int32(block_tables=block_tables, context_lens=context_lens)
    _args_ok(k_cache.device, q=q, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
             context_lens=context_lens)
    if q.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype or v_cache.shape != k_cache.shape:
        raise PhotonError(ERR_INVALID_ARG, "PHOTON_ERR_INVALID_ARG", "q and pools differ")
    if q.shape[2] != k_cache.shape[3] or block_tables.shape[0] != q.shape[0] \
            or tuple(context_lens.shape) != (q.shape[0],):
        raise PhotonError(ERR_INVALID_ARG, "PHOTON_ERR_INVALID_ARG", "shape mismatch")
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if context_lens.numel() else 0
    if out is not None:
        out_dtype = out.dtype
    elif out_dtype is None:
        out_dtype = q.dtype
    if out_dtype not in (q.dtype, torch.float32):
        raise PhotonError(ERR_INVALID_ARG, "PHOTON_ERR_INVALID_ARG",
                          f"output dtype {out_dtype} is neither {q.dtype} nor float32")
    flags = DECODE_OUT_F32 if out_dtype == torch.float32 and q.dtype != torch.float32 else 0
    desc = decode_desc(q, k_cache, block_tables, max_context_len, partition_tokens, flags)
    ws_need = workspace_bytes(desc)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    else:
        _args_ok(k_cache.device, out=out)
        if out.shape != q.shape:
            raise PhotonError(ERR_INVALID_ARG, "PHOTON_ERR_INVALID_ARG", "out shape")
    if ws_need and workspace is None:
        workspace = new_workspace(ws_need, q.device)
    if workspace is not None:
        _args_ok(k_cache.device, workspace=workspace)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check(get_lib().photon_paged_attn_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                       block_tables.data_ptr(), context_lens.data_ptr(),
                                       float(scale), ctypes.byref(desc), out.data_ptr(), ws_ptr,
                                       ws_len, _stream_ptr(q)))
    return out


def paged_attn_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale: float,
                              max_context_len: int, out, partition_tokens: int = 0):
    """:func:`paged_attn_decode` through the entry point that allocates
    nothing: the library's static per-GPU scratch serves as the workspace,
    and ``out`` (q's dtype, or float32) must be given, so the call makes no
    allocation at all.  Calls that may overlap in time on one GPU race."""
    import torch
    _int32(block_tables=block_tables, context_lens=context_lens)
    _args_ok(k_cache.device, q=q, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
             context_lens=context_lens, out=out)
    if q.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype or v_cache.shape != k_cache.shape:
        raise PhotonError(ERR_INVALID_ARG, "PHOTON_ERR_INVALID_ARG", "q and pools differ")
    if q.shape[2] != k_cache.shape[3] or block_tables.shape[0] != q.shape[0] \
            or tuple(context_lens.shape) != (q.shape[0],) or out.shape != q.shape:
        raise PhotonError(ERR_INVALID_ARG, "PHOTON_ERR_INVALID_ARG", "shape mismatch")
    if out.dtype not in (q.dtype, torch.float32):
        raise PhotonError(ERR_INVALID_ARG, "PHOTON_ERR_INVALID_ARG",
                          f"output dtype {out.dtype} is neither {q.dtype} nor float32")
    flags = DECODE_OUT_F32 if out.dtype == torch.float32 and q.dtype != torch.float32 else 0
    desc = decode_desc(q, k_cache, block_tables, max_context_len, partition_tokens, flags)
    with torch.cuda.device(q.device):  # the stream's device is the current one
        check(get_lib().photon_paged_attn_decode_noalloc(
            q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
            context_lens.data_ptr(), float(scale), ctypes.byref(desc), out.data_ptr(),
            _stream_ptr(q)))
    return out


def multi_query_desc(q, k_cache, block_tables, num_seqs: int, max_query_len: int,
                     max_context_len: int, split_tokens: int = 0, flags: int = 0) -> MultiQueryDesc:
    return MultiQueryDesc(num_seqs, q.shape[0], q.shape[1], block_tables.shape[1],
                          int(max_query_len), int(max_context_len), int(split_tokens), int(flags),
                          kv_desc(k_cache))


def multi_query_workspace_bytes(desc: MultiQueryDesc) -> int:
    n = ctypes.c_size_t(0)
    check(get_lib().photon_paged_attn_multi_query_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def paged_attn_multi_query(q, k_cache, v_cache, block_tables, context_lens, query_start,
                           scale: float, max_query_len: int | None = None,
                           max_context_len: int | None = None, out=None, out_dtype=None,
                           workspace=None, split_tokens: int = 0):
    """Causal multi-query paged attention (chunked prefill / speculative verification).

    q, out: [T, Hq, D]; sequence b owns rows query_start[b] .. query_start[b+1]-1,
    the last tokens of its context_lens[b]; row j attends to positions
    <= context_lens[b] - n_b + j.  ``max_query_len`` bounds every n_b (read
    back from the device, with a synchronisation, if None), and
    ``max_context_len`` every context length (likewise).  ``split_tokens``
    (0 = automatic) is the KV range one workgroup scans per 16-row tile;
    ``workspace`` is allocated through torch when needed and not given.
    """
    import torch
    _int32(block_tables=block_tables, context_lens=context_lens, query_start=query_start)
    _args_ok(k_cache.device, q=q, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
             context_lens=context_lens, query_start=query_start)
    if q.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype or v_cache.shape != k_cache.shape:
        raise PhotonError(ERR_INVALID_ARG, "PHOTON_ERR_INVALID_ARG", "q and pools differ")
    b = context_lens.shape[0]
    if q.shape[2] != k_cache.shape[3] or block_tables.shape[0] != b \
            or tuple(query_start.shape) != (b + 1,):
        raise PhotonError(ERR_INVALID_ARG, "PHOTON_ERR_INVALID_ARG", "shape mismatch")
    if max_query_len is None:
        max_query_len = int((query_start[1:] - query_start[:-1]).max().item()) if b else 0
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if b else 0
    if out is not None:
        out_dtype = out.dtype
    elif out_dtype is None:
        out_dtype = q.dtype
    if out_dtype not in (q.dtype, torch.float32):
        raise PhotonError(ERR_INVALID_ARG, "PHOTON_ERR_INVALID_ARG",
                          f"output dtype {out_dtype} is neither {q.dtype} nor float32")
    flags = DECODE_OUT_F32 if out_dtype == torch.float32 and q.dtype != torch.float32 else 0
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    else:
        _args_ok(k_cache.device, out=out)
        if out.shape != q.shape:
            raise PhotonError(ERR_INVALID_ARG, "PHOTON_ERR_INVALID_ARG", "out shape")
    desc = multi_query_desc(q, k_cache, block_tables, b, max_query_len, max_context_len,
                            split_tokens, flags)
    ws_need = multi_query_workspace_bytes(desc)
    if ws_need and workspace is None:
        workspace = new_workspace(ws_need, q.device)
    if workspace is not None:
        _args_ok(k_cache.device, workspace=workspace)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check(get_lib().photon_paged_attn_multi_query(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                            block_tables.data_ptr(), context_lens.data_ptr(),
                                            query_start.data_ptr(), float(scale), ctypes.byref(desc),
                                            out.data_ptr(), ws_ptr, ws_len, _stream_ptr(q)))
    return out


def paged_attn_decode_step(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens,
                           scale: float, max_context_len: int | None = None, out=None,
                           workspace=None, partition_tokens: int = 0):
    """One fused decode step: store k_new[b], v_new[b] ([B, Hkv, D]) at position
    context_lens[b] - 1 of each sequence, then attend as :func:`paged_attn_decode`."""
    import torch
    _int32(block_tables=block_tables, context_lens=context_lens)
    _args_ok(k_cache.device, q=q, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache,
             block_tables=block_tables, context_lens=context_lens)
    if any(t.dtype != k_cache.dtype for t in (q, k_new, v_new, v_cache)) or v_cache.shape != k_cache.shape:
        raise PhotonError(ERR_INVALID_ARG, "PHOTON_ERR_INVALID_ARG", "q, new rows and pools differ")
    b, _, d = q.shape
    _, hkv, _, _ = k_cache.shape
    if d != k_cache.shape[3] or tuple(k_new.shape) != (b, hkv, d) or v_new.shape != k_new.shape \
            or block_tables.shape[0] != b or tuple(context_lens.shape) != (b,):
        raise PhotonError(ERR_INVALID_ARG, "PHOTON_ERR_INVALID_ARG", "shape mismatch")
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if context_lens.numel() else 0
    desc = decode_desc(q, k_cache, block_tables, max_context_len, partition_tokens)
    ws_need = workspace_bytes(desc)
    if out is None:
        out = torch.empty_like(q)
    else:
        _args_ok(k_cache.device, out=out)
        if out.shape != q.shape or out.dtype != q.dtype:
            raise PhotonError(ERR_INVALID_ARG, "PHOTON_ERR_INVALID_ARG", "out shape or dtype")
    if ws_need and workspace is None:
        workspace = new_workspace(ws_need, q.device)
    if workspace is not None:
        _args_ok(k_cache.device, workspace=workspace)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check(get_lib().photon_paged_attn_decode_step(q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                                            k_cache.data_ptr(), v_cache.data_ptr(),
                                            block_tables.data_ptr(), context_lens.data_ptr(),
                                            float(scale), ctypes.byref(desc), out.data_ptr(),
                                            ws_ptr, ws_len, _stream_ptr(q)))
    return out


def probe_stream_read(buf, waves: int, sink=None):
    """Bandwidth probe: read every byte of ``buf`` (a contiguous GPU tensor)
    with ``waves`` wavefronts, no arithmetic.  Returns the uint32 ``sink``
    of per-wavefront XORs of the 32-bit words read (include/photon_probe.h)."""
    import torch
    _args_ok(buf.device, buf=buf)
    if sink is None:
        sink = torch.empty(waves, dtype=torch.int32, device=buf.device)
    check(get_lib().photon_probe_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(),
                                             int(waves), sink.data_ptr(), _stream_ptr(buf)))
    return sink


def _gather_desc(k_cache, v_cache, block_tables, context_lens, max_context_len: int):
    _int32(block_tables=block_tables, context_lens=context_lens)
    _args_ok(k_cache.device, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
             context_lens=context_lens)
    return DecodeDesc(context_lens.shape[0], k_cache.shape[1], block_tables.shape[1],
                      int(max_context_len), 0, kv_desc(k_cache), 0)


def probe_gather(k_cache, v_cache, block_tables, context_lens, max_context_len: int, waves: int,
                 sink=None):
    """Bandwidth probe: read every valid K and V row of the decode call over
    these tables and lengths, split evenly over ``waves`` wavefronts, no
    arithmetic.  Returns the per-wavefront XORs (include/photon_probe.h)."""
    import torch
    desc = _gather_desc(k_cache, v_cache, block_tables, context_lens, max_context_len)
    if sink is None:
        sink = torch.empty(waves, dtype=torch.int32, device=k_cache.device)
    check(get_lib().photon_probe_gather(k_cache.data_ptr(), v_cache.data_ptr(),
                                        block_tables.data_ptr(), context_lens.data_ptr(),
                                        ctypes.byref(desc), int(waves), sink.data_ptr(),
                                        _stream_ptr(k_cache)))
    return sink


def probe_gather_staged(k_cache, v_cache, block_tables, context_lens, max_context_len: int,
                        workgroups: int, ring_tiles: int, sink=None):
    """The rows of ``probe_gather`` over ``workgroups`` workgroups of four
    wavefronts, each wavefront keeping ``ring_tiles`` tiles in flight in
    LDS.  Returns the per-wavefront XORs (4 per workgroup)."""
    import torch
    desc = _gather_desc(k_cache, v_cache, block_tables, context_lens, max_context_len)
    if sink is None:
        sink = torch.empty(4 * workgroups, dtype=torch.int32, device=k_cache.device)
    check(get_lib().photon_probe_gather_staged(k_cache.data_ptr(), v_cache.data_ptr(),
                                               block_tables.data_ptr(), context_lens.data_ptr(),
                                               ctypes.byref(desc), int(workgroups),
                                               int(ring_tiles), sink.data_ptr(),
                                               _stream_ptr(k_cache)))
    return sink


def probe_gather_queue(k_cache, v_cache, block_tables, context_lens, max_context_len: int,
                       waves: int, static_permille: int, piece_tiles: int, queue, sink=None):
    """The rows of ``probe_gather``, the last (1000 - static_permille)
    thousandths handed out at run time in pieces of ``piece_tiles`` tiles
    through ``queue`` (one int64 on the device, zero before the call and
    zero again after it).  Returns the per-wavefront XORs."""
    import torch
    desc = _gather_desc(k_cache, v_cache, block_tables, context_lens, max_context_len)
    _args_ok(k_cache.device, queue=queue)
    if queue.dtype != torch.int64 or queue.numel() < 1:
        raise PhotonError(ERR_INVALID_ARG, "PHOTON_ERR_INVALID_ARG", "queue must hold one int64")
    if sink is None:
        sink = torch.empty(waves, dtype=torch.int32, device=k_cache.device)
    check(get_lib().photon_probe_gather_queue(k_cache.data_ptr(), v_cache.data_ptr(),
                                              block_tables.data_ptr(), context_lens.data_ptr(),
                                              ctypes.byref(desc), int(waves), int(static_permille),
                                              int(piece_tiles), queue.data_ptr(), sink.data_ptr(),
                                              _stream_ptr(k_cache)))
    return sink