"""Seeded synthetic inputs for batched paged-attention decode.

This module is shared by the CPU oracle's tests and by the GPU path's tests
and benchmark.  It only draws random numbers and lays out indices (context
lengths, block tables, slot mappings); it performs none of the attention or
cache-write arithmetic, so neither side of a parity check borrows the other's
computation through it.

Workload shapes follow the model families the PhotonInfer README names in its
"Performance highlights" section (Llama-3.2 1B, Qwen3): Llama-3.2-1B has 32
query heads, 8 KV heads and head_dim 64 over 16 layers; the Qwen3-0.6B-like
long-context case has 16 query heads, 8 KV heads and head_dim 128.  The block
pool follows the README's "Technical details -> Paged attention" section
(block-level KV cache, per-sequence block tables, one batched K/V write).

Recipe (all draws from ``numpy.random.default_rng``):

* context lengths and the physical-block permutation come from
  ``default_rng(seed)``, contexts first, then ``permutation(num_blocks)``;
  sequence b's table is the next ``ceil(ctx_b / block_size)`` entries of that
  permutation, so the pool is shared and shuffled;
* per-layer tensors come from ``default_rng([seed, layer])`` in the order
  q, K pool, V pool, new k, new v, each ``standard_normal`` in float32 and
  then rounded to nearest (ties to even) in the storage dtype;
* the decode-step slot of sequence b is the logical position ``ctx_b - 1``
  (the new token is written first and then attended to), which is also the
  position its q and k are rotated by.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

BLOCK_SIZE = 16
PAD_TABLE_ENTRY = -1

# numpy has no bfloat16: bf16 arrays are held as this one-field record of
# the 16 storage bits, so that they cannot be mistaken for integers.  Never
# ``astype`` into it (numpy would cast values to integers field-wise); use
# ``to_storage``.
BF16 = np.dtype([("bf16", "<u2")])

_NP_DTYPE = {"f32": np.dtype(np.float32), "f16": np.dtype(np.float16), "bf16": BF16}
# Quiet-NaN bit patterns, used to poison pool slots no sequence may read.
_NAN_BITS = {np.dtype(np.float32): (np.uint32, 0x7FC00000),
             np.dtype(np.float16): (np.uint16, 0x7E00),
             BF16: (np.uint16, 0x7FC0)}


def to_storage(x: np.ndarray, dtype) -> np.ndarray:
    """float32 values rounded to nearest-even in storage dtype ``dtype``.

    For bfloat16 (the upper half of a binary32) the rounding is done on the
    bits: add 0x7FFF plus the lowest kept bit, then drop the low 16 bits;
    NaN stays a quiet NaN of the same sign.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    dtype = np.dtype(dtype)
    if dtype != BF16:
        return x.astype(dtype)
    bits = x.view(np.uint32).astype(np.uint64)
    rounded = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    rounded[nan] = (bits[nan] >> 16).astype(np.uint16) | 0x7FC0
    return rounded.view(BF16)


def cast(x: np.ndarray, dtype) -> np.ndarray:
    """``x.astype(dtype)`` for float32/float16; ``to_storage`` (via float32) for ``BF16``."""
    dtype = np.dtype(dtype)
    if dtype == BF16:
        return to_storage(np.asarray(x, dtype=np.float32), BF16)
    return np.asarray(x).astype(dtype)


def as_float64(a: np.ndarray) -> np.ndarray:
    """Exact float64 values of a storage array (torch widens bfloat16)."""
    if a.dtype == BF16:
        return to_torch(a).double().numpy()
    return np.asarray(a).astype(np.float64)


def storage_bits(a: np.ndarray) -> np.ndarray:
    """Unsigned-integer view of a storage array's bits (same shape)."""
    return a.view(_NAN_BITS[a.dtype][0])


def to_torch(a: np.ndarray):
    """CPU torch tensor sharing ``a``'s bits (bfloat16 for ``BF16`` arrays)."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == BF16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(a)


def from_torch(t) -> np.ndarray:
    """numpy copy of a torch tensor's bits (``BF16`` for bfloat16)."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(BF16)
    return t.numpy()


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    """Shape and seed of one decode workload."""

    name: str
    seed: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str  # "f32", "f16" or "bf16": storage type of q, K/V pool and output
    ctx_kind: str  # "fixed", "uniform" or "loguniform"
    ctx_lo: int
    ctx_hi: int
    layers: int = 1
    block_size: int = BLOCK_SIZE
    pool_blocks: int | None = None  # None: exactly the blocks the tables use
    force_first_ctx: int | None = None
    rope_base: float = 500000.0  # rotary frequency base (Llama 3: 5e5, Qwen3: 1e6)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        # 1/sqrt(head_dim) rounded once to float32; both sides use this value.
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def np_dtype(self):
        return _NP_DTYPE[self.dtype]


CONFIGS: dict[str, DecodeConfig] = {
    # Tiny case: 37 tokens span two full blocks and 5 slots of a third.
    "tiny": DecodeConfig("tiny", 0, 1, 2, 1, 64, "f32", "fixed", 37, 37,
                         pool_blocks=8),
    # One Llama-3.2-1B attention layer at batch 1.
    "llama1b_b1": DecodeConfig("llama1b_b1", 1, 1, 32, 8, 64, "f32",
                               "fixed", 512, 512),
    # Llama-3.2-1B decode step at batch 16, 16 layers, one pool per layer.
    "llama1b_b16": DecodeConfig("llama1b_b16", 2, 16, 32, 8, 64, "f32",
                                "uniform", 64, 2048, layers=16),
    # Continuous-batching step: ragged log-uniform contexts, fp16 KV.
    "cb_b64": DecodeConfig("cb_b64", 3, 64, 32, 8, 64, "f16",
                           "loguniform", 1, 8192, force_first_ctx=1),
    # Qwen3-0.6B-shaped long context, fp16 KV, head_dim 128.
    "qwen3_long": DecodeConfig("qwen3_long", 4, 8, 16, 8, 128, "f16",
                               "fixed", 32768, 32768, rope_base=1e6),
    # The batch-16 Llama step with bfloat16 KV (same seed, contexts, tables).
    "llama1b_b16_bf16": DecodeConfig("llama1b_b16_bf16", 2, 16, 32, 8, 64, "bf16",
                                     "uniform", 64, 2048, layers=16),
}


def draw_context_lens(cfg: DecodeConfig, rng: np.random.Generator) -> np.ndarray:
    """Context lengths (tokens already in the cache, new token included)."""
    b = cfg.num_seqs
    if cfg.ctx_kind == "fixed":
        ctx = np.full(b, cfg.ctx_lo, dtype=np.int64)
    elif cfg.ctx_kind == "uniform":
        ctx = rng.integers(cfg.ctx_lo, cfg.ctx_hi, b, endpoint=True)
    elif cfg.ctx_kind == "loguniform":
        u = rng.uniform(0.0, math.log(cfg.ctx_hi), b)
        ctx = np.clip(np.floor(np.exp(u)), cfg.ctx_lo, cfg.ctx_hi).astype(np.int64)
    else:
        raise ValueError(cfg.ctx_kind)
    if cfg.force_first_ctx is not None:
        ctx[0] = cfg.force_first_ctx
    return ctx.astype(np.int32)


def blocks_needed(ctx: np.ndarray, block_size: int = BLOCK_SIZE) -> np.ndarray:
    return (np.asarray(ctx, dtype=np.int64) + block_size - 1) // block_size


@dataclasses.dataclass
class BatchLayout:
    """Index tensors of one decode step (shared by every layer)."""

    context_lens: np.ndarray  # [B] int32
    block_tables: np.ndarray  # [B, max_blocks] int32, unused entries = -1
    slot_mapping: np.ndarray  # [B] int32, slot of logical position ctx-1
    positions: np.ndarray     # [B] int32, position ctx-1 of the new token (0 if ctx is 0)
    num_blocks: int
    max_blocks_per_seq: int

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.size else 0


def make_layout(cfg: DecodeConfig, context_lens: np.ndarray | None = None,
                max_blocks_per_seq: int | None = None,
                num_blocks: int | None = None) -> BatchLayout:
    """Contexts, shuffled block tables and decode-step slots for ``cfg``."""
    rng = np.random.default_rng(cfg.seed)
    ctx = draw_context_lens(cfg, rng) if context_lens is None else \
        np.asarray(context_lens, dtype=np.int32)
    need = blocks_needed(ctx, cfg.block_size)
    used = int(need.sum())
    nb = num_blocks or cfg.pool_blocks or max(used, 1)
    if nb < used:
        raise ValueError(f"pool of {nb} blocks cannot hold {used}")
    perm = rng.permutation(nb).astype(np.int32)
    mb = max_blocks_per_seq or max(int(need.max()) if need.size else 1, 1)
    tables = np.full((len(ctx), mb), PAD_TABLE_ENTRY, dtype=np.int32)
    pos = 0
    for b, n in enumerate(need):
        tables[b, :n] = perm[pos:pos + n]
        pos += n
    slots = np.full(len(ctx), -1, dtype=np.int32)
    for b, c in enumerate(ctx):
        if c > 0:
            t = int(c) - 1
            slots[b] = tables[b, t // cfg.block_size] * cfg.block_size + t % cfg.block_size
    positions = np.maximum(ctx.astype(np.int32) - 1, 0)
    return BatchLayout(ctx.astype(np.int32), tables, slots, positions, nb, mb)


@dataclasses.dataclass
class LayerTensors:
    q: np.ndarray        # [B, Hq, D]
    k_cache: np.ndarray  # [NB, Hkv, bs, D]
    v_cache: np.ndarray  # [NB, Hkv, bs, D]
    k_new: np.ndarray    # [T, Hkv, D]
    v_new: np.ndarray    # [T, Hkv, D]


def make_layer(cfg: DecodeConfig, layout: BatchLayout, layer: int = 0,
               num_new_tokens: int | None = None) -> LayerTensors:
    """Per-layer q, pools and new-token K/V drawn from ``default_rng([seed, layer])``."""
    rng = np.random.default_rng([cfg.seed, layer])
    dt = cfg.np_dtype
    b, hq, hkv, d, bs = cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    b = len(layout.context_lens)
    t = b if num_new_tokens is None else num_new_tokens

    def draw(shape):
        return to_storage(rng.standard_normal(shape, dtype=np.float32), dt)

    q = draw((b, hq, d))
    k_cache = draw((layout.num_blocks, hkv, bs, d))
    v_cache = draw((layout.num_blocks, hkv, bs, d))
    k_new = draw((t, hkv, d))
    v_new = draw((t, hkv, d))
    return LayerTensors(q, k_cache, v_cache, k_new, v_new)


def random_injective_slots(num_blocks: int, block_size: int, n: int,
                           rng: np.random.Generator, pad_fraction: float = 0.0) -> np.ndarray:
    """``n`` distinct slots in ``[0, num_blocks*block_size)``; a fraction set to -1."""
    slots = rng.choice(num_blocks * block_size, n, replace=False).astype(np.int32)
    if pad_fraction > 0:
        slots[rng.random(n) < pad_fraction] = -1
    return slots


def poison_unused(cfg: DecodeConfig, layout: BatchLayout, pool: np.ndarray) -> np.ndarray:
    """Copy of ``pool`` with NaN in every slot no sequence may read.

    Poisoned: blocks no table references, and the slots of each sequence's
    last block at or past its context length.
    """
    out = pool.copy()
    bits = storage_bits(out)
    bs = cfg.block_size
    used = np.zeros(layout.num_blocks, dtype=bool)
    nan = _NAN_BITS[pool.dtype][1]
    for b, c in enumerate(layout.context_lens):
        n = int(blocks_needed(np.array([c]), bs)[0])
        used[layout.block_tables[b, :n]] = True
        if c % bs:
            last = layout.block_tables[b, n - 1]
            bits[last, :, c % bs:, :] = nan
    bits[~used] = nan
    return out


# ----------------------------------------------------------- request traces

@dataclasses.dataclass(frozen=True)
class TraceConfig:
    """A seeded stream of requests for the continuous-batching scheduler.

    Arrivals: exponential gaps of mean ``mean_gap`` steps (rounded down, so
    several requests may arrive at one step); prompt lengths log-uniform in
    [prompt_lo, prompt_hi]; generated lengths uniform in [new_lo, new_hi].
    The pool and step limits are the scheduler's configuration.
    """

    name: str
    seed: int
    num_requests: int
    mean_gap: float
    prompt_lo: int
    prompt_hi: int
    new_lo: int
    new_hi: int
    num_blocks: int
    max_seqs: int
    max_tokens_per_step: int
    max_blocks_per_seq: int
    block_size: int = BLOCK_SIZE

    def sched_config(self) -> dict:
        return dict(num_blocks=self.num_blocks, block_size=self.block_size,
                    max_seqs=self.max_seqs, max_tokens_per_step=self.max_tokens_per_step,
                    max_blocks_per_seq=self.max_blocks_per_seq)


TRACES: dict[str, TraceConfig] = {
    # Small and tight: the pool holds a few requests, so preemption is frequent.
    "tight": TraceConfig("tight", 10, 40, 0.7, 4, 120, 1, 40, num_blocks=24, max_seqs=6,
                         max_tokens_per_step=64, max_blocks_per_seq=12),
    # Larger pool, long prompts chunked by the token budget.
    "chunked": TraceConfig("chunked", 11, 120, 0.3, 16, 2048, 8, 128, num_blocks=600,
                           max_seqs=32, max_tokens_per_step=512, max_blocks_per_seq=136),
    # Llama-3.2-1B-like serving: batch up to 64, 2048-token budget, 4096 blocks.
    "serving": TraceConfig("serving", 12, 256, 0.25, 16, 2048, 16, 256, num_blocks=4096,
                           max_seqs=64, max_tokens_per_step=2048, max_blocks_per_seq=144),
}


def make_request_trace(tc: TraceConfig) -> list[tuple[int, int, int, int]]:
    """[(arrival_step, request_id, prompt_len, max_new_tokens)] sorted by arrival."""
    rng = np.random.default_rng(tc.seed)
    gaps = rng.exponential(tc.mean_gap, tc.num_requests)
    arrival = np.floor(np.cumsum(gaps)).astype(np.int64)
    u = rng.uniform(math.log(tc.prompt_lo), math.log(tc.prompt_hi + 1), tc.num_requests)
    prompt = np.clip(np.floor(np.exp(u)), tc.prompt_lo, tc.prompt_hi).astype(np.int64)
    new = rng.integers(tc.new_lo, tc.new_hi, tc.num_requests, endpoint=True)
    cap = min(tc.max_blocks_per_seq, tc.num_blocks) * tc.block_size
    new = np.minimum(new, cap + 1 - prompt)  # the longest a request may grow
    return [(int(a), i, int(p), int(n)) for i, (a, p, n) in enumerate(zip(arrival, prompt, new))]
