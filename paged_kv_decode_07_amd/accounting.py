"""Algorithmic byte and flop counts of one decode step (pure host arithmetic).

These are the bytes the method must move, not what a kernel happens to read:
over-read tail slots, split partials and cache refills are overhead and never
count as useful work.

KV growth per token follows the formula of "Building an LLM inference engine
from scratch: KV cache, operator fusion and quantisation practice", section
5.1: K and V each hold ``layers x heads x head_dim`` values per token.
"""

from __future__ import annotations

import numpy as np

Q_HEADS, KV_HEADS, HEAD_DIM, PAGE = 32, 8, 64, 16
BF16 = 2


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    """K plus V bytes one token adds to the cache over ``layers`` layers."""
    return 2 * layers * kv_heads * head_dim * dtype_bytes


KV_TOKEN_BYTES = kv_bytes_per_token(1, KV_HEADS, HEAD_DIM, BF16)    # 2048 per layer
PAGE_BYTES = PAGE * KV_TOKEN_BYTES                                   # 32 KiB (K+V)


def step_bytes(seq_lens, out_bytes: int = 4, append: bool = False) -> dict:
    """Algorithmic HBM bytes of one layer's decode step for these lengths.

    kv    K and V rows of every valid token (2 KiB per token)
    q     the new queries (32 x 64 BF16 per active sequence)
    out   the outputs (32 x 64 x ``out_bytes`` per active sequence)
    meta  the block-table entries in use plus the length of each sequence
    app   the one-token append: 2 KiB read, 2 KiB written, 8 B of metadata
    """
    lens = np.asarray(seq_lens, dtype=np.int64)
    active = int(np.count_nonzero(lens))
    pages = (lens + PAGE - 1) // PAGE
    kv = int(lens.sum()) * KV_TOKEN_BYTES
    q = active * Q_HEADS * HEAD_DIM * BF16
    out = active * Q_HEADS * HEAD_DIM * out_bytes
    meta = int(4 * pages.sum() + 4 * lens.shape[0])
    app = active * (2 * KV_TOKEN_BYTES + 8) if append else 0
    return {"kv": kv, "q": q, "out": out, "meta": meta, "app": app,
            "total": kv + q + out + meta + app}


def step_flops(seq_lens) -> int:
    """Multiply-adds of q.K^T and p.V, two flops each: 4 flops per KV byte."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    return int(lens.sum()) * Q_HEADS * HEAD_DIM * 2 * 2


# INT8 pages: one byte per value plus one FP32 scale per (token, KV head) row,
# for K and for V (the INT8 cache of the same section 5.1, with the symmetric
# quantiser of section 3.4 applied row by row)
Q8_TOKEN_BYTES = 2 * KV_HEADS * (HEAD_DIM + 4)                       # 1088 per layer
Q8_PAGE_BYTES = PAGE * Q8_TOKEN_BYTES                                # 17 KiB (K+V+scales)


def step_bytes_q8(seq_lens, out_bytes: int = 4, append: bool = False) -> dict:
    """As ``step_bytes`` for INT8 pages: ``kv`` counts 1088 bytes per valid token;
    the append reads a BF16 row pair and writes its codes and scales."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    base = step_bytes(lens, out_bytes=out_bytes, append=False)
    active = int(np.count_nonzero(lens))
    kv = int(lens.sum()) * Q8_TOKEN_BYTES
    app = active * (KV_TOKEN_BYTES + Q8_TOKEN_BYTES + 8) if append else 0
    out = dict(base, kv=kv, app=app)
    out["total"] = kv + base["q"] + base["out"] + base["meta"] + app
    return out


# INT4 pages: two codes per byte plus the same per-row FP32 scales (section
# 5.1's lower-precision cache at 4 bits)
Q4_TOKEN_BYTES = 2 * KV_HEADS * (HEAD_DIM // 2 + 4)                  # 576 per layer
Q4_PAGE_BYTES = PAGE * Q4_TOKEN_BYTES                                # 9 KiB (K+V+scales)


def step_bytes_q4(seq_lens, out_bytes: int = 4, append: bool = False) -> dict:
    """As ``step_bytes`` for INT4 pages: ``kv`` counts 576 bytes per valid token;
    the append reads a BF16 row pair and writes its codes and scales."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    base = step_bytes(lens, out_bytes=out_bytes, append=False)
    active = int(np.count_nonzero(lens))
    kv = int(lens.sum()) * Q4_TOKEN_BYTES
    app = active * (KV_TOKEN_BYTES + Q4_TOKEN_BYTES + 8) if append else 0
    out = dict(base, kv=kv, app=app)
    out["total"] = kv + base["q"] + base["out"] + base["meta"] + app
    return out

