"""Seeded synthetic workloads for the paged lightning indexer.

This module only draws inputs: context lengths, the paged pool's block
assignment, bf16 K and q values, fp32 head weights and the poison bytes that
fill every cache byte no token owns.  It holds none of the indexer's
arithmetic (no quantisation, no scoring, no selection); both the CPU oracle
and the HIP path start from what it returns.

Workload shapes follow the decode / MTP-decode / prefill / long-context
indexer calls of a DeepSeek-V3.2 serving step: 64 indexer heads of dimension
128, 64-token cache blocks, top-2048.  Values are N(0, 1) rounded to bf16; head
weights are N(0, 1) * 128^-0.5 * 64^-0.5 in fp32.  Physical blocks are a
random permutation of the pool, so neighbouring tokens of a request live in
unrelated blocks.

Every random stream is a child of ``numpy.random.SeedSequence(seed)``, so the
K rows of one request can be regenerated alone (the oracle only needs the
requests it samples at full size).
"""
from dataclasses import dataclass, field
import math

import numpy as np

BLOCK = 64
HEADS = 64
DIM = 128
BLOCK_BYTES = BLOCK * DIM + BLOCK * 4
TOPK = 2048

# Poison: an fp8 NaN code for every value byte and a float32 quiet NaN for
# every scale that no token owns (stale tails, unused blocks).
POISON_CODE = 0x7F
POISON_SCALE_BYTES = np.frombuffer(np.float32(np.nan).tobytes(), dtype=np.uint8)


def f32_to_bf16_bits(x):
    """Round float32 to the nearest bf16 (ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b):
    """Exact widening of bf16 bits to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def poison_block():
    """One 64-token block whose every byte is poison."""
    blk = np.full(BLOCK_BYTES, POISON_CODE, dtype=np.uint8)
    blk[BLOCK * DIM:] = np.tile(POISON_SCALE_BYTES, BLOCK)
    return blk


@dataclass
class Workload:
    name: str
    seed: int
    batch: int
    next_n: int                 # query tokens per request (decode); 0 = prefill
    ctx: np.ndarray             # int32 [batch] context length per request
    num_blocks: int             # pool size in blocks
    block_table: np.ndarray     # int32 [batch, bt_width], -1 beyond a request's blocks
    width: int                  # logits row width (columns) = bt_width * 64
    topk: int = TOPK
    _ss: list = field(default=None, repr=False)
    chunk: np.ndarray = None    # prefill only: query tokens per request (the last of its context)

    @property
    def prefill(self):
        return self.next_n == 0

    @property
    def chunked(self):
        return self.prefill and self.chunk is not None

    @property
    def rows(self):
        if self.chunked:
            return int(self.chunk.sum())
        return int(self.ctx.sum()) if self.prefill else self.batch * self.next_n

    @property
    def cu_q(self):
        """Prefill query rows per request (its chunk, or its whole context)."""
        n = self.chunk if self.chunked else self.ctx
        return np.concatenate([[0], np.cumsum(n)]).astype(np.int32)

    @property
    def total_tokens(self):
        return int(self.ctx.sum())

    @property
    def cu_seq_lens(self):
        return np.concatenate([[0], np.cumsum(self.ctx)]).astype(np.int32)

    # ---- values -------------------------------------------------------
    def k_request(self, b):
        """bf16 bits [ctx_b, 128] of request b's cached K rows."""
        rng = np.random.Generator(np.random.PCG64(self._ss[2 + b]))
        x = rng.standard_normal((int(self.ctx[b]), DIM), dtype=np.float32)
        return f32_to_bf16_bits(x)

    def slots_request(self, b):
        """Slot of every cached token of request b (block * 64 + offset)."""
        c = int(self.ctx[b])
        nb = -(-c // BLOCK)
        blocks = self.block_table[b, :nb].astype(np.int64)
        return (blocks[:, None] * BLOCK + np.arange(BLOCK)[None, :]).reshape(-1)[:c]

    def k_all(self):
        return np.concatenate([self.k_request(b) for b in range(self.batch)])

    def slot_mapping(self):
        return np.concatenate([self.slots_request(b) for b in range(self.batch)])

    def q(self):
        """bf16 bits [rows, 64, 128] of the query tokens (row = b*next_n + j,
        or the token index for prefill)."""
        rng = np.random.Generator(np.random.PCG64(self._ss[0]))
        x = rng.standard_normal((self.rows, HEADS, DIM), dtype=np.float32)
        return f32_to_bf16_bits(x)

    def w(self):
        """fp32 [rows, 64] head weights, N(0,1) * 128^-0.5 * 64^-0.5."""
        rng = np.random.Generator(np.random.PCG64(self._ss[1]))
        x = rng.standard_normal((self.rows, HEADS), dtype=np.float32)
        return (x * np.float32(DIM ** -0.5 * HEADS ** -0.5)).astype(np.float32)

    def poisoned_pool(self):
        """uint8 [num_blocks, 8448], every byte poison (the bytes of
        ``poison_block`` in every block)."""
        pool = np.empty((self.num_blocks, BLOCK_BYTES), dtype=np.uint8)
        pool[:, :BLOCK * DIM] = POISON_CODE
        pool[:, BLOCK * DIM:] = np.tile(POISON_SCALE_BYTES, BLOCK)[None, :]
        return pool


def _assign_blocks(rng, ctx, num_blocks, bt_width):
    need = [-(-int(c) // BLOCK) for c in ctx]
    assert sum(need) <= num_blocks, "pool too small"
    perm = rng.permutation(num_blocks).astype(np.int32)
    bt = np.full((len(ctx), bt_width), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    return bt


def make(cfg, seed=None):
    """Build workload ``cfg`` (0..4) with the default seed 1000 + cfg.

    0  tiny decode: batch 2, next_n 1, contexts 3000 and 5000, pool 256 blocks
    1  decode: batch 64, next_n 1, contexts uniform in [4096, 16384], pool 20000
    2  MTP decode: batch 128, next_n 2; 96 contexts log-uniform in
       [2048, 65536] and 32 (at seeded positions) uniform in [2, 2047];
       pool ceil(1.25 * blocks needed)
    3  prefill: one request of 8192 tokens, pool 256 blocks
    4  long-context decode: batch 32, next_n 1, contexts 131072, pool 70000
    5  chunked prefill: 4 requests with contexts 16384, 8192, 6144, 2048, each
       scoring its last 2048 tokens (8192 query rows), pool 640 blocks
    """
    seed = 1000 + cfg if seed is None else seed
    ss = np.random.SeedSequence(seed)
    meta = np.random.Generator(np.random.PCG64(ss.spawn(1)[0]))
    if cfg == 0:
        name, batch, next_n = "tiny_decode_b2", 2, 1
        ctx = np.array([3000, 5000], dtype=np.int32)
        num_blocks, bt_width = 256, 79
    elif cfg == 1:
        name, batch, next_n = "decode_b64_ctx4k-16k", 64, 1
        ctx = meta.integers(4096, 16384, size=batch, endpoint=True).astype(np.int32)
        num_blocks, bt_width = 20000, 256
    elif cfg == 2:
        name, batch, next_n = "mtp_decode_b128_n2_ctx2k-64k", 128, 2
        lg = np.exp(meta.uniform(math.log(2048), math.log(65536), size=96))
        long_ctx = np.minimum(np.floor(lg), 65536).astype(np.int32)
        short_ctx = meta.integers(2, 2047, size=32, endpoint=True).astype(np.int32)
        short_pos = np.sort(meta.choice(batch, size=32, replace=False))
        ctx = np.empty(batch, dtype=np.int32)
        mask = np.zeros(batch, dtype=bool)
        mask[short_pos] = True
        ctx[mask] = short_ctx
        ctx[~mask] = long_ctx
        need = sum(-(-int(c) // BLOCK) for c in ctx)
        num_blocks, bt_width = int(math.ceil(1.25 * need)), 1024
    elif cfg == 3:
        name, batch, next_n = "prefill_8192", 1, 0
        ctx = np.array([8192], dtype=np.int32)
        num_blocks, bt_width = 256, 128
    elif cfg == 4:
        name, batch, next_n = "long_decode_b32_ctx128k", 32, 1
        ctx = np.full(batch, 131072, dtype=np.int32)
        num_blocks, bt_width = 70000, 2048
    elif cfg == 5:
        name, batch, next_n = "chunked_prefill_b4_chunk2048", 4, 0
        ctx = np.array([16384, 8192, 6144, 2048], dtype=np.int32)
        num_blocks, bt_width = 640, 256
    else:
        raise ValueError(f"unknown workload {cfg}")
    bt = _assign_blocks(meta, ctx, num_blocks, bt_width)
    chunk = np.full(batch, 2048, dtype=np.int32) if cfg == 5 else None
    return Workload(name=name, seed=seed, batch=batch, next_n=next_n, ctx=ctx,
                    num_blocks=num_blocks, block_table=bt, width=bt_width * BLOCK,
                    _ss=ss.spawn(2 + batch), chunk=chunk)


def custom(batch, next_n, ctx, num_blocks, bt_width, seed, name="custom"):
    """A workload with caller-chosen shapes (tests of edge cases)."""
    ss = np.random.SeedSequence(seed)
    meta = np.random.Generator(np.random.PCG64(ss.spawn(1)[0]))
    ctx = np.asarray(ctx, dtype=np.int32)
    bt = _assign_blocks(meta, ctx, num_blocks, bt_width)
    return Workload(name=name, seed=seed, batch=batch, next_n=next_n, ctx=ctx,
                    num_blocks=num_blocks, block_table=bt, width=bt_width * BLOCK,
                    _ss=ss.spawn(2 + batch))
