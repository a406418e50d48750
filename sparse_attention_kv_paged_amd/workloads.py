"""Seeded synthetic inputs for the CSA indexer (score + top-k).

This module only draws random numbers and lays out bytes; it holds none of the
scoring or selection arithmetic.  Both the GPU path's tests/benchmark and the
CPU oracle consume what it returns, so neither depends on the other.

Value recipe (the same for every workload):
  * q      bf16, N(0, 1) rounded to nearest even                 [B, H, D]
  * w      fp32, N(0, 1) * D^-0.5 * H^-0.5  ("FlashMemory-DeepSeek-V4",
           "Retriever architecture": weights_proj output times the weight
           scale HEAD_DIM^-0.5 * N_HEADS^-0.5)                    [B, H]
  * keys   one 132-byte row per compressed entry ("FlashMemory-DeepSeek-V4",
           "compressed_k format"): D float8_e4m3fn bytes of clip(x / s, +-448)
           with x ~ N(0, 1), then the fp32 scale s ~ U(0.005, 0.05),
           little-endian.
  * poison rows (tail padding inside a request's last block, and pool blocks
    no request references) hold 0x7F bytes (e4m3fn NaN) and a NaN scale, so a
    stray read turns a logit into NaN.

Draw order from numpy's PCG64 `default_rng(seed)`: lengths -> block
permutation -> chunk lists -> q -> w -> key values -> scales.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

HEADS = 64
HEAD_DIM = 128
BLOCK = 64
ROW_BYTES = HEAD_DIM + 4
TOPK = 512
COMPRESS = 4          # one compressed record per 4 token positions (C4)
_POISON_SCALE = np.array([np.nan], dtype="<f4").view(np.uint8)
_KEY_CHUNK_ROWS = 1 << 17


@dataclasses.dataclass
class Workload:
    """Host (numpy) arrays of one scoring problem; layout matches the C ABI."""

    name: str
    q: np.ndarray                       # uint16 [B, H, D]  (bf16 bit patterns)
    w: np.ndarray                       # float32 [B, H]
    pool: np.ndarray                    # uint8 [n_pool_rows, D + 4]
    limits: np.ndarray                  # int32 [B]
    n_cols: int
    k: int = TOPK
    block_size: int = BLOCK
    block_table: Optional[np.ndarray] = None   # int32 [n_req, max_blocks]
    q_req: Optional[np.ndarray] = None         # int32 [B]
    chunk_ids: Optional[np.ndarray] = None     # int32 [B, max_chunks]
    n_chunks: Optional[np.ndarray] = None      # int32 [B]
    description: str = ""

    @property
    def B(self) -> int:
        return int(self.q.shape[0])

    @property
    def H(self) -> int:
        return int(self.q.shape[1])

    @property
    def D(self) -> int:
        return int(self.q.shape[2])

    @property
    def n_pool_rows(self) -> int:
        return int(self.pool.shape[0])

    @property
    def n_req(self) -> int:
        return 0 if self.block_table is None else int(self.block_table.shape[0])

    @property
    def max_blocks(self) -> int:
        return 0 if self.block_table is None else int(self.block_table.shape[1])

    @property
    def max_chunks(self) -> int:
        return 0 if self.chunk_ids is None else int(self.chunk_ids.shape[1])

    def valid_mask(self) -> np.ndarray:
        """bool [B, n_cols]: which columns name a scored entry (layout only)."""
        B, nc, bs = self.B, self.n_cols, self.block_size
        cols = np.arange(nc, dtype=np.int64)
        j, s = cols // bs, cols % bs
        out = np.zeros((B, nc), dtype=bool)
        for b in range(B):
            req = b if self.q_req is None else int(self.q_req[b])
            if req < 0:
                continue
            if self.chunk_ids is not None:
                ncb = min(int(self.n_chunks[b]), self.max_chunks)
                ok = j < ncb
                beta = np.where(ok, self.chunk_ids[b][np.minimum(j, self.max_chunks - 1)], -1)
                ok &= beta >= 0
            else:
                beta = j.copy()
                ok = np.ones(nc, dtype=bool)
            entry = beta * bs + s
            ok &= entry < int(self.limits[b])
            if self.block_table is not None:
                if req >= self.n_req:
                    continue
                inb = ok & (beta < self.max_blocks)
                pblk = np.full(nc, -1, dtype=np.int64)
                pblk[inb] = self.block_table[req][beta[inb]]
                ok = inb & (pblk >= 0) & ((pblk + 1) * bs <= self.n_pool_rows)
            else:
                ok &= entry < self.n_pool_rows
            out[b] = ok
        return out

    def pairs(self) -> int:
        """Scored (query row, entry) pairs."""
        return int(self.valid_mask().sum())

    def pairs_per_row(self) -> np.ndarray:
        """Scored entries of each query row."""
        return self.valid_mask().sum(axis=1)


# ----------------------------------------------------------------------------
# value helpers (library casts only)

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (torch's cast)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def e4m3_bytes(y: np.ndarray) -> np.ndarray:
    """float32 -> float8_e4m3fn bytes, round to nearest even (torch's cast).

    Callers clip to +-448 first: torch returns NaN for |y| >= 464."""
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def make_key_rows(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Key rows from values x [n, D] (float) and scales s [n]: bytes of
    e4m3fn(clip(x / s, +-448)) followed by the little-endian fp32 scale."""
    s = np.asarray(s, dtype=np.float32)
    y = np.array(x, dtype=np.float32, copy=True)
    n, d = y.shape
    rows = np.empty((n, d + 4), dtype=np.uint8)
    y /= s[:, None]
    np.clip(y, -448.0, 448.0, out=y)
    rows[:, :d] = e4m3_bytes(y)
    rows[:, d:] = s.astype("<f4").view(np.uint8).reshape(n, 4)
    return rows


def poison_rows(pool: np.ndarray, rows) -> None:
    """Overwrite pool rows with e4m3fn NaN bytes and a NaN scale."""
    d = pool.shape[1] - 4
    pool[rows, :d] = 0x7F
    pool[rows, d:] = _POISON_SCALE


def _draw_queries(rng, B, H, D):
    q = bf16_bits(rng.standard_normal((B, H, D), dtype=np.float32))
    w = (rng.standard_normal((B, H), dtype=np.float32)
         * np.float32(D ** -0.5 * H ** -0.5)).astype(np.float32)
    return q, w


def _draw_pool(rng, n_rows, D):
    """Key values are drawn before scales, both in fixed-size chunks."""
    x_parts = []
    for start in range(0, n_rows, _KEY_CHUNK_ROWS):
        m = min(_KEY_CHUNK_ROWS, n_rows - start)
        x_parts.append(rng.standard_normal((m, D), dtype=np.float32))
    s = rng.uniform(0.005, 0.05, size=n_rows).astype(np.float32)
    pool = np.empty((n_rows, D + 4), dtype=np.uint8)
    start = 0
    for xp in x_parts:
        m = xp.shape[0]
        pool[start:start + m] = make_key_rows(xp, s[start:start + m])
        start += m
    return pool


def _ceil_div(a, b):
    return -(-a // b)


# ----------------------------------------------------------------------------
# workload families

def contiguous(n_entries=2048, B=1, seed=0, H=HEADS, D=HEAD_DIM, k=TOPK,
               name="tiny-decode") -> Workload:
    """B query rows over one contiguous key array of n_entries rows (no block
    table); every row scores all n_entries entries."""
    rng = np.random.default_rng(seed)
    q, w = _draw_queries(rng, B, H, D)
    pool = _draw_pool(rng, n_entries, D)
    limits = np.full(B, n_entries, dtype=np.int32)
    return Workload(name=name, q=q, w=w, pool=pool, limits=limits,
                    n_cols=n_entries, k=k,
                    description=f"B={B}, contiguous N={n_entries}, seed {seed}")


def paged_decode(entries, seed, H=HEADS, D=HEAD_DIM, k=TOPK, max_blocks=None,
                 poison_frac=0.01, name="paged-decode") -> Workload:
    """One query per request; request b scores its entries[b] compressed
    entries through a shuffled block table of 64-entry blocks.

    entries: sequence of per-request entry counts (already divided by C4)."""
    rng = np.random.default_rng(seed)
    entries = np.asarray(entries, dtype=np.int64)
    return _paged_decode_from(rng, entries, H, D, k, max_blocks, poison_frac,
                              name, f"seed {seed}")


def _paged_decode_from(rng, entries, H, D, k, max_blocks, poison_frac, name,
                       tag):
    B = len(entries)
    nblk = [_ceil_div(int(n), BLOCK) for n in entries]
    if max_blocks is None:
        max_blocks = max(nblk) if nblk else 1
    used = int(sum(nblk))
    n_poison = _ceil_div(used * int(round(poison_frac * 1000)), 1000)
    n_blocks = used + n_poison
    perm = rng.permutation(n_blocks).astype(np.int32)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += nblk[b]
    q, w = _draw_queries(rng, B, H, D)
    pool = _draw_pool(rng, n_blocks * BLOCK, D)
    for b in range(B):                       # tail padding of the last block
        if nblk[b] and entries[b] % BLOCK:
            last = int(table[b, nblk[b] - 1])
            poison_rows(pool, slice(last * BLOCK + int(entries[b] % BLOCK),
                                    (last + 1) * BLOCK))
    for pb in perm[off:]:                    # blocks nobody references
        poison_rows(pool, slice(int(pb) * BLOCK, (int(pb) + 1) * BLOCK))
    return Workload(name=name, q=q, w=w, pool=pool,
                    limits=entries.astype(np.int32), n_cols=max_blocks * BLOCK,
                    k=k, block_table=table,
                    description=f"B={B}, paged, {used} blocks (+{n_poison} poison), {tag}")


def decode_batch(B=32, min_tokens=32768, max_tokens=131072, seed=1, **kw):
    """Context lengths L_b ~ integers U[min_tokens, max_tokens]; N_b = L_b // 4."""
    rng = np.random.default_rng(seed)
    L = rng.integers(min_tokens, max_tokens, size=B, endpoint=True)
    entries = L // COMPRESS
    max_blocks = _ceil_div(max_tokens // COMPRESS, BLOCK)
    return _paged_decode_from(rng, entries, kw.get("H", HEADS), kw.get("D", HEAD_DIM),
                              kw.get("k", TOPK), max_blocks, 0.01,
                              kw.get("name", "decode-batch"),
                              f"L~U[{min_tokens},{max_tokens}], seed {seed}")


def speculative_decode(n_req=16, draft=4, min_tokens=4096, max_tokens=16384, seed=8, k=TOPK,
                       name="speculative-decode") -> Workload:
    """Several query rows per request in one call (the draft tokens of
    speculative decoding): request r has L_r ~ integers U[min_tokens,
    max_tokens] tokens; its draft row i (0-based) scores entries
    < (L_r + i + 1) // 4, and all rows of a request share its shuffled block
    table through q_req.  Draw order: lengths, then the paged pool as in
    paged_decode, then the B = n_req * draft query rows."""
    rng = np.random.default_rng(seed)
    L = rng.integers(min_tokens, max_tokens, size=n_req, endpoint=True)
    entries = (L + draft) // COMPRESS
    base = _paged_decode_from(rng, entries, HEADS, HEAD_DIM, k, None, 0.01, name, f"seed {seed}")
    B = n_req * draft
    q, w = _draw_queries(rng, B, HEADS, HEAD_DIM)
    q_req = np.repeat(np.arange(n_req, dtype=np.int32), draft)
    i = np.tile(np.arange(draft, dtype=np.int64), n_req)
    limits = ((L[q_req] + i + 1) // COMPRESS).astype(np.int32)
    return Workload(name=name, q=q, w=w, pool=base.pool, limits=limits, n_cols=base.n_cols, k=k,
                    block_table=base.block_table, q_req=q_req,
                    description=f"{n_req} requests x {draft} draft rows, L~U[{min_tokens},{max_tokens}], seed {seed}")


def prefill(prefix_tokens=65536, n_queries=4096, seed=3, H=HEADS, D=HEAD_DIM,
            k=TOPK, name="chunked-prefill") -> Workload:
    """One request: query i (0-based) of the new chunk scores entries
    < (prefix_tokens + i + 1) // 4, all rows sharing one block list."""
    rng = np.random.default_rng(seed)
    total_entries = (prefix_tokens + n_queries) // COMPRESS
    nblk = _ceil_div(total_entries, BLOCK)
    n_poison = _ceil_div(nblk * 10, 1000)
    n_blocks = nblk + n_poison
    perm = rng.permutation(n_blocks).astype(np.int32)
    table = perm[:nblk].reshape(1, nblk).copy()
    q, w = _draw_queries(rng, n_queries, H, D)
    pool = _draw_pool(rng, n_blocks * BLOCK, D)
    if total_entries % BLOCK:
        last = int(table[0, -1])
        poison_rows(pool, slice(last * BLOCK + total_entries % BLOCK, (last + 1) * BLOCK))
    for pb in perm[nblk:]:
        poison_rows(pool, slice(int(pb) * BLOCK, (int(pb) + 1) * BLOCK))
    i = np.arange(n_queries, dtype=np.int64)
    limits = ((prefix_tokens + i + 1) // COMPRESS).astype(np.int32)
    return Workload(name=name, q=q, w=w, pool=pool, limits=limits,
                    n_cols=nblk * BLOCK, k=k, block_table=table,
                    q_req=np.zeros(n_queries, dtype=np.int32),
                    description=f"prefix {prefix_tokens} + {n_queries} queries, seed {seed}")


def resident(B=40, chunks_per_req=4096, n_resident=384, seed=4, H=HEADS,
             D=HEAD_DIM, k=TOPK, name="resident-subset") -> Workload:
    """Each request scores only n_resident chunks (64 entries each), drawn
    without replacement from its chunks_per_req chunks and passed as a chunk
    list; only resident chunks have pool blocks (the rest are -1)."""
    rng = np.random.default_rng(seed)
    used = B * n_resident
    n_poison = _ceil_div(used * 10, 1000)
    n_blocks = used + n_poison
    perm = rng.permutation(n_blocks).astype(np.int32)
    chunk_ids = np.stack([rng.choice(chunks_per_req, n_resident, replace=False)
                          for _ in range(B)]).astype(np.int32)
    table = np.full((B, chunks_per_req), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, chunk_ids[b]] = perm[off:off + n_resident]
        off += n_resident
    q, w = _draw_queries(rng, B, H, D)
    pool = _draw_pool(rng, n_blocks * BLOCK, D)
    for pb in perm[off:]:
        poison_rows(pool, slice(int(pb) * BLOCK, (int(pb) + 1) * BLOCK))
    limits = np.full(B, chunks_per_req * BLOCK, dtype=np.int32)
    return Workload(name=name, q=q, w=w, pool=pool, limits=limits,
                    n_cols=n_resident * BLOCK, k=k, block_table=table,
                    chunk_ids=chunk_ids,
                    n_chunks=np.full(B, n_resident, dtype=np.int32),
                    description=f"B={B}, {n_resident}/{chunks_per_req} resident chunks, seed {seed}")


@dataclasses.dataclass
class WriteLoad:
    """Host arrays of one index-plane write: keys k [n, D] (bf16 bits) go to
    pool rows slots [n] (int64, -1 = none) of a pool whose rows start out as
    poison."""

    name: str
    k: np.ndarray                       # uint16 [n, D]
    slots: np.ndarray                   # int64 [n]
    pool: np.ndarray                    # uint8 [n_pool_rows, D + 4] (before the write)
    block_table: np.ndarray             # int32 [1, n_blocks]: the request's blocks
    description: str = ""

    @property
    def n(self) -> int:
        return int(self.k.shape[0])


def index_fill(n_keys=262144, seed=5, D=HEAD_DIM, poison_frac=0.01,
               name="index-fill") -> WriteLoad:
    """The compressed keys of one request (n_keys entries, 262,144 = one
    1M-token context at C4) written into a shuffled paged pool of 64-entry
    blocks: entry e goes to row 64 * table[e // 64] + e % 64.  Key values are
    bf16(N(0, 1) * m) with a per-key magnitude m ~ U(1, 6), so the scales the
    writer derives (amax / 448) fall in about the range the scoring workloads
    draw theirs from.  Unreferenced blocks (1 %) and the tail of the last
    block keep their poison rows.  Draw order: permutation -> magnitudes ->
    values."""
    rng = np.random.default_rng(seed)
    nblk = _ceil_div(n_keys, BLOCK)
    n_blocks = nblk + _ceil_div(nblk * int(round(poison_frac * 1000)), 1000)
    perm = rng.permutation(n_blocks).astype(np.int32)
    table = perm[:nblk].reshape(1, nblk).copy()
    m = rng.uniform(1.0, 6.0, size=n_keys).astype(np.float32)
    x = rng.standard_normal((n_keys, D), dtype=np.float32)
    x *= m[:, None]
    k = bf16_bits(x)
    e = np.arange(n_keys, dtype=np.int64)
    slots = table[0, e // BLOCK].astype(np.int64) * BLOCK + e % BLOCK
    pool = np.empty((n_blocks * BLOCK, D + 4), dtype=np.uint8)
    poison_rows(pool, slice(None))
    return WriteLoad(name=name, k=k, slots=slots, pool=pool, block_table=table,
                     description=f"{n_keys} keys into {nblk} shuffled blocks (+{n_blocks - nblk} unreferenced), seed {seed}")


@dataclasses.dataclass
class ResidentLoad:
    """One Level-1 selection problem: per-layer scoring workloads (same rows,
    same limits, each layer its own q, w and paged index plane) and the
    selection settings."""

    name: str
    layers: list                        # [Workload] * n_layers
    kmax: int = 384
    threshold: float = 0.76
    n_sink: int = 1
    n_recent: int = 1
    ensemble: int = 0                   # 0 = max, 1 = mean
    description: str = ""

    @property
    def B(self) -> int:
        return self.layers[0].B

    @property
    def n_cols(self) -> int:
        return self.layers[0].n_cols

    @property
    def limits(self) -> np.ndarray:
        return self.layers[0].limits


def memory_indexer(entries=(262144,) * 8, n_layers=3, seed=6, kmax=384, threshold=0.76,
                   n_sink=1, n_recent=1, ensemble=0, H=HEADS, name="memory-indexer") -> ResidentLoad:
    """Level 1 over each request's whole history: layer l is a paged decode
    workload of the given per-request entry counts drawn from seed
    16 * seed + l (its own q, w, keys and block table, the same limits).
    Defaults: 8 requests at 1M tokens (262,144 entries), 3 layers, KMAX 384
    pages, one sink page and one recent page, threshold 0.76 (the maximum of
    three layers' synthetic scores passes it for about 12 % of the entries,
    inside the 10-15 % resident share the pages report).  H = 128 gives the
    trained retriever's head count."""
    entries = np.asarray(entries, dtype=np.int64)
    mb = _ceil_div(int(entries.max()), BLOCK)
    layers = [_paged_decode_from(np.random.default_rng(16 * seed + l), entries, H, HEAD_DIM, TOPK,
                                 mb, 0.01, f"{name}-layer{l}", f"seed {16 * seed + l}")
              for l in range(n_layers)]
    return ResidentLoad(name=name, layers=layers, kmax=kmax, threshold=threshold, n_sink=n_sink,
                        n_recent=n_recent, ensemble=ensemble,
                        description=(f"B={len(entries)}, {n_layers} layers, entries {int(entries.min())}.."
                                     f"{int(entries.max())}, KMAX {kmax}, threshold {threshold}, "
                                     f"sink {n_sink}, recent {n_recent}, seed {seed}"))


# ----------------------------------------------------------------------------
# the five named workloads at full size, and small variants of each

def config(i: int) -> Workload:
    """The five workloads at full size (seed = workload number)."""
    if i == 0:
        return contiguous(2048, B=1, seed=0, name="tiny-decode")
    if i == 1:
        return decode_batch(32, 32768, 131072, seed=1, name="decode-batch")
    if i == 2:
        return paged_decode([262144] * 8, seed=2, name="long-decode")
    if i == 3:
        return prefill(65536, 4096, seed=3, name="chunked-prefill")
    if i == 4:
        return resident(40, 4096, 384, seed=4, name="resident-subset")
    raise ValueError(f"no workload {i}")


def small_config(i: int, seed: Optional[int] = None) -> Workload:
    """Same recipe as config(i) at oracle-friendly sizes: several blocks per
    row and ragged tails."""
    s = (100 + i) if seed is None else seed
    if i == 0:
        return contiguous(2048, B=1, seed=s, name="tiny-decode")
    if i == 1:
        return decode_batch(6, 2048, 8192, seed=s, name="decode-batch-small")
    if i == 2:
        return paged_decode([16384, 16384], seed=s, name="long-decode-small")
    if i == 3:
        return prefill(4096, 64, seed=s, name="chunked-prefill-small")
    if i == 4:
        return resident(5, 256, 24, seed=s, name="resident-subset-small")
    raise ValueError(f"no workload {i}")


def reblock(wl: Workload, seed: int, block_size: int = 16, ragged: bool = True,
            name: Optional[str] = None) -> Workload:
    """The same keys in pool blocks of `block_size` rows ("DeepSeek-V4.1
    native paged runtime": a block id names 16 index rows).

    Each 64-row block of wl's pool is cut into 64 / block_size small blocks
    and every small block moves to its own place in a new pool (a seeded
    permutation), so the blocks one 64-entry stretch of a row reads lie
    apart; the block table grows to name the small blocks.  A chunk list is
    expanded the same way; with `ragged`, each row's small chunks are then
    shuffled and a few dropped, so chunk counts are not multiples of
    64 / block_size and one 64-column stretch mixes chunks of different
    64-entry blocks.  Without a block table only block_size changes (rows
    are entries).  Every key row keeps its bytes, so each logical entry
    scores as it did in wl."""
    bs = int(block_size)
    if bs <= 0 or BLOCK % bs:
        raise ValueError("block_size must divide 64")
    U = BLOCK // bs
    rng = np.random.default_rng(seed)
    out = dataclasses.replace(wl, block_size=bs, name=name or f"{wl.name}-b{bs}",
                              description=f"{wl.description}; {bs}-row blocks, seed {seed}")
    if wl.block_table is not None:
        n_small = wl.n_pool_rows // bs
        perm = rng.permutation(n_small)
        pool = np.empty_like(wl.pool)
        pool.reshape(n_small, bs, -1)[perm] = wl.pool.reshape(n_small, bs, -1)
        t = wl.block_table.astype(np.int64)
        small = perm[np.maximum(t, 0)[:, :, None] * U + np.arange(U)]
        table = np.where(t[:, :, None] >= 0, small, -1).reshape(t.shape[0], -1)
        out.pool = pool
        out.block_table = table.astype(np.int32)
    if wl.chunk_ids is not None:
        B, mc = wl.chunk_ids.shape
        ids = np.full((B, mc * U), -1, dtype=np.int32)
        counts = np.zeros(B, dtype=np.int32)
        for b in range(B):
            nc = min(int(wl.n_chunks[b]), mc)
            c = wl.chunk_ids[b, :nc].astype(np.int64)
            c = np.where(c[:, None] >= 0, c[:, None] * U + np.arange(U), -1).ravel()
            if ragged and c.size:
                c = c[rng.permutation(c.size)]
                c = c[:c.size - int(rng.integers(0, min(2 * U, c.size) + 1))]
            ids[b, :c.size] = c
            counts[b] = c.size
        out.chunk_ids = ids
        out.n_chunks = counts
    return out


WORKLOAD_NAMES = {0: "tiny-decode", 1: "decode-batch", 2: "long-decode",
                  3: "chunked-prefill", 4: "resident-subset"}
