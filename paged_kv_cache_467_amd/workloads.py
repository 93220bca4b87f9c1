"""Seeded synthetic decode batches for paged attention.

This module only builds inputs: sequence lengths, block tables, the K/V pool,
the new tokens to be written and their slot_mapping.  It holds none of the
attention arithmetic, and it is the one module that both the HIP path's tests
and the CPU oracle are fed from.

The layout follows the pages:
  * key_cache / value_cache are ``[num_blocks, block_size, num_kv_heads,
    head_dim]`` ("vLLM 源码解析 一", §三, the paged_attention_v1 description);
  * ``block_tables[s]`` lists the physical blocks of sequence ``s`` in logical
    order ("23.1 vLLM：高吞吐推理框架原理与部署", §二.2, steps 1-3);
  * ``slot_mapping[t]`` names the cell that new token ``t`` is written to
    ("大模型推理框架VLLM-0.7.3源码", §2.1), encoded as
    ``physical_block * block_size + offset`` to match the pool's two leading
    dimensions.

Element data are carried as raw bits: ``float32`` arrays for f32 and
``uint16`` arrays for f16 / bf16, so that every consumer reads the very same
bits.  Values are standard normal float32 samples, cast round-to-nearest-even.

Five named workloads stand in for the situations the pages describe (a tiny
unit case, a Llama-3-8B-shaped GQA batch, a Llama-13B-shaped MHA batch, a
32K-token long-context batch and a shared-prefix batch); ``make_custom``
builds arbitrary small shapes for property tests.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# dtype name -> (code used at the C boundary, bytes per element)
DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2}
DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
NAN_BITS = {"f32": np.float32(np.nan), "f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0)}


def f32_to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Cast float32 samples to the storage dtype, round-to-nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        u = x.view(np.uint32)
        # round half to even on the 16 dropped bits (finite inputs: no overflow)
        u = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
        return (u >> np.uint32(16)).astype(np.uint16)
    raise ValueError(dtype)


def bits_to_f32(b: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored bits to float32 (exact for all three dtypes)."""
    if dtype == "f32":
        return np.asarray(b, dtype=np.float32)
    if dtype == "f16":
        return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dtype)


def storage_dtype(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


@dataclass
class DecodeBatch:
    """One decode step's inputs: a paged K/V pool, its block tables and the
    new tokens (one per sequence) that the step writes before attending."""

    name: str
    dtype: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    scale: float                     # a float32 value
    query: np.ndarray                # [S, Hq, D] bits
    key_cache: np.ndarray            # [num_blocks, bs, Hkv, D] bits
    value_cache: np.ndarray          # [num_blocks, bs, Hkv, D] bits
    block_tables: np.ndarray         # [S, max_blocks_per_seq] int32
    context_lens: np.ndarray         # [S] int32
    new_key: np.ndarray              # [T, Hkv, D] bits
    new_value: np.ndarray            # [T, Hkv, D] bits
    slot_mapping: np.ndarray         # [T] int32
    referenced_blocks: np.ndarray    # sorted unique block ids reachable from block_tables
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def dtype_code(self) -> int:
        return DTYPE_CODES[self.dtype]

    @property
    def elem_bytes(self) -> int:
        return DTYPE_BYTES[self.dtype]

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def copy(self) -> "DecodeBatch":
        out = DecodeBatch(**{k: (v.copy() if isinstance(v, np.ndarray) else v)
                             for k, v in self.__dict__.items() if k != "meta"})
        out.meta = dict(self.meta)
        return out

    # ---- byte accounting used by the bench (algorithmic, not measured) ----
    def decode_algorithmic_bytes(self) -> int:
        """K and V rows of positions [0, L_s) for every kv head, the query
        read and the output written, the block-table entries used and the
        context lengths."""
        e = self.elem_bytes
        L = self.context_lens.astype(np.int64)
        kv = int(L.sum()) * self.num_kv_heads * self.head_dim * e * 2
        qo = 2 * self.num_seqs * self.num_q_heads * self.head_dim * e
        bt = int(np.sum((L + self.block_size - 1) // self.block_size)) * 4
        return kv + qo + bt + 4 * self.num_seqs

    def decode_unique_bytes(self) -> int:
        """decode_algorithmic_bytes with each distinct pool cell counted once:
        the least HBM traffic a decode of this batch can have when cells that
        several sequences share (a common prefix) are fetched once."""
        bs = self.block_size
        cells = set()
        for s in range(self.num_seqs):
            L = int(self.context_lens[s])
            for i in range((L + bs - 1) // bs):
                blk = int(self.block_tables[s, i])
                for off in range(min(bs, L - i * bs)):
                    cells.add(blk * bs + off)
        e = self.elem_bytes
        kv = len(cells) * self.num_kv_heads * self.head_dim * e * 2
        return self.decode_algorithmic_bytes() - \
            int(self.context_lens.astype(np.int64).sum()) * self.num_kv_heads * self.head_dim * e * 2 \
            + kv

    def write_algorithmic_bytes(self) -> int:
        t = len(self.slot_mapping)
        row = self.num_kv_heads * self.head_dim * self.elem_bytes
        return t * row * 2 * 2 + 4 * t

    def decode_flops(self) -> int:
        return int(self.context_lens.astype(np.int64).sum()) * self.num_q_heads * 4 * self.head_dim


def _normal_bits(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    return f32_to_bits(rng.standard_normal(size=shape, dtype=np.float32), dtype)


def _assemble(name, dtype, rng, *, S, Hq, Hkv, D, bs, lens, tables, num_blocks,
              max_blocks, scale, poison, seed, meta=None, keys_identical=False, values=True):
    """Fill the pool rows that block tables reach, poison or zero the rest,
    draw queries and the new tokens, and derive slot_mapping for a write of
    one new token per sequence at position L_s - 1.  With values=False the
    pool arrays are left empty (shape (0,)): only the structure is built."""
    sd = storage_dtype(dtype)
    lens = np.asarray(lens, dtype=np.int32)
    bt = np.asarray(tables, dtype=np.int32)
    assert bt.shape == (S, max_blocks)
    referenced = set()
    for s in range(S):
        nb = (int(lens[s]) + bs - 1) // bs
        referenced.update(int(b) for b in bt[s, :nb])
    referenced = np.array(sorted(referenced), dtype=np.int64)

    fill = NAN_BITS[dtype] if poison else sd(0)
    if not values:
        key_cache = value_cache = np.zeros((0,), dtype=sd)
        poison = keys_identical = False
    else:
        key_cache = np.full((num_blocks, bs, Hkv, D), fill, dtype=sd)
        value_cache = np.full((num_blocks, bs, Hkv, D), fill, dtype=sd)
    if values and len(referenced):
        key_cache[referenced] = _normal_bits(rng, (len(referenced), bs, Hkv, D), dtype)
        value_cache[referenced] = _normal_bits(rng, (len(referenced), bs, Hkv, D), dtype)
    if poison:
        # Tail slots of each sequence's last block hold stale data: positions
        # >= L_s must never be read, so make them NaN as well.  Shared blocks
        # are only ever shared whole (the prefix), so this never hits a slot
        # that another sequence uses.
        used = np.zeros((num_blocks, bs), dtype=bool)
        for s in range(S):
            L = int(lens[s])
            nb = (L + bs - 1) // bs
            for i in range(nb):
                n = min(bs, L - i * bs)
                used[bt[s, i], :n] = True
        key_cache[~used] = NAN_BITS[dtype]
        value_cache[~used] = NAN_BITS[dtype]
    query = _normal_bits(rng, (S, Hq, D), dtype)
    if keys_identical:
        one = _normal_bits(rng, (Hkv, D), dtype)
        for b in referenced:
            key_cache[b] = one[None]
    new_key = _normal_bits(rng, (S, Hkv, D), dtype)
    new_value = _normal_bits(rng, (S, Hkv, D), dtype)
    slots = np.empty(S, dtype=np.int32)
    for s in range(S):
        L = int(lens[s])
        if L <= 0:
            slots[s] = -1          # nothing to write for an empty sequence
            continue
        j = L - 1
        slots[s] = int(bt[s, j // bs]) * bs + j % bs
    return DecodeBatch(
        name=name, dtype=dtype, num_seqs=S, num_q_heads=Hq, num_kv_heads=Hkv,
        head_dim=D, block_size=bs, num_blocks=num_blocks, max_blocks_per_seq=max_blocks,
        scale=float(np.float32(scale)), query=query, key_cache=key_cache,
        value_cache=value_cache, block_tables=bt, context_lens=lens, new_key=new_key,
        new_value=new_value, slot_mapping=slots, referenced_blocks=referenced,
        seed=seed, meta=dict(meta or {}))


def _deal_tables(rng, lens, bs, max_blocks, pool_factor=1.5, min_pool=None):
    """Each sequence gets ceil(L/bs) blocks drawn, in order, from one random
    permutation of the pool; unused table entries point at a block no
    sequence uses (so that a stray read of padding lands on poisoned data)."""
    S = len(lens)
    need = [(int(L) + bs - 1) // bs for L in lens]
    total = sum(need)
    pool = int(math.ceil(pool_factor * total))
    if min_pool is not None:
        pool = max(pool, min_pool)
    pool = max(pool, total + 1)
    perm = rng.permutation(pool)
    free_block = int(perm[total])
    tables = np.full((S, max_blocks), free_block, dtype=np.int32)
    k = 0
    for s in range(S):
        assert need[s] <= max_blocks
        tables[s, :need[s]] = perm[k:k + need[s]]
        k += need[s]
    return tables, pool


WORKLOADS = ("tiny_f32", "llama3_8b_gqa_bf16", "llama13b_mha_f16",
             "long_context_bf16", "shared_prefix_bf16")


def make_workload(name: str, seed: int | None = None, poison: bool = False,
                  values: bool = True) -> DecodeBatch:
    """Build one of the five named workloads (seed defaults to 46700 + index).
    values=False builds only lengths, tables and slots (no pool contents)."""
    idx = WORKLOADS.index(name)
    seed = 46700 + idx + 1 if seed is None else seed
    rng = np.random.default_rng(seed)
    if name == "tiny_f32":
        S, Hq, Hkv, D, bs, pool, mb = 4, 4, 4, 64, 16, 64, 7
        lens = [1, 17, 33, 100]
        tables, _ = _deal_tables(rng, lens, bs, mb, min_pool=pool)
        tables_pool = pool
        return _assemble(name, "f32", rng, S=S, Hq=Hq, Hkv=Hkv, D=D, bs=bs, lens=lens,
                         tables=tables, num_blocks=tables_pool, max_blocks=mb,
                         scale=1.0 / math.sqrt(64), poison=poison, seed=seed, values=values)
    if name == "llama3_8b_gqa_bf16":
        S, Hq, Hkv, D, bs, mb = 256, 32, 8, 128, 16, 40
        lens = rng.integers(512, 640, size=S, endpoint=True)
        tables, pool = _deal_tables(rng, lens, bs, mb)
        return _assemble(name, "bf16", rng, S=S, Hq=Hq, Hkv=Hkv, D=D, bs=bs, lens=lens,
                         tables=tables, num_blocks=pool, max_blocks=mb,
                         scale=1.0 / math.sqrt(D), poison=poison, seed=seed, values=values)
    if name == "llama13b_mha_f16":
        S, Hq, Hkv, D, bs, mb = 50, 40, 40, 128, 16, 128
        lens = rng.integers(1, 2048, size=S, endpoint=True)
        tables, pool = _deal_tables(rng, lens, bs, mb)
        return _assemble(name, "f16", rng, S=S, Hq=Hq, Hkv=Hkv, D=D, bs=bs, lens=lens,
                         tables=tables, num_blocks=pool, max_blocks=mb,
                         scale=1.0 / math.sqrt(D), poison=poison, seed=seed, values=values)
    if name == "long_context_bf16":
        S, Hq, Hkv, D, bs, mb = 8, 32, 8, 128, 32, 1024
        lens = rng.integers(24576, 32768, size=S, endpoint=True)
        tables, pool = _deal_tables(rng, lens, bs, mb)
        return _assemble(name, "bf16", rng, S=S, Hq=Hq, Hkv=Hkv, D=D, bs=bs, lens=lens,
                         tables=tables, num_blocks=pool, max_blocks=mb,
                         scale=1.0 / math.sqrt(D), poison=poison, seed=seed, values=values)
    if name == "shared_prefix_bf16":
        S, Hq, Hkv, D, bs = 64, 32, 8, 128, 16
        prefix_blocks = 125                     # 2000 tokens
        z = rng.standard_normal(S)
        suffix = np.clip(np.rint(np.exp(math.log(64.0) + 0.5 * z)), 16, 256).astype(np.int64)
        priv = (suffix + bs - 1) // bs
        mb = prefix_blocks + 16
        total = prefix_blocks + int(priv.sum())
        pool = int(math.ceil(1.5 * total))
        perm = rng.permutation(pool)
        prefix = perm[:prefix_blocks]
        free_block = int(perm[total])
        tables = np.full((S, mb), free_block, dtype=np.int32)
        k = prefix_blocks
        for s in range(S):
            tables[s, :prefix_blocks] = prefix
            tables[s, prefix_blocks:prefix_blocks + priv[s]] = perm[k:k + priv[s]]
            k += int(priv[s])
        lens = prefix_blocks * bs + suffix
        return _assemble(name, "bf16", rng, S=S, Hq=Hq, Hkv=Hkv, D=D, bs=bs, lens=lens,
                         tables=tables, num_blocks=pool, max_blocks=mb,
                         scale=1.0 / math.sqrt(D), poison=poison, seed=seed, values=values,
                         meta={"prefix_blocks": prefix_blocks})
    raise ValueError(name)


def make_custom(seed: int, *, dtype="f32", num_seqs=2, num_q_heads=2, num_kv_heads=1,
                head_dim=64, block_size=16, context_lens=(5, 20), extra_blocks=3,
                max_blocks_per_seq=None, poison=False, scale=None,
                keys_identical=False) -> DecodeBatch:
    """A small batch of any shape: blocks dealt from a random permutation of a
    pool with ``extra_blocks`` spare blocks."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(context_lens, dtype=np.int64)
    assert len(lens) == num_seqs
    need = [(int(L) + block_size - 1) // block_size for L in lens]
    mb = max_blocks_per_seq if max_blocks_per_seq is not None else max(1, max(need))
    tables, pool = _deal_tables(rng, lens, block_size, mb, pool_factor=1.0,
                                min_pool=sum(need) + max(1, extra_blocks))
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return _assemble(f"custom{seed}", dtype, rng, S=num_seqs, Hq=num_q_heads,
                     Hkv=num_kv_heads, D=head_dim, bs=block_size, lens=lens,
                     tables=tables, num_blocks=pool, max_blocks=mb, scale=scale,
                     poison=poison, seed=seed, keys_identical=keys_identical)


def make_shared_prefix(seed: int, *, dtype="bf16", num_q_heads=8, num_kv_heads=2,
                       head_dim=128, block_size=16, prefix_len=64, suffix_lens=(0, 5),
                       max_blocks_per_seq=None, poison=False, scale=None) -> DecodeBatch:
    """A batch whose sequences all begin with the same prefix_len positions
    in the same physical blocks (the first prefix_len / block_size of a
    random permutation of the pool), each followed by suffix_lens[s]
    positions in blocks of its own; like the shared-prefix workload, at any
    shape."""
    assert prefix_len % block_size == 0
    rng = np.random.default_rng(seed)
    S = len(suffix_lens)
    bs = block_size
    suffix = np.asarray(suffix_lens, dtype=np.int64)
    pb = prefix_len // bs
    priv = (suffix + bs - 1) // bs
    need = pb + int(priv.max()) if S else pb
    mb = max_blocks_per_seq if max_blocks_per_seq is not None else max(1, need)
    assert mb >= need
    total = pb + int(priv.sum())
    pool = total + 3
    perm = rng.permutation(pool)
    free_block = int(perm[total])
    tables = np.full((S, mb), free_block, dtype=np.int32)
    k = pb
    for s in range(S):
        tables[s, :pb] = perm[:pb]
        tables[s, pb:pb + priv[s]] = perm[k:k + priv[s]]
        k += int(priv[s])
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return _assemble(f"shared{seed}", dtype, rng, S=S, Hq=num_q_heads, Hkv=num_kv_heads,
                     D=head_dim, bs=bs, lens=prefix_len + suffix, tables=tables,
                     num_blocks=pool, max_blocks=mb, scale=scale, poison=poison, seed=seed,
                     meta={"prefix_blocks": pb})


@dataclass
class PrefillBatch:
    """Multi-token (chunked-prefill) inputs: a paged pool whose sequences
    already hold their q_len new tokens at positions L - q_len .. L - 1, and
    the queries of those new tokens, all sequences one after another
    (``query_start[s] .. query_start[s+1] - 1`` are sequence s's rows)."""

    base: DecodeBatch                # pool, tables, context_lens (L includes the new tokens)
    query: np.ndarray                # [total_q, Hq, D] bits
    query_start: np.ndarray          # [S + 1] int32

    def __getattr__(self, name):
        # pool, shapes and lengths come from the decode batch underneath
        if name in ("base", "query", "query_start"):
            raise AttributeError(name)
        return getattr(self.base, name)

    @property
    def query_lens(self) -> np.ndarray:
        return np.diff(self.query_start).astype(np.int32)

    @property
    def total_q(self) -> int:
        return int(self.query_start[-1])

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if self.base.num_seqs else 0

    def copy(self) -> "PrefillBatch":
        return PrefillBatch(self.base.copy(), self.query.copy(), self.query_start.copy())

    def flops(self) -> int:
        """Causal attention FLOPs: new token i of sequence s scores and
        averages L - q_len + i + 1 positions, 4 * head_dim flops each, for
        every query head."""
        total = 0
        for L, q in zip(self.base.context_lens.astype(np.int64), self.query_lens.astype(np.int64)):
            if 0 < q <= L:
                total += int(q * (L - q) + q * (q + 1) // 2)
        return total * self.base.num_q_heads * 4 * self.base.head_dim

    def algorithmic_bytes(self, elem_bytes: int | None = None) -> int:
        """Each sequence's K/V rows once, the queries read, the outputs
        written, block-table entries and the two length arrays (elements of
        elem_bytes bytes, default the batch's own)."""
        b = self.base
        e = b.elem_bytes if elem_bytes is None else elem_bytes
        L = b.context_lens.astype(np.int64)
        kv = int(L.sum()) * b.num_kv_heads * b.head_dim * e * 2
        qo = 2 * self.total_q * b.num_q_heads * b.head_dim * e
        bt = int(np.sum((L + b.block_size - 1) // b.block_size)) * 4
        return kv + qo + bt + 4 * (2 * b.num_seqs + 1)


def make_prefill(seed: int, *, dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=128,
                 block_size=16, context_lens=(40, 17), query_lens=(8, 17), extra_blocks=3,
                 pool_factor=1.0, poison=False, scale=None, values=True,
                 name=None) -> PrefillBatch:
    """A multi-token batch: sequence s holds context_lens[s] tokens, the last
    query_lens[s] of them new (their queries are drawn here, their K/V are
    already in the pool).  Blocks are dealt as for make_custom."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(context_lens, dtype=np.int64)
    qlens = np.asarray(query_lens, dtype=np.int64)
    assert lens.shape == qlens.shape
    need = [(int(L) + block_size - 1) // block_size for L in lens]
    mb = max(1, max(need))
    tables, pool = _deal_tables(rng, lens, block_size, mb, pool_factor=pool_factor,
                                min_pool=sum(need) + max(1, extra_blocks))
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    base = _assemble(name or f"prefill{seed}", dtype, rng, S=len(lens), Hq=num_q_heads,
                     Hkv=num_kv_heads, D=head_dim, bs=block_size, lens=lens, tables=tables,
                     num_blocks=pool, max_blocks=mb, scale=scale, poison=poison, seed=seed,
                     values=values)
    qs = np.zeros(len(lens) + 1, dtype=np.int32)
    qs[1:] = np.cumsum(qlens)
    query = _normal_bits(rng, (int(qs[-1]), num_q_heads, head_dim), dtype)
    return PrefillBatch(base, query, qs)


PREFILL_WORKLOADS = ("llama3_8b_chunked_prefill_bf16",)


def make_prefill_workload(name: str, seed: int | None = None, poison: bool = False,
                          values: bool = True) -> PrefillBatch:
    """Chunked prefill on the Llama-3-8B shape: 16 prompts of 1024..2048
    tokens whose last 512 tokens are processed as one chunk (the earlier ones
    already cached), 32 query / 8 kv heads, head_dim 128, block_size 16;
    bf16 (llama3_8b_chunked_prefill_bf16), or the same draws in f16 or f32
    (the name's suffix)."""
    stem = "llama3_8b_chunked_prefill_"
    dtype = name[len(stem):] if name.startswith(stem) else None
    if dtype not in ("bf16", "f16", "f32"):
        raise ValueError(name)
    seed = 46710 if seed is None else seed
    rng = np.random.default_rng(seed)
    lens = rng.integers(1024, 2048, size=16, endpoint=True)
    return make_prefill(seed, dtype=dtype, num_q_heads=32, num_kv_heads=8, head_dim=128,
                        block_size=16, context_lens=lens, query_lens=np.full(16, 512),
                        pool_factor=1.5, poison=poison, values=values, name=name)


def permute_blocks(batch: DecodeBatch, seed: int) -> DecodeBatch:
    """Relabel physical blocks by a random permutation pi: pool row b moves
    to pi[b] and every table entry b becomes pi[b].  The logical contents of
    every sequence are unchanged."""
    rng = np.random.default_rng(seed)
    pi = rng.permutation(batch.num_blocks).astype(np.int64)
    out = batch.copy()
    out.key_cache = np.empty_like(batch.key_cache)
    out.value_cache = np.empty_like(batch.value_cache)
    out.key_cache[pi] = batch.key_cache
    out.value_cache[pi] = batch.value_cache
    out.block_tables = pi[batch.block_tables].astype(np.int32)
    bs = batch.block_size
    sl = batch.slot_mapping.astype(np.int64)
    ok = sl >= 0
    new_sl = sl.copy()
    new_sl[ok] = pi[sl[ok] // bs] * bs + sl[ok] % bs
    out.slot_mapping = new_sl.astype(np.int32)
    out.referenced_blocks = np.sort(pi[batch.referenced_blocks])
    return out


# ---- prefix caching ----
@dataclass
class PrefixBatch:
    """Token sequences for prefix-cache hashing: tokens one after another,
    token_start [S+1] and block_start [S+1] (prefix sums of full-block
    counts)."""
    name: str
    block_size: int
    tokens: np.ndarray       # [T] int32
    token_start: np.ndarray  # [S + 1] int32
    block_start: np.ndarray  # [S + 1] int32
    shared_blocks: int       # full blocks of the prompt every sequence starts with

    @property
    def num_seqs(self) -> int:
        return len(self.token_start) - 1

    @property
    def total_blocks(self) -> int:
        return int(self.block_start[-1])

    def seq_tokens(self, s: int) -> np.ndarray:
        return self.tokens[self.token_start[s]:self.token_start[s + 1]]


def make_prefix_batch(seed: int, *, num_seqs=256, block_size=16, system_len=512,
                      doc_len=1024, num_docs=8, doc_share=0.5, suffix=(64, 1024),
                      vocab=152064, name="prefix") -> PrefixBatch:
    """Requests that all begin with one system prompt of system_len tokens
    (the pages' long shared system prompt); a doc_share fraction of them
    then carry one of num_docs retrieved documents of doc_len tokens (the
    RAG case, documents placed right after the prompt so that requests on
    the same document share it), then a private suffix of U{suffix} tokens.
    Token ids uniform in [0, vocab)."""
    rng = np.random.default_rng(seed)
    system = rng.integers(0, vocab, size=system_len).astype(np.int32)
    docs = [rng.integers(0, vocab, size=doc_len).astype(np.int32) for _ in range(num_docs)]
    seqs = []
    for _ in range(num_seqs):
        parts = [system]
        if num_docs and rng.random() < doc_share:
            parts.append(docs[int(rng.integers(0, num_docs))])
        parts.append(rng.integers(0, vocab, size=int(rng.integers(suffix[0], suffix[1],
                                                                   endpoint=True))
                                  ).astype(np.int32))
        seqs.append(np.concatenate(parts))
    lens = np.array([len(x) for x in seqs], dtype=np.int64)
    token_start = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    block_start = np.concatenate([[0], np.cumsum(lens // block_size)]).astype(np.int32)
    return PrefixBatch(name, block_size, np.concatenate(seqs).astype(np.int32), token_start,
                       block_start, system_len // block_size)


PREFIX_WORKLOADS = ("shared_system_prompt_rag",)


def make_prefix_workload(name: str) -> PrefixBatch:
    """256 requests behind one 512-token system prompt, half of them with
    one of 8 retrieved 1024-token documents, private suffixes of 64..1024
    tokens, 16-token blocks."""
    if name != "shared_system_prompt_rag":
        raise ValueError(name)
    return make_prefix_batch(46720, name=name)
