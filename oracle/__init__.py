"""CPU oracle for paged-attention decode, the paged KV write and the gather.

TEST INFRASTRUCTURE: only the tests, ``__graft_entry__.smoke()`` and the
bench's CPU-baseline leg may import this package.  The product path never
calls it.  It wraps ``liboracle.so`` (built from ``paged_attention_oracle.c``
by ``oracle/build.py``), a plain fp64 implementation that shares no code with
the HIP library.

Arrays are numpy, element data as stored bits (float32 for f32, uint16 for
f16/bf16); dtype codes are 0 = f32, 1 = f16, 2 = bf16.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import LIBRARY, build

_CODES = {"f32": 0, "f16": 1, "bf16": 2}


def _code(dtype) -> int:
    return _CODES[dtype] if isinstance(dtype, str) else int(dtype)


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """ctypes wrapper around one build of the oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        sig = {
            "oracle_paged_attention_decode": [vp, vp, vp, vp, vp, cf] + [ci] * 7 + [vp, vp, ci],
            "oracle_paged_attention_decode_partitioned": [vp, vp, vp, vp, vp, cf] + [ci] * 8 + [vp],
            "oracle_kv_cache_write": [vp, vp, vp, vp, vp] + [ci] * 5,
            "oracle_paged_kv_gather": [vp, vp, vp, vp, vp, vp] + [ci] * 7,
            "oracle_copy_blocks": [vp, vp, vp] + [ci] * 5,
            "oracle_swap_blocks": [vp, vp, ci, vp, vp, ci, vp] + [ci] * 5,
            "oracle_prefix_block_hashes": [vp, ci, ci, ctypes.c_uint64, ctypes.c_uint64, vp],
            "oracle_paged_attention_prefill": [vp] * 6 + [cf] + [ci] * 7 + [vp],
            "oracle_elements_to_double": [vp, ctypes.c_int64, ci, vp],
            "oracle_set_threads": [ci],
            "oracle_max_threads": [],
        }
        for name, args in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ci if name == "oracle_max_threads" else None
        self.lib = lib
        self.path = path

    def max_threads(self) -> int:
        return self.lib.oracle_max_threads()

    def set_threads(self, n: int) -> None:
        self.lib.oracle_set_threads(int(n))

    def elements_to_double(self, bits: np.ndarray, dtype) -> np.ndarray:
        bits = np.ascontiguousarray(bits)
        out = np.empty(bits.size, dtype=np.float64)
        self.lib.oracle_elements_to_double(_ptr(bits), bits.size, _code(dtype), _ptr(out))
        return out.reshape(bits.shape)

    def paged_attention_decode(self, query, key_cache, value_cache, block_tables,
                               context_lens, scale, dtype, *, return_weights=False):
        """fp64 decode attention -> out [S, Hq, D] (and weights [S, Hq, max L])."""
        S, Hq, D = query.shape
        nb, bs, Hkv, D2 = key_cache.shape
        assert D2 == D and value_cache.shape == key_cache.shape and Hq % Hkv == 0
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        cl = np.ascontiguousarray(context_lens, dtype=np.int32)
        out = np.empty((S, Hq, D), dtype=np.float64)
        wstride = max(1, int(cl.max()) if S else 1)
        weights = np.zeros((S, Hq, wstride), dtype=np.float64) if return_weights else None
        self.lib.oracle_paged_attention_decode(
            _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(bt), _ptr(cl),
            ctypes.c_float(scale), S, Hq, Hkv, D, bs, bt.shape[1], _code(dtype), _ptr(out),
            _ptr(weights), wstride)
        return (out, weights) if return_weights else out

    def paged_attention_decode_partitioned(self, query, key_cache, value_cache, block_tables,
                                           context_lens, scale, dtype, partition_size):
        S, Hq, D = query.shape
        nb, bs, Hkv, _ = key_cache.shape
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        cl = np.ascontiguousarray(context_lens, dtype=np.int32)
        out = np.empty((S, Hq, D), dtype=np.float64)
        self.lib.oracle_paged_attention_decode_partitioned(
            _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(bt), _ptr(cl),
            ctypes.c_float(scale), S, Hq, Hkv, D, bs, bt.shape[1], _code(dtype),
            int(partition_size), _ptr(out))
        return out

    def kv_cache_write(self, key, value, slot_mapping, key_cache, value_cache, dtype):
        """Writes into key_cache / value_cache in place."""
        T, Hkv, D = key.shape
        nb, bs, Hkv2, D2 = key_cache.shape
        assert (Hkv2, D2) == (Hkv, D)
        sm = np.ascontiguousarray(slot_mapping, dtype=np.int32)
        self.lib.oracle_kv_cache_write(_ptr(key), _ptr(value), _ptr(sm), _ptr(key_cache),
                                       _ptr(value_cache), T, Hkv, D, bs, _code(dtype))

    def paged_kv_gather(self, key_cache, value_cache, block_tables, context_lens,
                        max_context_len, dtype, fill=0):
        nb, bs, Hkv, D = key_cache.shape
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        cl = np.ascontiguousarray(context_lens, dtype=np.int32)
        S = bt.shape[0]
        out_k = np.full((S, max_context_len, Hkv, D), fill, dtype=key_cache.dtype)
        out_v = np.full((S, max_context_len, Hkv, D), fill, dtype=key_cache.dtype)
        self.lib.oracle_paged_kv_gather(_ptr(key_cache), _ptr(value_cache), _ptr(bt), _ptr(cl),
                                        _ptr(out_k), _ptr(out_v), S, Hkv, D, bs, bt.shape[1],
                                        int(max_context_len), _code(dtype))
        return out_k, out_v

    def paged_attention_prefill(self, query, key_cache, value_cache, block_tables,
                                context_lens, query_start, scale, dtype):
        """Multi-token causal attention over the paged cache; returns fp64
        [total_q, Hq, D].  Row i of sequence s sits at position
        context_lens[s] - q_len_s + i and attends over positions 0 .. that."""
        total_q, Hq, D = query.shape
        nb, bs, Hkv, D2 = key_cache.shape
        assert D2 == D
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        cl = np.ascontiguousarray(context_lens, dtype=np.int32)
        qs = np.ascontiguousarray(query_start, dtype=np.int32)
        S = bt.shape[0]
        assert qs.shape == (S + 1,) and qs[-1] == total_q
        out = np.zeros((total_q, Hq, D), dtype=np.float64)
        self.lib.oracle_paged_attention_prefill(
            _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(bt), _ptr(cl), _ptr(qs),
            ctypes.c_float(scale), S, Hq, Hkv, D, bs, bt.shape[1], _code(dtype), _ptr(out))
        return out

    def copy_blocks(self, key_cache, value_cache, block_mapping, dtype):
        """Copy-on-write block copy, in place: for each (src, dst) row of
        block_mapping, in order, block dst of both pools becomes a copy of
        block src; a negative id skips the row."""
        nb, bs, Hkv, D = key_cache.shape
        bm = np.ascontiguousarray(block_mapping, dtype=np.int32).reshape(-1, 2)
        self.lib.oracle_copy_blocks(_ptr(key_cache), _ptr(value_cache), _ptr(bm), bm.shape[0],
                                    Hkv, D, bs, _code(dtype))

    def swap_blocks(self, src_key, src_value, dst_key, dst_value, block_mapping, dtype):
        """Block swap between two pool pairs of the same block shape (device
        to host, or back): for each (from, to) row of block_mapping, block to
        of dst_key/dst_value becomes a copy of block from of src_key/src_value;
        a row with an id outside its pool is skipped.  dst is updated in
        place."""
        ns, bs, Hkv, D = src_key.shape
        assert dst_key.shape[1:] == src_key.shape[1:] and dst_value.shape == dst_key.shape
        bm = np.ascontiguousarray(block_mapping, dtype=np.int32).reshape(-1, 2)
        self.lib.oracle_swap_blocks(_ptr(src_key), _ptr(src_value), ns, _ptr(dst_key),
                                    _ptr(dst_value), dst_key.shape[0], _ptr(bm), bm.shape[0],
                                    Hkv, D, bs, _code(dtype))

    def prefix_block_hashes(self, tokens, block_size, seed, base):
        """Chained prefix hashes of one token sequence, one per full block:
        out[k] is the polynomial hash (mod 2^61 - 1, from ``seed``, Horner's
        rule with ``base``, token t entering as t + 1) of the first
        (k + 1) * block_size tokens.  Returns uint64 [len(tokens) // bs]."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        out = np.zeros(t.size // block_size, dtype=np.uint64)
        if out.size:
            self.lib.oracle_prefix_block_hashes(_ptr(t), t.size, block_size, seed, base,
                                                _ptr(out))
        return out

    @staticmethod
    def prefix_match(block_hashes, block_start, cached):
        """Longest cached prefix of each sequence.  block_hashes holds the
        full-block hashes of all sequences, sequence s owning entries
        block_start[s] .. block_start[s+1] - 1 in order; cached maps a hash
        to the block that holds it.  Returns (blocks, lengths): lengths[s] =
        the number of leading blocks of s whose hashes are all cached, and
        blocks[block_start[s] + k] = cached[hash] for k < lengths[s] (-1
        elsewhere)."""
        blocks = np.full(len(block_hashes), -1, dtype=np.int32)
        lengths = np.zeros(len(block_start) - 1, dtype=np.int32)
        for s in range(len(block_start) - 1):
            for i in range(int(block_start[s]), int(block_start[s + 1])):
                h = int(block_hashes[i])
                if h not in cached:
                    break
                blocks[i] = cached[h]
                lengths[s] += 1
        return blocks, lengths

    # ---- conveniences on a workloads.DecodeBatch ----
    def decode_batch(self, batch, *, return_weights=False):
        return self.paged_attention_decode(batch.query, batch.key_cache, batch.value_cache,
                                           batch.block_tables, batch.context_lens, batch.scale,
                                           batch.dtype, return_weights=return_weights)

    def write_batch(self, batch):
        """Apply the batch's KV write to its own pool (in place)."""
        self.kv_cache_write(batch.new_key, batch.new_value, batch.slot_mapping,
                            batch.key_cache, batch.value_cache, batch.dtype)


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY):
            build()
        _default = Oracle(LIBRARY)
    return _default


def __getattr__(name):
    # module-level access to the default instance's methods: oracle.decode_batch(...)
    if name.startswith("_"):
        raise AttributeError(name)
    return getattr(default(), name)
