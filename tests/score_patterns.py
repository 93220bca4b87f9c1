"""Decode inputs whose scores sit at the extremes of the online softmax.

Input generation only (scales, queries and keys on top of the seeded
N(0, 1) batches of the workloads module); it holds no attention arithmetic.
tests/test_score_patterns.py checks on the CPU that each pattern has the
margins stated here; tests/test_gpu_parity.py runs every decode kernel on
them against the oracle.

The kernels: the matrix-core decode (f16/bf16 with 4 or 8 query heads per
kv head), the vector decode (f16/bf16 with one query head per kv head, f32
with 1 or 4), each at partition_size 0 (no split below 1024 tokens on this
shape) and 32 (the reduce merges up to 32 partitions).

The cases:
 * scale 0 (uniform weights: the mean of V), negative scales (the max is
   then the most negative dot product) and |scale| = 3 on N(0, 1) data
   (dot products of about +-11, so exponents of up to about +-150: the
   softmax is nearly one-hot);
 * "rise" / "steep": the scores climb a staircase along the context, one
   step per 16-token tile, so that every tile's maximum exceeds the running
   maximum by more than 2^8 (2^20 per tile on average), respectively by
   more than 2^40 (2^58 on average; the partitions' maxima then differ by
   hundreds of binary orders and the earlier partitions' weights underflow
   to 0 in the merge);
 * "first": the first 16 tokens of every context outscore the rest by more
   than 2^100, so every later tile, and every partition after the first,
   underflows to 0 relative to them;
 * "last": the same for the last tile of every context, which then arrives
   after all the others (every earlier partial result is rescaled to 0).
"""
import functools

import numpy as np

from paged_kv_cache_467_amd import workloads as W

EXTREME_KERNELS = [("bf16", 4), ("bf16", 8), ("f16", 4), ("f16", 8), ("f16", 1), ("bf16", 1),
                   ("f32", 1), ("f32", 4)]
EXTREME_CASES = ["scale0", "scale_neg", "scale3", "scale_neg3", "rise", "steep", "first", "last"]
EXTREME_LENS = (1, 15, 16, 17, 100, 255, 513, 1000)


def with_scores(b, case):
    """b with its scale, queries and keys set for one of EXTREME_CASES.  The
    patterned cases set every query to 1 + N(0, 0.1^2) and add a staircase or
    a step along the context to the N(0, 1) keys, so that every query head's
    dot product with token j carries about head_dim times the offset added
    at j.  Inputs only: no attention arithmetic."""
    b = b.copy()
    D, dt = b.head_dim, b.dtype
    base = 1.0 / np.sqrt(D)
    if case.startswith("scale"):
        b.scale = float(np.float32({"scale0": 0.0, "scale_neg": -base, "scale3": 3.0,
                                    "scale_neg3": -3.0}[case]))
        return b
    q = W.bits_to_f32(b.query, dt)
    b.query = W.f32_to_bits(1.0 + 0.1 * q, dt)
    # offset added to every element of a key: it raises that token's score by
    # about offset * head_dim * scale (natural-log units)
    per_tile = {"rise": 14.0, "steep": 40.0}.get(case)  # score step per 16-token tile
    kc = W.bits_to_f32(b.key_cache, dt)
    # a pool cell that several sequences share (a common prefix, at the same
    # position in each) takes its offset once, from the first of them
    done = np.zeros(kc.shape[:2], dtype=bool)
    for s in range(b.num_seqs):
        L = int(b.context_lens[s])
        j = np.arange(L)
        if per_tile is not None:
            # a staircase: one step per 16-token tile (a partial tile included)
            off = (j // 16) * per_tile / (D * b.scale)
        elif case == "first":
            off = np.where(j < 16, 80.0 / (D * b.scale), 0.0)     # +80 nats = +115 binary orders
        else:                                                    # "last"
            first_of_last = ((L - 1) // 16) * 16
            off = np.where(j >= first_of_last, 80.0 / (D * b.scale), 0.0)
        blk = b.block_tables[s, j // b.block_size]
        slot = j % b.block_size
        new = ~done[blk, slot]
        kc[blk[new], slot[new]] += off[new][:, None, None].astype(np.float32)
        done[blk, slot] = True
    b.key_cache = W.f32_to_bits(kc, dt)
    return b


@functools.lru_cache(maxsize=None)
def extreme_batch(dtype, G):
    return W.make_custom(5100 + 10 * G + len(dtype), dtype=dtype, num_seqs=len(EXTREME_LENS),
                         num_q_heads=2 * G, num_kv_heads=2, head_dim=128, block_size=16,
                         context_lens=EXTREME_LENS, extra_blocks=6, poison=True)
