"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that the pins catch every one of them.

Each mutant is the oracle's C source with one textual change, compiled to a
temporary library.  A mutant that passes every pin would mean the pins do
not pin that part of the oracle.
"""
import os
import subprocess
import sys

import pytest

from oracle import Oracle
from oracle.build import SOURCE
from oracle_pins import ALL_PINS

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

MUTANTS = {
    # wrong index: offset used to pick the block in the attention loops
    "block_index_uses_modulo": ("const int block_id = blocks[j / block_size];\n            const int offset = j % block_size;\n            const int64_t k0",
                                "const int block_id = blocks[j % block_size];\n            const int offset = j % block_size;\n            const int64_t k0"),
    # dropped term: scale left out of the scores
    "scale_dropped": ("x[j] = (double)scale * dot;", "x[j] = dot;"),
    # wrong head mapping: interleaved instead of consecutive groups
    "gqa_head_mapping": ("const int kv_head = h / group;\n        const int context_len = context_lens[s];\n        const int32_t *blocks = block_tables + (int64_t)s * max_blocks_per_seq;\n        const int64_t q0 = ((int64_t)s * num_q_heads + h) * head_dim;\n        double *o = out + unit * head_dim;\n        for (int d = 0; d < head_dim; ++d)\n            o[d] = 0.0;\n        if (context_len <= 0)\n            continue;\n\n",
                         "const int kv_head = h % num_kv_heads;\n        const int context_len = context_lens[s];\n        const int32_t *blocks = block_tables + (int64_t)s * max_blocks_per_seq;\n        const int64_t q0 = ((int64_t)s * num_q_heads + h) * head_dim;\n        double *o = out + unit * head_dim;\n        for (int d = 0; d < head_dim; ++d)\n            o[d] = 0.0;\n        if (context_len <= 0)\n            continue;\n\n"),
    # off by one: last token left out of the weighted sum
    "last_token_dropped": ("    for (int j = 0; j < context_len; ++j) {\n            const double w = exp(x[j] - m) / sum;",
                           "    for (int j = 0; j < context_len - 1; ++j) {\n            const double w = exp(x[j] - m) / sum;"),
    # missing normalisation
    "no_normalisation": ("const double w = exp(x[j] - m) / sum;", "const double w = exp(x[j] - m);"),
    # transposed pool layout: [num_blocks, num_kv_heads, block_size, head_dim]
    "pool_axes_swapped": ("return ((block_id * block_size + offset) * num_kv_heads + kv_head) * (int64_t)head_dim;",
                          "return ((block_id * num_kv_heads + kv_head) * block_size + offset) * (int64_t)head_dim;"),
    # f16 exponent bias off by one
    "half_bias": ("exponent - 25); /* (1 + f/1024)", "exponent - 24); /* (1 + f/1024)"),
    # kv write: block and offset swapped
    "write_slot_split": ("const int64_t block_id = slot / block_size;\n        const int offset = slot % block_size;",
                         "const int64_t block_id = slot % block_size;\n        const int offset = slot / block_size;"),
    # no max subtraction: first score used as the shift
    "no_running_max": ("        double m = x[0];\n        for (int j = 1; j < context_len; ++j)\n            if (x[j] > m)\n                m = x[j];",
                       "        double m = x[0];"),
    # split merge: rescale factor with the wrong sign
    "merge_sign": ("const double c = exp(m_p[p] - M) / total;", "const double c = exp(M - m_p[p]) / total;"),
    # multi-token: causal bound off by one (a new token does not see itself)
    "prefill_causal_off_by_one": ("const int n = position + 1; /* positions 0 .. position */",
                                  "const int n = position > 0 ? position : 1;"),
    # multi-token: new token i placed at position i instead of L - q_len + i
    "prefill_position": ("const int position = context_len - q_len + i;",
                         "const int position = i;"),
    # block copy: source and destination swapped
    "copy_direction": ("const int src = block_mapping[2 * i];\n        const int dst = block_mapping[2 * i + 1];",
                       "const int src = block_mapping[2 * i + 1];\n        const int dst = block_mapping[2 * i];"),
    # block copy: value pool filled from the key pool
    "copy_v_from_k": ("memmove((char *)value_cache + (size_t)dst * block_bytes,\n                (const char *)value_cache",
                      "memmove((char *)value_cache + (size_t)dst * block_bytes,\n                (const char *)key_cache"),
    # block swap: pair read the wrong way round
    "swap_direction": ("const int from = block_mapping[2 * i];\n        const int to = block_mapping[2 * i + 1];",
                       "const int from = block_mapping[2 * i + 1];\n        const int to = block_mapping[2 * i];"),
    # block swap: value pool filled from the key pool
    "swap_v_from_k": ("(const char *)src_value + (size_t)from * bytes",
                      "(const char *)src_key + (size_t)from * bytes"),
    # block swap: off-by-one range check (reads one block past the source)
    "swap_range": ("from >= num_src_blocks", "from > num_src_blocks"),
    # prefix hash: token t enters as t instead of t + 1
    "hash_plus_one_dropped": ("+ (uint64_t)(uint32_t)tokens[i] + 1)", "+ (uint64_t)(uint32_t)tokens[i])"),
    # prefix hash: a block's hash taken one token early
    "hash_boundary": ("if ((i + 1) % block_size == 0)", "if ((i + 2) % block_size == 0)"),
    # prefix hash: seed ignored
    "hash_seed_ignored": ("uint64_t h = seed % ORACLE_HASH_P;", "uint64_t h = 0;"),
    # gather: value rows taken from the key pool
    "gather_v_from_k": ("memcpy((char *)out_v + dst * element_bytes(dtype),\n                   (const char *)value_cache",
                        "memcpy((char *)out_v + dst * element_bytes(dtype),\n                   (const char *)key_cache"),
}


def _build_mutant(tmp_path, name, old, new):
    src = open(SOURCE).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", str(path), "-o",
                    str(lib), "-lm"], check=True)
    return Oracle(str(lib))


def _run_pins(lib_path):
    """Run every pin against one library in this process; return the names
    of the pins that fail."""
    orc = Oracle(lib_path)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
            print("FAILED " + pin.__name__, flush=True)
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    orc = _build_mutant(tmp_path, name, old, new)
    # A mutant may also read out of bounds and crash, so its pins run in a
    # child process; a crash counts as detected.
    code = ("import sys, json; sys.path[:0] = [%r, %r]; import test_oracle_mutants as T; "
            "print(json.dumps(T._run_pins(%r)))" % (ROOT, HERE, orc.path))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    failed = [ln.split()[1] for ln in r.stdout.splitlines() if ln.startswith("FAILED ")]
    if r.returncode != 0:
        # crashed part-way; still require that a pin had failed, or that it
        # crashed (a mutant reading outside the pool) before any could
        assert failed or r.returncode < 0, r.stderr[-2000:]
        return
    assert failed, f"no pin detects mutant {name}"
