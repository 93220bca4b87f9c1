"""The attention-output bar shared by the GPU parity tests.

Decode and multi-token attention outputs are compared with the fp64 oracle
element by element:

* max-abs error <= 2e-3 for f32 inputs and <= 2e-2 for f16 / bf16 inputs,
  with fp32 accumulation;
* for f16 / bf16 a relative error <= 1e-2, taken normwise
  (||got - ref||_2 / ||ref||_2) over the whole output AND over every single
  output row (one sequence -- or one new token -- and one query head, the
  last axis being head_dim).  Outputs are weighted means of N(0, 1) values,
  so their size falls like 1/sqrt(L): at 32K-token contexts every element is
  about 0.01 and the max-abs bar alone checks nothing; the per-row bound
  catches one wrong (sequence, head) that the batch-wide norm would average
  away;
* for f32 the same per-row normwise bound at 1e-3.  The only rounding on the
  f32 path is fp32 arithmetic: per row a sum of at most 32768 weighted
  terms, split into partitions of at most 1024 tokens and merged, and the
  hardware exp2 (about 1 ulp).  A per-row error near 1e-3 (n * 2^-24 at
  n = 16384) would already take the worst-case rounding of every term
  adding up; the measured figures are around 1e-6.

A row whose reference is exactly zero (an empty context) must come out
exactly zero (max-abs covers it, and its relative error is not defined).
"""
import sys

import numpy as np

# dtype -> (max-abs bound, whole-output normwise bound, per-row normwise bound)
TOL = {"f32": (2e-3, None, 1e-3), "f16": (2e-2, 1e-2, 1e-2), "bf16": (2e-2, 1e-2, 1e-2)}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check_close(got, ref, dtype, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} != {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    amax, rmax, rowmax = TOL[dtype]
    err = np.abs(got - ref).max() if got.size else 0.0
    nrm = np.linalg.norm(ref)
    rel = np.linalg.norm(got - ref) / nrm if nrm > 0 else 0.0
    worst_row, worst_rel = None, 0.0
    if got.size:
        D = got.shape[-1]
        g2, r2 = got.reshape(-1, D), ref.reshape(-1, D)
        rn = np.linalg.norm(r2, axis=1)
        en = np.linalg.norm(g2 - r2, axis=1)
        live = rn > 0
        if np.any(live):
            rows = en[live] / rn[live]
            k = int(np.argmax(rows))
            worst_rel = float(rows[k])
            worst_row = int(np.flatnonzero(live)[k])
        # rows whose reference is exactly zero must be exactly zero
        assert np.all(en[~live] == 0), f"{what}: nonzero output where the reference is 0"
    say(f"  {what}: max|err| {err:.3e}  normwise rel {rel:.3e}  "
        f"worst row rel {worst_rel:.3e} (row {worst_row})")
    assert err <= amax, f"{what}: max abs error {err}"
    if rmax is not None:
        assert rel <= rmax, f"{what}: normwise relative error {rel}"
    assert worst_rel <= rowmax, \
        f"{what}: row {worst_row} (sequence/token x head) normwise relative error {worst_rel}"
