"""The parity comparisons themselves (CPU): the per-(b, h) gradient check
catches one wrong short sequence among thousands, which the tensor-wide
relative L2 dilutes below the bar, and the forward bar is the raw max-abs
error wherever |O_ref| < 2."""
import numpy as np
import torch

import oracle
from helpers import BF16_TOL, compare_backward, compare_forward, rel_l2
from variable_length_attention_jfa_amd import inputs as gen


def _many_short():
    wl = gen.Workload("many", 4096, 1, 64, "bf16", False, False, gen.LengthDist("uniform", 1, 8), seed=10)
    return gen.make_batch(wl)


def test_one_wrong_short_slice_fails_per_slice_check():
    batch = _many_short()
    dq, dk, dv = (torch.from_numpy(g.astype(np.float32)) for g in
                  oracle.backward(batch.q, batch.k, batch.v, batch.dout, batch.q_offsets, batch.kv_offsets))
    assert max(compare_backward(batch, dq, dk, dv)) < 1e-6
    # dV of one length-1 sequence lost (written as zeros)
    b = int(np.flatnonzero(batch.kv_lengths == 1)[0])
    r0 = int(batch.kv_offsets[b])
    bad = dv.clone()
    bad[r0] = 0.0
    whole = rel_l2(bad.numpy(), dv.numpy())
    assert whole < BF16_TOL["grad"], "the tensor-wide figure alone would pass it"
    assert compare_backward(batch, dq, dk, bad)[2] > BF16_TOL["grad"]


def test_forward_bar_is_raw_below_two():
    batch = _many_short()
    o_ref, l_ref = oracle.forward(batch.q, batch.k, batch.v, batch.q_offsets, batch.kv_offsets)
    out = torch.from_numpy(o_ref.astype(np.float32))
    lse = torch.from_numpy(l_ref.astype(np.float32))
    # an error of 0.011 on one element with |O_ref| < 2 fails ...
    idx = np.argwhere(np.abs(o_ref) < 1.0)[0]
    bad = out.clone()
    bad[tuple(idx)] += 0.011
    assert compare_forward(batch, bad, lse)[0] > BF16_TOL["out"]
    # ... while at |O_ref| >= 2 the same error is within half a bf16 ulp (2^-7) plus the bar
    big = np.argwhere(np.abs(o_ref) >= 2.0)
    assert len(big) > 0
    ok = out.clone()
    ok[tuple(big[0])] += 0.011
    e = compare_forward(batch, ok, lse)
    assert e[0] <= BF16_TOL["out"] and e.n_large > 0
