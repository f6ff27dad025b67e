"""Parity at the full sizes of the five benchmark workloads, in the launch
configuration the benchmark times (same library calls, same workspaces).

The oracle cannot redo a whole workload in seconds, so each check covers
sampled (sequence, head) slices: the longest and the shortest sequence and two
random ones, compared row by row over every output of those slices.
"""
import gc

import numpy as np
import pytest
import torch

from helpers import compare_backward, compare_forward, raw_forward_error, sample_pairs, to_device, tol_for
from variable_length_attention_jfa_amd import inputs as gen
from variable_length_attention_jfa_amd import jfa

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_full_workload_sampled_parity(cfg):
    wl = gen.WORKLOADS[cfg]
    print(f"[case] full workload {cfg} ({wl.name}) generating", flush=True)
    batch = gen.make_batch(wl)
    d = to_device(batch)
    print(f"   B={wl.B} Tq={batch.total_q} Tk={batch.total_kv} on device", flush=True)
    out, lse = jfa.forward(d["q"], d["k"], d["v"], d["q_offsets"], d["kv_offsets"], d["bias"], wl.causal)
    dq, dk, dv = jfa.backward(d["q"], d["k"], d["v"], out, lse, d["dout"], d["q_offsets"], d["kv_offsets"], d["bias"],
                              wl.causal)
    torch.cuda.synchronize()
    for t in (out, lse, dq, dk, dv):
        assert torch.isfinite(t.float()).all(), "non-finite output"
    pairs = sample_pairs(batch, n_random=2, seed=cfg)
    print(f"   sampled (b, h): {pairs} lengths {[int(batch.q_lengths[b]) for b, _ in pairs]}", flush=True)
    tol = tol_for(batch)
    e_o, e_l, o_ref, _ = compare_forward(batch, out, lse, pairs)
    raw = raw_forward_error(batch, out, o_ref, pairs)
    print(f"   fwd max|dO| beyond output rounding={e_o:.3e} (raw {raw:.3e}) max|dlse|={e_l:.3e}", flush=True)
    r = compare_backward(batch, dq, dk, dv, pairs)
    print(f"   bwd relL2 dq={r[0]:.3e} dk={r[1]:.3e} dv={r[2]:.3e}", flush=True)
    assert e_o <= tol["out"] and e_l <= tol["lse"] and max(r) <= tol["grad"]
    del d, out, lse, dq, dk, dv, batch
    gc.collect()
    torch.cuda.empty_cache()
