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
    # the key-count bound the benchmark passes (the batch's longest key side)
    max_kv = int(batch.kv_lengths.max())
    out, lse = jfa.forward(d["q"], d["k"], d["v"], d["q_offsets"], d["kv_offsets"], d["bias"], wl.causal,
                           max_kv_len=max_kv)
    dq, dk, dv = jfa.backward(d["q"], d["k"], d["v"], out, lse, d["dout"], d["q_offsets"], d["kv_offsets"], d["bias"],
                              wl.causal, max_kv_len=max_kv)
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


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_full_workload_padded_baseline_sampled_parity(cfg):
    """The padded-dense baseline at full size (slots of the batch's longest
    lengths, as the benchmark runs it), sampled slices against the oracle."""
    from variable_length_attention_jfa_amd import padded
    wl = gen.WORKLOADS[cfg]
    print(f"[case] padded baseline, full workload {cfg} ({wl.name})", flush=True)
    batch = gen.make_batch(wl)
    d = to_device(batch)
    qo, ko = batch.q_offsets, batch.kv_offsets
    q_slot, kv_slot = int(batch.q_lengths.max()), int(batch.kv_lengths.max())
    qp, dop = padded.to_slots(d["q"], qo, q_slot), padded.to_slots(d["dout"], qo, q_slot)
    kp, vp = padded.to_slots(d["k"], ko, kv_slot), padded.to_slots(d["v"], ko, kv_slot)
    kv_lens = torch.from_numpy(batch.kv_lengths.astype(np.int32)).cuda()
    out_p, lse_p = jfa.forward_padded(qp, kp, vp, kv_lens, d["bias"], wl.causal)
    dq_p, dk_p, dv_p = jfa.backward_padded(qp, kp, vp, out_p, lse_p, dop, kv_lens, d["bias"], wl.causal)
    torch.cuda.synchronize()
    out, lse = padded.from_slots(out_p, qo), padded.from_slots(lse_p, qo)
    dq, dk, dv = padded.from_slots(dq_p, qo), padded.from_slots(dk_p, ko), padded.from_slots(dv_p, ko)
    for t in (out, lse, dq, dk, dv):
        assert torch.isfinite(t.float()).all(), "non-finite output"
    pairs = sample_pairs(batch, n_random=2, seed=cfg)
    tol = tol_for(batch)
    e_o, e_l, _, _ = compare_forward(batch, out, lse, pairs)
    r = compare_backward(batch, dq, dk, dv, pairs)
    print(f"   slots {q_slot}/{kv_slot}: fwd {e_o:.3e} lse {e_l:.3e} bwd relL2 {r[0]:.2e}/{r[1]:.2e}/{r[2]:.2e}", flush=True)
    assert e_o <= tol["out"] and e_l <= tol["lse"] and max(r) <= tol["grad"]
    del d, qp, dop, kp, vp, out_p, lse_p, dq_p, dk_p, dv_p, batch
    gc.collect()
    torch.cuda.empty_cache()
