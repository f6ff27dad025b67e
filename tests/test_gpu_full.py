"""Parity at the full sizes of the five benchmark workloads, in the launch
configuration the benchmark times (same library calls, same workspaces).

Workloads 1, 2 and 4 are compared whole: every (sequence, head) slice, every
row of every output. Workloads 3 and 5 (hundreds of millions to billions of
causal pairs per head) are compared on 16 slices each: the 4 longest
sequences, the shortest, and random others, every row of those slices.
"""
import gc

import numpy as np
import pytest
import torch

from helpers import compare_backward, compare_forward, longest_and_random_pairs, to_device, tol_for
from variable_length_attention_jfa_amd import inputs as gen
from variable_length_attention_jfa_amd import jfa

pytestmark = pytest.mark.gpu

WHOLE = (1, 2, 4)


def _pairs(batch, cfg):
    if cfg in WHOLE:
        return None  # every slice
    return longest_and_random_pairs(batch, n=16, n_longest=4, seed=cfg)


def _describe(batch, pairs):
    if pairs is None:
        return f"all {len(batch.q_lengths) * batch.wl.H} slices"
    return f"{len(pairs)} slices {pairs} query lengths {[int(batch.q_lengths[b]) for b, _ in pairs]}"


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_full_workload_parity(cfg):
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
    pairs = _pairs(batch, cfg)
    print(f"   comparing {_describe(batch, pairs)}", flush=True)
    tol = tol_for(batch)
    e_o, e_l, _, _ = compare_forward(batch, out, lse, pairs)
    r = compare_backward(batch, dq, dk, dv, pairs)
    assert e_o <= tol["out"] and e_l <= tol["lse"] and max(r) <= tol["grad"]
    del d, out, lse, dq, dk, dv, batch
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_full_workload_padded_baseline_parity(cfg):
    """The padded-dense baseline at full size (slots of the batch's longest
    lengths, as the benchmark runs it) against the oracle, on the same slices
    as the jagged path."""
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
    pairs = _pairs(batch, cfg)
    print(f"   slots {q_slot}/{kv_slot}; comparing {_describe(batch, pairs)}", flush=True)
    tol = tol_for(batch)
    e_o, e_l, _, _ = compare_forward(batch, out, lse, pairs)
    r = compare_backward(batch, dq, dk, dv, pairs)
    assert e_o <= tol["out"] and e_l <= tol["lse"] and max(r) <= tol["grad"]
    del d, qp, dop, kp, vp, out_p, lse_p, dq_p, dk_p, dv_p, batch
    gc.collect()
    torch.cuda.empty_cache()
