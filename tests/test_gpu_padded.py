"""GPU parity of the padded-dense baseline (jfa_fwd_padded / jfa_bwd_padded):
the jagged batch is copied into zeroed fixed-length slots, run through the
baseline, and the rows inside each sequence are compared with the fp64 oracle
at the same tolerances as the jagged path."""
import numpy as np
import pytest
import torch

from helpers import compare_backward, compare_forward, to_device, tol_for
from variable_length_attention_jfa_amd import inputs as gen
from variable_length_attention_jfa_amd import jfa, padded

pytestmark = pytest.mark.gpu


def _check_padded(batch, label, extra_slot=0):
    wl = batch.wl
    q_slot = int(batch.q_lengths.max()) + extra_slot
    kv_slot = int(batch.kv_lengths.max()) + extra_slot
    print(f"[case] padded {label} B={len(batch.q_lengths)} H={wl.H} D={wl.D} causal={wl.causal} bias={wl.bias} "
          f"q_slot={q_slot} kv_slot={kv_slot}", flush=True)
    d = to_device(batch)
    qo, ko = batch.q_offsets, batch.kv_offsets
    qp, dop = padded.to_slots(d["q"], qo, q_slot), padded.to_slots(d["dout"], qo, q_slot)
    kp, vp = padded.to_slots(d["k"], ko, kv_slot), padded.to_slots(d["v"], ko, kv_slot)
    kv_lens = torch.from_numpy(batch.kv_lengths.astype(np.int32)).cuda()
    out_p, lse_p = jfa.forward_padded(qp, kp, vp, kv_lens, d["bias"], wl.causal)
    dq_p, dk_p, dv_p = jfa.backward_padded(qp, kp, vp, out_p, lse_p, dop, kv_lens, d["bias"], wl.causal)
    torch.cuda.synchronize()
    out, lse = padded.from_slots(out_p, qo), padded.from_slots(lse_p, qo)
    dq, dk, dv = padded.from_slots(dq_p, qo), padded.from_slots(dk_p, ko), padded.from_slots(dv_p, ko)
    tol = tol_for(batch)
    e_o, e_l, _, _ = compare_forward(batch, out, lse)
    r = compare_backward(batch, dq, dk, dv)
    assert e_o <= tol["out"] and e_l <= tol["lse"]
    assert max(r) <= tol["grad"], r
    assert torch.isfinite(dq.float()).all() and torch.isfinite(dk.float()).all() and torch.isfinite(dv.float()).all()


SMALL = {
    2: gen.small_workload(gen.WORKLOADS[2], B=6, lo=1, hi=700, seed=21),
    3: gen.small_workload(gen.WORKLOADS[3], B=5, lo=1, hi=600, seed=31),
    4: gen.small_workload(gen.WORKLOADS[4], B=5, lo=1, hi=64, kv=(64, 900), seed=41),
    5: gen.small_workload(gen.WORKLOADS[5], B=3, lo=16, hi=1100, seed=51),
}


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_padded_small_workloads(cfg):
    _check_padded(gen.make_batch(SMALL[cfg]), f"small cfg{cfg}")


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("causal,bias", [(False, False), (True, False), (False, True), (True, True)])
def test_padded_features(D, causal, bias):
    """Slots longer than the longest sequence (whole blocks of pad keys and
    rows), asymmetric query and key lengths, one-token sequences."""
    ql, kl = [1, 70, 130, 5], [9, 1, 200, 129]
    if causal:
        kl = ql  # the causal workloads are self-attention
    wl = gen.Workload("padgrid", len(ql), 2, D, "bf16", causal, bias, gen.LengthDist("fixed", 1, 1), seed=70 + D)
    _check_padded(gen.make_batch(wl, q_lengths=ql, kv_lengths=kl), f"D={D}", extra_slot=77)


def test_padded_sequence_without_keys():
    """A slot with no valid key: O = 0, lse = -inf, dQ = 0 (the backward's P is 0 on such rows)."""
    ql, kl = [3, 40, 7], [0, 50, 0]
    wl = gen.Workload("pad0", len(ql), 2, 64, "bf16", False, False, gen.LengthDist("fixed", 1, 1), seed=72)
    _check_padded(gen.make_batch(wl, q_lengths=ql, kv_lengths=kl), "zero keys", extra_slot=10)


def test_padded_backward_very_negative_scores():
    """Every valid score ~20 below the pad keys' score: a pad key's P =
    exp(-lse) is ~e^18 there, and the dQ pass must drop the pad keys (it masks
    them at kv_lens) for dQ to stay finite and exact."""
    ql, kl = [4, 70, 9], [5, 70, 130]
    wl = gen.Workload("pad_neg", len(ql), 2, 64, "bf16", False, False, gen.LengthDist("fixed", 1, 1), seed=83)
    batch = gen.make_batch(wl, q_lengths=ql, kv_lengths=kl)
    for s in (0, 2):
        qs = slice(batch.q_offsets[s], batch.q_offsets[s + 1])
        ks = slice(batch.kv_offsets[s], batch.kv_offsets[s + 1])
        batch.q[qs] = 0.0
        batch.q[qs, :, 0] = 16.0
        batch.k[ks, :, 0] = -10.0
    batch.q_bits = gen.bf16_round(batch.q)
    batch.k_bits = gen.bf16_round(batch.k)
    _check_padded(batch, "very negative scores", extra_slot=200)
