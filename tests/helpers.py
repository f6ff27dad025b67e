"""Shared test helpers: move a synthetic batch to the GPU, run the library,
compare with the oracle at the stated tolerances."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from variable_length_attention_jfa_amd import inputs as gen

# Tolerances for unit-normal bf16 inputs with fp32 accumulation: forward
# max-abs error on O, max-abs error on lse, relative L2 error per gradient.
BF16_TOL = dict(out=1e-2, lse=1e-3, grad=2e-2)
# fp32 inputs (no bf16 rounding of P or of the outputs): the error is fp32
# accumulation over at most a few thousand terms, ~1e-6 relative.
F32_TOL = dict(out=2e-5, lse=2e-5, grad=2e-5)


def tol_for(batch: gen.Batch):
    return F32_TOL if batch.wl.dtype == "f32" else BF16_TOL


def to_device(batch: gen.Batch, device="cuda"):
    def t(vals, bits):
        if bits is not None:
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(vals).to(device)

    d = dict(
        q=t(batch.q, batch.q_bits), k=t(batch.k, batch.k_bits), v=t(batch.v, batch.v_bits),
        q_offsets=torch.from_numpy(batch.q_offsets.astype(np.int32)).to(device),
        kv_offsets=torch.from_numpy(batch.kv_offsets.astype(np.int32)).to(device),
        bias=None if batch.bias is None else torch.from_numpy(batch.bias).to(device),
    )
    if batch.dout is not None:
        d["dout"] = t(batch.dout, batch.dout_bits)
    return d


def valid_rows_mask(offsets: np.ndarray, pairs, H: int, T: int):
    """[T, H] boolean mask of rows that belong to the selected (b, h) pairs."""
    m = np.zeros((T, H), dtype=bool)
    for b, h in pairs:
        m[offsets[b]:offsets[b + 1], h] = True
    return m


def all_pairs(batch: gen.Batch):
    return [(b, h) for b in range(len(batch.q_offsets) - 1) for h in range(batch.wl.H)]


def longest_and_random_pairs(batch: gen.Batch, n: int = 16, n_longest: int = 4, seed: int = 0):
    """n distinct (b, h) slices: the n_longest longest sequences (by query x
    key length; head b mod H), the shortest non-empty one, and random others."""
    B, H = len(batch.q_lengths), batch.wl.H
    size = batch.q_lengths.astype(np.int64) * np.maximum(batch.kv_lengths, 1)
    order = np.argsort(-size, kind="stable")
    pairs = [(int(b), int(b) % H) for b in order[:n_longest]]
    nonempty = [int(b) for b in order[::-1] if batch.q_lengths[b] > 0]
    if nonempty:
        pairs.append((nonempty[0], H - 1))
    rng = np.random.default_rng(seed)
    while len(set(pairs)) < min(n, B * H):
        pairs.append((int(rng.integers(0, B)), int(rng.integers(0, H))))
    return sorted(set(pairs))


# Forward bar on O: the raw max-abs error must stay within the tolerance
# wherever |O_ref| and the stored |O| are both below ROUNDING_ALLOWANCE_FROM.
# Above it the bf16 store alone can break the bar (half a bf16 ulp is 2^-7 =
# 0.0078 for |O| in [2, 4) and 2^-6 = 0.0156 in [4, 8)), so there the
# tolerance applies to the error beyond half an ulp of the larger of the two
# magnitudes (the store rounds in the computed value's binade, which an
# element just below 2 can leave); the elements that take this allowance are
# counted and printed.
ROUNDING_ALLOWANCE_FROM = 2.0


class FwdErrors(tuple):
    """(e_o, e_l, o_ref, l_ref) plus the split of the O error: ``raw`` over all
    compared elements, ``small`` (raw, |O_ref| and |O| below 2), ``large``
    (beyond half a bf16 ulp, either at 2 or above) and ``n_large`` (elements
    in the second group)."""

    def __new__(cls, e_o, e_l, o_ref, l_ref, raw, small, large, n_large):
        t = super().__new__(cls, (e_o, e_l, o_ref, l_ref))
        t.raw, t.small, t.large, t.n_large = raw, small, large, n_large
        return t


def compare_forward(batch, out, lse, pairs=None, verbose=True):
    """Returns (max O error under the bar's reading, max-abs error on lse,
    o_ref, l_ref) over the selected rows. The O error is the raw max-abs where
    |O_ref| and |O| are below 2 and, for bf16 outputs, the error beyond half a
    bf16 ulp of max(|O_ref|, |O|) where either is at 2 or above (fp32 outputs:
    raw everywhere)."""
    wl = batch.wl
    pairs = all_pairs(batch) if pairs is None else pairs
    o_ref, l_ref = oracle.forward(batch.q, batch.k, batch.v, batch.q_offsets, batch.kv_offsets, batch.bias,
                                  wl.causal, pairs=pairs)
    m = valid_rows_mask(batch.q_offsets, pairs, wl.H, batch.total_q)
    o = out.float().cpu().numpy()
    l = lse.float().cpu().numpy()
    if not m.any():
        return FwdErrors(0.0, 0.0, o_ref, l_ref, 0.0, 0.0, 0.0, 0)
    ref = o_ref[m]
    got = o[m]
    err = np.abs(got - ref)
    raw = float(err.max())
    mag = np.maximum(np.abs(ref), np.abs(got))
    if batch.wl.dtype == "bf16":
        big = mag >= ROUNDING_ALLOWANCE_FROM
    else:
        big = np.zeros(ref.shape, dtype=bool)
    small = float(err[~big].max()) if (~big).any() else 0.0
    large = float(np.maximum(err[big] - half_ulp_bf16(mag[big]), 0.0).max()) if big.any() else 0.0
    n_large = int(big.sum())
    e_o = max(small, large)
    lm = m & np.isfinite(l_ref)
    e_l = float(np.abs(l[lm] - l_ref[lm]).max()) if lm.any() else 0.0
    # rows with no keys: lse must be -inf and O exactly 0
    em = m & ~np.isfinite(l_ref)
    if em.any():
        assert np.all(np.isneginf(l[em])), "rows without keys must have lse = -inf"
        assert np.all(o[em] == 0), "rows without keys must have O = 0"
    if verbose:
        print(f"   fwd max|dO| raw={raw:.3e}: below 2 {small:.3e}; at 2 or above, beyond half a bf16 ulp {large:.3e} "
              f"({n_large} of {err.size} elements); max|dlse|={e_l:.3e}", flush=True)
    return FwdErrors(e_o, e_l, o_ref, l_ref, raw, small, large, n_large)


ZERO_REF = 1e-9  # a reference gradient below this everywhere is exactly 0 up to fp64 noise


def half_ulp_bf16(x):
    """Half the spacing of bf16 values at |x| (8 significant bits)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.where(a > 0, 2.0 ** (e - 8), 0.0)


def rel_l2(x, ref):
    """Relative L2 error; where the exact gradient is identically zero (for
    example dQ and dK when every sequence has one key) there is no scale to be
    relative to, and the max-abs error is returned instead."""
    if ref.size == 0:
        return 0.0
    if float(np.abs(ref).max()) < ZERO_REF:
        return float(np.abs(x - ref).max())
    return float(np.linalg.norm(x - ref) / np.linalg.norm(ref))


def slice_errors(x, ref, offsets, pairs, H, tensor_norm, n_rows):
    """Per-(b, h) relative L2 errors of one gradient over the selected slices.

    Returns (worst strict, worst floored, slices that took the floor, where).
    Strict: ||x - ref|| / ||ref|| over the slice (max-abs where ref is
    identically 0, as for the whole tensor). Floored: the same error divided
    by max(||ref||_slice, ||ref||_tensor * sqrt(rows_slice / rows_tensor)),
    the slice's share of the tensor's norm at the tensor's RMS per row. The
    floor keeps the ratio meaningful for slices whose gradient is small next
    to the backward's unavoidable absolute error: Delta = rowsum(dO * O) is
    formed from the stored bf16 O, which moves dS by ~2^-9 |dO||O| per row
    whatever the slice's gradient is (a 2-token slice whose two dP nearly
    agree has a tiny exact dQ, and there the strict ratio reaches 0.15 even
    when every other step is exact). A wrong slice still fails: its error is
    of the order of its rows' gradients, far above 2% of that share."""
    worst, worst_f, n_floor, where = 0.0, 0.0, 0, None
    for b, h in pairs:
        r0, r1 = int(offsets[b]), int(offsets[b + 1])
        if r1 == r0:
            continue
        a, g = ref[r0:r1, h], x[r0:r1, h]
        e = float(np.linalg.norm(g - a))
        if float(np.abs(a).max()) < ZERO_REF:
            strict = floored = float(np.abs(g - a).max())
        else:
            na = float(np.linalg.norm(a))
            share = tensor_norm * np.sqrt((r1 - r0) / max(n_rows, 1))
            strict = e / na
            floored = e / max(na, share)
            n_floor += int(share > na)
        worst = max(worst, strict)
        if floored > worst_f:
            worst_f, where = floored, (b, h, r1 - r0)
    return worst, worst_f, n_floor, where


def compare_backward(batch, dq, dk, dv, pairs=None, verbose=True):
    """Returns, for dQ, dK, dV, the larger of the tensor-wide relative L2
    error and the worst per-(b, h) floored relative L2 error (slice_errors)."""
    wl = batch.wl
    pairs = all_pairs(batch) if pairs is None else pairs
    r_dq, r_dk, r_dv = oracle.backward(batch.q, batch.k, batch.v, batch.dout, batch.q_offsets, batch.kv_offsets,
                                       batch.bias, wl.causal, pairs=pairs)
    mq = valid_rows_mask(batch.q_offsets, pairs, wl.H, batch.total_q)
    mk = valid_rows_mask(batch.kv_offsets, pairs, wl.H, batch.total_kv)
    g = [dq.float().cpu().numpy(), dk.float().cpu().numpy(), dv.float().cpu().numpy()]
    refs = (r_dq, r_dk, r_dv)
    masks = (mq, mk, mk)
    offs = (batch.q_offsets, batch.kv_offsets, batch.kv_offsets)
    out = []
    lines = []
    for name, x, ref, m, off in zip(("dq", "dk", "dv"), g, refs, masks, offs):
        whole = rel_l2(x[m], ref[m])
        tn = float(np.linalg.norm(ref[m]))
        strict, floored, n_floor, where = slice_errors(x, ref, off, pairs, wl.H, tn, int(m.sum()))
        out.append(max(whole, floored))
        lines.append(f"{name} {whole:.2e} (slices: {floored:.2e} floored at {where}, strict {strict:.2e}, "
                     f"{n_floor} floored)")
    if verbose:
        print("   bwd relL2 " + "; ".join(lines), flush=True)
    return tuple(out)
