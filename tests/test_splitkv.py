"""GPU parity of the split-KV forward (fa_fwd_splitkv) against the fp64 oracle.

The split-KV path computes the same attention as fa_fwd_kv -- every query row
against its visible keys -- by cutting the keys into ranges whose partial
(O, LSE) are merged afterwards, so the oracle is the same plain definition and
the bar is the same: max |dO| <= 1e-2, mean |dO| <= 1e-3, max |dLSE| <= 1e-3.

Cases: single-query decoding with every grouped-query ratio; a few queries
(row blocks of packed query rows and heads); ragged key counts that end
inside a 32-key block; more splits than key blocks (empty splits); one split;
the causal mask with rows that see no key; no keys at all; both head dims;
wide logits.  Then the two decoding workloads at full size, compared on every
output row, and properties: bitwise determinism, agreement with the forward
kernel, a caller-provided workspace reused across calls.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import tiled_attention_flash_amd as fa
from tiled_attention_flash_amd.inputs import WORKLOADS, make_qkv, workload_inputs

pytestmark = pytest.mark.gpu

MAX_O, MEAN_O, MAX_LSE = 1e-2, 1e-3, 1e-3


def check(o, lse, o_ref, lse_ref, what):
    o = o.cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    empty = np.isneginf(lse_ref)  # [B, H, Lq] rows that see no key
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: rows with no key differ"
    rows = np.transpose(empty, (0, 2, 1))  # [B, Lq, H]
    assert np.all(o[rows] == 0.0), f"{what}: a row with no key has nonzero output"
    if (~rows).any():
        d = np.abs(o[~rows] - o_ref[~rows])
        dl = np.abs(lse[~empty] - lse_ref[~empty])
        msg = (f"{what}: max|dO|={d.max():.3e} mean|dO|={d.mean():.3e} "
               f"max|dLSE|={dl.max():.3e}")
        print(msg, flush=True)
        assert d.max() <= MAX_O and d.mean() <= MEAN_O and dl.max() <= MAX_LSE, msg


CASES = [
    # B, Lq, Lk, H, Hkv, D, past_len (None = Lk - Lq), n_splits (None = library's choice)
    (4, 1, 3000, 8, 8, 128, None, None),    # MHA decoding
    (2, 1, 4097, 32, 8, 128, None, None),   # GQA 4, ragged by one key
    (2, 1, 2000, 16, 2, 64, None, 7),       # GQA 8, D = 64
    (1, 1, 1000, 4, 1, 128, None, 1),       # GQA 4, a single split
    (1, 1, 333, 2, 2, 128, None, 64),       # more splits than 32-key blocks
    (2, 3, 1500, 8, 2, 128, None, 5),       # 3 queries x 4 heads = 12 packed rows
    (1, 40, 2500, 8, 1, 64, None, 6),       # 320 packed rows: 10 row blocks
    (1, 9, 700, 4, 4, 128, 5, 4),           # causal offset 5: keys 0..13 seen at most
    (1, 8, 500, 4, 2, 64, -3, 3),           # negative offset: the first rows see no key
    (1, 5, 0, 4, 2, 128, None, 2),          # no keys at all
    (2, 2, 64, 4, 4, 128, None, 2),         # one block per split
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", CASES, ids=[f"q{c[1]}-k{c[2]}-h{c[3]}-kv{c[4]}-d{c[5]}-p{c[6]}-n{c[7]}"
                                            for c in CASES])
def test_splitkv_matches_oracle(case, causal):
    B, Lq, Lk, H, Hkv, D, past, n = case
    q, k, v = make_qkv(B, Lq, H, Hkv, D, seed=900 + Lq + Lk, Lk=Lk)
    o_ref, lse_ref = oracle.forward(q, k, v, causal=causal, past_len=past)
    o, lse = fa.forward_splitkv(q.cuda(), k.cuda(), v.cuda(), causal=causal, past_len=past,
                                n_splits=n)
    torch.cuda.synchronize()
    check(o, lse, o_ref, lse_ref, f"B{B} Lq{Lq} Lk{Lk} H{H} Hkv{Hkv} D{D} past={past} "
                                  f"n={n} causal={causal}")


def test_splitkv_wide_logits():
    q, k, v = make_qkv(2, 2, 8, 2, 128, seed=950, qk_mult=3.0, Lk=5000)
    o_ref, lse_ref = oracle.forward(q, k, v, causal=True)
    o, lse = fa.forward_splitkv(q.cuda(), k.cuda(), v.cuda(), causal=True, n_splits=9)
    torch.cuda.synchronize()
    check(o, lse, o_ref, lse_ref, "Q, K x3, 9 splits")


@pytest.mark.parametrize("name", ["decode-b8-h32-kv8-q1-k32768-d128-causal",
                                  "decode-b8-h32-q1-k4096-d128-causal"])
def test_decode_workloads_every_row(name):
    """The decoding workloads at full size, in the benchmark's launch
    configuration (the library's choice of splits): every output row against
    the oracle, plus bitwise determinism."""
    w = WORKLOADS[name]
    print(f"workload {name}", flush=True)
    q, k, v = workload_inputs(w, seed=0)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o1, l1 = fa.forward_splitkv(qd, kd, vd, causal=w.causal, scale=w.scale)
    o2, l2 = fa.forward_splitkv(qd, kd, vd, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o_ref, lse_ref = oracle.forward(q, k, v, causal=w.causal, scale=w.scale)
    check(o1, l1, o_ref, lse_ref, name)


def test_splitkv_agrees_with_forward_kernel():
    """Both entry points compute the same attention; only the order in which
    keys are summed differs, so they agree to rounding."""
    q, k, v = make_qkv(2, 16, 8, 2, 128, seed=960, Lk=3000)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    for causal in (False, True):
        o1, l1 = fa.forward(qd, kd, vd, causal=causal)
        o2, l2 = fa.forward_splitkv(qd, kd, vd, causal=causal, n_splits=11)
        torch.cuda.synchronize()
        assert (o1.float() - o2.float()).abs().max().item() <= 4e-3
        assert (l1 - l2).abs().max().item() <= 1e-4


def test_splitkv_workspace_reused_and_lse_optional():
    q, k, v = make_qkv(1, 2, 4, 4, 64, seed=970, Lk=900)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    need = fa.fa_splitkv_workspace_bytes(1, 2, 4, 64, 8)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN-filled fp32
    o1, l1 = fa.forward_splitkv(qd, kd, vd, causal=True, n_splits=8, workspace=ws)
    o2, l2 = fa.forward_splitkv(qd, kd, vd, causal=True, n_splits=8, workspace=ws,
                                with_lse=False)
    torch.cuda.synchronize()
    assert l2 is None and torch.equal(o1, o2)
    o_ref, lse_ref = oracle.forward(q, k, v, causal=True)
    check(o1, l1, o_ref, lse_ref, "caller workspace")
    with pytest.raises(fa.FaError) as e:
        fa.forward_splitkv(qd, kd, vd, causal=True, n_splits=8, workspace=ws[:need - 16])
    assert e.value.status == 10


def test_splitkv_empty_inputs():
    z = torch.empty((0, 1, 4, 64), dtype=torch.float16, device="cuda")
    o, l = fa.forward_splitkv(z, z, z)
    assert o.shape == z.shape and l.shape == (0, 4, 1)


@pytest.mark.parametrize("pattern", ["rising", "spike"])
def test_splitkv_reference_maximum_overruns(pattern):
    """Decoding rows whose scores outgrow each split's first block (rising by
    0.1 per key over 3000 keys), or jump once (one key 60 above the rest):
    the overrun path inside the splits, then the merge, against the oracle."""
    D, Lk, Lq, H, Hkv = 128, 3000, 2, 4, 1
    g = torch.Generator().manual_seed(23)
    u = torch.randn(D, generator=g, dtype=torch.float64)
    u = u / u.norm()
    scale = 1.0 / np.sqrt(D)
    if pattern == "rising":
        c = 0.1 * torch.arange(Lk, dtype=torch.float64)
    else:
        c = torch.zeros(Lk, dtype=torch.float64)
        c[1234] = 60.0
    k = (c / scale)[:, None] * u[None, :] + 0.05 * torch.randn(Lk, D, generator=g, dtype=torch.float64)
    q = u.expand(1, Lq, H, D).clone().half()
    k = k[None, :, None, :].clone().half()
    v = torch.randn(1, Lk, Hkv, D, generator=g, dtype=torch.float64).half()
    assert torch.isfinite(k).all()
    o_ref, lse_ref = oracle.forward(q, k, v, causal=True)
    o, lse = fa.forward_splitkv(q.cuda(), k.cuda(), v.cuda(), causal=True, n_splits=7)
    torch.cuda.synchronize()
    check(o, lse, o_ref, lse_ref, f"overrun {pattern}, 7 splits")
