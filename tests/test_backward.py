"""GPU parity of the backward pass (fa_bwd) against the fp64 oracle.

The GPU path runs the forward (fa_fwd) and then the backward on the same
seeded inputs; the oracle computes the exact gradients of sum(O * dO) from
Q, K, V and dO alone.

Bar, per gradient tensor G in {dQ, dK, dV}, derived from the arithmetic:
fp16 operands P and dS carry a relative rounding of 2^-11 into fp32 sums,
and the fp16 result another 2^-12, so errors are a few 1e-4 of the
gradient's own scale:
    max |G_gpu - G_ref|  <= 1e-2 * max |G_ref|
    mean |G_gpu - G_ref| <= 2e-3 * mean |G_ref|
and every gradient finite.

Cases: ragged lengths around the 32-row blocks and 64-key tiles, both head
dimensions, causal and not; every grouped-query ratio; wide logits (Q, K x3);
a non-default scale; queries and keys of different lengths (fa_bwd_kv:
cross-attention, rows after a cached prefix, rows that see no key, keys
that no row sees, no keys or no rows at all); the page's workload (B=8,
H=32, L=1024, D=64) and the
long B=8, H=32, L=4096, D=128 shape at full size, compared on whole
(batch, K/V head) slices, which the oracle computes exactly because
different slices do not interact; determinism; GQA equal to MHA with K/V
repeated and dK/dV summed; argument errors.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import tiled_attention_flash_amd as fa
from tiled_attention_flash_amd.inputs import make_qkvdo

pytestmark = pytest.mark.gpu

REL_MAX, REL_MEAN = 1e-2, 2e-3


def gpu_grads(q, k, v, do, causal, scale=None):
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv, _ = fa.backward(qd, kd, vd, o, lse, dod, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def check(got, ref, what):
    for g, r, name in zip(got, ref, ("dq", "dk", "dv")):
        g = g.double().numpy()
        assert np.isfinite(g).all(), f"{what} {name}: non-finite"
        d = np.abs(g - r)
        scale_max, scale_mean = np.abs(r).max(), np.abs(r).mean()
        msg = (f"{what} {name}: max|d|={d.max():.3e} (ref max {scale_max:.3e}) "
               f"mean|d|={d.mean():.3e} (ref mean {scale_mean:.3e})")
        print(msg, flush=True)
        assert d.max() <= REL_MAX * scale_max + 1e-6, msg
        assert d.mean() <= REL_MEAN * scale_mean + 1e-7, msg


def case(B, L, H, Hkv, D, causal, seed, qk_mult=1.0, scale=None):
    q, k, v, do = make_qkvdo(B, L, H, Hkv, D, seed=seed, qk_mult=qk_mult)
    ref = oracle.backward(q, k, v, do, causal=causal, scale=scale)
    got = gpu_grads(q, k, v, do, causal, scale)
    check(got, ref, f"B{B} L{L} H{H} Hkv{Hkv} D{D} causal={causal} seed={seed}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("L", [1, 7, 31, 32, 33, 64, 65, 100, 127, 128, 129, 255, 300])
def test_backward_ragged(L, D, causal):
    case(1, L, 2, 1, D, causal, seed=1000 + L)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("groups", [1, 2, 4, 8])
def test_backward_gqa(groups, causal):
    case(2, 200, 8, 8 // groups, 128, causal, seed=1100 + groups)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_backward_multi_block(D, causal):
    case(2, 600, 4, 2, D, causal, seed=1200 + D)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_wide_logits(causal):
    case(1, 400, 4, 4, 128, causal, seed=1300, qk_mult=3.0)


def test_backward_nondefault_scale():
    case(1, 257, 2, 2, 64, True, seed=1400, scale=0.3)


@pytest.mark.parametrize("B,L,H,Hkv,D,slices", [
    (8, 1024, 32, 32, 64, [(0, 0), (3, 17), (7, 31)]),
    (8, 4096, 32, 32, 128, [(5, 9)]),
])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_full_size_slices(B, L, H, Hkv, D, slices, causal):
    q, k, v, do = make_qkvdo(B, L, H, Hkv, D, seed=0)
    print(f"full size B{B} L{L} H{H} D{D} causal={causal}", flush=True)
    got = gpu_grads(q, k, v, do, causal)
    g = H // Hkv
    for b, hk in slices:
        hs = slice(hk * g, (hk + 1) * g)
        qs, dos = q[b:b + 1, :, hs].contiguous(), do[b:b + 1, :, hs].contiguous()
        ks, vs = k[b:b + 1, :, hk:hk + 1].contiguous(), v[b:b + 1, :, hk:hk + 1].contiguous()
        ref = oracle.backward(qs, ks, vs, dos, causal=causal)
        sub = (got[0][b:b + 1, :, hs], got[1][b:b + 1, :, hk:hk + 1], got[2][b:b + 1, :, hk:hk + 1])
        check(sub, ref, f"slice b={b} hk={hk}")


def gpu_grads_kv(q, k, v, do, causal, past_len):
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = fa.forward(qd, kd, vd, causal=causal, past_len=past_len)
    dq, dk, dv, _ = fa.backward(qd, kd, vd, o, lse, dod, causal=causal, past_len=past_len)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Lq,Lk,H,Hkv,D,past", [
    (1, 77, 300, 4, 2, 128, None),     # cross-attention / rows after a 223-key prefix
    (2, 300, 77, 2, 1, 64, None),      # more rows than keys (negative default offset)
    (1, 70, 50, 4, 4, 128, -20),       # the first 20 rows see no key
    (1, 33, 129, 2, 2, 64, 500),       # every key visible
    (1, 129, 257, 8, 2, 128, 0),       # offset 0 with more keys: keys past row 128 unseen when causal
    (2, 1, 333, 4, 1, 64, None),       # one row after 332 cached keys
    (1, 1024, 4096, 4, 2, 128, None),  # a prefill of 1024 rows after 3072 cached keys
])
def test_backward_unequal_lengths(B, Lq, Lk, H, Hkv, D, past, causal):
    q, _, _, do = make_qkvdo(B, Lq, H, Hkv, D, seed=1600 + Lq)
    _, k, v, _ = make_qkvdo(B, Lk, H, Hkv, D, seed=1700 + Lk)
    what = f"B{B} Lq{Lq} Lk{Lk} H{H} Hkv{Hkv} D{D} past={past} causal={causal}"
    print(what, flush=True)
    ref = oracle.backward(q, k, v, do, causal=causal, past_len=past)
    got = gpu_grads_kv(q, k, v, do, causal, past)
    check(got, ref, what)
    # rows that see no key have dq = 0 exactly, keys that no row sees dk = dv = 0 exactly
    pl = Lk - Lq if past is None else past
    if causal:
        for i in range(Lq):
            if i + pl < 0:
                assert torch.all(got[0][:, i] == 0), (what, i)
        first_unseen = max(0, Lq - 1 + pl + 1)
        if first_unseen < Lk:
            assert torch.all(got[1][:, first_unseen:] == 0) and torch.all(got[2][:, first_unseen:] == 0)


def test_backward_no_rows_or_no_keys():
    """No query rows: dk = dv = 0.  No keys: every row sees nothing, dq = 0."""
    B, H, Hkv, D = 2, 4, 2, 128
    _, k, v, _ = make_qkvdo(B, 50, H, Hkv, D, seed=1800)
    q = torch.empty(B, 0, H, D, dtype=torch.float16)
    o = torch.empty_like(q).cuda()
    lse = torch.empty(B, H, 0, dtype=torch.float32, device="cuda")
    dq, dk, dv, _ = fa.backward(q.cuda(), k.cuda(), v.cuda(), o, lse, q.cuda(), causal=False)
    torch.cuda.synchronize()
    assert dq.numel() == 0 and torch.all(dk == 0) and torch.all(dv == 0)
    q, _, _, do = make_qkvdo(B, 40, H, Hkv, D, seed=1801)
    k0 = torch.empty(B, 0, Hkv, D, dtype=torch.float16, device="cuda")
    for causal in (False, True):
        o, lse = fa.forward(q.cuda(), k0, k0, causal=causal)
        dq, dk, dv, _ = fa.backward(q.cuda(), k0, k0, o, lse, do.cuda(), causal=causal)
        torch.cuda.synchronize()
        assert torch.all(dq == 0) and dk.numel() == 0 and dv.numel() == 0


def test_backward_deterministic_and_gqa_equals_repeated():
    q, k, v, do = make_qkvdo(2, 333, 8, 2, 128, seed=1500)
    g = 4
    for causal in (False, True):
        a = gpu_grads(q, k, v, do, causal)
        b = gpu_grads(q, k, v, do, causal)
        for x, y in zip(a, b):
            assert torch.equal(x, y)
        # repeated K/V heads: dq equal; dk, dv of the group sum to the GQA ones
        kr, vr = k.repeat_interleave(g, dim=2).contiguous(), v.repeat_interleave(g, dim=2).contiguous()
        r = gpu_grads(q, kr, vr, do, causal)
        assert torch.equal(a[0], r[0])
        for x, y in ((a[1], r[1]), (a[2], r[2])):
            s = y.double().reshape(2, 333, 2, g, 128).sum(dim=3)
            assert (x.double() - s).abs().max().item() <= 2e-2 * s.abs().max().item()


def test_backward_rejects_bad_arguments():
    q, k, v, do = make_qkvdo(1, 64, 2, 2, 64, seed=1600)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = fa.forward(qd, kd, vd)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    delta = torch.empty_like(lse)
    with pytest.raises(fa.FaError) as e:
        fa.backward(qd, kd, vd, o, lse, dod, dq=qd)  # dq aliases q
    assert e.value.status == 7
    with pytest.raises(fa.FaError) as e:
        fa.backward(qd, kd, vd, o, lse, dod, dk=dv, dv=dv)  # outputs overlap
    assert e.value.status == 7
    st = fa.fa_bwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), dod.data_ptr(),
                   lse.data_ptr(), delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                   1, 64, 2, 2, 96, 0, 0.125, None)
    assert st == 4
    z = torch.empty((0, 8, 2, 64), dtype=torch.float16, device="cuda")
    zl = torch.empty((0, 2, 8), dtype=torch.float32, device="cuda")
    r = fa.backward(z, z, z, z, zl, z)
    assert r[0].shape == z.shape


def test_backward_rejects_wrong_gradient_buffers():
    """Caller-supplied dq, dk, dv must match q (dq) or k (dk, dv) in shape,
    dtype, contiguity and device; anything else is a ValueError raised in the
    binding before any launch."""
    q, k, v, do = make_qkvdo(1, 64, 4, 2, 64, seed=1601)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = fa.forward(qd, kd, vd)
    good_k = torch.empty_like(kd)
    bad = [dict(dq=torch.empty_like(kd)),                                   # dq shaped like k
           dict(dq=torch.empty(qd.shape, dtype=torch.float32, device="cuda")),
           dict(dq=torch.empty((1, 4, 64, 64), dtype=torch.float16, device="cuda").transpose(1, 2)),
           dict(dk=torch.empty_like(qd)),                                   # dk shaped like q
           dict(dk=good_k, dv=torch.empty(kd.shape, dtype=torch.float16)),  # dv in host memory
           dict(dv=torch.empty((1, 32, 2, 64), dtype=torch.float16, device="cuda"))]
    for kw in bad:
        with pytest.raises(ValueError):
            fa.backward(qd, kd, vd, o, lse, dod, **kw)
