"""The allocation-free split-KV entry point (fa_fwd_splitkv_noalloc: the
library's static device scratch instead of a caller workspace) against the
workspace entry point fa_fwd_splitkv, through the C ABI.

Both run the same kernels with the same split count, so the outputs must be
bitwise equal; they are also held to the parity bar (max |dO| <= 1e-2, mean
|dO| <= 1e-3, max |dLSE| <= 1e-3).  Calls come in a row on one stream, a
large problem first and then smaller ones, so later calls find the scratch
holding an earlier call's partial results.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import tiled_attention_flash_amd as fa
from tiled_attention_flash_amd.inputs import make_qkv

pytestmark = pytest.mark.gpu

MAX_O, MEAN_O, MAX_LSE = 1e-2, 1e-3, 1e-3


def run_both(B, Lq, Lk, H, Hkv, D, causal, seed, n_splits=0):
    q, k, v = make_qkv(B, Lq, H, Hkv, D, seed=seed, Lk=Lk)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    past, scale = Lk - Lq, 1.0 / math.sqrt(D)
    splits = n_splits or fa.fa_splitkv_splits(B, Lq, Lk, H, Hkv, D, causal, past)
    need = fa.fa_splitkv_workspace_bytes(B, Lq, H, D, splits)
    assert 0 < need <= fa.SPLITKV_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o1 = torch.full_like(qd, float("nan"))
    l1 = torch.full((B, H, Lq), float("nan"), dtype=torch.float32, device="cuda")
    o2 = torch.full_like(qd, float("nan"))
    l2 = torch.full((B, H, Lq), float("nan"), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    print(f"noalloc B{B} Lq{Lq} Lk{Lk} H{H} Hkv{Hkv} D{D} causal={causal} splits={splits} "
          f"scratch bytes={need}", flush=True)
    st1 = fa.fa_fwd_splitkv(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o1.data_ptr(),
                            l1.data_ptr(), B, Lq, Lk, H, Hkv, D, causal, past, scale, splits,
                            ws.data_ptr(), need, stream)
    st2 = fa.fa_fwd_splitkv_noalloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o2.data_ptr(),
                                    l2.data_ptr(), B, Lq, Lk, H, Hkv, D, causal, past, scale,
                                    splits, stream)
    assert st1 == 0 and st2 == 0, (st1, st2)
    torch.cuda.synchronize()
    assert torch.isfinite(o1).all() and torch.isfinite(l1).all()
    d = (o2.double() - o1.double()).abs()
    dl = (l2.double() - l1.double()).abs()
    assert d.max().item() <= MAX_O and d.mean().item() <= MEAN_O and dl.max().item() <= MAX_LSE
    assert torch.equal(o1, o2) and torch.equal(l1, l2)  # same kernels, same splits


def test_noalloc_matches_workspace_entry_point_on_calls_in_a_row():
    # B=8, H=32 (8 K/V heads) decode step, 127 splits: 16.6 of the 16.8 MB of scratch
    per_split = fa.fa_splitkv_workspace_bytes(8, 1, 32, 128, 1)
    n_fit = fa.SPLITKV_SCRATCH_BYTES // per_split
    run_both(8, 1, 8192, 32, 8, 128, True, seed=1, n_splits=n_fit)
    # then smaller problems on the same scratch: a few query rows at D = 64,
    # the library's own split count, and one split
    run_both(2, 3, 1000, 8, 2, 64, True, seed=2)
    run_both(1, 5, 777, 4, 4, 128, False, seed=3, n_splits=1)


def test_noalloc_binding_and_oracle_free_properties():
    q, k, v = make_qkv(2, 1, 32, 8, 128, seed=4, Lk=4096)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o1, l1 = fa.forward_splitkv(qd, kd, vd, causal=True)
    o2, l2 = fa.forward_splitkv_noalloc(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    with pytest.raises(fa.FaError) as e:  # more partials than the scratch holds
        fa.forward_splitkv_noalloc(qd, kd, vd, causal=True, n_splits=4096)
    assert e.value.status == 11
