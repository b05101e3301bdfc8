"""Pins of the backward oracle (fp64 gradients of sum(O * dO)), CPU only.

Each pin checks oracle.backward against something other than itself:
* a library routine: torch autograd through scaled_dot_product_attention in
  float64 on the CPU (grouped-query heads, causal and not);
* central finite differences of torch's float64 attention forward;
* identities that follow from the softmax: with dO = 0 every gradient is 0;
  the dV rows of a head sum to the dO rows (each probability row sums to 1);
  the dK rows sum to 0 (each softmax-derivative row sums to 0); shifting
  every key, or every value, by one common vector leaves all gradients
  unchanged; under the causal mask query row 0 gets dQ = 0 exactly;
* grouped-query heads equal multi-head attention with K/V repeated and the
  repeated heads' dK, dV summed; the thread count changes nothing;
* query and key lengths that differ, with the causal position offset
  past_len: torch autograd in float64 through the plain masked softmax
  (rows that keep no key have output 0); the last Lq rows of a square causal
  problem whose other rows carry dO = 0; rows before the first key (negative
  past_len) have dQ = 0 and change nothing else.
Plausible mistakes planted in copies of the C source must each fail a pin.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tiled_attention_flash_amd.inputs import make_qkvdo

TOL = 1e-10


def torch_grads(q, k, v, do, causal, scale):
    """Reference gradients from torch autograd in float64 (BSHD in and out)."""
    Q, K, V, DO = [t.double().permute(0, 2, 1, 3).contiguous() for t in (q, k, v, do)]
    for t in (Q, K, V):
        t.requires_grad_(True)
    O = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=causal, scale=scale,
                                                         enable_gqa=True)
    O.backward(DO)
    return [t.grad.permute(0, 2, 1, 3).numpy() for t in (Q, K, V)]


def pin_autograd(lib):
    for (B, L, H, Hkv, D, seed) in [(1, 1, 1, 1, 8, 1), (2, 37, 4, 2, 16, 2), (1, 64, 4, 1, 64, 3),
                                    (1, 20, 2, 2, 128, 4), (2, 9, 8, 2, 32, 5)]:
        q, k, v, do = make_qkvdo(B, L, H, Hkv, D, seed=seed)
        for causal in (False, True):
            scale = 1.0 / np.sqrt(D)
            got = oracle.backward(q, k, v, do, causal=causal, lib=lib)
            ref = torch_grads(q, k, v, do, causal, scale)
            for g, r, name in zip(got, ref, ("dq", "dk", "dv")):
                err = np.max(np.abs(g - r))
                assert err <= TOL * max(1.0, np.max(np.abs(r))), (B, L, H, Hkv, D, causal, name, err)


def pin_finite_differences(lib):
    """d sum(O*dO) / d x by central differences of torch's float64 forward,
    for a few entries of Q, K and V (independent of any backward code)."""
    B, L, H, Hkv, D = 1, 6, 2, 1, 4
    q, k, v, do = make_qkvdo(B, L, H, Hkv, D, seed=11)
    scale = 0.7
    for causal in (False, True):
        dq, dk, dv = oracle.backward(q, k, v, do, causal=causal, scale=scale, lib=lib)
        base = [t.double().permute(0, 2, 1, 3).clone() for t in (q, k, v)]
        DO = do.double().permute(0, 2, 1, 3)

        def loss(ts):
            o = torch.nn.functional.scaled_dot_product_attention(*ts, is_causal=causal, scale=scale,
                                                                 enable_gqa=True)
            return float((o * DO).sum())

        eps = 1e-5
        for which, grad in ((0, dq), (1, dk), (2, dv)):
            n_heads = base[which].shape[1]
            for (b, i, hh, d) in [(0, 0, 0, 0), (0, 3, n_heads - 1, 2), (0, L - 1, 0, D - 1)]:
                plus = [t.clone() for t in base]
                minus = [t.clone() for t in base]
                plus[which][b, hh, i, d] += eps
                minus[which][b, hh, i, d] -= eps
                fd = (loss(plus) - loss(minus)) / (2 * eps)
                assert abs(fd - grad[b, i, hh, d]) <= 1e-7, (causal, which, (b, i, hh, d), fd,
                                                              grad[b, i, hh, d])


def pin_zero_dout(lib):
    q, k, v, do = make_qkvdo(1, 19, 4, 2, 16, seed=12)
    for causal in (False, True):
        for g in oracle.backward(q, k, v, torch.zeros_like(do), causal=causal, lib=lib):
            assert np.all(g == 0.0)


def pin_sums(lib):
    """sum_j dV[j] = sum_{i, heads of the group} dO[i]; sum_j dK[j] = 0."""
    B, L, H, Hkv, D = 2, 23, 4, 2, 32
    q, k, v, do = make_qkvdo(B, L, H, Hkv, D, seed=13)
    g = H // Hkv
    dof = do.double().numpy()
    for causal in (False, True):
        dq, dk, dv = oracle.backward(q, k, v, do, causal=causal, lib=lib)
        want = dof.reshape(B, L, Hkv, g, D).sum(axis=(1, 3))
        assert np.max(np.abs(dv.sum(axis=1) - want)) <= TOL * 100
        assert np.max(np.abs(dk.sum(axis=1))) <= TOL * 100


def pin_shift_invariance(lib):
    """Adding one vector to every key (scores move by a per-row constant) or
    to every value (the output moves by that vector) leaves the gradients."""
    B, L, H, Hkv, D = 1, 17, 2, 1, 16
    q, k, v, do = make_qkvdo(B, L, H, Hkv, D, seed=14)
    # K and V on a grid of 1/64 within (-8, 8): adding small integers keeps
    # every entry exact in float16 (11 significant bits cover 16 * 64)
    k = (torch.round(k.float().clamp(-7, 7) * 64) / 64).half()
    v = (torch.round(v.float().clamp(-7, 7) * 64) / 64).half()
    u = torch.tensor([1.0, -2.0, 0.0, 1.0] * 4, dtype=torch.float32)
    ks, vs = (k.float() + u).half(), (v.float() + u).half()
    assert torch.equal(ks.float(), k.float() + u) and torch.equal(vs.float(), v.float() + u)
    for causal in (False, True):
        base = oracle.backward(q, k, v, do, causal=causal, lib=lib)
        shifted_k = oracle.backward(q, ks, v, do, causal=causal, lib=lib)
        shifted_v = oracle.backward(q, k, vs, do, causal=causal, lib=lib)
        for a, b2, c in zip(base, shifted_k, shifted_v):
            assert np.max(np.abs(a - b2)) <= 1e-9
            assert np.max(np.abs(a - c)) <= 1e-9


def pin_causal_row0(lib):
    q, k, v, do = make_qkvdo(2, 15, 4, 2, 32, seed=15)
    dq, _, _ = oracle.backward(q, k, v, do, causal=True, lib=lib)
    assert np.all(dq[:, 0] == 0.0)


def pin_gqa_equals_repeated(lib):
    B, L, H, Hkv, D = 1, 21, 8, 2, 16
    q, k, v, do = make_qkvdo(B, L, H, Hkv, D, seed=16)
    g = H // Hkv
    for causal in (False, True):
        dq, dk, dv = oracle.backward(q, k, v, do, causal=causal, lib=lib)
        dq2, dk2, dv2 = oracle.backward(q, k.repeat_interleave(g, dim=2).contiguous(),
                                        v.repeat_interleave(g, dim=2).contiguous(), do,
                                        causal=causal, lib=lib)
        assert np.array_equal(dq, dq2)
        assert np.max(np.abs(dk - dk2.reshape(B, L, Hkv, g, D).sum(axis=3))) <= 1e-12
        assert np.max(np.abs(dv - dv2.reshape(B, L, Hkv, g, D).sum(axis=3))) <= 1e-12


def pin_threads(lib):
    q, k, v, do = make_qkvdo(2, 33, 4, 2, 32, seed=17)
    a = oracle.backward(q, k, v, do, causal=True, nthreads=1, lib=lib)
    b = oracle.backward(q, k, v, do, causal=True, nthreads=5, lib=lib)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def torch_grads_kv(q, k, v, do, causal, scale, past):
    """Reference gradients for Lq != Lk from torch autograd in float64 through
    the plain definition: masked scores, softmax over the kept keys (a row
    that keeps none has output 0), weighted sum of V."""
    Lq, Lk = q.shape[1], k.shape[1]
    g = q.shape[2] // k.shape[2]
    Q, K, V = [t.double().permute(0, 2, 1, 3).contiguous().requires_grad_(True) for t in (q, k, v)]
    DO = do.double().permute(0, 2, 1, 3)
    keep = torch.ones(Lq, Lk, dtype=torch.bool)
    if causal:
        keep = torch.arange(Lq)[:, None] + past >= torch.arange(Lk)[None, :]
    s = torch.matmul(Q, K.repeat_interleave(g, dim=1).transpose(-1, -2)) * scale
    s = s.masked_fill(~keep, float("-inf"))
    m = s.amax(dim=-1, keepdim=True)
    m = torch.where(torch.isfinite(m), m, torch.zeros_like(m)).detach()
    p = torch.exp(s - m)
    z = p.sum(dim=-1, keepdim=True)
    O = torch.matmul(p / torch.where(z > 0, z, torch.ones_like(z)), V.repeat_interleave(g, dim=1))
    O.backward(DO)
    return [t.grad.permute(0, 2, 1, 3).numpy() for t in (Q, K, V)]


BWD_KV_CASES = [  # B, Lq, Lk, H, Hkv, D, past_len (None: Lk - Lq)
    (1, 5, 17, 2, 1, 16, None),
    (2, 13, 7, 4, 2, 32, None),    # more queries than keys
    (1, 9, 25, 2, 2, 64, -4),      # the first 4 rows keep no key
    (1, 6, 20, 4, 1, 8, 100),      # every key kept
    (1, 33, 40, 2, 2, 128, 3),
]


def pin_autograd_kv(lib):
    for n, (B, Lq, Lk, H, Hkv, D, past) in enumerate(BWD_KV_CASES):
        q, _, _, do = make_qkvdo(B, Lq, H, Hkv, D, seed=500 + n)
        _, k, v, _ = make_qkvdo(B, Lk, H, Hkv, D, seed=600 + n)
        pl = Lk - Lq if past is None else past
        scale = 1.0 / np.sqrt(D)
        for causal in (False, True):
            got = oracle.backward(q, k, v, do, causal=causal, past_len=past, lib=lib)
            ref = torch_grads_kv(q, k, v, do, causal, scale, pl if causal else 0)
            for g, r, name in zip(got, ref, ("dq", "dk", "dv")):
                err = np.max(np.abs(g - r))
                assert err <= TOL * max(1.0, np.max(np.abs(r))), (n, causal, name, err)


def pin_prefix_kv(lib):
    """Causal rows placed after a cached prefix (past_len = Lk - Lq) have the
    gradients of the last Lq rows of the square causal problem over all Lk
    positions in which the first Lk - Lq rows carry dO = 0 (those rows then
    add nothing to dK and dV)."""
    B, L, H, Hkv, D = 2, 29, 4, 2, 32
    q, k, v, do = make_qkvdo(B, L, H, Hkv, D, seed=700)
    for Lq in (1, 11, 29):
        do_full = do.clone()
        do_full[:, :L - Lq] = 0
        dq_f, dk_f, dv_f = oracle.backward(q, k, v, do_full, causal=True, lib=lib)
        dq, dk, dv = oracle.backward(q[:, L - Lq:].contiguous(), k, v, do[:, L - Lq:].contiguous(),
                                     causal=True, lib=lib)
        for a, b in ((dq, dq_f[:, L - Lq:]), (dk, dk_f), (dv, dv_f)):
            assert np.max(np.abs(a - b)) <= TOL * max(1.0, np.max(np.abs(b))), Lq


def pin_rows_before_first_key(lib):
    """With past_len = -c (c > 0) the first c rows keep no key: their dQ is 0,
    and the rest equals the problem without those rows at past_len = 0."""
    B, Lq, Lk, H, Hkv, D, c = 1, 12, 15, 2, 1, 64, 5
    q, _, _, do = make_qkvdo(B, Lq, H, Hkv, D, seed=710)
    _, k, v, _ = make_qkvdo(B, Lk, H, Hkv, D, seed=711)
    dq, dk, dv = oracle.backward(q, k, v, do, causal=True, past_len=-c, lib=lib)
    assert np.all(dq[:, :c] == 0.0)
    dq2, dk2, dv2 = oracle.backward(q[:, c:].contiguous(), k, v, do[:, c:].contiguous(), causal=True,
                                    past_len=0, lib=lib)
    for a, b in ((dq[:, c:], dq2), (dk, dk2), (dv, dv2)):
        assert np.max(np.abs(a - b)) <= TOL * max(1.0, np.max(np.abs(b)))


PINS = [pin_autograd, pin_finite_differences, pin_zero_dout, pin_sums, pin_shift_invariance,
        pin_causal_row0, pin_gqa_equals_repeated, pin_threads, pin_autograd_kv, pin_prefix_kv,
        pin_rows_before_first_key]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_backward_oracle_pin(pin):
    pin(None)


MUTANTS = {
    "Delta dropped": ("dprob[j] = prob[j] * (dprob[j] - delta);", "dprob[j] = prob[j] * dprob[j];"),
    "Delta sign": ("dprob[j] = prob[j] * (dprob[j] - delta);",
                   "dprob[j] = prob[j] * (dprob[j] + delta);"),
    "dQ without scale": ("dq[q_index(p, b, i, h, d)] = p->scale * acc;",
                         "dq[q_index(p, b, i, h, d)] = acc;"),
    "dK from K": ("p->scale * dprob[j] * h2d(p->q[q_index(p, b, i, h, d)]);",
                  "p->scale * dprob[j] * h2d(p->k[kv_index(p, b, j, hk, d)]);"),
    "dV weighted by dS": ("dv[kv_index(p, b, j, hk, d)] += prob[j] * h2d(dout[q_index(p, b, i, h, d)]);",
                          "dv[kv_index(p, b, j, hk, d)] += dprob[j] * h2d(dout[q_index(p, b, i, h, d)]);"),
    "dP from K": ("acc += h2d(dout[q_index(p, b, i, h, d)]) * h2d(p->v[kv_index(p, b, j, hk, d)]);",
                  "acc += h2d(dout[q_index(p, b, i, h, d)]) * h2d(p->k[kv_index(p, b, j, hk, d)]);"),
    "group sum: last head only": ("            dk[kv_index(p, b, j, hk, d)] = 0.0;\n            dv[kv_index(p, b, j, hk, d)] = 0.0;\n        }\n    for (int h = hk * groups; h < (hk + 1) * groups; ++h) {",
                                  "            dk[kv_index(p, b, j, hk, d)] = 0.0;\n            dv[kv_index(p, b, j, hk, d)] = 0.0;\n        }\n    for (int h = (hk + 1) * groups - 1; h < (hk + 1) * groups; ++h) {"),
    "unequal lengths: past_len dropped": ("problem_t p = {q, k, v, B, Lq, Lk, H, Hkv, D, causal ? 1 : 0, causal ? past_len : 0, scale};\n    bwd_job_t job;",
                                          "problem_t p = {q, k, v, B, Lq, Lk, H, Hkv, D, causal ? 1 : 0, 0, scale};\n    bwd_job_t job;"),
    "dQ over masked keys": ("for (int j = 0; j < n; ++j) acc += dprob[j] * h2d(p->k[kv_index(p, b, j, hk, d)]);",
                            "for (int j = 0; j < n + (n < p->Lk); ++j) acc += (j < n ? dprob[j] : 1.0) * h2d(p->k[kv_index(p, b, j, hk, d)]);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_pins_reject_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = oracle.source_text()
    assert src.count(old) >= 1, f"mutation site for '{name}' not found"
    lib = oracle.build_variant(src.replace(old, new, 1), str(tmp_path / "mutant.so"))
    failed = []
    for pin in PINS:
        try:
            with np.errstate(invalid="ignore"):
                pin(lib)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin rejects the planted mistake '{name}'"
