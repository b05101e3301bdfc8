"""Pins for the fp64 oracle: it is checked against things other than itself.

Each pin is a function of an oracle build (``lib``) that raises AssertionError
when the build is wrong.  The real oracle must pass every pin; a set of copies
of the oracle, each with one plausible mistake planted in its C source (a
dropped scale, a wrong K/V head, an off-by-one mask, a missing max term in the
log-sum-exp, ...), must each fail at least one pin.  What pins what:

* binary16 decoding      -- numpy's float16 -> float64 conversion, all 65536 patterns
* whole O and LSE        -- torch's scaled_dot_product_attention (enable_gqa) and
                            logsumexp in float64 on the CPU, a library routine
                            that computes the same definition
* softmax normalisation  -- each row of probabilities sums to one
* weighted sum           -- constant V returns that constant
* causal mask            -- row 0 equals V[0] with LSE = s_00; Q = 0 gives the
                            running mean of V and LSE = ln(i + 1) (closed form)
* large logits/selection -- one-hot keys and a large one-hot query select one V row
* grouped-query heads    -- equals multi-head attention with K/V heads repeated
* small cases            -- L = 1 gives V and s_00; L = 2 is a two-way sigmoid mix
* invariances            -- key permutation (non-causal), per-row logit shift,
                            per-(b, h) slicing, thread count, the row API
* Lq != Lk, past_len     -- torch's attention with an explicit boolean mask
                            (keep j iff i + past_len >= j); Q = 0 gives the mean
                            of the visible V rows and ln(count); rows that see no
                            key give O = 0 and LSE = -inf; past_len >= Lk - 1
                            equals the unmasked result; the queries of a prefill
                            after a cached prefix equal the last rows of causal
                            self-attention over the whole sequence
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from tiled_attention_flash_amd.inputs import make_qkv

TOL = 1e-12


def f64(x: torch.Tensor) -> np.ndarray:
    return x.to(torch.float64).numpy()


def sdpa_reference(q, k, v, causal, scale):
    """torch's fused attention in float64 on the CPU, with GQA head sharing.
    BSHD -> BHSD for torch, and back."""
    qt = q.to(torch.float64).permute(0, 2, 1, 3)
    kt = k.to(torch.float64).permute(0, 2, 1, 3)
    vt = v.to(torch.float64).permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, is_causal=causal, scale=scale, enable_gqa=qt.shape[1] != kt.shape[1])
    g = qt.shape[1] // kt.shape[1]
    kr = kt.repeat_interleave(g, dim=1)
    s = torch.matmul(qt, kr.transpose(-1, -2)) * scale
    if causal:
        L = s.shape[-1]
        mask = torch.ones(L, L, dtype=torch.bool).triu(1)
        s = s.masked_fill(mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.permute(0, 2, 1, 3).numpy(), lse.numpy()


# ------------------------------------------------------------------- pins

def pin_decoder(lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b), lib=lib) for b in bits])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), "NaN patterns decode differently"
    assert np.array_equal(got[~nan], want[~nan]), "binary16 decode differs from numpy"


SDPA_SHAPES = [
    # B, L, H, Hkv, D
    (1, 1, 1, 1, 64),
    (1, 7, 2, 2, 64),
    (2, 33, 4, 2, 64),
    (1, 64, 4, 1, 128),
    (2, 17, 4, 4, 16),
    (1, 40, 8, 2, 8),
]


def pin_sdpa(lib):
    for n, (B, L, H, Hkv, D) in enumerate(SDPA_SHAPES):
        q, k, v = make_qkv(B, L, H, Hkv, D, seed=100 + n)
        for causal in (False, True):
            scale = 1.0 / math.sqrt(D)
            o, lse = oracle.forward(q, k, v, causal=causal, lib=lib)
            o_ref, lse_ref = sdpa_reference(q, k, v, causal, scale)
            assert np.max(np.abs(o - o_ref)) <= 1e-12, (B, L, H, Hkv, D, causal)
            assert np.max(np.abs(lse - lse_ref)) <= 1e-12, (B, L, H, Hkv, D, causal)


def pin_rows_sum_to_one(lib):
    q, k, v = make_qkv(1, 50, 2, 1, 64, seed=7)
    for causal in (False, True):
        for i in (0, 1, 25, 49):
            p = oracle.row_probs(q, k, v, 0, 1, i, causal=causal, lib=lib)
            assert abs(p.sum() - 1.0) <= TOL
            assert np.all(p >= 0)
            if causal:
                assert np.all(p[i + 1:] == 0)
                assert np.all(p[: i + 1] > 0)


def pin_constant_v(lib):
    q, k, _ = make_qkv(2, 31, 4, 2, 64, seed=8)
    c = torch.linspace(-3, 3, 64).half()
    v = c.expand(2, 31, 2, 64).contiguous()
    for causal in (False, True):
        o, _ = oracle.forward(q, k, v, causal=causal, lib=lib)
        assert np.max(np.abs(o - f64(c))) <= TOL


def pin_causal_row0(lib):
    q, k, v = make_qkv(2, 20, 4, 2, 64, seed=9)
    o, lse = oracle.forward(q, k, v, causal=True, lib=lib)
    qd, kd, vd = f64(q), f64(k), f64(v)
    for b in range(2):
        for h in range(4):
            hk = h // 2
            assert np.max(np.abs(o[b, 0, h] - vd[b, 0, hk])) <= TOL
            s00 = (qd[b, 0, h] @ kd[b, 0, hk]) / 8.0
            assert abs(lse[b, h, 0] - s00) <= TOL


def pin_zero_q(lib):
    _, k, v = make_qkv(1, 24, 2, 2, 64, seed=10)
    q = torch.zeros(1, 24, 2, 64, dtype=torch.float16)
    vd = f64(v)
    o, lse = oracle.forward(q, k, v, causal=True, lib=lib)
    for i in range(24):
        want = vd[0, : i + 1].mean(axis=0)  # [Hkv, D]
        assert np.max(np.abs(o[0, i] - want)) <= TOL
        assert np.max(np.abs(lse[0, :, i] - math.log(i + 1))) <= TOL
    o, lse = oracle.forward(q, k, v, causal=False, lib=lib)
    assert np.max(np.abs(o[0] - vd[0].mean(axis=0)[None])) <= TOL
    assert np.max(np.abs(lse - math.log(24))) <= TOL


def pin_one_hot_selection(lib):
    L, D = 48, 64
    perm = np.random.default_rng(11).permutation(L)
    k = torch.zeros(1, L, 1, D, dtype=torch.float16)
    for j in range(L):
        k[0, j, 0, j] = 1.0
    q = torch.zeros(1, L, 1, D, dtype=torch.float16)
    for i in range(L):
        q[0, i, 0, perm[i]] = 1000.0  # logit gap 1000/8 = 125 -> others weigh < L*e^-125
    _, _, v = make_qkv(1, L, 1, 1, D, seed=12)
    o, lse = oracle.forward(q, k, v, causal=False, lib=lib)
    vd = f64(v)
    for i in range(L):
        assert np.max(np.abs(o[0, i, 0] - vd[0, perm[i], 0])) <= TOL
        assert abs(lse[0, 0, i] - 125.0) <= TOL


def pin_gqa_equals_repeated_mha(lib):
    q, k, v = make_qkv(2, 37, 8, 2, 64, seed=13)
    kr = k.repeat_interleave(4, dim=2).contiguous()
    vr = v.repeat_interleave(4, dim=2).contiguous()
    for causal in (False, True):
        o1, l1 = oracle.forward(q, k, v, causal=causal, lib=lib)
        o2, l2 = oracle.forward(q, kr, vr, causal=causal, lib=lib)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def pin_small_L(lib):
    q, k, v = make_qkv(1, 1, 2, 1, 64, seed=14)
    for causal in (False, True):
        o, lse = oracle.forward(q, k, v, causal=causal, lib=lib)
        assert np.max(np.abs(o[0, 0] - f64(v)[0, 0, 0][None])) <= TOL
        s00 = f64(q)[0, 0] @ f64(k)[0, 0, 0] / 8.0
        assert np.max(np.abs(lse[0, :, 0] - s00)) <= TOL
    # L = 2, non-causal: O = sigmoid(s0 - s1) V0 + sigmoid(s1 - s0) V1
    q, k, v = make_qkv(1, 2, 1, 1, 64, seed=15)
    qd, kd, vd = f64(q)[0, :, 0], f64(k)[0, :, 0], f64(v)[0, :, 0]
    o, lse = oracle.forward(q, k, v, causal=False, lib=lib)
    for i in range(2):
        s0, s1 = qd[i] @ kd[0] / 8.0, qd[i] @ kd[1] / 8.0
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        w1 = 1.0 / (1.0 + math.exp(s0 - s1))
        assert np.max(np.abs(o[0, i, 0] - (w0 * vd[0] + w1 * vd[1]))) <= TOL
        assert abs(lse[0, 0, i] - np.logaddexp(s0, s1)) <= TOL


def pin_key_permutation(lib):
    q, k, v = make_qkv(1, 29, 2, 2, 64, seed=16)
    perm = torch.from_numpy(np.random.default_rng(17).permutation(29))
    o1, l1 = oracle.forward(q, k, v, causal=False, lib=lib)
    o2, l2 = oracle.forward(q, k[:, perm].contiguous(), v[:, perm].contiguous(), causal=False,
                            lib=lib)
    assert np.max(np.abs(o1 - o2)) <= TOL and np.max(np.abs(l1 - l2)) <= TOL


def pin_logit_shift(lib):
    """Adding the same vector u to every key shifts row i's logits by
    scale * (q_i . u): O is unchanged and LSE moves by exactly that amount.
    Values are multiples of 2^-6 below 4 in magnitude so K + u stays exact in fp16."""
    rng = np.random.default_rng(18)
    B, L, H, D = 1, 26, 2, 64
    q = torch.from_numpy(np.round(np.clip(rng.normal(size=(B, L, H, D)), -3.9, 3.9) * 64) / 64).half()
    k = torch.from_numpy(np.round(np.clip(rng.normal(size=(B, L, H, D)), -3.9, 3.9) * 64) / 64).half()
    v = torch.from_numpy(rng.normal(size=(B, L, H, D))).half()
    u = torch.from_numpy(rng.integers(-1, 2, size=D).astype(np.float64)).half()
    k2 = (k.double() + u.double()).half()
    assert torch.equal(k2.double(), k.double() + u.double())
    for causal in (False, True):
        o1, l1 = oracle.forward(q, k, v, causal=causal, lib=lib)
        o2, l2 = oracle.forward(q, k2, v, causal=causal, lib=lib)
        shift = np.einsum("bihd,d->bhi", f64(q), f64(u)) / 8.0
        assert np.max(np.abs(o1 - o2)) <= 1e-11
        assert np.max(np.abs((l2 - l1) - shift)) <= 1e-11


def pin_slices(lib):
    q, k, v = make_qkv(2, 21, 4, 2, 64, seed=19)
    for causal in (False, True):
        o, lse = oracle.forward(q, k, v, causal=causal, lib=lib)
        for b in range(2):
            for h in range(4):
                hk = h // 2
                o1, l1 = oracle.forward(q[b:b + 1, :, h:h + 1].contiguous(),
                                        k[b:b + 1, :, hk:hk + 1].contiguous(),
                                        v[b:b + 1, :, hk:hk + 1].contiguous(), causal=causal,
                                        lib=lib)
                assert np.array_equal(o1[0, :, 0], o[b, :, h])
                assert np.array_equal(l1[0, 0], lse[b, h])


def pin_threads_and_rows(lib):
    q, k, v = make_qkv(1, 150, 4, 1, 64, seed=20)
    for causal in (False, True):
        o1, l1 = oracle.forward(q, k, v, causal=causal, nthreads=1, lib=lib)
        o8, l8 = oracle.forward(q, k, v, causal=causal, nthreads=8, lib=lib)
        assert np.array_equal(o1, o8) and np.array_equal(l1, l8)
        ids = np.array([[0, 0, 0], [0, 3, 149], [0, 2, 77], [0, 1, 64]])
        orow, lrow = oracle.rows(q, k, v, ids, causal=causal, lib=lib)
        for n, (b, h, i) in enumerate(ids):
            assert np.array_equal(orow[n], o1[b, i, h]) and lrow[n] == l1[b, h, i]


def visible_counts(Lq, Lk, causal, past_len):
    """Keys query row i keeps: all Lk, or those with i + past_len >= j."""
    if not causal:
        return np.full(Lq, Lk)
    return np.clip(np.arange(Lq) + past_len + 1, 0, Lk)


KV_CASES = [
    # B, Lq, Lk, H, Hkv, D, past_len (None = Lk - Lq)
    (1, 5, 19, 2, 1, 64, None),
    (2, 17, 40, 4, 2, 64, None),
    (1, 33, 33, 2, 2, 16, 7),      # queries shifted forward
    (1, 30, 12, 2, 1, 64, None),   # more queries than keys: early rows see nothing
    (2, 9, 25, 4, 4, 8, -4),       # negative offset: first 4 rows see nothing
    (1, 6, 20, 2, 2, 32, 100),     # offset past the end: every key visible
]


def pin_sdpa_kv(lib):
    for n, (B, Lq, Lk, H, Hkv, D, past) in enumerate(KV_CASES):
        q, _, _ = make_qkv(B, Lq, H, Hkv, D, seed=200 + n)
        _, k, v = make_qkv(B, Lk, H, Hkv, D, seed=300 + n)
        pl = Lk - Lq if past is None else past
        scale = 1.0 / math.sqrt(D)
        for causal in (False, True):
            o, lse = oracle.forward(q, k, v, causal=causal, past_len=past, lib=lib)
            keep = torch.ones(Lq, Lk, dtype=torch.bool)
            if causal:
                keep = torch.arange(Lq)[:, None] + pl >= torch.arange(Lk)[None, :]
            qt = q.to(torch.float64).permute(0, 2, 1, 3)
            kt = k.to(torch.float64).permute(0, 2, 1, 3).repeat_interleave(H // Hkv, dim=1)
            vt = v.to(torch.float64).permute(0, 2, 1, 3).repeat_interleave(H // Hkv, dim=1)
            o_ref = torch.nn.functional.scaled_dot_product_attention(
                qt, kt, vt, attn_mask=keep, scale=scale).permute(0, 2, 1, 3).numpy()
            s = (torch.matmul(qt, kt.transpose(-1, -2)) * scale).masked_fill(~keep, float("-inf"))
            lse_ref = torch.logsumexp(s, dim=-1).numpy()
            seen = visible_counts(Lq, Lk, causal, pl) > 0
            assert np.max(np.abs(o[:, seen] - o_ref[:, seen]), initial=0) <= 1e-12, (n, causal)
            assert np.max(np.abs(lse[:, :, seen] - lse_ref[:, :, seen]), initial=0) <= 1e-12
            assert np.all(o[:, ~seen] == 0.0), (n, causal)
            assert np.all(lse[:, :, ~seen] == -np.inf), (n, causal)


def pin_zero_q_kv(lib):
    B, Lq, Lk, H, D = 1, 12, 20, 2, 32
    _, k, v = make_qkv(B, Lk, H, H, D, seed=400)
    q = torch.zeros(B, Lq, H, D, dtype=torch.float16)
    vd = f64(v)
    for past in (Lk - Lq, -3, 0):
        o, lse = oracle.forward(q, k, v, causal=True, past_len=past, lib=lib)
        for i, n in enumerate(visible_counts(Lq, Lk, True, past)):
            if n == 0:
                assert np.all(o[0, i] == 0.0) and np.all(lse[0, :, i] == -np.inf)
            else:
                assert np.max(np.abs(o[0, i] - vd[0, :n].mean(axis=0))) <= TOL
                assert np.max(np.abs(lse[0, :, i] - math.log(n))) <= TOL


def pin_past_beyond_end_is_unmasked(lib):
    q, _, _ = make_qkv(1, 10, 2, 1, 64, seed=401)
    _, k, v = make_qkv(1, 23, 2, 1, 64, seed=402)
    o1, l1 = oracle.forward(q, k, v, causal=False, lib=lib)
    for past in (22, 40):
        o2, l2 = oracle.forward(q, k, v, causal=True, past_len=past, lib=lib)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def pin_prefill_after_prefix(lib):
    """The last Lq query rows of causal self-attention over Lk positions equal
    a causal forward of just those rows, placed at past_len = Lk - Lq."""
    q, k, v = make_qkv(2, 41, 4, 2, 64, seed=403)
    o_full, l_full = oracle.forward(q, k, v, causal=True, lib=lib)
    for Lq in (1, 13, 41):
        qs = q[:, 41 - Lq:].contiguous()
        o, lse = oracle.forward(qs, k, v, causal=True, lib=lib)  # default past_len = Lk - Lq
        assert np.array_equal(o, o_full[:, 41 - Lq:]) and np.array_equal(lse, l_full[:, :, 41 - Lq:])


PINS = [pin_decoder, pin_sdpa, pin_rows_sum_to_one, pin_constant_v, pin_causal_row0, pin_zero_q,
        pin_one_hot_selection, pin_gqa_equals_repeated_mha, pin_small_L, pin_key_permutation,
        pin_logit_shift, pin_slices, pin_threads_and_rows, pin_sdpa_kv, pin_zero_q_kv,
        pin_past_beyond_end_is_unmasked, pin_prefill_after_prefix]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(None)


# Plausible mistakes, each planted in a copy of the oracle's source.  Every
# one must be rejected by at least one pin.
MUTANTS = {
    "scale dropped": ("s[j] = p->scale * dot;", "s[j] = dot;"),
    "kv head h mod Hkv": ("int hk = h / groups;", "int hk = h % p->Hkv;"),
    "mask admits one future key": ("long n = (long)i + p->past_len + 1;",
                                   "long n = (long)i + p->past_len + 2;"),
    "mask drops the diagonal": ("long n = (long)i + p->past_len + 1;",
                                "long n = (long)i + p->past_len;"),
    "past_len ignored": ("long n = (long)i + p->past_len + 1;", "long n = (long)i + 1;"),
    "past_len sign flipped": ("long n = (long)i + p->past_len + 1;",
                              "long n = (long)i - p->past_len + 1;"),
    "key rows indexed with the query length": (
        "return (((size_t)b * p->Lk + j) * p->Hkv + hk) * p->D + d;",
        "return (((size_t)b * p->Lq + j) * p->Hkv + hk) * p->D + d;"),
    "K used in place of V": ("acc += s[j] * h2d(p->v[kv_index(p, b, j, hk, d)]);",
                             "acc += s[j] * h2d(p->k[kv_index(p, b, j, hk, d)]);"),
    "no normalisation": ("s[j] = s[j] / z;", "s[j] = s[j] / (double)n;"),
    "lse without max": ("*lse_out = m + log(z);", "*lse_out = log(z);"),
    "log2 lse": ("*lse_out = m + log(z);", "*lse_out = m + log2(z);"),
    "last d dropped": ("for (int d = 0; d < p->D; ++d)\n            dot +=",
                       "for (int d = 0; d < p->D - 1; ++d)\n            dot +="),
    "subnormal exponent": ("ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    "exponent bias": ("ldexp(1.0 + (double)frac / 1024.0, e - 15)",
                      "ldexp(1.0 + (double)frac / 1024.0, e - 14)"),
    "query row transposed with head": ("return (((size_t)b * p->Lq + i) * p->H + h) * p->D + d;",
                                       "return (((size_t)b * p->H + h) * p->Lq + i) * p->D + d;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = oracle.source_text()
    assert src.count(old) >= 1, f"mutation site for '{name}' not found"
    lib = oracle.build_variant(src.replace(old, new, 1), str(tmp_path / "mutant.so"))
    failed = []
    for pin in PINS:
        try:
            with np.errstate(invalid="ignore"):  # a broken copy may produce inf - inf
                pin(lib)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin rejects the planted mistake '{name}'"
