"""Pins of the fp8 oracle (forward on E4M3 inputs, and its error bound), CPU only.

Each pin checks oracle.forward_fp8 against something other than itself:
* the E4M3 decoder against torch's float8_e4m3fn for all 256 codes;
* the whole O and LSE against torch scaled_dot_product_attention and
  logsumexp in float64 on the decoded, descaled tensors (grouped-query heads,
  causal with past_len, ragged lengths);
* descale arithmetic: doubling the V descale doubles O exactly; doubling the
  Q (or K) descale while halving the scale changes nothing, bit for bit; with
  unit descales the result equals the fp16 oracle on the same values (every
  E4M3 value is an fp16 value);
* the error bound: the probabilities are rounded by torch's own E4M3 cast,
  after the offset a kernel applies (8 times the weight relative to a
  reference maximum R times below the row's maximum, R from 1 to 56), and the
  O that results must lie within the bound for every element, while the bound
  must not be vacuous (some element uses a good part of it).
Plausible mistakes planted in copies of the C source must each fail a pin.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tiled_attention_flash_amd.inputs import make_qkv_fp8

TOL = 1e-12
# Rounding model of the probabilities in E4M3 with the x8 offset: relative
# error 2^-4 (3 fraction bits, round to nearest) for weights >= 2^-9 (8 * w at
# or above E4M3's smallest normal 2^-6), below that at most the weight itself
# or half the subnormal spacing 2^-9 / 8.
MODEL = (2.0 ** -4, 2.0 ** -9, 2.0 ** -13)


def decoded(x8, descale):
    return x8.view(torch.float8_e4m3fn).double() * descale


def torch_attention(q8, k8, v8, ds, causal, scale, past_len):
    Q, K, V = (decoded(t, d).permute(0, 2, 1, 3) for t, d in zip((q8, k8, v8), ds))
    B, H, Lq, D = Q.shape
    Hkv, Lk = K.shape[1], K.shape[2]
    g = H // Hkv
    K = K.repeat_interleave(g, dim=1)
    V = V.repeat_interleave(g, dim=1)
    s = scale * (Q @ K.transpose(-1, -2))
    if causal:
        i = torch.arange(Lq).view(-1, 1)
        j = torch.arange(Lk).view(1, -1)
        s = s.masked_fill(~(i + past_len >= j), float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    o = torch.softmax(s, dim=-1) @ V
    return o.permute(0, 2, 1, 3).numpy(), lse.numpy(), s


CASES = [  # B, Lq, Lk, H, Hkv, D, causal, past_len, seed, qk_mult
    (1, 1, 1, 1, 1, 16, False, 0, 1, 1.0),
    (2, 37, 37, 4, 2, 16, True, 0, 2, 1.0),
    (1, 64, 64, 4, 1, 64, False, 0, 3, 3.0),
    (1, 20, 50, 2, 2, 128, True, 30, 4, 1.0),
    (2, 9, 9, 8, 2, 32, True, 0, 5, 3.0),
    (1, 12, 40, 2, 1, 64, True, -5, 6, 1.0),
]


def pin_decode(lib):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.e4m3_to_double(c, lib=lib) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def pin_torch(lib):
    for (B, Lq, Lk, H, Hkv, D, causal, past, seed, mult) in CASES:
        q8, k8, v8, ds = make_qkv_fp8(B, Lq, H, Hkv, D, seed=seed, qk_mult=mult, Lk=Lk)
        scale = 1.0 / np.sqrt(D)
        o, lse, _ = oracle.forward_fp8(q8, k8, v8, ds, causal=causal, scale=scale, past_len=past,
                                       lib=lib)
        ro, rl, _ = torch_attention(q8, k8, v8, ds, causal, scale, past)
        seen = np.isfinite(rl)
        assert np.array_equal(np.isfinite(lse), seen)
        assert np.max(np.abs(lse[seen] - rl[seen]), initial=0.0) <= TOL
        # rows that see no key: O = 0 (torch gives NaN there)
        row_seen = np.transpose(seen, (0, 2, 1))[..., None].repeat(D, axis=3)
        assert np.all(o[~row_seen] == 0.0)
        assert np.max(np.abs(o[row_seen] - ro[row_seen]), initial=0.0) <= TOL


def pin_descales(lib):
    q8, k8, v8, ds = make_qkv_fp8(2, 33, 4, 2, 64, seed=7)
    base_o, base_l, _ = oracle.forward_fp8(q8, k8, v8, ds, causal=True, lib=lib)
    scale = 1.0 / 8.0
    o2, l2, _ = oracle.forward_fp8(q8, k8, v8, (ds[0], ds[1], 2 * ds[2]), causal=True, lib=lib)
    assert np.array_equal(o2, 2 * base_o) and np.array_equal(l2, base_l)
    o3, l3, _ = oracle.forward_fp8(q8, k8, v8, (2 * ds[0], ds[1], ds[2]), causal=True,
                                   scale=scale / 2, lib=lib)
    assert np.array_equal(o3, base_o) and np.array_equal(l3, base_l)
    o4, l4, _ = oracle.forward_fp8(q8, k8, v8, (ds[0], 2 * ds[1], ds[2]), causal=True,
                                   scale=scale / 2, lib=lib)
    assert np.array_equal(o4, base_o) and np.array_equal(l4, base_l)
    # unit descales: the fp16 oracle on the same values
    q16, k16, v16 = (t.view(torch.float8_e4m3fn).half() for t in (q8, k8, v8))
    o5, l5, _ = oracle.forward_fp8(q8, k8, v8, (1.0, 1.0, 1.0), causal=True, lib=lib)
    r5, rl5 = oracle.forward(q16, k16, v16, causal=True)
    assert np.max(np.abs(o5 - r5)) <= TOL * np.max(np.abs(r5)) and np.max(np.abs(l5 - rl5)) <= TOL


def simulated_o(s_row, vals, r):
    """O of one row when each weight w_j = exp(s_j - max) is stored as the
    E4M3 rounding of 8*r*w_j (torch's cast), divided back, over the exact
    sum of the weights."""
    w = torch.exp(s_row - s_row.max())
    q = (8.0 * r * w).float().to(torch.float8_e4m3fn).double() / (8.0 * r)
    return (q @ vals) / w.sum()


def pin_bound(lib):
    rng = np.random.default_rng(11)
    worst = 0.0
    for (B, Lq, Lk, H, Hkv, D, causal, past, seed, mult) in CASES + [
            (1, 48, 300, 2, 1, 64, False, 0, 8, 3.0), (1, 16, 200, 2, 2, 32, True, 184, 9, 4.0)]:
        q8, k8, v8, ds = make_qkv_fp8(B, Lq, H, Hkv, D, seed=seed, qk_mult=mult, Lk=Lk)
        scale = 1.0 / np.sqrt(D)
        o, lse, bound = oracle.forward_fp8(q8, k8, v8, ds, causal=causal, scale=scale,
                                           past_len=past, bound_model=MODEL, lib=lib)
        _, _, s = torch_attention(q8, k8, v8, ds, causal, scale, past)
        V = decoded(v8, ds[2]).permute(0, 2, 1, 3).repeat_interleave(H // Hkv, dim=1)
        for b in range(B):
            for h in range(H):
                for i in range(Lq):
                    row = s[b, h, i]
                    keep = torch.isfinite(row)
                    if not keep.any():
                        assert np.all(bound[b, i, h] == 0.0)
                        continue
                    for r in (1.0, float(2.0 ** rng.uniform(0, np.log2(56.0)))):
                        sim = simulated_o(row[keep], V[b, h][keep], r).numpy()
                        err = np.abs(sim - o[b, i, h])
                        lim = bound[b, i, h]
                        assert np.all(err <= lim * (1 + 1e-9) + 1e-15), (b, h, i, r)
                        worst = max(worst, float(np.max(err / np.maximum(lim, 1e-300))))
    # the bound is attained to within a small factor somewhere
    assert worst > 0.25, worst
    # a row where the subnormal rounding dominates: key 0 has weight 1 and
    # V = 0; 100 keys have weight w = 1.4 * 2^-12 (8w = 1.4 * 2^-9, just above
    # E4M3's smallest subnormal, rounded down by 29 %) and V = 1, so every
    # rounding error has the same sign
    n, D = 100, 16
    q8 = torch.zeros((1, 1, 1, D), dtype=torch.uint8)
    q8[0, 0, 0, 0] = 0x38  # 1.0
    k8 = torch.zeros((1, n + 1, 1, D), dtype=torch.uint8)
    k8[0, 1:, 0, 0] = 0xB8  # -1.0
    v8 = torch.zeros((1, n + 1, 1, D), dtype=torch.uint8)
    v8[0, 1:, 0, :] = 0x38
    scale = -float(np.log(1.4 * 2.0 ** -12))  # s_0 = 0, s_j = -scale
    o, _, bound = oracle.forward_fp8(q8, k8, v8, (1.0, 1.0, 1.0), scale=scale,
                                     bound_model=MODEL, lib=lib)
    srow = torch.tensor([0.0] + [-scale] * n, dtype=torch.float64)
    sim = simulated_o(srow, decoded(v8, 1.0)[0, :, 0, :], 1.0).numpy()
    err = np.abs(sim - o[0, 0, 0])
    assert np.all(err <= bound[0, 0, 0] * (1 + 1e-9)) and np.all(err > 0.5 * bound[0, 0, 0])


PINS = [pin_decode, pin_torch, pin_descales, pin_bound]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_fp8_oracle_pin(pin):
    pin(None)


MUTANTS = {
    "exponent bias 8": ("mag = ldexp(1.0 + (double)frac / 8.0, e - 7);",
                        "mag = ldexp(1.0 + (double)frac / 8.0, e - 8);"),
    "subnormal scale": ("mag = ldexp((double)frac, -9); /* 2^-6 * frac / 2^3 */",
                        "mag = ldexp((double)frac, -10);"),
    "q descale dropped": ("dot += (p->qd * g_e4m3[p->q[q8_index(p, b, i, h, d)]]) *",
                          "dot += (g_e4m3[p->q[q8_index(p, b, i, h, d)]]) *"),
    "k descale dropped": ("(p->kd * g_e4m3[p->k[kv8_index(p, b, j, hk, d)]]);",
                          "(g_e4m3[p->k[kv8_index(p, b, j, hk, d)]]);"),
    "v descale dropped": ("double val = p->vd * g_e4m3[p->v[kv8_index(p, b, j, hk, d)]];",
                          "double val = g_e4m3[p->v[kv8_index(p, b, j, hk, d)]];"),
    "bound: no absolute floor": (
        "double e = s[j] >= p->b_floor ? p->b_rel * s[j] : (s[j] < p->b_abs ? s[j] : p->b_abs);",
        "double e = p->b_rel * s[j];"),
    "bound: signed V": ("err += e * fabs(val);", "err += e * val;"),
    "bound: unnormalised": ("if (bound_row) bound_row[d] = err / z;",
                            "if (bound_row) bound_row[d] = err / (z * z);"),
    "fp8 mask ignores past_len": ("long n = (long)i + p->past_len + 1;\n    return n < 0 ? 0 : (n > p->Lk ? p->Lk : (int)n);\n}\n\n/* One output row on the decoded",
                                  "long n = (long)i + 1;\n    return n < 0 ? 0 : (n > p->Lk ? p->Lk : (int)n);\n}\n\n/* One output row on the decoded"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_fp8_pins_reject_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = oracle.source_text()
    assert src.count(old) == 1, f"mutation site for '{name}' not found once"
    lib = oracle.build_variant(src.replace(old, new, 1), str(tmp_path / "mutant.so"))
    failed = []
    for pin in PINS:
        try:
            with np.errstate(invalid="ignore", over="ignore"):
                pin(lib)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin rejects the planted mistake '{name}'"
