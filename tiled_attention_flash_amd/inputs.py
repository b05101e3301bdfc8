"""Seeded synthetic inputs and the workload registry.

This module is the only code that both the HIP path's tests/benchmark and the
fp64 oracle consume: it draws the random Q/K/V and nothing else.  It holds none
of the attention arithmetic.

Recipe (every workload): a CPU ``torch.Generator`` seeded with ``seed`` draws,
in this order, Q ``[B, Lq, H, D]``, K ``[B, Lk, Hkv, D]`` and V ``[B, Lk, Hkv, D]``
as i.i.d. N(0, 1) float32 (Lq = Lk = L unless a workload says otherwise); the
long-sequence workload then multiplies Q and K by 3 in float32 to widen the
softmax's logit range; finally all three are
rounded to float16 (round-to-nearest-even).  The same float16 tensors go to the
oracle (host) and to the GPU.  Layout is BSHD, contiguous.  The scale is
1/sqrt(D), the value the TileLang AMD page sets up at kernel entry.

FP8 workloads draw Q, K, V the same way (float32, before any rounding) and
store each tensor as OCP E4M3 codes with one descale factor per tensor:
descale = max|x| / 448 (448 is E4M3's largest finite value), rounded to
float32, and code = E4M3(x / descale) by torch's float8_e4m3fn cast
(round-to-nearest-even), the quotient clamped to +-448 first.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Hkv: int
    L: int
    D: int
    causal: bool
    qk_mult: float = 1.0  # Q and K are multiplied by this before the fp16 cast
    Lk: int | None = None  # key rows; None = L (queries and keys equally long)
    path: str = "forward"  # entry point: "forward", "splitkv", "backward" or "fp8"

    @property
    def Lq(self) -> int:
        return self.L

    @property
    def keys(self) -> int:
        return self.L if self.Lk is None else self.Lk

    @property
    def past_len(self) -> int:
        """Key position of query row 0: the queries are the last L of the keys."""
        return self.keys - self.L

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def flops(self) -> float:
        """Attention forward work: two contractions of 2*D flops per (query,
        key) pair.  Equal lengths: 4*B*H*L^2*D, counted as exactly half when
        causal.  Queries after past_len cached keys, causal: the rectangle of
        past keys plus half of the Lq x Lq square."""
        pairs = float(self.L) * self.keys
        if self.causal:
            pairs = float(self.L) * self.past_len + self.L * self.L / 2
        return 4.0 * self.B * self.H * self.D * pairs

    @property
    def step_flops(self) -> float:
        """Flops of one step of the workload's path: the forward's, or for
        the backward its five products (S recomputed, dP, dV, dK, dQ) of
        2*D flops per (query, key) pair: 2.5 times the forward's."""
        return 2.5 * self.flops if self.path == "backward" else self.flops

    @property
    def algorithmic_bytes(self) -> int:
        """Each tensor moved once: Q and O (fp16), K and V (fp16), LSE (fp32);
        with fp8 inputs Q, K, V take one byte per element."""
        ein = 1 if self.path == "fp8" else 2
        q = self.B * self.L * self.H * self.D
        kv = 2 * self.B * self.keys * self.Hkv * self.D * ein
        return q * ein + q * 2 + kv + self.B * self.H * self.L * 4


# The workloads the method is measured on (B, H, Hkv, L, D, causal[, qk_mult, Lk]).
WORKLOADS = {
    "tiny-mha-L128-d64": Workload("tiny-mha-L128-d64", 1, 2, 2, 128, 64, False),
    "tiny-mha-L128-d64-causal": Workload("tiny-mha-L128-d64-causal", 1, 2, 2, 128, 64, True),
    "mha-b8-h32-L1024-d64": Workload("mha-b8-h32-L1024-d64", 8, 32, 32, 1024, 64, False),
    "mha-b8-h32-L1024-d64-causal": Workload("mha-b8-h32-L1024-d64-causal", 8, 32, 32, 1024, 64, True),
    "mha-b8-h32-L4096-d128": Workload("mha-b8-h32-L4096-d128", 8, 32, 32, 4096, 128, False),
    "mha-b8-h32-L4096-d128-causal": Workload("mha-b8-h32-L4096-d128-causal", 8, 32, 32, 4096, 128, True),
    # the same tokens as B=8 L=4096 at half the length: the causal instance
    # with four wavefronts per workgroup (fewer than 4096 keys)
    "mha-b16-h32-L2048-d128-causal": Workload("mha-b16-h32-L2048-d128-causal", 16, 32, 32, 2048, 128, True),
    "gqa-b2-h32-kv8-L8192-d128-causal": Workload("gqa-b2-h32-kv8-L8192-d128-causal", 2, 32, 8, 8192, 128, True),
    "mha-b1-h32-L16384-d128-causal-qk3": Workload("mha-b1-h32-L16384-d128-causal-qk3", 1, 32, 32, 16384, 128, True, 3.0),
    # 1024 new queries after 3072 cached positions (a prefill continuing a prefix)
    "prefill-b8-h32-q1024-kv4096-d128-causal": Workload(
        "prefill-b8-h32-q1024-kv4096-d128-causal", 8, 32, 32, 1024, 128, True, 1.0, 4096),
    # one new query per sequence after a long cache (decoding), by key splits
    "decode-b8-h32-kv8-q1-k32768-d128-causal": Workload(
        "decode-b8-h32-kv8-q1-k32768-d128-causal", 8, 32, 8, 1, 128, True, 1.0, 32768, "splitkv"),
    "decode-b8-h32-q1-k4096-d128-causal": Workload(
        "decode-b8-h32-q1-k4096-d128-causal", 8, 32, 32, 1, 128, True, 1.0, 4096, "splitkv"),
    # backward: the backward page's workload (LLaMA-7B head shape) and the long shape
    "bwd-b8-h32-L1024-d64": Workload("bwd-b8-h32-L1024-d64", 8, 32, 32, 1024, 64, False,
                                     path="backward"),
    "bwd-b8-h32-L1024-d64-causal": Workload("bwd-b8-h32-L1024-d64-causal", 8, 32, 32, 1024, 64,
                                            True, path="backward"),
    "bwd-b8-h32-L4096-d128": Workload("bwd-b8-h32-L4096-d128", 8, 32, 32, 4096, 128, False,
                                      path="backward"),
    "bwd-b8-h32-L4096-d128-causal": Workload("bwd-b8-h32-L4096-d128-causal", 8, 32, 32, 4096, 128,
                                             True, path="backward"),
    # fp8 (E4M3) inputs, fp16 output
    "fp8-mha-b8-h32-L4096-d128": Workload("fp8-mha-b8-h32-L4096-d128", 8, 32, 32, 4096, 128, False,
                                          path="fp8"),
    "fp8-mha-b8-h32-L4096-d128-causal": Workload("fp8-mha-b8-h32-L4096-d128-causal", 8, 32, 32,
                                                 4096, 128, True, path="fp8"),
}

HEADLINE = "mha-b8-h32-L4096-d128"

E4M3_MAX = 448.0


def make_qkv(B: int, L: int, H: int, Hkv: int, D: int, seed: int = 0, qk_mult: float = 1.0,
             device: str | torch.device = "cpu", Lk: int | None = None):
    """Seeded fp16 Q, K, V (BSHD, contiguous) following the recipe above;
    K and V have Lk rows (default L)."""
    Lk = L if Lk is None else Lk
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn((B, L, H, D), generator=g, dtype=torch.float32)
    k = torch.randn((B, Lk, Hkv, D), generator=g, dtype=torch.float32)
    v = torch.randn((B, Lk, Hkv, D), generator=g, dtype=torch.float32)
    if qk_mult != 1.0:
        q = q * qk_mult
        k = k * qk_mult
    q, k, v = q.half(), k.half(), v.half()
    if str(device) != "cpu":
        q, k, v = q.to(device), k.to(device), v.to(device)
    return q, k, v


def make_qkvdo(B: int, L: int, H: int, Hkv: int, D: int, seed: int = 0, qk_mult: float = 1.0,
               device: str | torch.device = "cpu"):
    """Backward-pass inputs: Q, K, V exactly as make_qkv draws them, then,
    from the same generator, the output gradient dO [B, L, H, D] as i.i.d.
    N(0, 1) float32 rounded to float16."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn((B, L, H, D), generator=g, dtype=torch.float32)
    k = torch.randn((B, L, Hkv, D), generator=g, dtype=torch.float32)
    v = torch.randn((B, L, Hkv, D), generator=g, dtype=torch.float32)
    do = torch.randn((B, L, H, D), generator=g, dtype=torch.float32)
    if qk_mult != 1.0:
        q = q * qk_mult
        k = k * qk_mult
    out = [t.half() for t in (q, k, v, do)]
    if str(device) != "cpu":
        out = [t.to(device) for t in out]
    return tuple(out)


def _to_e4m3(x: torch.Tensor):
    """float32 tensor -> (E4M3 codes as uint8, float32 descale) per the recipe."""
    amax = float(x.abs().max()) if x.numel() else 0.0
    descale = float(torch.tensor(amax / E4M3_MAX if amax > 0 else 1.0, dtype=torch.float32))
    codes = (x / descale).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, descale


def make_qkv_fp8(B: int, L: int, H: int, Hkv: int, D: int, seed: int = 0, qk_mult: float = 1.0,
                 device: str | torch.device = "cpu", Lk: int | None = None):
    """Seeded fp8 Q, K, V: the float32 draws of make_qkv (same generator and
    order, times qk_mult for Q and K), stored as E4M3 codes (uint8 tensors,
    BSHD) with one descale per tensor.  Returns (q8, k8, v8, (qd, kd, vd))."""
    Lk = L if Lk is None else Lk
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn((B, L, H, D), generator=g, dtype=torch.float32)
    k = torch.randn((B, Lk, Hkv, D), generator=g, dtype=torch.float32)
    v = torch.randn((B, Lk, Hkv, D), generator=g, dtype=torch.float32)
    if qk_mult != 1.0:
        q = q * qk_mult
        k = k * qk_mult
    (q8, qd), (k8, kd), (v8, vd) = _to_e4m3(q), _to_e4m3(k), _to_e4m3(v)
    if str(device) != "cpu":
        q8, k8, v8 = q8.to(device), k8.to(device), v8.to(device)
    return q8, k8, v8, (qd, kd, vd)


def workload_inputs(w: Workload, seed: int = 0, device: str | torch.device = "cpu"):
    if w.path == "fp8":
        return make_qkv_fp8(w.B, w.L, w.H, w.Hkv, w.D, seed=seed, qk_mult=w.qk_mult,
                            device=device, Lk=w.keys)
    return make_qkv(w.B, w.L, w.H, w.Hkv, w.D, seed=seed, qk_mult=w.qk_mult, device=device,
                    Lk=w.keys)
