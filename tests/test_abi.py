"""The C ABI of libfa.so, on the host: it loads, exports every symbol that
include/fa.h declares, and rejects every invalid argument with the documented
status before any HIP call (fake, never-dereferenced addresses are passed, so
a launch would be a bug)."""
import math
import os
import re
import subprocess

import pytest

import tiled_attention_flash_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

# fake device addresses, 256-byte aligned, far apart (never dereferenced)
Q, K, V, O, LSE = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000
OK_ARGS = dict(q=Q, k=K, v=V, o=O, lse=LSE, B=1, L=128, H=2, Hkv=2, D=64, causal=0,
               scale=0.125, stream=None)


def call(**kw):
    a = dict(OK_ARGS)
    a.update(kw)
    return fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["L"], a["H"], a["Hkv"],
                     a["D"], a["causal"], a["scale"], a["stream"])


def declared_symbols():
    text = open(HEADER).read()
    return re.findall(r"^FA_API\s+[\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)


def test_library_loads_and_exports_header_symbols():
    lib = fa.library()
    names = declared_symbols()
    assert set(names) == {"fa_fwd", "fa_fwd_kv", "fa_fwd_fp8", "fa_fwd_splitkv",
                          "fa_fwd_splitkv_noalloc", "fa_splitkv_splits",
                          "fa_splitkv_workspace_bytes", "fa_bwd", "fa_bwd_kv", "fa_status_string",
                          "fa_abi_version"}
    out = subprocess.run(["nm", "-D", "--defined-only", fa.library_path()], check=True,
                         stdout=subprocess.PIPE, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)
    # nothing beyond the declared C ABI leaks out of the library
    assert exported == set(names)
    assert lib.fa_abi_version() == 7


def test_status_strings():
    for code, name in fa.STATUS.items():
        assert fa.fa_status_string(code).startswith(name)
    assert fa.fa_status_string(12345) == "FA_ERR_UNKNOWN"


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(o=None), 1),
    (dict(B=-1), 2), (dict(L=-5), 2), (dict(D=-64), 2), (dict(H=-2), 2),
    (dict(B=1 << 30, L=1 << 30, H=1 << 30, Hkv=1 << 30, D=128), 2),
    (dict(H=3, Hkv=2), 3), (dict(Hkv=0), 3), (dict(H=0), 3), (dict(H=4, Hkv=8), 3),
    (dict(D=96), 4), (dict(D=32), 4), (dict(D=256), 4), (dict(D=0), 4),
    (dict(scale=0.0), 5), (dict(scale=-0.125), 5), (dict(scale=math.nan), 5),
    (dict(scale=math.inf), 5),
    (dict(q=Q + 8), 6), (dict(k=K + 2), 6), (dict(v=V + 4), 6), (dict(o=O + 1), 6),
    (dict(lse=LSE + 2), 6),
    (dict(o=Q), 7), (dict(o=K + 64), 7), (dict(lse=V + 256), 7), (dict(lse=O + 16), 7),
    (dict(o=Q - 1024), 7),
])
def test_invalid_arguments_rejected_without_launch(kw, status):
    assert call(**kw) == status


def test_empty_problems_are_noops():
    assert call(B=0, q=None, k=None, v=None, o=None, lse=None) == 0
    assert call(L=0, q=None, k=None, v=None, o=None, lse=None) == 0
    # still validated
    assert call(B=0, D=96) == 4
    assert call(L=0, H=3, Hkv=2) == 3


def test_binding_rejects_host_tensors():
    import torch
    q = torch.zeros(1, 8, 1, 64, dtype=torch.float16)
    with pytest.raises(TypeError):
        fa.forward(q, q, q)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(fa, "_lib", None)
    monkeypatch.setattr(fa, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        fa.library()


KV_ARGS = dict(q=Q, k=K, v=V, o=O, lse=LSE, B=1, Lq=64, Lk=192, H=2, Hkv=2, D=64, causal=1,
               past_len=128, scale=0.125, stream=None)


def call_kv(**kw):
    a = dict(KV_ARGS)
    a.update(kw)
    return fa.fa_fwd_kv(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Lq"], a["Lk"],
                        a["H"], a["Hkv"], a["D"], a["causal"], a["past_len"], a["scale"],
                        a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(k=None), 1), (dict(v=None), 1),
    (dict(Lq=-1), 2), (dict(Lk=-1), 2), (dict(Lq=(1 << 30) + 1), 2), (dict(Lk=(1 << 30) + 1), 2),
    (dict(past_len=(1 << 30) + 1), 2), (dict(past_len=-(1 << 30) - 1), 2),
    (dict(H=3, Hkv=2), 3), (dict(D=96), 4), (dict(scale=0.0), 5),
    (dict(k=K + 8), 6), (dict(lse=LSE + 1), 6),
    # o (Lq rows) overlapping the longer k/v (Lk rows), and k's range reaching o
    (dict(o=K + 64 * 2 * 64 * 2), 7), (dict(k=O - 64 * 2 * 64 * 2), 7),
])
def test_kv_invalid_arguments_rejected_without_launch(kw, status):
    assert call_kv(**kw) == status


def test_kv_empty_problems_are_noops():
    assert call_kv(B=0, q=None, k=None, v=None, o=None, lse=None) == 0
    assert call_kv(Lq=0, q=None, k=None, v=None, o=None, lse=None) == 0
    assert call_kv(Lq=0, D=96) == 4
    # past_len is range-checked even where the mask is off
    assert call_kv(causal=0, past_len=(1 << 31) - 1) == 2


def test_binding_routes_unequal_lengths_to_the_kv_entry_point(monkeypatch):
    """forward() marshals Lq != Lk (or an explicit past_len) to fa_fwd_kv with
    the default offset Lk - Lq, and equal lengths to fa_fwd; nothing is
    launched here (the entry points are replaced)."""
    torch = pytest.importorskip("torch")
    seen = {}

    class FakeTensor:
        def __init__(self, shape):
            self.shape = shape
            self.dtype = torch.float16
            self.is_cuda = True
            self.device = "dev"

        def dim(self):
            return 4

        def is_contiguous(self):
            return True

        def data_ptr(self):
            return 0x1000

    monkeypatch.setattr(fa, "fa_fwd", lambda *a: seen.setdefault("fwd", a) and 0)
    monkeypatch.setattr(fa, "fa_fwd_kv", lambda *a: seen.setdefault("kv", a) and 0)
    monkeypatch.setattr(torch, "Tensor", FakeTensor)

    class Dev:
        def __init__(self, d):
            pass

        def __enter__(self):
            return self

        def __exit__(self, *e):
            return False

    class Stream:
        cuda_stream = None

    monkeypatch.setattr(torch.cuda, "device", Dev)
    monkeypatch.setattr(torch.cuda, "current_stream", lambda d=None: Stream())
    q, k = FakeTensor((1, 16, 2, 64)), FakeTensor((1, 48, 2, 64))
    o = FakeTensor((1, 16, 2, 64))
    fa.forward(q, k, k, causal=True, out=o, with_lse=False)
    assert "kv" in seen and "fwd" not in seen
    args = seen["kv"]
    assert args[5:13] == (1, 16, 48, 2, 2, 64, True, 32)  # B, Lq, Lk, H, Hkv, D, causal, past_len
    seen.clear()
    fa.forward(q, q, q, causal=True, out=o, with_lse=False)
    assert "fwd" in seen and "kv" not in seen


# ------------------------------------------------------------ split-KV ABI

WS = 0x60000000
SPLIT_ARGS = dict(KV_ARGS, Lq=4, Lk=4096, past_len=4092, n_splits=8, workspace=WS,
                  workspace_bytes=1 << 20)


def call_split(**kw):
    a = dict(SPLIT_ARGS)
    a.update(kw)
    return fa.fa_fwd_splitkv(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Lq"], a["Lk"],
                             a["H"], a["Hkv"], a["D"], a["causal"], a["past_len"], a["scale"],
                             a["n_splits"], a["workspace"], a["workspace_bytes"], a["stream"])


def test_splitkv_workspace_bytes():
    # fp32 partial outputs [B][H][Lq][n][D] then partial LSEs [B][H][Lq][n]
    assert fa.fa_splitkv_workspace_bytes(2, 3, 4, 128, 5) == 2 * 3 * 4 * 5 * (128 + 1) * 4
    assert fa.fa_splitkv_workspace_bytes(1, 1, 1, 64, 1) == 65 * 4
    assert fa.fa_splitkv_workspace_bytes(0, 1, 1, 64, 1) == 0
    for bad in [dict(D=96), dict(n=0), dict(n=4097), dict(B=-1)]:
        a = dict(B=1, Lq=1, H=1, D=64, n=1)
        a.update(bad)
        assert fa.fa_splitkv_workspace_bytes(a["B"], a["Lq"], a["H"], a["D"], a["n"]) == -1
    big = 1 << 30
    assert fa.fa_splitkv_workspace_bytes(big, big, big, 128, 4096) == -1  # int64 overflow


def _splits_model(B, Lq, Lk, H, Hkv, D, causal, past_len):
    """The documented choice: minimise rounds * (blocks per split + 2) over
    1..min(64, blocks // 4) splits, rounds of 256 * (160 KiB // (384 * D))
    resident work items; ties to fewer splits."""
    if B <= 0 or Lq <= 0 or H <= 0 or Hkv <= 0 or H % Hkv or D not in (64, 128):
        return 1
    rows = Lq * (H // Hkv)
    base = B * Hkv * ((rows + 31) // 32)
    vis = Lk if not causal else max(0, min(Lk, Lq + past_len))
    blocks = (vis + 31) // 32
    slots = 256 * ((160 * 1024) // (384 * D))
    cap = max(1, min(64, blocks // 4))
    costs = [((base * n + slots - 1) // slots) * (-(-blocks // n) + 2) for n in range(1, cap + 1)]
    return 1 + costs.index(min(costs))


def test_splitkv_default_splits():
    # hand-checked: 768 resident items at D = 128; 64 items per split -> 12 splits, one round
    assert fa.fa_splitkv_splits(8, 1, 32768, 32, 8, 128, 1, 32767) == 12
    # 256 items, 128 blocks: three splits fill one round with the least work per split
    assert fa.fa_splitkv_splits(8, 1, 4096, 32, 32, 128, 1, 4095) == 3
    # one query row of one K/V head over 2^17 keys: capped at 64 splits
    assert fa.fa_splitkv_splits(1, 1, 131072, 32, 8, 128, 1, 131071) == 64
    # 8 blocks: at most 2 splits of >= 4 blocks; 2 blocks: 1
    assert fa.fa_splitkv_splits(1, 1, 256, 8, 8, 128, 0, 0) == 2
    assert fa.fa_splitkv_splits(1, 1, 64, 8, 8, 128, 0, 0) == 1
    # causal: only keys up to the last query's position count
    assert fa.fa_splitkv_splits(1, 1, 1 << 20, 1, 1, 64, 1, 4095) == 32
    assert fa.fa_splitkv_splits(0, 1, 100, 1, 1, 64, 0, 0) == 1
    for B in (1, 2, 8, 32):
        for Lq in (1, 3, 16, 64):
            for Lk in (100, 4096, 32768, 200000):
                for H, Hkv in ((32, 8), (32, 32), (8, 1)):
                    for D in (64, 128):
                        for causal in (0, 1):
                            args = (B, Lq, Lk, H, Hkv, D, causal, Lk - Lq)
                            assert fa.fa_splitkv_splits(*args) == _splits_model(*args), args


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(Lk=-1), 2), (dict(H=3, Hkv=2), 3),
    (dict(D=96), 4), (dict(scale=math.nan), 5), (dict(v=V + 2), 6),
    (dict(n_splits=-1), 2), (dict(n_splits=4097), 2),
    (dict(workspace=None), 10), (dict(workspace=WS + 8), 10),
    (dict(workspace_bytes=4 * 2 * 8 * 65 * 4 - 1), 10),
    (dict(workspace=Q), 7), (dict(workspace=O - 1024), 7), (dict(workspace=LSE + 16), 7),
    (dict(workspace=K + 4096 * 2 * 64 * 2 - 16), 7),
])
def test_splitkv_invalid_arguments_rejected_without_launch(kw, status):
    assert call_split(**kw) == status


def test_splitkv_exact_workspace_size_accepted_by_validation():
    """The documented size is enough: validation passes it (a NULL stream and
    fake pointers would then reach the launch, so only the checks before it
    are exercised, via a size one byte short being rejected above and the
    empty problem here)."""
    need = fa.fa_splitkv_workspace_bytes(1, 4, 2, 64, 8)
    assert need == 4 * 2 * 8 * 65 * 4
    assert call_split(Lq=0, workspace=None, workspace_bytes=0) == 0
    assert call_split(B=0, workspace=None, workspace_bytes=0) == 0
    assert call_split(B=0, n_splits=5000) == 2  # still validated


def call_noalloc(**kw):
    a = dict(SPLIT_ARGS)
    a.update(kw)
    return fa.fa_fwd_splitkv_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Lq"],
                                     a["Lk"], a["H"], a["Hkv"], a["D"], a["causal"],
                                     a["past_len"], a["scale"], a["n_splits"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(Lk=-1), 2), (dict(H=3, Hkv=2), 3),
    (dict(D=96), 4), (dict(scale=math.nan), 5), (dict(v=V + 2), 6), (dict(o=Q), 7),
    (dict(n_splits=-1), 2), (dict(n_splits=4097), 2),
])
def test_splitkv_noalloc_invalid_arguments_rejected_without_launch(kw, status):
    assert call_noalloc(**kw) == status


def test_splitkv_noalloc_rejects_problems_beyond_its_scratch():
    """Partial results larger than the static scratch (16 MiB) are refused
    with FA_ERR_SCRATCH before any HIP call; the limit is exact."""
    assert fa.SPLITKV_SCRATCH_BYTES == 16 << 20
    # B*H*Lq*n*(D+1)*4 bytes: 8 query rows of 2 heads over 4096 splits need 17 MB
    assert fa.fa_splitkv_workspace_bytes(1, 8, 2, 64, 4096) > fa.SPLITKV_SCRATCH_BYTES
    assert call_noalloc(Lq=8, past_len=4088, n_splits=4096) == 11
    # the largest n_splits that still fits a B=8, H=32, Lq=1, D=128 decode step
    need = lambda n: fa.fa_splitkv_workspace_bytes(8, 1, 32, 128, n)  # noqa: E731
    n_fit = max(n for n in range(1, 4097) if need(n) <= fa.SPLITKV_SCRATCH_BYTES)
    assert need(n_fit + 1) > fa.SPLITKV_SCRATCH_BYTES
    big = dict(SPLIT_ARGS, B=8, H=32, Hkv=8, Lq=1, D=128, past_len=4095)
    assert call_noalloc(**dict(big, n_splits=n_fit + 1)) == 11
    assert "FA_ERR_SCRATCH" in fa.fa_status_string(11)


def test_splitkv_noalloc_empty_problems_are_noops():
    assert call_noalloc(Lq=0) == 0
    assert call_noalloc(B=0) == 0
    assert call_noalloc(B=0, n_splits=5000) == 2  # still validated


# ------------------------------------------------------------ backward ABI

DO, DELTA, DQ, DK, DV = 0x70000000, 0x80000000, 0x90000000, 0xA0000000, 0xB0000000
BWD_ARGS = dict(q=Q, k=K, v=V, o=O, dout=DO, lse=LSE, delta=DELTA, dq=DQ, dk=DK, dv=DV, B=1, L=128,
                H=2, Hkv=2, D=64, causal=0, scale=0.125, stream=None)


def call_bwd(**kw):
    a = dict(BWD_ARGS)
    a.update(kw)
    return fa.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["delta"], a["dq"],
                     a["dk"], a["dv"], a["B"], a["L"], a["H"], a["Hkv"], a["D"], a["causal"],
                     a["scale"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(dout=None), 1), (dict(lse=None), 1),
    (dict(delta=None), 1), (dict(dq=None), 1), (dict(dk=None), 1), (dict(dv=None), 1),
    (dict(L=-1), 2), (dict(L=(1 << 30) + 1), 2), (dict(H=3, Hkv=2), 3), (dict(D=96), 4),
    (dict(scale=0.0), 5), (dict(dout=DO + 8), 6), (dict(delta=DELTA + 2), 6), (dict(dk=DK + 4), 6),
    (dict(dq=Q), 7), (dict(dk=DV), 7), (dict(delta=LSE), 7), (dict(dv=O + 64), 7),
    (dict(dq=DO - 1024), 7), (dict(delta=DQ + 256), 7),
    # 256 rows of a 32768-head, D = 128 tensor span 2 GiB: tile offsets would not fit 32 bits
    (dict(H=32768, Hkv=32768, D=128, L=1), 2),
])
def test_bwd_invalid_arguments_rejected_without_launch(kw, status):
    assert call_bwd(**kw) == status


def test_bwd_empty_problems_are_noops():
    nulls = dict(q=None, k=None, v=None, o=None, dout=None, lse=None, delta=None, dq=None,
                 dk=None, dv=None)
    assert call_bwd(B=0, **nulls) == 0
    assert call_bwd(L=0, **nulls) == 0
    assert call_bwd(L=0, D=96) == 4


BWD_KV_ARGS = dict(BWD_ARGS, Lq=100, Lk=300, past_len=200)
del BWD_KV_ARGS["L"]


def call_bwd_kv(**kw):
    a = dict(BWD_KV_ARGS)
    a.update(kw)
    return fa.fa_bwd_kv(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["delta"], a["dq"],
                        a["dk"], a["dv"], a["B"], a["Lq"], a["Lk"], a["H"], a["Hkv"], a["D"],
                        a["causal"], a["past_len"], a["scale"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(dout=None), 1), (dict(dq=None), 1), (dict(k=None), 1), (dict(dv=None), 1),
    (dict(Lq=-1), 2), (dict(Lk=-1), 2), (dict(Lk=(1 << 30) + 1), 2), (dict(past_len=(1 << 30) + 1), 2),
    (dict(past_len=-(1 << 30) - 1), 2), (dict(H=4, Hkv=3), 3), (dict(D=32), 4), (dict(scale=-1.0), 5),
    (dict(dk=DK + 4), 6), (dict(dq=Q), 7), (dict(dk=DV), 7),
    # rows with no keys need no k, v, dk, dv -- but q-side pointers are still required
    (dict(Lk=0, k=None, v=None, dk=None, dv=None, lse=None), 1),
    # keys with no rows need no q-side pointers -- but k-side pointers are still required
    (dict(Lq=0, q=None, o=None, dout=None, lse=None, delta=None, dq=None, dk=None), 1),
])
def test_bwd_kv_invalid_arguments_rejected_without_launch(kw, status):
    assert call_bwd_kv(**kw) == status


def test_bwd_kv_empty_problems_are_noops():
    nulls = dict(q=None, k=None, v=None, o=None, dout=None, lse=None, delta=None, dq=None,
                 dk=None, dv=None)
    assert call_bwd_kv(B=0, **nulls) == 0
    assert call_bwd_kv(Lq=0, Lk=0, **nulls) == 0
    assert call_bwd_kv(Lq=0, Lk=0, D=96) == 4


# ------------------------------------------------------------ fp8 forward ABI

FP8_ARGS = dict(q=Q, k=K, v=V, o=O, lse=LSE, B=1, Lq=128, Lk=128, H=2, Hkv=2, D=64, causal=0,
                past_len=0, scale=0.125, qd=0.01, kd=0.02, vd=0.03, stream=None)
Q8_BYTES = 128 * 2 * 64  # one byte per element


def call_fp8(**kw):
    a = dict(FP8_ARGS)
    a.update(kw)
    return fa.fa_fwd_fp8(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Lq"], a["Lk"], a["H"],
                         a["Hkv"], a["D"], a["causal"], a["past_len"], a["scale"], a["qd"], a["kd"],
                         a["vd"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(v=None), 1), (dict(o=None), 1),
    (dict(B=-1), 2), (dict(Lk=(1 << 30) + 1), 2), (dict(past_len=-(1 << 30) - 1), 2),
    (dict(H=3, Hkv=2), 3), (dict(D=96), 4),
    (dict(scale=0.0), 5), (dict(qd=0.0), 5), (dict(kd=-1.0), 5), (dict(vd=math.nan), 5),
    (dict(qd=math.inf), 5), (dict(scale=1e30, qd=1e30, kd=1e30), 5),
    (dict(q=Q + 8), 6), (dict(k=K + 4), 6), (dict(o=O + 2), 6), (dict(lse=LSE + 1), 6),
    # q, k, v span one byte per element, o two
    (dict(o=Q + Q8_BYTES - 16), 7), (dict(o=K - 2 * Q8_BYTES + 16), 7), (dict(lse=V + 16), 7),
    (dict(lse=O + 2 * Q8_BYTES - 16), 7),
])
def test_fp8_invalid_arguments_rejected_without_launch(kw, status):
    assert call_fp8(**kw) == status


def test_fp8_empty_problems_are_noops():
    assert call_fp8(B=0, q=None, k=None, v=None, o=None, lse=None) == 0
    assert call_fp8(Lq=0, q=None, k=None, v=None, o=None, lse=None) == 0
    assert call_fp8(B=0, qd=0.0) == 5  # still validated
    assert call_fp8(Lq=0, D=96) == 4
