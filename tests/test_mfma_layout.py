"""Lane layouts of the gfx950 instructions the attention kernel is built on,
checked on the GPU against host arithmetic (all values exact in fp16/fp32).

The kernel assumes, for v_mfma_f32_32x32x16_f16 (D = A[32x16] . B[16x32]):
  lane l holds A[l % 32][8 * (l // 32) + i]          for i in 0..7
  lane l holds B[8 * (l // 32) + i][l % 32]          for i in 0..7
  lane l holds D[8 * I + 4 * (l // 32) + J][l % 32]  in register 4 * I + J
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def probe():
    from tests import probe_lib
    return probe_lib.load()


def test_mfma_32x32x16_f16_layout(probe):
    rng = np.random.default_rng(0)
    A = rng.integers(-4, 5, size=(32, 16)).astype(np.float16)
    B = rng.integers(-4, 5, size=(16, 32)).astype(np.float16)
    a_lanes = np.zeros((64, 8), np.float16)
    b_lanes = np.zeros((64, 8), np.float16)
    for l in range(64):
        for i in range(8):
            a_lanes[l, i] = A[l % 32, 8 * (l // 32) + i]
            b_lanes[l, i] = B[8 * (l // 32) + i, l % 32]
    a = torch.from_numpy(a_lanes).cuda()
    b = torch.from_numpy(b_lanes).cuda()
    c = torch.zeros((64, 16), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert probe.probe_mfma_32x32x16_f16(a.data_ptr(), b.data_ptr(), c.data_ptr(), s) == 0
    torch.cuda.synchronize()
    got = c.cpu().numpy()
    want = A.astype(np.float32) @ B.astype(np.float32)
    for l in range(64):
        for I in range(4):
            for J in range(4):
                assert got[l, 4 * I + J] == want[8 * I + 4 * (l // 32) + J, l % 32], (l, I, J)


def test_permlane32_swap_pairs_halves(probe):
    x = torch.arange(64, dtype=torch.float32, device="cuda")
    out = torch.zeros((2, 64), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert probe.probe_permlane32_swap(x.data_ptr(), out.data_ptr(), s) == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    for l in range(64):
        assert sorted((o[0, l], o[1, l])) == sorted((float(l), float(l ^ 32))), l


def test_fp16_pack_rounds_to_nearest_even(probe):
    rng = np.random.default_rng(1)
    x = rng.normal(size=4096).astype(np.float32) * 3
    # exact ties between two fp16 neighbours, both parities
    base = rng.normal(size=512).astype(np.float16).astype(np.float32)
    ulp = np.spacing(np.abs(base).astype(np.float16)).astype(np.float32)
    x = np.concatenate([x, base + ulp / 2, base - ulp / 2]).astype(np.float32)
    x = x[: len(x) // 2 * 2]
    xt = torch.from_numpy(x).cuda()
    y = torch.zeros(len(x), dtype=torch.float16, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert probe.probe_cvt_f16(xt.data_ptr(), y.data_ptr(), len(x), s) == 0
    torch.cuda.synchronize()
    want = x.astype(np.float16)  # numpy rounds to nearest even
    assert np.array_equal(y.cpu().numpy().view(np.uint16), want.view(np.uint16))
