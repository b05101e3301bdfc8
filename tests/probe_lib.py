"""Builds and loads the test-only probe library (tests/csrc/mfma_probe.hip)."""
from __future__ import annotations

import ctypes
import os

from tiled_attention_flash_amd import build as fa_build

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "mfma_probe.hip")
LIB = os.path.join(HERE, "csrc", "libmfma_probe.so")


def build() -> str:
    return fa_build.build_shared([SRC], LIB)


def load():
    if not os.path.exists(LIB):
        raise ImportError(f"{LIB} is not built; run build() first")
    lib = ctypes.CDLL(LIB)
    vp = ctypes.c_void_p
    lib.probe_mfma_32x32x16_f16.argtypes = [vp, vp, vp, vp]
    lib.probe_permlane32_swap.argtypes = [vp, vp, vp]
    lib.probe_cvt_f16.argtypes = [vp, vp, ctypes.c_int, vp]
    lib.probe_mfma_32x32x64_f8.argtypes = [vp, vp, vp, ctypes.c_int, vp]
    lib.probe_ds_read_tr8.argtypes = [vp, ctypes.POINTER(ctypes.c_int), vp, vp, vp]
    lib.probe_cvt_fp8.argtypes = [vp, vp, ctypes.c_int, vp]
    lib.probe_mfma_4x4x4_16b_f16.argtypes = [vp, vp, vp, vp]
    lib.probe_mfma_32x32x64_f8_batch.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp]
    lib.probe_mfma_32x32x16_f16_batch.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp]
    for f in (lib.probe_mfma_32x32x16_f16, lib.probe_permlane32_swap, lib.probe_cvt_f16,
              lib.probe_mfma_32x32x64_f8, lib.probe_ds_read_tr8, lib.probe_cvt_fp8,
              lib.probe_mfma_4x4x4_16b_f16, lib.probe_mfma_32x32x64_f8_batch,
              lib.probe_mfma_32x32x16_f16_batch):
        f.restype = ctypes.c_int
    return lib
