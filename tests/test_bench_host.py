"""Host-side pieces of bench.py (no GPU): the kernel-source hash that keys the
committed HBM traffic figures."""
from __future__ import annotations

import os
import shutil

import bench


def _copy_sources(tmp_path):
    out = {}
    for path, srcs in bench.KERNEL_SRCS.items():
        out[path] = []
        for src in srcs:
            dst = tmp_path / os.path.basename(src)
            if not dst.exists():
                shutil.copy(src, dst)
            out[path].append(str(dst))
    return out


def test_kernel_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    srcs = _copy_sources(tmp_path)
    monkeypatch.setattr(bench, "KERNEL_SRCS", srcs)
    before = {p: bench.kernel_sha(p) for p in srcs}
    fwd = tmp_path / "fa_fwd_kernel.hip"
    text = fwd.read_text()
    # comments, blank lines and trailing spaces only: every hash unchanged
    fwd.write_text("// a new leading comment\n\n" + text.replace("{\n", "{  /* note */\n", 1) + "\n// end\n")
    assert {p: bench.kernel_sha(p) for p in srcs} == before
    # one changed constant: the forward hash moves, the other paths' do not
    fwd.write_text(text.replace("constexpr int kBN = 64;", "constexpr int kBN = 128;", 1))
    after = {p: bench.kernel_sha(p) for p in srcs}
    assert after["forward"] != before["forward"]
    assert all(after[p] == before[p] for p in srcs if p != "forward")


def test_kernel_hash_covers_each_paths_sources():
    for path, srcs in bench.KERNEL_SRCS.items():
        names = [os.path.basename(s) for s in srcs]
        assert "fa_device.h" in names and "fa_internal.h" in names, path
        assert all(os.path.exists(s) for s in srcs), path


def test_kernel_hash_covers_build_flags(monkeypatch):
    """A change of the extra flags a kernel source is built with moves that
    path's hash (the counters were taken on the code those flags produce)."""
    from tiled_attention_flash_amd import build as fa_build

    before = {p: bench.kernel_sha(p) for p in bench.KERNEL_SRCS}
    flags = dict(fa_build.SOURCE_FLAGS)
    flags["fa_bwd_kernel.hip"] = ["-mllvm", "-some-other-option"]
    monkeypatch.setattr(fa_build, "SOURCE_FLAGS", flags)
    after = {p: bench.kernel_sha(p) for p in bench.KERNEL_SRCS}
    assert after["backward"] != before["backward"]
    assert all(after[p] == before[p] for p in after if p != "backward")
