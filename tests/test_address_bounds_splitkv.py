"""Every memory address the split-KV decoding kernels touch, computed on the
CPU with the hardware's own arithmetic, lies inside its buffer.

A model of the address arithmetic of ``fa_splitkv_kernel.hip``: the work
item decode (batch, K/V head, split, block of 32 packed query rows), the
packing of a K/V head's query rows (row R = query i * groups + member), the
split's key range, the ring of 32-key stages and their direct loads (uint32
lane offsets, the zero-extended address, the tail re-read of row Lk - 1),
the Q loads, the partial O and LSE stores into the workspace, and the merge
kernel's reads of the partials and its O and LSE stores.  It must follow any
change to that arithmetic.
"""
from __future__ import annotations

import numpy as np
import pytest

SB = 32          # keys per stage
NST = 3          # ring depth
U32 = 1 << 32
MERGE_LANES = 16
MERGE_ROWS = 256 // MERGE_LANES


def k_chunk(D, row, c):
    return c ^ (row & 15) if D == 128 else c ^ ((row >> 1) & 7)


def v_chunk(D, row, c):
    return c ^ ((row & 3) << 2) if D == 128 else c ^ (((row >> 1) & 1) << 2)


class SplitChecker:
    def __init__(self, B, Lq, Lk, H, Hkv, D, causal, past_len, n_splits):
        self.B, self.Lq, self.Lk, self.H, self.Hkv, self.D = B, Lq, Lk, H, Hkv, D
        self.causal, self.past = causal, past_len
        self.g = H // Hkv
        self.n_splits = n_splits
        self.rows = Lq * self.g
        self.n_rb = (self.rows + 31) // 32
        kv_vis = Lk
        if causal:
            last = Lq + past_len
            kv_vis = 0 if last < 0 else min(last, Lk)
        self.kv_vis = kv_vis
        blocks = (kv_vis + SB - 1) // SB
        self.split_blocks = (blocks + n_splits - 1) // n_splits
        self.chunks = D // 8
        self.rpl = 64 // self.chunks
        self.n_loads = SB // self.rpl
        self.kv_row = Hkv * D
        self.kv_bytes = 2 * B * Lk * Hkv * D
        self.q_bytes = 2 * B * Lq * H * D
        self.n_rows = B * H * Lq
        self.ws_o_floats = self.n_rows * n_splits * D
        self.ws_lse_floats = self.n_rows * n_splits
        self.lane = np.arange(64)
        pc = self.lane % self.chunks
        self.load_rows = [self.rpl * n + self.lane // self.chunks for n in range(self.n_loads)]
        self.k_offs = [(2 * (r.astype(np.int64) * self.kv_row + 8 * k_chunk(D, r, pc))) % U32
                       for r in self.load_rows]
        self.v_offs = [(2 * (r.astype(np.int64) * self.kv_row + 8 * v_chunk(D, r, pc))) % U32
                       for r in self.load_rows]
        self.n_checked = 0

    def issue_stage(self, b, hk, k0):
        base = 2 * (b * self.Lk * self.kv_row + hk * self.D + k0 * self.kv_row)
        full = k0 + SB <= self.Lk
        for n in range(self.n_loads):
            back = 0
            if not full:
                over = k0 + self.load_rows[n] - (self.Lk - 1)
                back = (2 * np.maximum(over, 0).astype(np.int64) * self.kv_row) % U32
            for offs in (self.k_offs, self.v_offs):
                addr = base + (offs[n] - back) % U32
                assert np.all(addr >= 0) and np.all(addr + 16 <= self.kv_bytes), (
                    f"stage k0={k0} b={b} hk={hk}: bytes {addr.min()}..{addr.max() + 16} "
                    f"outside 0..{self.kv_bytes}")
                self.n_checked += addr.size
            assert 512 * n + 512 <= SB * self.D  # LDS halves of the stage

    def item(self, b, hk, sp, rb):
        col, half = self.lane & 31, self.lane >> 5
        R0 = 32 * rb
        R = R0 + col
        qi = R // self.g
        h = hk * self.g + (R - qi * self.g)
        R_last = min(R0 + 31, self.rows - 1)
        wpl = R_last // self.g + self.past
        ks = sp * self.split_blocks * SB
        ke = self.kv_vis if self.kv_vis - ks < self.split_blocks * SB else ks + self.split_blocks * SB
        if self.causal and wpl < ke - 1:
            ke = wpl + 1
        nb = (ke - ks + SB - 1) // SB if ke > ks else 0
        if nb > 0:
            # every stage starts at a key that exists (the tail re-read
            # assumes it): ks + 32 s < ke <= Lk for s < nb
            assert ks + SB * (nb - 1) < min(ke, self.Lk)
            for s in range(NST - 1):
                if s < nb:
                    self.issue_stage(b, hk, ks + SB * s)
            for t in range(nb):
                tn = t + NST - 1
                if tn < nb:
                    self.issue_stage(b, hk, ks + SB * tn)
            ok = qi < self.Lq
            for s in range(self.D // 16):
                a = 2 * ((b * self.Lq + qi) * self.H * self.D + h * self.D + 16 * s + 8 * half)
                assert np.all(a[ok] >= 0) and np.all(a[ok] + 16 <= self.q_bytes)
        w = R < self.rows
        prow = ((b * self.H + h) * self.Lq + qi) * self.n_splits + sp
        for i in range(self.D // 32):
            for r4 in range(4):
                f = prow * self.D + 32 * i + 8 * r4 + 4 * half
                assert np.all(f[w] >= 0) and np.all(f[w] + 4 <= self.ws_o_floats)
        assert np.all(prow[w] >= 0) and np.all(prow[w] < self.ws_lse_floats)

    def merge(self):
        blocks = (self.n_rows + MERGE_ROWS - 1) // MERGE_ROWS
        t = np.arange(256)
        per = self.D // MERGE_LANES
        for blk in range(blocks):
            row = blk * MERGE_ROWS + t // MERGE_LANES
            live = row < self.n_rows
            row, d0 = row[live], per * (t[live] % MERGE_LANES)
            for p in range(self.n_splits):
                assert np.all(row * self.n_splits + p < self.ws_lse_floats)
                f = row * self.n_splits * self.D + d0 + p * self.D
                assert np.all(f >= 0) and np.all(f + per <= self.ws_o_floats)
            bh, i = row // self.Lq, row % self.Lq
            b, h = bh // self.H, bh % self.H
            o = 2 * (((b * self.Lq + i) * self.H + h) * self.D + d0)
            assert np.all(o >= 0) and np.all(o + 2 * per <= self.q_bytes)
            assert np.all(row < self.n_rows)

    def run(self):
        for b in range(self.B):
            for hk in range(self.Hkv):
                for sp in range(self.n_splits):
                    for rb in range(self.n_rb):
                        self.item(b, hk, sp, rb)
        self.merge()
        return self.n_checked


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", [
    (2, 1, 1, 4, 2, None, 1), (2, 1, 33, 4, 2, None, 2), (1, 1, 4096, 8, 1, None, 16),
    (1, 3, 1000, 4, 4, None, 7), (2, 5, 333, 8, 2, None, 5), (1, 1, 65, 2, 2, None, 12),
    (1, 40, 300, 4, 1, None, 3), (1, 64, 64, 2, 2, 0, 4), (1, 17, 200, 4, 2, -5, 6),
    (1, 2, 100, 2, 1, 500, 3), (1, 1, 31, 32, 8, None, 2), (1, 1, 32, 32, 8, None, 2)])
def test_splitkv_in_bounds(case, causal, D):
    B, Lq, Lk, H, Hkv, past, n_splits = case
    past = Lk - Lq if past is None else past
    assert SplitChecker(B, Lq, Lk, H, Hkv, D, causal, past if causal else 0, n_splits).run() > 0


@pytest.mark.parametrize("shape", [(2, 32768, 32, 8), (2, 4096, 32, 32)])
def test_splitkv_decoding_workloads_in_bounds(shape):
    """The decoding shapes (one query after the cached keys, D = 128) at the
    split count the library picks for them, on two batches (the others
    differ by whole batches)."""
    import tiled_attention_flash_amd as fa
    B, Lk, H, Hkv = shape
    n_splits = fa.fa_splitkv_splits(8, 1, Lk, H, Hkv, 128, 1, Lk - 1)
    assert 1 <= n_splits <= 64
    assert SplitChecker(B, 1, Lk, H, Hkv, 128, True, Lk - 1, n_splits).run() > 0


def test_splitkv_model_catches_a_stage_past_the_keys():
    """Not vacuous: a stage whose first key lies past the last one wraps the
    tail re-read offset and is reported."""
    c = SplitChecker(1, 1, 40, 2, 1, 128, False, 0, 1)
    with pytest.raises(AssertionError):
        c.issue_stage(0, 0, 39 + 64)
