"""Every memory address the E4M3 forward kernel touches, computed on the CPU
with the hardware's own arithmetic, lies inside its buffer, and the K operand
reads find the bytes the S product expects.

A model of the address arithmetic of ``fa_fwd_fp8_kernel.hip`` (the
tile-load lane offsets and their XOR swizzle, the tile schedule, the Q loads,
the O and LSE stores, the K and V operand reads from LDS), written out again
here in numpy; it must follow any change to that arithmetic.  As in the fp16
model, a direct load adds the 64-bit scalar base and the 32-bit lane offset
zero-extended, so every lane offset is a uint32 that wraps; a tile that
reaches past the last key re-reads row Lk - 1 by subtracting whole rows from
that offset.  Elements are one byte.

Instances as the launcher picks them: 8 wavefronts for the full pass, 4 for
causal, at D = 64 and 128.
"""
from __future__ import annotations

import numpy as np
import pytest

BLK = 64  # keys per score block and per LDS tile
U32 = 1 << 32


def swz(D, row):
    row = np.asarray(row)
    if D == 128:
        return ((row >> 2) & 1) | (((row >> 1) & 1) << 1) | (((row >> 3) & 1) << 2)
    return ((row >> 2) & 1) | (((row >> 3) & 1) << 1)


class Checker8:
    def __init__(self, B, Lq, Lk, H, Hkv, D, causal, past_len):
        self.B, self.Lq, self.Lk, self.H, self.Hkv, self.D = B, Lq, Lk, H, Hkv, D
        self.causal, self.past = causal, past_len
        self.W = 4 if causal else 8
        self.BM = 32 * self.W
        self.nq = (Lq + self.BM - 1) // self.BM
        self.chunks = D // 16
        self.rpl = 64 // self.chunks                    # rows one load fills (1 KiB)
        self.per_tile = BLK // self.rpl                 # load instructions per tile
        self.lpw = (self.per_tile + self.W - 1) // self.W
        self.kv_row = Hkv * D                           # bytes between key rows
        self.q_row = H * D
        self.kv_bytes = B * Lk * Hkv * D
        self.q_bytes = B * Lq * H * D
        self.o_bytes = 2 * B * Lq * H * D
        self.tile = BLK * D
        self.lane = np.arange(64)
        # LDS contents as the global byte each LDS byte was loaded from
        # (-1: never written): klds[0], klds[1], vlds[0], vlds[1]
        self.lds = np.full((4, self.tile), -1, dtype=np.int64)
        self.read_swz = swz  # the swizzle the K operand reads undo
        self.n_checked = 0

    def lane_offsets(self):
        """The uint32 offsets offs[n] of every wave's n-th load, as the item
        prologue computes them, with the instruction index blk = wave + W n;
        instructions with blk >= loads per tile are not issued."""
        out = []
        pc = self.lane % self.chunks
        for wave in range(self.W):
            for n in range(self.lpw):
                blk = wave + self.W * n
                if blk >= self.per_tile:
                    continue
                row = self.rpl * blk + self.lane // self.chunks
                off = (row.astype(np.int64) * self.kv_row + 16 * (pc ^ swz(self.D, row))) % U32
                out.append((blk, row, off))
        return out

    def issue(self, b, hk, j, is_v, buf):
        """issue_tile8_at for tile j (keys 64 j ..) into buffer `buf`."""
        k0 = BLK * j
        head = b * self.Lk * self.kv_row + hk * self.D   # byte offset of key 0 of this head
        tile_base = head + (j * ((BLK * self.kv_row) % U32))  # (uint32_t)(kBlk * kv_row), < 2^31
        edge = not (k0 + BLK <= self.Lk)
        slot = (2 if is_v else 0) + buf
        for blk, row, off in self.lane_offsets():
            if edge:
                over = k0 + row - (self.Lk - 1)
                sub = (np.maximum(over, 0).astype(np.int64) * self.kv_row) % U32
                off = (off - sub) % U32
            addr = tile_base + off  # 64-bit base + zero-extended offset
            assert np.all(addr >= 0) and np.all(addr + 16 <= self.kv_bytes), (
                f"{'V' if is_v else 'K'} tile {j} b={b} hk={hk}: bytes "
                f"{addr.min()}..{addr.max() + 16} outside 0..{self.kv_bytes}")
            m0 = 1024 * blk
            assert m0 + 16 * 64 <= self.tile
            dst = m0 + 16 * self.lane[:, None] + np.arange(16)[None, :]
            self.lds[slot][dst] = addr[:, None] + np.arange(16)[None, :]
            self.n_checked += addr.size

    def check_k_reads(self, b, hk, j, buf):
        """kfrag(a, s) of every lane reads bytes 64 s + 32 h .. + 31 of key
        row 32 a + col of tile j (two 16-byte LDS reads at kb ^ 64 s and
        kb ^ (64 s + 16))."""
        D = self.D
        col, h = self.lane & 31, self.lane >> 5
        kb = col * D + 16 * ((2 * h) ^ self.read_swz(D, col))
        head = b * self.Lk * self.kv_row + hk * self.D
        for a in range(2):
            key = np.minimum(BLK * j + 32 * a + col, self.Lk - 1)  # tail rows re-read Lk - 1
            for s in range(D // 64):
                for part in range(2):
                    la = 32 * a * D + (kb ^ (64 * s + 16 * part))
                    assert np.all(la >= 0) and np.all(la + 16 <= self.tile)
                    got = self.lds[buf][la[:, None] + np.arange(16)[None, :]]
                    want = (head + key * self.kv_row + 64 * s + 32 * h + 16 * part)[:, None] + np.arange(16)
                    assert np.array_equal(got, want), (j, a, s, part)

    def check_v_reads(self, b, hk, j, buf):
        """vfrag(i): four 8-byte transpose reads at (vb ^ 32 i) + 16 t D stay
        inside the tile; the read of lane (g, h, row pair b', e) finds bytes
        32 i + 16 (g & 1) + 8 e .. + 7 of key row 16 t + row0 of tile j."""
        D = self.D
        lane = self.lane
        g, m, h = lane >> 4, lane & 15, lane >> 5
        bb, e = m >> 1, m & 1
        row0 = 4 * h + (bb & 3) + 8 * (bb >> 2)
        vb = row0 * D + 16 * ((g & 1) ^ swz(D, row0)) + 8 * e
        head = b * self.Lk * self.kv_row + hk * self.D
        for i in range(D // 32):
            for t in range(4):
                la = (vb ^ (32 * i)) + 16 * t * D
                assert np.all(la >= 0) and np.all(la + 8 <= self.tile)
                got = self.lds[2 + buf][la[:, None] + np.arange(8)[None, :]]
                key = np.minimum(BLK * j + 16 * t + row0, self.Lk - 1)
                want = (head + key * self.kv_row + 32 * i + 16 * (g & 1) + 8 * e)[:, None] + np.arange(8)
                assert np.array_equal(got, want), (j, i, t)

    def item(self, b, hk, g, qb):
        hq = hk * (self.H // self.Hkv) + g
        q0 = qb * self.BM
        kv_end = self.Lk
        if self.causal:
            last = min(q0 + self.BM, self.Lq) - 1 + self.past
            kv_end = last + 1 if last < self.Lk - 1 else self.Lk
        n_blocks = (kv_end + BLK - 1) // BLK if kv_end > 0 else 0
        if n_blocks > 0:
            self.issue(b, hk, 0, False, 0)
            self.issue(b, hk, 0, True, 0)
            if n_blocks > 1:
                self.issue(b, hk, 1, False, 1)
            self.check_k_reads(b, hk, 0, 0)          # prologue S of block 0
            for u in range(n_blocks):                # block<P, NEXT, MASK> for step u
                P = u % 2
                if u + 2 < n_blocks:
                    self.issue(b, hk, u + 2, False, P)
                if u + 1 < n_blocks:
                    self.issue(b, hk, u + 1, True, P ^ 1)
                    self.check_k_reads(b, hk, u + 1, P ^ 1)  # S(u + 1)
                self.check_v_reads(b, hk, u, P)      # P.V(u)
        col, h = self.lane & 31, self.lane >> 5
        for wave in range(self.W):
            qi = q0 + 32 * wave + col
            ok = qi < self.Lq
            qa = b * self.Lq * self.q_row + hq * self.D + qi * self.q_row
            for s in range(self.D // 64):
                a = qa + 64 * s + 32 * h
                assert np.all(a[ok] >= 0) and np.all(a[ok] + 32 <= self.q_bytes)
            orow = 2 * ((b * self.Lq + qi) * self.H * self.D + hq * self.D)
            for i in range(self.D // 32):
                for e in range(2):
                    a = orow + 2 * (32 * i + 16 * e + 8 * h)
                    assert np.all(a[ok] >= 0) and np.all(a[ok] + 16 <= self.o_bytes)
            li = (b * self.H + hq) * self.Lq + qi
            assert np.all(li[ok] >= 0) and np.all(li[ok] < self.B * self.H * self.Lq)

    def run(self, corners_only=False):
        groups = self.H // self.Hkv
        bs = sorted({0, self.B - 1}) if corners_only else range(self.B)
        hks = sorted({0, self.Hkv - 1}) if corners_only else range(self.Hkv)
        gs = sorted({0, groups - 1}) if corners_only else range(groups)
        for b in bs:
            for hk in hks:
                for g in gs:
                    for qb in range(self.nq):
                        self.lds[:] = -1
                        self.item(b, hk, g, qb)
        return self.n_checked


RAGGED = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 333, 1000]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_fp8_ragged_lengths_in_bounds(D, causal):
    n = 0
    for L in RAGGED:
        n += Checker8(2, L, L, 4, 2, D, causal, 0).run()
    assert n > 0


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", [
    (1, 1, 300, 4, 2, None), (2, 100, 333, 4, 2, None), (1, 257, 1000, 2, 1, None),
    (1, 300, 120, 2, 2, None), (2, 200, 200, 4, 4, 37), (1, 129, 64, 2, 1, -20),
    (1, 77, 500, 4, 1, 600), (1, 64, 1, 2, 2, None)])
def test_fp8_queries_after_cached_keys_in_bounds(case, causal):
    B, Lq, Lk, H, Hkv, past = case
    past = Lk - Lq if past is None else past
    for D in (64, 128):
        assert Checker8(B, Lq, Lk, H, Hkv, D, causal, past if causal else 0).run() > 0


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_full_size_workload_in_bounds(causal):
    """The E4M3 benchmark shape (B 8, 32 heads, 4096 keys, D 128) on the
    items at the corners of the tensors, every q block."""
    assert Checker8(8, 4096, 4096, 32, 32, 128, causal, 0).run(corners_only=True) > 0


def test_fp8_model_catches_a_tile_past_the_end():
    """Not vacuous: a K tile whose first key is past the last one wraps the
    tail re-read offset and is reported."""
    c = Checker8(1, 20, 20, 1, 1, 128, False, 0)
    with pytest.raises(AssertionError):
        c.issue(0, 0, 1, False, 0)


def test_fp8_model_catches_a_wrong_swizzle():
    """Not vacuous: K reads that do not undo the loads' swizzle find other
    bytes."""
    c = Checker8(1, 64, 64, 1, 1, 128, False, 0)
    c.issue(0, 0, 0, False, 0)
    c.check_k_reads(0, 0, 0, 0)
    c.read_swz = lambda D, row: np.zeros_like(np.asarray(row))
    with pytest.raises(AssertionError):
        c.check_k_reads(0, 0, 0, 0)
