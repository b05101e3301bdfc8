"""Every memory address the fp16 forward kernel touches, computed on the CPU
with the hardware's own arithmetic, lies inside its buffer.

This is a model of the address arithmetic of ``fa_fwd_kernel.hip`` (the
tile-load offsets, the tile schedule, the Q loads, the O and LSE stores and
the LDS operand reads), written out again here in numpy; it must follow any
change to that arithmetic.  What it models that a plain integer emulation
would not:

* a direct HBM -> LDS load (``global_load_lds_dwordx4 v_off, s[base]``) adds
  the 64-bit scalar base and the 32-bit per-lane offset *zero-extended*: an
  offset that goes below zero wraps to about +4 GiB instead of stepping
  backwards, so every lane offset is kept as a uint32 and wrapped as the
  kernel's ``uint32_t`` arithmetic wraps it;
* the first K tile starts at key -32 (its scalar base lies before the tensor
  for the first batch and head; the load instructions whose rows are all
  before key 0 are skipped, and no instruction straddles key 0);
* a tile that reaches past the last key re-reads row Lk - 1 by subtracting
  whole rows from the lane offset (the tail re-read);
* lane i of a direct load writes LDS bytes m0 + 16 i .. m0 + 16 i + 15, m0
  being the destination of the load instruction.

Instances are chosen as the launcher chooses them: D = 128 full pass with 8
wavefronts, causal with 4 below 4096 keys and 8 from 4096 on; D = 64 with 4.
"""
from __future__ import annotations

import numpy as np
import pytest

BN, SB = 64, 32  # keys per K/V tile, keys per score block
U32 = np.uint64(1 << 32)


def waves_for(D, causal, Lk):
    if D == 128 and causal:
        return 8 if Lk >= 4096 else 4
    return 4 if D == 64 else 8


def k_chunk(D, row, c):
    return c ^ (row & 15) if D == 128 else c ^ ((row >> 1) & 7)


def v_chunk(D, row, c):
    return c ^ ((row & 3) << 2) if D == 128 else c ^ (((row >> 1) & 1) << 2)


class Checker:
    def __init__(self, B, Lq, Lk, H, Hkv, D, causal, past_len):
        self.B, self.Lq, self.Lk, self.H, self.Hkv, self.D = B, Lq, Lk, H, Hkv, D
        self.causal, self.past = causal, (past_len if causal else 0)
        self.W = waves_for(D, causal, Lk)
        self.BM = 32 * self.W
        self.nq = (Lq + self.BM - 1) // self.BM
        self.chunks = D // 8
        self.rpl = 64 // self.chunks           # rows one load instruction fills
        per_tile = BN // self.rpl              # load instructions per tile
        self.loaders = min(self.W, per_tile)   # waves that load (the first ones)
        self.lpw = per_tile // self.loaders    # load instructions per loading wave
        self.kv_row = Hkv * D                  # elements between key rows
        self.q_row = H * D
        self.kv_bytes = 2 * B * Lk * Hkv * D
        self.q_bytes = 2 * B * Lq * H * D
        self.tile_bytes = 2 * BN * D
        lane = np.arange(64)
        self.lane = lane
        self.n_checked = 0

    # ---------------------------------------------------------- direct loads
    def lane_offsets(self, is_v):
        """init_load_offsets for every (wave, n) at once: rows [W*lpw, 64] and
        the lane offsets (uint32_t)(2 * (row * kv_row + 8 * chunk))."""
        blk = np.arange(self.loaders * self.lpw)[:, None]  # blk = lpw * wave + n
        row = self.rpl * blk + self.lane[None, :] // self.chunks
        pc = np.broadcast_to(self.lane[None, :] % self.chunks, row.shape)
        ch = v_chunk(self.D, row, pc) if is_v else k_chunk(self.D, row, pc)
        off = (2 * (row.astype(np.int64) * self.kv_row + 8 * ch)) % (1 << 32)
        return blk, row, off.astype(np.uint64)

    def issue(self, b, hk, k0, is_v, buf):
        """issue_loads for the tile starting at key k0 into LDS buffer `buf`,
        every wavefront's share."""
        full = k0 + BN <= self.Lk
        sbase = 2 * ((b * self.Lk * self.kv_row + hk * self.D) + k0 * self.kv_row)  # signed bytes
        lds_base = (2 + buf if is_v else buf) * self.tile_bytes  # klds[2] then vlds[2]
        blk, row, off = self.lane_offsets(is_v)
        issued = (k0 + self.rpl * blk[:, 0]) >= 0  # instructions wholly before key 0 are skipped
        blk, row, off = blk[issued], row[issued], off[issued]
        if not full:
            over = k0 + row - (self.Lk - 1)
            sub = (2 * np.maximum(over, 0).astype(np.int64) * self.kv_row) % (1 << 32)
            off = (off + U32 - sub.astype(np.uint64)) % U32  # uint32 subtraction
        addr = sbase + off.astype(np.int64)  # 64-bit base + zero-extended offset
        assert np.all(addr >= 0) and np.all(addr + 16 <= self.kv_bytes), (
            f"{'V' if is_v else 'K'} tile k0={k0} b={b} hk={hk}: "
            f"global bytes {addr.min()}..{addr.max() + 16} outside 0..{self.kv_bytes}")
        m0 = lds_base + 1024 * blk[:, 0]  # lane i writes m0 + 16 i .. m0 + 16 i + 15
        assert np.all(m0 >= lds_base) and np.all(m0 + 16 * 64 <= lds_base + self.tile_bytes), (k0, buf)
        self.n_checked += addr.size

    # ------------------------------------------------------------- one item
    def item(self, b, hk, g, qb):
        h = hk * (self.H // self.Hkv) + g
        q0 = qb * self.BM
        if self.causal:
            last = min(q0 + self.BM, self.Lq) - 1 + self.past
            kv_end = last + 1 if last < self.Lk - 1 else self.Lk
        else:
            kv_end = self.Lk
        n_blocks = (kv_end + SB - 1) // SB if kv_end > 0 else 0
        n_tiles = (kv_end + BN - 1) // BN if kv_end > 0 else 0
        if n_blocks > 0:
            self.issue(b, hk, -SB, False, 0)
            self.issue(b, hk, 0, True, 0)
            if n_blocks > 1:
                self.issue(b, hk, SB, False, 1)
            n_main = (n_blocks - 1) // 2
            for t in range(n_main):  # tile_start of every tile with a successor
                if 2 * t + 3 < n_blocks:
                    self.issue(b, hk, BN * (t + 1) + SB, False, t % 2)
                if t + 1 < n_tiles:
                    self.issue(b, hk, BN * (t + 1), True, (t + 1) % 2)
        # Q loads and O / LSE stores of every lane, guarded by qi < Lq
        col, half = self.lane & 31, self.lane >> 5
        for wave in range(self.W):
            qi = q0 + 32 * wave + col
            ok = qi < self.Lq
            base = 2 * (b * self.Lq * self.q_row + qi * self.q_row + h * self.D)
            for s in range(self.D // 16):
                a = base + 2 * (16 * s + 8 * half)
                assert np.all(a[ok] >= 0) and np.all(a[ok] + 16 <= self.q_bytes)
            for i in range(self.D // 32):
                for e in range(2):
                    a = base + 2 * (32 * i + 16 * e + 8 * half)
                    assert np.all(a[ok] >= 0) and np.all(a[ok] + 16 <= self.q_bytes)
            li = (b * self.H + h) * self.Lq + qi
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
                        self.item(b, hk, g, qb)
        return self.n_checked


def lds_operand_reads(D, W):
    """K operand reads (ds_read_b128, 16 bytes) and V transpose reads
    (ds_read_b64_tr_b16, 8 bytes) of one score block: every lane stays
    inside the 64-key tile it reads (WaveMath::init_lds_bases, k_offset,
    v_offset, vfrag)."""
    lane = np.arange(64)
    col, half = lane & 31, lane >> 5
    tile_halves = BN * D
    k_base = col * D + 8 * k_chunk(D, col, half)
    gg, j = lane >> 4, lane & 15
    row = 4 * (gg >> 1) + (j >> 2)
    d = 16 * (gg & 1) + 4 * (j & 3)
    v_base = row * D + 8 * v_chunk(D, row, d >> 3) + (d & 7)
    for blk in (0, 1):  # the lower and upper score block of a tile
        for s in range(D // 16):
            a = blk * SB * D + (k_base ^ (16 * s))
            assert np.all(a >= 0) and np.all(a + 8 <= tile_halves)
        for i in range(D // 32):
            for cs in range(SB // 16):
                for hi in (0, 8):
                    a = blk * SB * D + (v_base ^ (32 * i)) + 16 * cs * D + hi * D
                    assert np.all(a >= 0) and np.all(a + 4 <= tile_halves)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("W", [4, 8])
def test_lds_operand_reads_stay_in_their_tile(D, W):
    lds_operand_reads(D, W)


RAGGED = [1, 2, 31, 32, 33, 63, 64, 65, 95, 96, 97, 127, 128, 129, 255, 256, 257, 333, 1000]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_ragged_lengths_in_bounds(D, causal):
    n = 0
    for L in RAGGED:
        n += Checker(2, L, L, 4, 2, D, causal, 0).run()
    assert n > 0


def test_faulted_schedule_shape_in_bounds():
    """The parity shape a discarded 128-key-tile variant faulted on (L = 333,
    two batches, four query heads on two K/V heads), on every instance."""
    for D in (64, 128):
        for causal in (False, True):
            assert Checker(2, 333, 333, 4, 2, D, causal, 0).run() > 0


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", [
    (1, 1, 300, 4, 2, None), (2, 100, 333, 4, 2, None), (1, 257, 1000, 2, 1, None),
    (1, 300, 120, 2, 2, None), (2, 200, 200, 4, 4, 37), (1, 129, 64, 2, 1, -20),
    (1, 77, 500, 4, 1, 600), (1, 64, 1, 2, 2, None)])
def test_queries_after_cached_keys_in_bounds(case, causal):
    B, Lq, Lk, H, Hkv, past = case
    past = Lk - Lq if past is None else past
    for D in (64, 128):
        assert Checker(B, Lq, Lk, H, Hkv, D, causal, past).run() > 0


@pytest.mark.parametrize("Lk", [4095, 4096, 4097, 4161, 8193, 8257])
def test_eight_wavefront_causal_in_bounds(Lk):
    """Causal over 4096 keys or more selects the 8-wavefront D = 128 instance."""
    assert Checker(1, Lk, Lk, 2, 1, 128, True, 0).run() > 0
    assert Checker(1, 300, Lk, 2, 2, 128, True, Lk - 300).run() > 0


@pytest.mark.parametrize("shape", [
    (8, 1024, 32, 32, 64, False), (8, 1024, 32, 32, 64, True), (8, 4096, 32, 32, 128, False),
    (8, 4096, 32, 32, 128, True), (2, 8192, 32, 8, 128, True)])
def test_full_size_workloads_in_bounds(shape):
    """The benchmark shapes, on the items at the corners of the tensors
    (first and last batch, K/V head and group member; every q block): the
    addresses of the other items differ only by whole rows and heads."""
    B, L, H, Hkv, D, causal = shape
    assert Checker(B, L, L, H, Hkv, D, causal, 0).run(corners_only=True) > 0


def test_model_catches_a_wrapped_offset():
    """The model is not vacuous: a tail re-read taken one row too far (past
    key 0 of a short sequence) wraps the 32-bit offset and is reported."""
    c = Checker(1, 20, 20, 1, 1, 128, False, 0)
    with pytest.raises(AssertionError):
        c.issue(0, 0, BN, False, 0)  # a K tile starting past the last key: rows wrap
