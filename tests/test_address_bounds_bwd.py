"""Every global address the backward kernels (Delta, dK/dV, dQ) touch,
computed on the CPU with the hardware's arithmetic, lies inside its buffer --
for equal and for different query and key lengths (``fa_bwd_kv``).

A model of the address arithmetic of ``fa_bwd_kernels.h`` (the Delta
kernel's O and dO row reads and Delta stores, the staged tile loads of
``TileLoad::issue``, the LSE/Delta loads, the K, Q and dO row loads
and the gradient stores), written out again here; it must follow any change
to that arithmetic.  As in the forward's model, a direct HBM -> LDS load adds
the 64-bit scalar base (the tile's first row) and the 32-bit lane offset
*zero-extended*: an offset that goes below zero wraps to about +4 GiB, so
the lane offsets are kept as uint32 and wrapped as the kernels' uint32_t
arithmetic wraps them.  Rows at or past the end re-read the last row by
moving the offset back from the tile's first row.
"""
from __future__ import annotations

import random

import numpy as np
import pytest

U32 = 1 << 32


def rt_chunk(D, row, c):
    if D == 128:
        return c ^ (((row & 3) << 2) | ((row >> 2) & 3))
    return c ^ ((((row >> 1) & 1) << 2) | ((row >> 2) & 3))


class Buf:
    """A tensor of `elems` halves (or floats) at byte address `base`."""

    def __init__(self, name, base, nbytes):
        self.name, self.base, self.nbytes = name, base, nbytes

    def check(self, addr, width, what):
        a = np.asarray(addr, dtype=np.int64)
        bad = (a < self.base) | (a + width > self.base + self.nbytes)
        assert not bad.any(), f"{what}: {self.name} address out of bounds ({int(a[bad][0]) - self.base:+d})"


def tile_load(buf, D, W, kRows, base_elem, row_stride, r0, n_rows, what):
    """TileLoad<D, W, kRows>::issue: every lane of every wave's instructions."""
    chunks = D // 8
    rpl = 64 // chunks
    loads = kRows // rpl
    per_wave = loads // W
    lane = np.arange(64)
    pc = lane % chunks
    tile = buf.base + 2 * (base_elem + r0 * row_stride)  # scalar base: the tile's first row
    for wave in range(W):
        for n in range(per_wave):
            blk = per_wave * wave + n
            row = rpl * blk + lane // chunks
            lrow = row.copy()
            row = np.where(r0 + row > n_rows - 1, n_rows - 1 - r0, row)
            off = (2 * (row * row_stride + 8 * np.array([rt_chunk(D, int(r), int(c)) for r, c in zip(lrow, pc)])))
            off = off % U32  # uint32_t arithmetic, zero-extended by the instruction
            buf.check(tile + off, 16, what)


def run_model(B, Lq, Lk, H, Hkv, D, causal, past_len):
    past = past_len if causal else 0
    g = H // Hkv
    qs, kvs = H * D, Hkv * D
    bufs = {
        "q": Buf("q", 1 << 40, 2 * B * Lq * qs), "dout": Buf("dout", 2 << 40, 2 * B * Lq * qs),
        "k": Buf("k", 3 << 40, 2 * B * Lk * kvs), "v": Buf("v", 4 << 40, 2 * B * Lk * kvs),
        "lse": Buf("lse", 5 << 40, 4 * B * H * Lq), "delta": Buf("delta", 6 << 40, 4 * B * H * Lq),
        "dq": Buf("dq", 7 << 40, 2 * B * Lq * qs), "dk": Buf("dk", 8 << 40, 2 * B * Lk * kvs),
        "dv": Buf("dv", 9 << 40, 2 * B * Lk * kvs), "o": Buf("o", 10 << 40, 2 * B * Lq * qs),
    }
    # Delta: one (b, i, h) row of O and dO per 16 lanes, rows in BSHD order
    n_rows = B * Lq * H
    blocks = (n_rows + 15) // 16
    t = np.arange(256)
    row = (np.arange(blocks)[:, None] * 16 + t[None, :] // 16).ravel()
    sub = np.tile(t % 16, blocks)
    live = row < n_rows
    row, sub = row[live], sub[live]
    per = D // 16
    for name in ("o", "dout"):
        bufs[name].check(bufs[name].base + 2 * (row * D + per * sub), 2 * per, f"delta {name}")
    h, bi = row % H, row // H
    i, bb = bi % Lq, bi // Lq
    bufs["delta"].check(bufs["delta"].base + 4 * ((bb * H + h) * Lq + i), 4, "delta store")
    # dK, dV: items (b, hk, key block of 32 W keys)
    W = 8 if (D == 128 and not causal) else 4
    n_kb = (Lk + 32 * W - 1) // (32 * W)
    n_qb = (Lq + 31) // 32
    for b in range(B):
        for hk in range(Hkv):
            for kb in range(n_kb):
                k_wg = kb * 32 * W
                keys = k_wg + np.arange(32 * W)
                ok = keys < Lk  # K row loads and dK/dV stores are guarded
                for name in ("k", "dk", "dv"):
                    bufs[name].check(bufs[name].base + 2 * ((b * Lk + keys[ok]) * kvs + hk * D), 2 * D, name)
                tile_load(bufs["v"], D, W, 32 * W, b * Lk * kvs + hk * D, kvs, k_wg, Lk, "dkdv V tile")
                qb0 = 0
                if causal:
                    first = k_wg - past
                    qb0 = 0 if first <= 0 else (n_qb if first >= n_qb * 32 else first // 32)
                per_head = n_qb - qb0
                for t in range(per_head * g):
                    h = hk * g + t // per_head
                    q0 = (qb0 + t % per_head) * 32
                    for name in ("q", "dout"):
                        tile_load(bufs[name], D, W, 32, b * Lq * qs + h * D, qs, q0, Lq, f"dkdv {name} tile")
                    i = np.minimum(q0 + np.arange(32), Lq - 1)
                    r0 = (b * H + h) * Lq
                    for name in ("lse", "delta"):
                        bufs[name].check(bufs[name].base + 4 * r0 + (4 * i) % U32, 4, name)
    # dQ: items (b, h, query block of 32 W rows)
    W = 4 if (causal or D == 64) else 8
    BM = 32 * W
    for b in range(B):
        for h in range(H):
            hk = h // g
            for qb in range((Lq + BM - 1) // BM):
                q0 = qb * BM
                rows = q0 + np.arange(BM)
                ok = rows < Lq
                for name in ("q", "dout", "dq"):
                    bufs[name].check(bufs[name].base + 2 * ((b * Lq + rows[ok]) * qs + h * D), 2 * D, name)
                for name in ("lse", "delta"):
                    bufs[name].check(bufs[name].base + 4 * ((b * H + h) * Lq + rows[ok]), 4, name)
                kv_end = Lk
                if causal:
                    last = min(q0 + BM, Lq) - 1 + past
                    kv_end = 0 if last < 0 else (last + 1 if last < Lk - 1 else Lk)
                for t in range((kv_end + 63) // 64):
                    for name in ("k", "v"):
                        tile_load(bufs[name], D, W, 64, b * Lk * kvs + hk * D, kvs, 64 * t, Lk, f"dq {name} tile")


CASES = [  # B, Lq, Lk, H, Hkv, D, past_len (None: Lk - Lq)
    (1, 1, 1, 2, 2, 128, None), (1, 77, 300, 4, 2, 128, None), (2, 300, 77, 2, 1, 64, None),
    (1, 70, 50, 4, 4, 128, -20), (1, 33, 129, 2, 2, 64, 500), (1, 129, 257, 8, 2, 128, 0),
    (2, 1, 333, 4, 1, 64, None), (1, 1024, 4096, 4, 2, 128, None), (1, 300, 300, 2, 2, 128, None),
    (1, 5, 1000, 2, 1, 64, -3), (1, 1000, 5, 2, 1, 128, None), (1, 64, 64, 2, 2, 64, -64),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", CASES)
def test_backward_addresses_in_bounds(case, causal):
    B, Lq, Lk, H, Hkv, D, past = case
    run_model(B, Lq, Lk, H, Hkv, D, causal, Lk - Lq if past is None else past)


def test_backward_addresses_random_shapes():
    r = random.Random(5)
    for _ in range(40):
        D = r.choice([64, 128])
        Lq, Lk = r.randint(1, 400), r.randint(1, 400)
        Hkv = r.choice([1, 2])
        H = Hkv * r.choice([1, 2, 4])
        past = r.choice([Lk - Lq, 0, -r.randint(1, 50), r.randint(1, 500)])
        run_model(1, Lq, Lk, H, Hkv, D, r.random() < 0.6, past)


def test_model_catches_a_tile_past_the_end():
    """A tile whose first row lies past the last row (r0 > n_rows - 1) has
    its tail re-read before the tile: the offset wraps, and the model flags it."""
    D, W, Lk, kvs = 128, 4, 10, 128
    buf = Buf("v", 1 << 40, 2 * Lk * kvs)
    with pytest.raises(AssertionError):
        tile_load(buf, D, W, 64, 0, kvs, 64, Lk, "tile past the end")
