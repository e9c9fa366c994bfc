"""Host-side models of two LDS/HBM layouts the matrix-core kernels rely on.

They restate, in Python, the index arithmetic of the device code and check
it against the layouts' definitions on every lane, so that a change to one
side of an address computation fails on the CPU:

- the k-major W_out stage of the direct-to-LDS projection (mfma_tile.hpp,
  KMajorBOp): copies into LDS with a per-row XOR swizzle, fragments read
  with ds_read_b64_tr_b16.  The lane semantics of that instruction, as
  taken from an in-bounds LDS probe on gfx950: within each group of 16
  lanes, lane i receives element i % 4 of the 64-bit words addressed by
  lanes i // 4, 4 + i // 4, 8 + i // 4 and 12 + i // 4;
- the K-blocked H written by the H pass and read by the projection
  (k_route.hip, hbuild_kernel; k_proj.hip, proj_direct_kernel<C, true>).
"""
import numpy as np
import pytest

BK = 32


def swz(r):
    return (r & 3) << 2


def kmajor_stage(BN, waves, ncols, k0=0):
    """LDS contents (16-bit element ids) after one stage's copies."""
    k_row = BN * 2
    loads = BN // 16 // waves
    lds = np.full(BK * k_row // 2, -1, dtype=np.int64)
    for wave in range(waves):
        for j in range(loads):
            q = wave * loads + j
            for lane in range(64):
                byte = q * 1024 + lane * 16
                r = byte // k_row
                c = ((byte % k_row) >> 4) ^ swz(r)
                col = c * 8 if c * 8 < ncols else 0
                assert 0 <= r < BK
                dst = (q * 1024 + 16 * lane) // 2  # lane's 16 bytes land in order
                for e in range(8):
                    lds[dst + e] = (k0 + r) * 100000 + col + e
    return lds


def tr16_read(lds, addr):
    """ds_read_b64_tr_b16 over a wavefront: addr[lane] is a byte address."""
    out = np.zeros((64, 4), dtype=np.int64)
    for lane in range(64):
        g, i = lane & ~15, lane & 15
        for jw in range(4):
            src = g + 4 * jw + (i >> 2)
            out[lane, jw] = lds[addr[src] // 2 + (i & 3)]
    return out


def kmajor_frag_addr(BN, WN, wn, jf, kk, half):
    k_row = BN * 2
    addr = []
    for lane in range(64):
        cb = wn * WN + jf * 32 + (lane & 16)
        kb = kk * 16 + ((lane >> 5) << 3)
        jj = (lane >> 2) & 3
        col = cb + ((lane & 3) << 2)
        r = kb + jj
        off = r * k_row + (((col >> 3) ^ swz(r)) << 4) + ((col & 7) << 1) + half * 4 * k_row
        addr.append(off)
    return addr


@pytest.mark.parametrize("BN,WN,waves,ncols", [(256, 64, 8, 256), (256, 64, 8, 136),
                                               (128, 64, 4, 128), (128, 64, 8, 8),
                                               (128, 64, 4, 40)])
def test_kmajor_fragments(BN, WN, waves, ncols):
    k_row = BN * 2
    lds = kmajor_stage(BN, waves, ncols)
    assert (lds >= 0).all()  # every byte of the stage is written
    for wn in range(BN // WN):
        for jf in range(WN // 32):
            for kk in range(2):
                lo = kmajor_frag_addr(BN, WN, wn, jf, kk, 0)
                hi = kmajor_frag_addr(BN, WN, wn, jf, kk, 1)
                for addr in (lo, hi):
                    assert all(a % 8 == 0 and 0 <= a and a + 8 <= BK * k_row for a in addr)
                    # 32 lanes of a half wavefront, 8 bytes each, cover 64 banks
                    for h in range(2):
                        banks = set()
                        for lane in range(32 * h, 32 * h + 32):
                            banks.update({(addr[lane] // 4) % 64, (addr[lane] // 4 + 1) % 64})
                        assert len(banks) == 64
                frag = np.concatenate([tr16_read(lds, lo), tr16_read(lds, hi)], axis=1)
                for lane in range(64):
                    n = wn * WN + jf * 32 + (lane & 31)
                    if n >= ncols:
                        continue  # clamped columns: results unused
                    want = [(kk * 16 + 8 * (lane >> 5) + e) * 100000 + n for e in range(8)]
                    assert list(frag[lane]) == want


def test_kblocked_h_roundtrip():
    # The H pass stores 16-byte pieces of columns p*h + ja (and + h/2) of
    # token t; the projection's A loader reads, for K step k0, row r, chunk c,
    # the element at (H + r*32) + k0*T + c*8.  Both must address element
    # (t, k) at ((k // 32) * T + t) * 32 + k % 32.
    T, P, h = 300, 3, 64
    K = P * h
    Hblk = np.full(T * K, -1, dtype=np.int64)
    for t in range(T):
        for p in range(P):
            for ja in range(0, h // 2, 8):
                for base in (ja, h // 2 + ja):
                    k = p * h + base
                    off = (k >> 5) * (T << 5) + t * 32 + (k & 31)
                    for e in range(8):
                        assert Hblk[off + e] == -1
                        Hblk[off + e] = t * 10000 + k + e
    assert (Hblk >= 0).all()
    for k0 in range(0, K, 32):
        for r in range(T):
            for c in range(4):
                off = r * 32 + k0 * T + c * 8
                for e in range(8):
                    assert Hblk[off + e] == r * 10000 + k0 + c * 8 + e
