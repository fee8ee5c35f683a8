"""Host-side check of the tile kernel's staging and LDS index arithmetic.

Restates, for every tile shape the library compiles (head_dim 128 and 256 with
their key-block sizes and pipeline depths), the mapping of direct-to-LDS load
lanes to K/V chunks and the K-row and V-transpose read addresses, and checks
that every LDS access stays inside its buffer and every chunk of a block is
written exactly once.  Runs without a GPU; a failure here means a kernel
change would read or write LDS out of bounds.
"""

import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _shape(hd):
    text = open(os.path.join(ROOT, "varlen_prefill_amd", "csrc", "rp_internal.h")).read()
    bk = int(re.search(rf"#define RP_HD{hd}_BK (\d+)", text).group(1))
    st = int(re.search(rf"#define RP_HD{hd}_STAGES (\d+)", text).group(1))
    return bk, st


@pytest.mark.parametrize("hd", [128, 256])
def test_staging_and_reads_stay_in_bounds(hd):
    bk, stages = _shape(hd)
    threads = 256
    rb, cpr = hd * 2, hd // 8
    tile = bk * rb
    nload = tile // 1024 // (threads // 64)
    assert nload * 1024 * (threads // 64) == tile
    stage = 2 * tile
    lds = stages * stage
    assert lds <= 160 * 1024

    def swz_k(r):
        return r & 15

    def swz_v(r):
        return (r & 3) << 2

    wk, wv = set(), set()
    for w in range(threads // 64):
        for i in range(nload):
            for lane in range(64):
                chunk = (nload * w + i) * 64 + lane
                rr, pp = divmod(chunk, cpr)
                assert rr < bk
                assert 0 <= (pp ^ swz_k(rr)) < cpr and 0 <= (pp ^ swz_v(rr)) < cpr
                dk = (nload * w + i) * 1024 + 16 * lane
                assert dk + 16 <= tile
                assert (stages - 1) * stage + tile + dk + 16 <= lds
                wk.add((rr, pp ^ swz_k(rr)))
                wv.add((rr, pp ^ swz_v(rr)))
    assert len(wk) == bk * cpr and len(wv) == bk * cpr

    nb, ds_steps, dblocks = bk // 32, hd // 16, hd // 32
    for lane in range(64):
        h, qc, grp, s16 = lane >> 5, lane & 31, lane >> 4, lane & 15
        for ds in range(ds_steps):
            for n in range(nb):
                row = 32 * n + qc
                pos = (2 * ds + h) ^ swz_k(row)
                assert row < bk and 0 <= pos < cpr
                assert row * rb + 16 * pos + 16 <= tile
        for db in range(dblocks):
            for n in range(nb):
                for t in range(2):
                    row = 32 * n + 16 * t + 4 * h + (s16 >> 2)
                    cc = 4 * db + 2 * (grp & 1) + ((s16 & 3) >> 1)
                    pos = cc ^ swz_v(row)
                    assert 0 <= pos < cpr and row + 8 < bk
                    assert (row + 8) * rb + 16 * pos + 8 * (s16 & 1) + 8 <= tile


@pytest.mark.parametrize("hd", [128, 256])
def test_paged_wave_rows_share_one_page(hd):
    """The paged loader reads one block-table entry per wave and block, for
    key kb*BK + w*WAVE_ROWS (clamped to the last key).  That is right only if
    every row a wave's loads touch lies in the same 16-key-aligned group as
    that key, also after clamping rows past the request's end."""
    bk, _ = _shape(hd)
    threads = 256
    rb, cpr = hd * 2, hd // 8
    nload = bk * rb // 1024 // (threads // 64)
    wave_rows = nload * 1024 // rb
    assert 16 % wave_rows == 0
    for w in range(threads // 64):
        rows = {((nload * w + i) * 64 + lane) // cpr for i in range(nload) for lane in range(64)}
        assert min(rows) == w * wave_rows and max(rows) < (w + 1) * wave_rows
        for kb in range(3):
            for kv_len in range(1, 4 * bk + 1):
                key0 = min(kb * bk + w * wave_rows, kv_len - 1)
                for r in rows:
                    key = kb * bk + min(r, kv_len - 1 - kb * bk)
                    assert key // 16 == key0 // 16


def _cycles(addrs, width, group):
    """LDS cycles beyond the ideal for one wave-wide access: 64 four-byte
    banks; lanes are served `group` at a time in lane order (16 for 16-byte
    accesses, 32 for the 8-byte transpose read, the grouping a GPU probe of
    these access shapes confirmed); within a group, a bank hit by several
    different dwords costs one cycle per extra dword."""
    extra = 0
    for g0 in range(0, 64, group):
        banks = {}
        for lane in range(g0, g0 + group):
            for k in range(width // 4):
                d = addrs[lane] // 4 + k
                banks.setdefault(d % 64, set()).add(d)
        extra += max(len(v) for v in banks.values()) - 1
    return extra


@pytest.mark.parametrize("hd", [128, 256])
def test_loop_lds_accesses_are_bank_conflict_free(hd):
    """Bank model of the key loop's LDS traffic: the K-fragment reads
    (16 bytes per lane) and the V transpose reads (8 bytes per lane) hit
    every bank at most once per group of lanes served together, and the
    direct-to-LDS loads write 64 consecutive 16-byte pieces."""
    bk, _ = _shape(hd)
    rb = hd * 2

    def swz_k(r):
        return r & 15

    def swz_v(r):
        return (r & 3) << 2

    for ds in range(hd // 16):
        for n in range(bk // 32):
            addrs = []
            for lane in range(64):
                h, qc = lane >> 5, lane & 31
                row = 32 * n + qc
                addrs.append(row * rb + 16 * ((2 * ds + h) ^ swz_k(row)))
            assert _cycles(addrs, 16, 16) == 0, (ds, n)
    for db in range(hd // 32):
        for n in range(bk // 32):
            for t in range(2):
                for second in (0, 8):
                    addrs = []
                    for lane in range(64):
                        h, grp, s16 = lane >> 5, lane >> 4, lane & 15
                        row = 32 * n + 16 * t + 4 * h + (s16 >> 2)
                        cc = 4 * db + 2 * (grp & 1) + ((s16 & 3) >> 1)
                        addrs.append((row + second) * rb + 16 * (cc ^ swz_v(row)) + 8 * (s16 & 1))
                    assert _cycles(addrs, 8, 32) == 0, (db, n, t)
    assert _cycles([16 * lane for lane in range(64)], 16, 16) == 0
