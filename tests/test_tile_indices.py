"""Host-side check of the tile kernel's staging and LDS index arithmetic.

Restates, for every tile shape the library compiles (head_dim 128 and 256 with
their key-block sizes, pipeline depths and wave layouts: 4 waves of 32 rows at
head_dim 128, 8 waves of 16 rows at 256), the mapping of direct-to-LDS load
lanes to K/V chunks and the K-row, V-transpose and epilogue addresses, and
checks that every LDS access stays inside its buffer and every chunk of a
block is written exactly once.  Runs without a GPU; a failure here means a
kernel change would read or write LDS out of bounds.
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


def _waves(hd):
    """(rows per wave, waves per workgroup) of the tile kernel at head_dim hd"""
    rpw = 32 if hd == 128 else 16
    return rpw, 128 // rpw


def swz_k(r):
    return r & 15


def _swz_v(hd):
    return (lambda r: (r & 3) << 2) if hd == 128 else (lambda r: (r & 7) << 1)


def _f8_lane(hd, lane):
    """(row within one fp8 load instruction, 16-byte fp8 chunk) of a lane"""
    cpr = hd // 16
    return lane // cpr, lane % cpr


def _k_reads(hd, bk):
    """(row, 16-byte position) of every K-fragment read, per lane, in issue groups"""
    rpw, _ = _waves(hd)
    out = []
    if rpw == 32:
        for ds in range(hd // 16):
            for n in range(bk // 32):
                out.append([(32 * n + (lane & 31), (2 * ds + (lane >> 5)) ^ swz_k(32 * n + (lane & 31)))
                            for lane in range(64)])
    else:
        for ks in range(hd // 32):
            for t in range(2):
                out.append([(16 * t + (lane & 15), (4 * ks + (lane >> 4)) ^ swz_k(16 * t + (lane & 15)))
                            for lane in range(64)])
    return out


def _v_reads(hd, bk):
    """byte address of every 8-byte V transpose read, per lane, in issue groups"""
    rpw, _ = _waves(hd)
    rb, swz_v = hd * 2, _swz_v(hd)
    out = []
    if rpw == 32:
        for db in range(hd // 32):
            for n in range(bk // 32):
                for t in range(2):
                    for second in (0, 8):
                        addrs = []
                        for lane in range(64):
                            h, grp, s16 = lane >> 5, lane >> 4, lane & 15
                            row = 32 * n + 16 * t + 4 * h + (s16 >> 2)
                            cc = 4 * db + 2 * (grp & 1) + ((s16 & 3) >> 1)
                            addrs.append((row + second, (row + second) * rb + 16 * (cc ^ swz_v(row)) + 8 * (s16 & 1)))
                        out.append(addrs)
    else:
        for dt in range(hd // 16):
            for u in range(2):
                addrs = []
                for lane in range(64):
                    j, n16 = lane >> 4, lane & 15
                    row = 16 * u + 4 * j + (n16 >> 2)
                    cc = 2 * dt + ((n16 & 3) >> 1)
                    addrs.append((row, row * rb + 16 * (cc ^ swz_v(row)) + 8 * (n16 & 1)))
                out.append(addrs)
    return out


@pytest.mark.parametrize("hd", [128, 256])
def test_staging_and_reads_stay_in_bounds(hd):
    bk, stages = _shape(hd)
    rpw, nw = _waves(hd)
    threads = 64 * nw
    rb, cpr = hd * 2, hd // 8
    tile = bk * rb
    nload = tile // 1024 // (threads // 64)
    assert nload * 1024 * (threads // 64) == tile
    stage = 2 * tile
    lds = stages * stage
    assert lds <= 160 * 1024
    swz_v = _swz_v(hd)

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

    for group in _k_reads(hd, bk):
        for row, pos in group:
            assert row < bk and 0 <= pos < cpr
            assert row * rb + 16 * pos + 16 <= tile
    for group in _v_reads(hd, bk):
        for row, addr in group:
            assert row < bk and addr + 8 <= tile
    # epilogue: each wave's rows of O (bf16) or of one half of a partial
    # state (fp32), through the freed K/V stages
    for row_bytes in (rb, 2 * hd):
        assert nw * rpw * row_bytes <= lds


@pytest.mark.parametrize("hd", [256])
def test_16_row_epilogue_writes_cover_each_row_once(hd):
    """16-row waves write O as 8-byte halves of 16-byte chunks: lanes part and
    part ^ 1 fill chunk 2 dt + part // 2 of row n16; every byte of the wave's
    rows is written exactly once, and the fp32 passes likewise."""
    rpw, _ = _waves(hd)
    rb, cpr = hd * 2, hd // 8
    seen = {}
    for lane in range(64):
        n16, part = lane & 15, lane >> 4
        for dt in range(hd // 16):
            cc = 2 * dt + (part >> 1)
            off = n16 * rb + 16 * (cc ^ (n16 & (cpr - 1))) + 8 * (part & 1)
            for b in range(8):
                assert off + b not in seen
                seen[off + b] = 1
    assert len(seen) == rpw * rb
    cprf = hd // 8
    for _pass in range(2):
        seen = set()
        for lane in range(64):
            n16, part = lane & 15, lane >> 4
            for dtl in range(hd // 32):
                cc = 4 * dtl + part
                off = n16 * cprf * 16 + 16 * (cc ^ (n16 & (cprf - 1)))
                assert off + 16 <= rpw * cprf * 16
                assert off not in seen
                seen.add(off)
        assert len(seen) == rpw * cprf


@pytest.mark.parametrize("hd", [128, 256])
def test_paged_wave_rows_share_one_page(hd):
    """The paged loader reads one block-table entry per wave and block, for
    key kb*BK + w*WAVE_ROWS (clamped to the last key).  That is right only if
    every row a wave's loads touch lies in the same 16-key-aligned group as
    that key, also after clamping rows past the request's end."""
    bk, _ = _shape(hd)
    _, nw = _waves(hd)
    threads = 64 * nw
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
    for i, group in enumerate(_k_reads(hd, bk)):
        assert _cycles([row * rb + 16 * pos for row, pos in group], 16, 16) == 0, i
    for i, group in enumerate(_v_reads(hd, bk)):
        assert _cycles([addr for _, addr in group], 8, 32) == 0, i
    assert _cycles([16 * lane for lane in range(64)], 16, 16) == 0


def test_16_row_epilogue_lds_writes_are_bank_conflict_free():
    """head_dim 256: the 8-byte O writes (lanes part and part ^ 1 fill one
    16-byte chunk) and the 16-byte fp32 partial-state writes"""
    hd = 256
    rb, cpr = hd * 2, hd // 8
    for dt in range(hd // 16):
        addrs = []
        for lane in range(64):
            n16, part = lane & 15, lane >> 4
            cc = 2 * dt + (part >> 1)
            addrs.append(n16 * rb + 16 * (cc ^ (n16 & (cpr - 1))) + 8 * (part & 1))
        assert _cycles(addrs, 8, 32) == 0, dt
    for dtl in range(hd // 32):
        addrs = []
        for lane in range(64):
            n16, part = lane & 15, lane >> 4
            cc = 4 * dtl + part
            addrs.append(n16 * cpr * 16 + 16 * (cc ^ (n16 & (cpr - 1))))
        assert _cycles(addrs, 16, 16) == 0, dtl


def test_32_row_epilogue_lds_writes_are_bank_conflict_free():
    """head_dim 128: after the permlane32 swap the lower lane of a row writes
    chunk 4 db + 2 p and the upper lane chunk 4 db + 2 p + 1 (16 bytes each);
    the fp32 partial-state writes are 16-byte chunks 8 dbl + 2 jj + h"""
    hd = 128
    rb, cpr = hd * 2, hd // 8
    for db in range(hd // 32):
        for p in range(2):
            addrs = []
            for lane in range(64):
                h, qc = lane >> 5, lane & 31
                cc = 4 * db + 2 * p + h
                addrs.append(qc * rb + 16 * (cc ^ (qc & (cpr - 1))))
            assert _cycles(addrs, 16, 16) == 0, (db, p)
    # every 16-byte chunk of the wave's 32 rows is written exactly once
    seen = set()
    for lane in range(64):
        h, qc = lane >> 5, lane & 31
        for db in range(hd // 32):
            for p in range(2):
                cc = 4 * db + 2 * p + h
                seen.add((qc, cc ^ (qc & (cpr - 1))))
    assert len(seen) == 32 * cpr
    cprf = hd // 32 // 2 * 8
    for dbl in range(hd // 64):
        for jj in range(4):
            addrs = []
            for lane in range(64):
                h, qc = lane >> 5, lane & 31
                cc = 8 * dbl + 2 * jj + h
                addrs.append(qc * cprf * 16 + 16 * (cc ^ (qc & (cprf - 1))))
            assert _cycles(addrs, 16, 16) == 0, (dbl, jj)


@pytest.mark.parametrize("hd", [128, 256])
def test_fp8_staging_and_conversion_writes(hd):
    """FP8 K/V: each wave loads F8_W key rows per block (one 64-lane load per
    HD/16-chunk group of rows); the lane -> (row, chunk) map must cover every
    fp8 chunk of the wave's rows once.  The conversion's 16-byte bf16 writes
    (chunks 2 fc and 2 fc + 1 of the lane's row) are at most two-way
    conflicted: the K writes at head_dim 128 are conflict-free, the V writes
    (and both at head_dim 256) cost one extra cycle per 16 lanes.  A lane map
    and V swizzle that remove these measured 1-2 % slower (more address
    arithmetic), so the bound is what is kept."""
    bk, _ = _shape(hd)
    rpw, nw = _waves(hd)
    rb = hd * 2
    f8w = bk // nw
    f8cpr = hd // 16
    rpl = 64 // f8cpr
    nl = f8w // rpl
    assert nl * rpl == f8w
    swz_v = _swz_v(hd)
    for wu in range(nw):
        seen = set()
        for i in range(nl):
            for swz in (swz_k, swz_v):
                for half in (0, 1):
                    addrs = []
                    for lane in range(64):
                        r_in, fc = _f8_lane(hd, lane)
                        row = wu * f8w + i * rpl + r_in
                        seen.add((row, fc))
                        pos = (2 * fc + half) ^ swz(row)
                        assert 0 <= pos < hd // 8 and row < bk
                        addrs.append(row * rb + 16 * pos)
                    assert _cycles(addrs, 16, 16) <= 4, (wu, i, half)
        assert len(seen) == f8w * f8cpr
