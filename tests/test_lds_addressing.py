"""The LDS addresses of the backward's dK/dV step, formed by XOR (host check).

The dK/dV step of fa_bwd.hip forms every LDS read address from four per-lane
offsets (``dkdv_offsets``): the address of read kk of a row is the offset XORed
with 32*kk, and that of a transposed read (u, db) the offset XORed with 64*db
plus 16*u rows.  This holds because the swizzles of fa_common.h only flip bits
inside a row's 16-byte-chunk field.  Here the swizzles and both address forms
are written out and compared for every lane, every wave and every stage base
the kernel uses, at d = 128 and d = 64.
"""
import pytest


def k_swz(d, row, ch):
    return ch ^ (row & 15) if d == 128 else ch ^ ((row >> 1) & 7)


def kv_swz(d, row, ch):
    if d == 128:
        return ch ^ ((row & 15) ^ ((row & 3) << 2))
    return ch ^ (((row >> 1) & 7) ^ (((row >> 1) & 1) << 2))


def lane_coords(lane):
    col, hi = lane & 31, lane >> 5
    tg, ti = lane >> 4, lane & 15
    return col, hi, hi * 4 + (ti >> 2), 16 * (tg & 1) + 4 * (ti & 3)


@pytest.mark.parametrize("d", [128, 64])
def test_dkdv_step_addresses(d):
    rb, dch, kk_n, db_n = d * 2, d // 8, d // 16, d // 32
    vb = 128 * rb                    # the V block (128 keys), then Q and dO stages of 32 rows
    qtb = 32 * rb
    bases = [0] + [vb + i * qtb for i in range(4)]
    for base in bases:
        assert base % 256 == 0
        for wave in range(4):
            for lane in range(64):
                col, hi, tr_row, tr_dd = lane_coords(lane)
                vrow = wave * 32 + col
                c0, w = tr_dd >> 3, (tr_dd & 7) * 2
                qa = col * rb + kv_swz(d, col, hi) * 16
                va = vrow * rb + k_swz(d, vrow, hi) * 16
                ta0 = tr_row * rb + kv_swz(d, tr_row, c0) * 16 + w
                ta1 = (tr_row + 8) * rb + kv_swz(d, tr_row + 8, c0) * 16 + w
                for kk in range(kk_n):
                    want_q = base + (col * dch + kv_swz(d, col, 2 * kk + hi)) * 16
                    assert (base + qa) ^ (32 * kk) == want_q
                    want_v = base + (vrow * dch + k_swz(d, vrow, 2 * kk + hi)) * 16
                    assert (base + va) ^ (32 * kk) == want_v
                for i in range(2 * db_n):
                    u, db = i // db_n, i % db_n
                    r0 = 16 * u + tr_row
                    r1 = r0 + 8
                    dd = db * 32 + tr_dd
                    c, ww = dd >> 3, (dd & 7) * 2
                    assert ((base + ta0) ^ (64 * db)) + 16 * u * rb == base + r0 * rb + kv_swz(d, r0, c) * 16 + ww
                    assert ((base + ta1) ^ (64 * db)) + 16 * u * rb == base + r1 * rb + kv_swz(d, r1, c) * 16 + ww


def test_a_wrong_form_fails():
    """The check is not vacuous: adding instead of XORing the chunk constant breaks it."""
    d, rb, dch = 128, 256, 16
    bad = 0
    for lane in range(64):
        col, hi, _, _ = lane_coords(lane)
        qa = col * rb + kv_swz(d, col, hi) * 16
        for kk in range(8):
            bad += (qa + 32 * kk) != (col * dch + kv_swz(d, col, 2 * kk + hi)) * 16
    assert bad > 0
