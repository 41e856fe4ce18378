"""CPU models of the cross-lane reduce-scatters the kernels use (no GPU).

The one-row GEMV (`row_sums_rs` in csrc/device.h) and the one-row decode
attention (`k_attn_dec1`'s score reduction in csrc/attn.hip) sum many values
over the lanes of a wave with DPP permutes and a swizzle, each step pairing
lanes that differ in one bit and halving what a lane holds.  The kernels then
read each row's (or score's) sum from one particular lane, so these tests
replay the steps on a 64-lane model built from the permutes' definitions in
the CDNA ISA and check that lane mapping for random inputs.
"""
import random

import pytest

WAVE = 64


# lane i reads its operand from lane src(i)
def row_mirror(i):  # DPP row_mirror: within a 16-lane row, lane 15 - i
    return (i // 16) * 16 + 15 - i % 16


def row_half_mirror(i):  # DPP row_half_mirror: within 8 lanes, lane 7 - i
    return (i // 8) * 8 + 7 - i % 8


def quad_xor1(i):  # DPP quad_perm [1, 0, 3, 2]
    return i ^ 1


def quad_xor2(i):  # DPP quad_perm [2, 3, 0, 1]
    return i ^ 2


def row_ror(n):  # DPP row_ror:n: within a 16-lane row, lane (i + n) mod 16
    return lambda i: (i // 16) * 16 + (i % 16 + n) % 16


def swap16(i):  # ds_swizzle, bitmask mode, xor mask 0x10: lane i ^ 16 within 32
    return (i // 32) * 32 + ((i % 32) ^ 16)


def permute(vals, src):
    return [vals[src(i)] for i in range(WAVE)]


def rs_step(cur, bit, src):
    """One halving step: lane i keeps the half of its values selected by its
    bit `bit` (the upper half when set), sends the other half, and adds what
    its partner src(i) sends."""
    n = len(cur[0])
    half = n // 2
    out = [[0.0] * half for _ in range(WAVE)]
    for k in range(half):
        send = [cur[i][k] if (i >> bit) & 1 else cur[i][half + k] for i in range(WAVE)]
        keep = [cur[i][half + k] if (i >> bit) & 1 else cur[i][k] for i in range(WAVE)]
        got = permute(send, src)
        for i in range(WAVE):
            out[i][k] = keep[i] + got[i]
    return out


def gemv_row_sums(vals, rows):
    """The steps of row_sums_rs<rows>: returns one value per lane."""
    steps = {
        32: [(4, swap16), (3, row_mirror), (2, row_half_mirror), (1, quad_xor2), (0, quad_xor1)],
        16: [(3, row_mirror), (2, row_half_mirror), (1, quad_xor2), (0, quad_xor1)],
        8: [(2, row_half_mirror), (1, quad_xor2), (0, quad_xor1)],
        4: [(1, quad_xor2), (0, quad_xor1)],
    }[rows]
    cur = [list(v) for v in vals]
    for bit, src in steps:
        cur = rs_step(cur, bit, src)
    r = [c[0] for c in cur]
    if rows == 32:
        return r
    if rows <= 8:
        t = permute(r, row_ror(8))
        r = [a + b for a, b in zip(r, t)]
    if rows <= 4:
        t = permute(r, row_ror(4))
        r = [a + b for a, b in zip(r, t)]
    t = permute(r, swap16)
    return [a + b for a, b in zip(r, t)]


@pytest.mark.parametrize("rows", [4, 8, 16, 32])
def test_gemv_reduce_scatter_leaves_row_sums_in_the_first_lanes_of_each_half(rows):
    rng = random.Random(rows)
    vals = [[rng.uniform(-1, 1) for _ in range(rows)] for _ in range(WAVE)]
    out = gemv_row_sums(vals, rows)
    for i in range(WAVE):
        if i % 32 >= rows:
            continue  # the kernel reads only lanes i % 32 < rows
        half = i // 32
        want = sum(vals[l][i % 32] for l in range(32 * half, 32 * half + 32))
        assert out[i] == pytest.approx(want, abs=1e-12), (rows, i)


def test_decode_attention_reduce_scatter_leaves_value_dq_in_lane_dq():
    """k_attn_dec1's score reduction: 32 values a lane (4 heads x 8 keys, value
    v = 4 it + h); each step keeps, of every pair of values differing in the
    step's bit of v, the one whose bit equals the lane's bit of dq (lane % 32)
    and adds the partner's copy; after the five steps lane dq holds value dq
    summed over its 32-lane half."""
    rng = random.Random(7)
    vals = [[rng.uniform(-1, 1) for _ in range(32)] for _ in range(WAVE)]
    cur = [list(v) for v in vals]
    for bit, done, src in [(3, 0, row_mirror), (2, 8, row_half_mirror), (0, 12, quad_xor1),
                           (1, 13, quad_xor2), (4, 15, swap16)]:
        new = [list(c) for c in cur]
        for lane in range(WAVE):
            hi = ((lane & 31) >> bit) & 1
            p = src(lane)
            hi_p = ((p & 31) >> bit) & 1
            for v in range(32):
                if (v & done) or (v & (1 << bit)):
                    continue
                lo, hv = cur[lane][v], cur[lane][v | (1 << bit)]
                send_p = cur[p][v] if hi_p else cur[p][v | (1 << bit)]
                new[lane][v] = (hv if hi else lo) + send_p
        cur = new
    for lane in range(WAVE):
        half, dq = lane // 32, lane % 32
        want = sum(vals[l][dq] for l in range(32 * half, 32 * half + 32))
        assert cur[lane][0] == pytest.approx(want, abs=1e-12), lane
