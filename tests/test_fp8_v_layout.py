"""CPU model of the FP8 forward's V-tile reads (no GPU).

The kernel stores a 64-key V tile in LDS at pitch d + 32 bytes with rows exchanged by swap23
(LDS row r holds key swap23(r)), and gathers the V^T operand of each 64-key P V product with
four 8-bit transpose reads. Semantics of the transpose read (measured on gfx950): within each
16-lane group, lane i receives as its byte e the byte i % 8 of the 8-byte piece addressed by
source lane 2e + i / 8 of the same group.

Checked here, with the lane offsets written as the kernel computes them:
  * every lane receives, for read j and output block i, the V bytes of exactly the keys its P
    bytes hold (byte b of lane half h is key 32(b/16) + 8((b%16)/4) + 4h + b%4), at dim
    32 i + lane % 32;
  * the 32 lanes of each half (one LDS pass of 8-byte reads) touch each of the 64 four-byte
    banks at most once, while the former layout (pitch d + 16, rows in key order) did not.
"""
import pytest


def swap23(r):
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1)


def lane_off_swapped(lane, pitch):
    s, h = lane & 15, lane >> 5
    return (8 * h + 4 * (s >> 3) + ((s >> 1) & 3)) * pitch + 16 * ((lane >> 4) & 1) + 8 * (s & 1)


def lane_off_plain(lane, pitch):
    s, h = lane & 15, lane >> 5
    return (8 * (s >> 3) + 4 * h + ((s >> 1) & 3)) * pitch + 16 * ((lane >> 4) & 1) + 8 * (s & 1)


def gather(d, pitch, lane_off, row_of_key):
    where = {}
    for key in range(64):
        for dim in range(d):
            where[row_of_key(key) * pitch + dim] = (key, dim)
    out, conflicts = {}, 0
    for j in range(4):
        for i in range(d // 32):
            addr = {l: lane_off(l, pitch) + 16 * j * pitch + 32 * i for l in range(64)}
            for half in range(2):
                banks = [((addr[l] >> 2) + w) % 64 for l in range(32 * half, 32 * half + 32) for w in range(2)]
                conflicts += len(banks) - len(set(banks))
            for l in range(64):
                g, li = l // 16, l % 16
                out[(j, i, l)] = [where.get(addr[16 * g + 2 * e + li // 8] + li % 8) for e in range(8)]
    return out, conflicts


@pytest.mark.parametrize("d", [64, 128, 256])
def test_swapped_v_tile_gathers_the_p_keys_without_bank_conflicts(d):
    out, conflicts = gather(d, d + 32, lane_off_swapped, swap23)
    for (j, i, l), got in out.items():
        h = l >> 5
        # P bytes 8j .. 8j+7 of lane half h
        keys = [32 * (b // 16) + 8 * ((b % 16) // 4) + 4 * h + b % 4 for b in range(8 * j, 8 * j + 8)]
        assert got == [(k, 32 * i + l % 32) for k in keys], (d, j, i, l)
    assert conflicts == 0
    _, old_conflicts = gather(d, d + 16, lane_off_plain, lambda k: k)
    assert old_conflicts > 0
