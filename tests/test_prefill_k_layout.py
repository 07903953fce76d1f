"""CPU model of the prefill attention kernel's K tile stage (prefill.hip).

The kernel moves a 32-key x 256-dim BF16 K tile into LDS with loads that write LDS
directly (64 lanes x 16 bytes per instruction, contiguous in LDS), two key pairs per
wave, and reads it back as the A operand of v_mfma_f32_32x32x16_bf16 (lane l: key
l % 32, dims 16 s + 8 (l / 32) .. +7 in step s).  This test restates the kernel's
index arithmetic -- the load offsets, the LDS slot of each instruction and the read
address k_base + 32 s -- and checks, for several row strides, that every load stays
inside the stage, no LDS byte is written twice, every read returns the (key, chunk)
its MFMA step needs, and the 16 lanes that one LDS pass serves hit 64 distinct banks.
"""

from collections import Counter

import pytest

K_DIM = 256  # dims per key
P_KEYS = 32  # keys per tile
P_WAVES = 8  # waves per workgroup
PAIRS = P_KEYS // 2 // P_WAVES  # key pairs each wave loads per tile
PAIR_BYTES = 2 * K_DIM * 2 + 16  # one key pair + 16 unused bytes
STAGE_BYTES = P_KEYS // 2 * PAIR_BYTES
BANKS = 64  # 4-byte LDS banks


def stage_contents(stride):
    """LDS byte offset of each 16-byte chunk -> (key within the tile, chunk)."""
    lds = {}
    for wave in range(P_WAVES):
        for i in range(PAIRS):
            pr = PAIRS * wave + i
            for lane in range(64):
                lo_off = (lane >> 5) * stride
                voff = 16 * lo_off + ((lane & 31) << 4)
                soff = pr * stride  # tile's first key at offset 0
                key, rem = divmod(voff + soff, stride)
                assert rem % 16 == 0 and rem < 2 * K_DIM
                dst = pr * PAIR_BYTES + 16 * lane
                assert 0 <= dst and dst + 16 <= STAGE_BYTES
                assert dst not in lds, "an LDS chunk written twice"
                lds[dst] = (key, rem // 16)
    return lds


def k_base(lane):
    rl, hh = lane & 31, lane >> 5
    return (rl & 15) * PAIR_BYTES + (rl >> 4) * (2 * K_DIM) + 16 * hh


@pytest.mark.parametrize("stride", [2 * K_DIM, 4 * 2 * K_DIM, 7 * 512 + 32])
def test_every_read_returns_its_operand(stride):
    lds = stage_contents(stride)
    assert len(lds) == P_KEYS * K_DIM * 2 // 16
    assert sorted({k for k, _ in lds.values()}) == list(range(P_KEYS))
    for lane in range(64):
        rl, hh = lane & 31, lane >> 5
        for s in range(16):
            assert lds[k_base(lane) + 32 * s] == (rl, 2 * s + hh), (lane, s)


def test_reads_are_free_of_bank_conflicts():
    for s in range(16):
        for group in range(4):
            banks = Counter()
            for lane in range(16 * group, 16 * group + 16):
                a = k_base(lane) + 32 * s
                banks.update(((a // 4) + j) % BANKS for j in range(4))
            assert max(banks.values()) == 1, (s, group)


def test_stage_fits_beside_the_other_buffers():
    v_stage = P_KEYS * K_DIM * 2
    tables = 2 * 64 * P_WAVES * 16
    assert 4 * (STAGE_BYTES + v_stage) + tables <= 160 * 1024
