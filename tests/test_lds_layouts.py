"""LDS layouts of the 256-query attention kernel's direct staging (CPU model).

The kernel stages K and V tiles straight into LDS: a wave's buffer load with
the LDS flag writes lane l's 16 bytes at the load's LDS base + 16 l, so a
tile is a sequence of 16-byte slots, 64 per load.  K rows keep a 272-byte
stride (17 slots: 16 data + 1 padding), V rows a 320-byte stride (20 slots).
The value product reads V^T fragments with the CDNA4 transposing LDS read
(ds_read_b64_tr_b16): within each 16-lane group, lane i receives element
i mod 4 of the 4-element row addressed by lane 4 r + i // 4 of the group,
r = 0..3 (behaviour probed on the GPU).

These tests restate the kernel's address formulas and check, on a model of
the hardware, that (a) every data byte of a tile is loaded exactly once and
padding slots are the only ones left out, (b) the transposing reads hand each
lane the MFMA A-operand it needs (8 consecutive keys of one dim), and (c) the
fragment reads are free of LDS bank conflicts (64 banks of 4 bytes; 16 lanes
per clock for 16-byte reads, 32 for 8-byte reads) -- the counter run reports
zero conflicts, and a plausible slip in a stride or an index fails here.
"""
import numpy as np
import pytest

D, BN = 128, 64
KSTR_B, VROW_B = 272, 320            # row strides in bytes
K_SLOTS, V_SLOTS = KSTR_B // 16, VROW_B // 16
K_LOADS, V_LOADS = BN * K_SLOTS // 64, BN * V_SLOTS // 64


def dma_lane(w, lane, ch, nloads):
    """(row, chunk) of each of a wave's loads for one lane, None for padding
    or for a load the wave does not issue (mirrors dma_lane)."""
    out = []
    for m in range(5):
        i = w + 4 * m
        q = 64 * i + lane
        row, c = divmod(q, ch)
        out.append((i, row, c) if i < nloads and c < 16 else None)
    return out


@pytest.mark.parametrize("ch,nloads", [(K_SLOTS, K_LOADS), (V_SLOTS, V_LOADS)])
def test_direct_loads_cover_each_tile_byte_once(ch, nloads):
    assert nloads * 64 == BN * ch                    # whole wave loads per tile
    seen = {}
    for w in range(4):                               # the four waves of a stager group
        n = (nloads - w + 3) // 4
        for lane in range(64):
            for m, e in enumerate(dma_lane(w, lane, ch, nloads)):
                if e is None:
                    continue
                i, row, c = e
                assert m < n
                # LDS byte of the slot = load base 1024 i + 16 lane = row stride * row + 16 c
                assert 1024 * i + 16 * lane == 16 * ch * row + 16 * c
                assert (row, c) not in seen
                seen[(row, c)] = (w, m)
    assert set(seen) == {(r, c) for r in range(BN) for c in range(16)}


def tr_read(lds_words, addrs):
    """ds_read_b64_tr_b16 on a model LDS (array of 16-bit words): addrs[l] is
    lane l's byte address of a 4-element row; returns [64][4] elements."""
    rows = np.array([[lds_words[(a >> 1) + k] for k in range(4)] for a in addrs])
    out = np.zeros((64, 4), dtype=lds_words.dtype)
    for g in range(4):
        for i in range(16):
            for r in range(4):
                out[16 * g + i, r] = rows[16 * g + 4 * r + i // 4, i % 4]
    return out


def vtr_lane_offset(lane):
    g, a = lane >> 4, lane & 15
    return (8 * (g >> 1) + (a >> 2)) * VROW_B + 32 * (g & 1) + 8 * (a & 3)


def test_transposing_reads_give_the_value_product_operand():
    # V tile: element (key, dim) holds key * 256 + dim (distinct values).
    words = np.zeros(BN * VROW_B // 2, dtype=np.int64)
    for key in range(BN):
        for dim in range(D):
            words[key * VROW_B // 2 + dim] = key * 256 + dim
    for st in range(4):                              # 16-key steps of the tile
        for db in range(4):                          # 32-dim output blocks
            base = [vtr_lane_offset(l) + st * 16 * VROW_B + db * 64 for l in range(64)]
            x = tr_read(words, base)
            y = tr_read(words, [b + 4 * VROW_B for b in base])
            frag = np.concatenate([x, y], axis=1)    # the 8 bf16 of the A operand
            for l in range(64):
                keys = 16 * st + 8 * (l // 32) + np.arange(8)
                dim = 32 * db + l % 32
                assert list(frag[l]) == list(keys * 256 + dim), (st, db, l)


def conflict_free(addrs, nbytes, per_clock):
    """No two lanes served in the same clock touch one bank at different
    4-byte words (64 banks of 4 bytes)."""
    for c0 in range(0, 64, per_clock):
        words = {}
        for l in range(c0, c0 + per_clock):
            for b in range(0, nbytes, 4):
                word = (addrs[l] + b) // 4
                words.setdefault(word % 64, set()).add(word)
        if any(len(w) > 1 for w in words.values()):
            return False
    return True


def test_value_fragment_reads_are_conflict_free():
    for st in range(4):
        for db in range(4):
            for extra in (0, 4 * VROW_B):
                addrs = [vtr_lane_offset(l) + st * 16 * VROW_B + db * 64 + extra for l in range(64)]
                assert conflict_free(addrs, 8, 32), (st, db, extra)


def permuted_row(i):
    return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1)


def test_score_fragment_reads_are_conflict_free():
    for kb in range(2):
        for kk in range(8):
            addrs = [(32 * kb + permuted_row(l & 31)) * KSTR_B + 32 * kk + 16 * (l >> 5)
                     for l in range(64)]
            assert conflict_free(addrs, 16, 16), (kb, kk)


def test_conflict_model_catches_an_unpadded_stride():
    # The same V reads with 256-byte rows put the four rows one read touches
    # on the same 16 banks.
    addrs = [((8 * ((l >> 4) >> 1) + ((l & 15) >> 2)) * 256 + 32 * ((l >> 4) & 1) + 8 * (l & 3))
             for l in range(64)]
    assert not conflict_free(addrs, 8, 32)
