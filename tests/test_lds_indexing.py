"""CPU model of the decode kernels' LDS indexing: every LDS word a launch reads was written
earlier in the same launch, behind a barrier, and every access lies inside the launch's LDS
allocation.

The index formulas are those of the device code, transcribed one by one (each function below
names the one it follows in csrc/decode_impl.hpp, decode_kernels.hpp or decode_parts.hpp):
the activation staging in MFMA operand order, its zero padding up to whole slots, the
per-(row, group) activation sums and their zero padding groups, the operand and bias reads of
every slot, the parts kernel's hand-off of partial sums, and the streaming kernel's output
staging area.  The phases are separated by the kernels' workgroup barriers:
  staging + padding  |  sums of x  |  slot loop (operand and bias reads; hand-off rounds).
The same property is checked on the GPU by filling the LDS with NaN before each call
(test_gpu_lds_poison.py); this model covers every code width, group size, staged-row
layout and row count at once, including the K = 640, group 32 shapes of the 2- and 6-bit
kernels whose repeated calls once differed."""
import itertools

import pytest

THREADS = 512            # kStreamThreads: 8 waves of 64
WAVES = 8
STAGE_BATCH = 8          # kStageBatch
SX_PAD = 3               # kSxPad
Y_AREA_STRIDE = 40       # kYAreaStride (halfwords per activation row of the output area)


def slot_span(bits, gs):
    """Slot<BITS, GS>::kSpan."""
    return 64 if bits == 8 and gs == 64 else 128


def lane_group_of_sub(bits, sub):
    """lane_group_of_sub<BITS>: 8-bit codes swap the middle two 8-k chunks of a 32-k step."""
    if bits == 8:
        return 2 if sub == 1 else (1 if sub == 2 else sub)
    return sub


def sx_floats(ng, xrl):
    return (((ng + SX_PAD) << xrl) + 3) & ~3


def xs_index(bits, j8, m, xrl):
    """Entry of 8-k chunk j8 of staged row m (stage_x_commit, zero_x_pad)."""
    return ((((j8 >> 2) * 4 + lane_group_of_sub(bits, j8 & 3)) << xrl) + m)


def stage_writes(bits, K, Kp, xrl):
    """stage_x_commit over all batches, then zero_x_pad: the xs entries written."""
    per = THREADS >> xrl
    c8 = K >> 3
    nb = (c8 + STAGE_BATCH * per - 1) // (STAGE_BATCH * per)
    out = set()
    for tid in range(THREADS):
        m = tid & ((1 << xrl) - 1)
        for batch in range(nb):
            j0 = (tid >> xrl) + batch * STAGE_BATCH * per
            for b in range(STAGE_BATCH):
                j8 = j0 + b * per
                if j8 < c8:
                    out.add(xs_index(bits, j8, m, xrl))
        j8 = c8 + (tid >> xrl)
        while j8 < (Kp >> 3):
            out.add(xs_index(bits, j8, m, xrl))
            j8 += per
    return out


def sum_x_access(gs, mt, K, xrl):
    """sum_x: (xs entries read, sxs floats written)."""
    spg = gs // 32
    xmask = (1 << xrl) - 1
    ng = K // gs
    reads, writes = set(), set()
    for p in range(mt * ng):            # spread over the waves, all of them covered
        mtt, g = divmod(p, ng)
        for c in range(spg):
            for lg in range(4):
                for col in range(16):
                    reads.add((((g * spg + c) * 4 + lg) << xrl) + ((mtt * 16 + col) & xmask))
        for lg in range(4):
            for r in range(4):
                if mtt * 16 + 4 * lg + r <= xmask:
                    writes.add((g << xrl) + mtt * 16 + 4 * lg + r)
    return reads, writes


def slot_reads(bits, gs, mt, K, xrl):
    """consume_slot operand reads and bias_mfma reads over every slot of a row, with the bias
    of one slot or of two (kPairBias: group sizes 64 and 128 with an even slot count)."""
    span = slot_span(bits, gs)
    steps = span // 32
    Kp = -(-K // span) * span
    nit = Kp // span
    d = 2 if nit % 2 == 0 else 1
    pair_bias = gs >= 64 and d >= 2
    xmask = (1 << xrl) - 1
    xr, sr = set(), set()
    for kit in range(nit):
        step0 = (kit * span) >> 5
        for c in range(steps):
            for lg in range(4):
                for mtt in range(mt):
                    for col in range(16):
                        xr.add((((step0 + c) * 4 + lg) << xrl) + ((mtt * 16 + col) & xmask))
        if pair_bias:
            if kit % 2 == 0:
                continue
            g0 = (kit - 1) * span // gs
        else:
            g0 = kit * span // gs
        for lg in range(4):
            for mtt in range(mt):
                for col in range(16):
                    sr.add(((g0 + lg) << xrl) + ((mtt * 16 + col) & xmask))
    return xr, sr


def stream_lds_bytes(bits, gs, mt, K, xrl):
    span = slot_span(bits, gs)
    Kp = -(-K // span) * span
    return ((Kp * 2) << xrl) + sx_floats(K // gs, xrl) * 4 + 16 * mt * 8


def parts_lds_bytes(bits, gs, mt, K, xrl):
    return stream_lds_bytes(bits, gs, mt, K, xrl) + WAVES * 2 * mt * 64 * 16


def check_shape(bits, gs, mt, xrl, K, parts=None):
    span = slot_span(bits, gs)
    Kp = -(-K // span) * span
    ng = K // gs
    xs_entries = ((Kp // 32) * 4) << xrl            # u32x4 entries before sxs
    assert xs_entries * 16 == (Kp * 2) << xrl
    sx_base = xs_entries * 4                        # sxs, in 4-byte words
    kl_base = sx_base + sx_floats(ng, xrl)          # argmax keys: 16 * mt 8-byte words
    assert kl_base % 2 == 0 and (kl_base * 4) % 16 == 0, "keys and hand-off entries aligned"
    end_words = kl_base + 2 * 16 * mt
    limit = (stream_lds_bytes(bits, gs, mt, K, xrl) if parts is None else parts_lds_bytes(bits, gs, mt, K, xrl)) // 4
    assert end_words * 4 == stream_lds_bytes(bits, gs, mt, K, xrl)

    # phase 1: staging, x padding, Σx padding groups
    xw = stage_writes(bits, K, Kp, xrl)
    sw = {(ng << xrl) + t for t in range(SX_PAD << xrl)}
    # phase 2 (after a barrier): the sums read the staged x, write Σx
    sr2, sw2 = sum_x_access(gs, mt, K, xrl)
    assert sr2 <= xw, sorted(sr2 - xw)[:8]
    sw |= sw2
    # phase 3 (after a barrier): the slot loop
    xr3, sr3 = slot_reads(bits, gs, mt, K, xrl)
    assert xr3 <= xw, sorted(xr3 - xw)[:8]
    assert sr3 <= sw, sorted(sr3 - sw)[:8]
    # bounds: x entries (4 words each) and Σx words inside the area before the keys
    assert max(xw | xr3) < xs_entries
    assert max(sw | sr3) < sx_floats(ng, xrl)
    assert end_words <= limit

    if parts is not None:
        # hand-off of a round: parts 1.. of each group write their sums, barrier, part 0 of
        # the group reads the P - 1 entries of its group (decode_parts.hpp, round end)
        p = parts
        hs_base4 = end_words // 4                   # f32x4 entries after the keys
        hs_entries = WAVES * 2 * mt * 64
        writes = set()
        for wave in range(WAVES):
            if wave % p != 0:
                for t in range(2):
                    for mtt in range(mt):
                        for lane in range(64):
                            writes.add(((wave * 2 + t) * mt + mtt) * 64 + lane)
        for wave in range(0, WAVES, p):
            for jj in range(1, p):
                for t in range(2):
                    for mtt in range(mt):
                        for lane in range(64):
                            i = (((wave + jj) * 2 + t) * mt + mtt) * 64 + lane
                            assert i in writes and i < hs_entries
        assert (hs_base4 + hs_entries) * 16 == parts_lds_bytes(bits, gs, mt, K, xrl)


def check_y_area(mt, lds_bytes, pairs=1):
    """stage_pair_lds / flush_pair_lds: wave w's area of `pairs` slots of 16 * mt rows x
    kYAreaStride halfwords after the keys (one slot: each pair stored as it completes; more:
    every pair of the wave's range kept until its stream ends); each slot's 16-byte reads
    find all 8 halfwords written by that slot's 2-byte writes, and every access stays inside
    the wave's own area and the launch's LDS."""
    rows_area = 16 * mt
    pair_bytes = rows_area * Y_AREA_STRIDE * 2
    for wave in range(WAVES):
        lo = lds_bytes + wave * pairs * pair_bytes
        hi = lo + pairs * pair_bytes
        for q in range(pairs):
            base = lo + q * pair_bytes
            written = set()
            for lane in range(64):
                lg, col = lane >> 4, lane & 15
                for t in range(2):
                    for mtt in range(mt):
                        for r in range(4):
                            h = (mtt * 16 + 4 * lg + r) * Y_AREA_STRIDE + t * 16 + col
                            written.add(base + 2 * h)
            assert min(written) >= lo and max(written) + 2 <= hi
            for mtt in range(mt):
                for lane in range(64):
                    m = mtt * 16 + (lane >> 2)
                    c = lane & 3
                    off = base + 2 * (m * Y_AREA_STRIDE + c * 8)
                    assert off % 16 == 0
                    assert all(off + 2 * i in written for i in range(8))   # all 8 halfwords written
                    assert off + 16 <= hi


# staged-row layouts the launchers use: (MT, XRL)
LAYOUTS = [(1, 0), (1, 3), (1, 4), (2, 5)]
WIDTHS = [(2, 32), (3, 32), (3, 64), (4, 32), (4, 64), (4, 128), (5, 64), (6, 32), (8, 32), (8, 64), (8, 128)]


@pytest.mark.parametrize("bits,gs", WIDTHS)
@pytest.mark.parametrize("mt,xrl", LAYOUTS)
def test_every_lds_read_is_written_first(bits, gs, mt, xrl):
    # one group, short rows, the lm_head K, and K that is not a multiple of the slot span
    # (4128 at group 32, 4160 at group 64: the last slot is padded)
    for K in (gs, 3 * gs, 640, 1024, 1408, 4128, 4160):
        if K % gs == 0:
            check_shape(bits, gs, mt, xrl, K)


@pytest.mark.parametrize("bits,gs", [(4, 64), (8, 64), (4, 32), (6, 32), (2, 32), (4, 128)])
@pytest.mark.parametrize("parts", [2, 4, 8])
def test_parts_hand_off_reads_written_sums(bits, gs, parts):
    for (mt, xrl), K in itertools.product(LAYOUTS, (640, 2048, 3072, 4096)):
        if K % gs:
            continue
        check_shape(bits, gs, mt, xrl, K, parts=parts)


@pytest.mark.parametrize("mt,xrl", LAYOUTS)
def test_output_staging_area_inside_lds(mt, xrl):
    for bits, gs, K in [(4, 64, 1024), (8, 32, 1408), (3, 32, 640)]:
        for pairs in (1, 2, 3):
            check_y_area(mt, stream_lds_bytes(bits, gs, mt, K, xrl), pairs)


def test_model_detects_a_missing_pad():
    # the model itself: without the Σx padding groups the last slot's bias reads (at group 128
    # one group per slot, so the MFMA's three unused k lanes reach three groups past the
    # last) find unwritten words; with them the same shape passes
    global SX_PAD
    check_shape(4, 128, 1, 4, 640)
    saved = SX_PAD
    try:
        SX_PAD = 0
        with pytest.raises(AssertionError):
            check_shape(4, 128, 1, 4, 640)
    finally:
        SX_PAD = saved


PREFILL_Y_STRIDE = 136   # kYStride in csrc/prefill.hip


def test_prefill_epilogue_staging():
    """store_wave_tile (csrc/prefill.hip): each wave stages its 64 x 128 outputs as two
    halves of 32 rows in its own 16 KB of the operand buffers; every 16-byte read of a half
    finds its 8 halfwords written by that half's 2-byte writes, reads are 16-byte aligned,
    and every access stays inside the wave's 16 KB."""
    region = 16 * 1024
    for h in range(2):
        written = {}
        for lane in range(64):
            lg, col = lane >> 4, lane & 15
            for ii in range(2):
                for j in range(8):
                    for r in range(4):
                        row_in_half = 16 * ii + 4 * lg + r
                        off = 2 * (row_in_half * PREFILL_Y_STRIDE + 16 * j + col)
                        assert off + 2 <= region
                        assert off not in written
                        written[off] = (32 * h + row_in_half, 16 * j + col)   # (tile row, tile column)
        for q in range(8):
            for lane in range(64):
                lg, col = lane >> 4, lane & 15
                rr = 4 * q + lg
                off = 2 * (rr * PREFILL_Y_STRIDE + 8 * col)
                assert off % 16 == 0 and off + 16 <= region
                # the 8 halfwords are row 32h + rr, columns 8col .. 8col + 7, in order
                assert [written[off + 2 * e] for e in range(8)] == [(32 * h + rr, 8 * col + e) for e in range(8)]
