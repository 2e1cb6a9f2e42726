"""Host checks of the LDS layouts of the multi-query decode passes
(decode_wide_bf16.hip, decode_wide_int8.hip), restated from the kernels'
index formulas: the direct global-to-LDS copies of one 32-position chunk
fill every byte of the staged tile exactly once (a wave's surplus copy
slots issue nothing, or go to a sink in rings of three or more buffers), and
every operand read -- K rows as matrix-core A operands, V
through the 16-bit transposed read -- finds the element it stands for.
Exhaustive over d in {64, 128} and 2..8 waves; no GPU."""
import pytest


def _bf16_k_swizzle(D, r):
    return r & (D // 8 - 1)


def _bf16_v_swizzle(D, r):
    return ((r >> 1) & 3) << 1 if D == 64 else (r & 7) << 1


def _check_bf16_reads(D, kt, vt):
    """kt/vt: element offset -> (row, dim) of a staged bf16 chunk."""
    for lane in range(64):
        n, g = lane & 15, lane >> 4
        for mt in range(2):
            for s in range(D // 32):   # K operand: row 16mt + n, dims 32s + 8g .. +7
                off = 16 * mt * D + n * D + ((4 * s + g) ^ _bf16_k_swizzle(D, n)) * 8
                for e in range(8):
                    assert kt[off + e] == (16 * mt + n, 32 * s + 8 * g + e)
        tr_row = 4 * g + (n >> 2)      # transposed V read: rows 4g + n/4 (+16), dims 16t + 4(n%4) .. +3
        for t in range(D // 16):
            vb = tr_row * D + ((2 * t + ((n & 3) >> 1)) ^ _bf16_v_swizzle(D, tr_row)) * 8 + 4 * (n & 1)
            for hi in range(2):
                for e in range(4):
                    assert vt[vb + 16 * D * hi + e] == (tr_row + 16 * hi, 16 * t + 4 * (n & 3) + e)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("W", range(2, 9))
def test_wide_bf16_copies_and_reads(D, W):
    LPR, RPW = D // 8, 64 // (D // 8)
    NINST = 32 // RPW
    NI = (NINST + W - 1) // W
    kt, vt = {}, {}
    for wave in range(W):
        for c in range(NI):
            i = wave + c * W
            ir = i % NINST
            for lane in range(64):
                r, ph = (64 * ir + lane) // LPR, lane % LPR
                assert r // RPW == ir                      # one RPW-row group per instruction
                if i >= NINST:
                    continue                               # surplus copy: into the sink
                base = 512 * i + 8 * lane                  # lane l lands at 16 l bytes
                assert base == r * D + 8 * ph
                for e in range(8):
                    assert base + e not in kt
                    kt[base + e] = (r, 8 * (ph ^ _bf16_k_swizzle(D, r)) + e)
                    vt[base + e] = (r, 8 * (ph ^ _bf16_v_swizzle(D, r)) + e)
    assert len(kt) == len(vt) == 32 * D
    _check_bf16_reads(D, kt, vt)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("W", range(2, 9))
def test_wide_int8_copies_conversion_and_reads(D, W):
    CPR, LPR = D // 16, D // 8
    NINST = 32 * D // 1024
    NI = (NINST + W - 1) // W
    staged = {}
    for wave in range(W):
        for c in range(NI):
            i = wave + c * W
            if i >= NINST:
                continue
            for lane in range(64):
                pc = 64 * i + lane
                r, ph = pc // CPR, pc % CPR
                assert 1024 * i + 16 * lane == r * D + 16 * ph
                staged[r * D + 16 * ph] = (r, ph ^ (r & (CPR - 1)))   # logical 16-code piece
    assert len(staged) == 32 * CPR
    # conversion units: the K pieces, then the V pieces, one thread each;
    # whole waves past the last unit convert nothing, and no bf16 element is
    # written twice
    NP = 32 * CPR
    NU = 2 * NP
    NCONV = (NU + 64 * W - 1) // (64 * W)
    kt, vt = {}, {}
    for tid in range(64 * W):
        for i in range(NCONV):
            u = tid + 64 * W * i
            first = (tid - tid % 64) + 64 * W * i            # lane 0 of this thread's wave
            assert (u < NU) == (first < NU)                  # activity is wave-uniform
            if u >= NU:
                continue
            isv = u >= NP
            assert isv == (first >= NP)                      # so is the tensor
            pc = u - NP if isv else u
            r, lp = pc // CPR, pc % CPR
            assert staged[r * D + 16 * (lp ^ (r & (CPR - 1)))] == (r, lp)
            tile = vt if isv else kt
            dst = r * D + 8 * ((2 * lp) ^ (_bf16_v_swizzle(D, r) if isv else _bf16_k_swizzle(D, r)))
            for e in range(8):
                for off, val in ((dst + e, (r, 16 * lp + e)), ((dst ^ 8) + e, (r, 16 * lp + 8 + e))):
                    assert off not in tile
                    tile[off] = val
    assert len(kt) == len(vt) == 32 * D
    _check_bf16_reads(D, kt, vt)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("W", range(1, 9))
def test_f32_copies_and_reads(D, W):
    """fp32 pass (decode_f32.hip): 16-byte chunks of fp32 rows, K chunk ^
    (row % 16), V chunk ^ 4 ((row / 4) % 4); K read as float4 pieces of row
    16mt + n, V read one float per product; also the bank groups of the K
    reads (16 lanes of a lane group) and of the V reads (all 64 lanes)."""
    CPR = D // 4
    NINST = 32 * D // 256
    NI = (NINST + W - 1) // W
    kt, vt = {}, {}
    for wave in range(W):
        for c in range(NI):
            i = wave + c * W
            ir = i % NINST
            for lane in range(64):
                r, ph = (64 * ir + lane) // CPR, lane % CPR
                if i >= NINST:
                    continue                                   # surplus copy: into the sink
                base = 256 * i + 4 * lane                      # lane l lands at 16 l bytes
                assert base == r * D + 4 * ph
                for e in range(4):
                    assert base + e not in kt
                    kt[base + e] = (r, 4 * (ph ^ (r & 15)) + e)
                    vt[base + e] = (r, 4 * (ph ^ (((r >> 2) & 3) << 2)) + e)
    assert len(kt) == len(vt) == 32 * D
    for mt in range(2):
        for j in range(D // 16):
            banks = {}
            for lane in range(64):
                n, g = lane & 15, lane >> 4
                off = 16 * mt * D + n * D + 4 * ((4 * j + g) ^ n)
                for c in range(4):                             # product (j, c): dim 16j + 4g + c
                    assert kt[off + c] == (16 * mt + n, 16 * j + 4 * g + c)
                banks.setdefault(g, set()).add((off * 4 // 16) % 16)   # 16-byte bank group
            assert all(len(v) == 16 for v in banks.values())
    for mt in range(2):
        for i in range(4):
            for t in range(D // 16):
                banks = set()
                for lane in range(64):
                    n, g = lane & 15, lane >> 4
                    vb = 4 * g * D + 4 * ((4 * t + (n >> 2)) ^ (g << 2)) + (n & 3)
                    off = vb + (16 * mt + i) * D
                    assert vt[off] == (16 * mt + 4 * g + i, 16 * t + n)
                    banks.add(off % 64)                        # 64 four-byte banks
                assert len(banks) == 64


@pytest.mark.parametrize("D", [64, 128])
def test_f32_prefill_copies_and_reads(D):
    """fp32 prefill (prefill_f32.hip): 32-key tiles copied by the four waves
    (copy r of wave w is instruction w + 4r), the fp32 decode pass's
    swizzles; every element lands once and every K / V read finds it."""
    CPR = D // 4
    COPIES = 32 * D // 256 // 4
    kt, vt = {}, {}
    for wave in range(4):
        for r in range(COPIES):
            i = wave + 4 * r
            for lane in range(64):
                c = 64 * i + lane
                row, cp = c // CPR, c % CPR
                base = 256 * i + 4 * lane
                assert base == row * D + 4 * cp
                for e in range(4):
                    assert base + e not in kt
                    kt[base + e] = (row, 4 * (cp ^ (row & 15)) + e)
                    vt[base + e] = (row, 4 * (cp ^ (((row >> 2) & 3) << 2)) + e)
    assert len(kt) == len(vt) == 32 * D
    for lane in range(64):
        n, g = lane & 15, lane >> 4
        for mt in range(2):
            for jj in range(D // 16):
                off = 16 * mt * D + n * D + 4 * ((4 * jj + g) ^ n)
                for c in range(4):
                    assert kt[off + c] == (16 * mt + n, 16 * jj + 4 * g + c)
            for i in range(4):
                for t in range(D // 16):
                    vb = 4 * g * D + 4 * ((4 * t + (n >> 2)) ^ (g << 2)) + (n & 3)
                    assert vt[vb + (16 * mt + i) * D] == (16 * mt + 4 * g + i, 16 * t + n)
