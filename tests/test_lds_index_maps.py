"""Host checks of the LDS layouts of the multi-query decode passes
(decode_wide_bf16.hip, decode_wide_int8.hip), restated from the kernels'
index formulas: the direct global-to-LDS copies of one 32-position chunk
fill every byte of the staged tile exactly once (a wave's surplus copies go
to a sink), and every operand read -- K rows as matrix-core A operands, V
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
    # every thread converts its share of pieces into the bf16 tiles
    NP = 32 * CPR
    NCONV = (NP + 64 * W - 1) // (64 * W)
    kt, vt = {}, {}
    for tid in range(64 * W):
        for i in range(NCONV):
            pc = min(tid + 64 * W * i, NP - 1)
            r, lp = pc // CPR, pc % CPR
            assert staged[r * D + 16 * (lp ^ (r & (CPR - 1)))] == (r, lp)
            ck = r * D + 8 * ((2 * lp) ^ _bf16_k_swizzle(D, r))
            cv = r * D + 8 * ((2 * lp) ^ _bf16_v_swizzle(D, r))
            for e in range(8):
                kt[ck + e], kt[(ck ^ 8) + e] = (r, 16 * lp + e), (r, 16 * lp + 8 + e)
                vt[cv + e], vt[(cv ^ 8) + e] = (r, 16 * lp + e), (r, 16 * lp + 8 + e)
    assert len(kt) == len(vt) == 32 * D
    _check_bf16_reads(D, kt, vt)
