"""Host model of the flat work split shared by the decode partition passes
and the combine pass (the rules of grouped_query_kv_amd/csrc/decode_flat.h,
restated in Python): every valid cached position of every (sequence, KV
head) pair is covered by exactly one workgroup segment, segments start on
32-position boundaries, partial slots are distinct and below n_wg + B*K,
and the combine's slot range for a pair is exactly the set of slots the
partition pass wrote for it."""
import random

import pytest


def pad32(L):
    return (L + 31) & ~31


def flat_range(total, n_wg, row_bytes, r_min, r_max):
    r = pad32((total + n_wg - 1) // n_wg)
    r = max(r, r_min)
    if (r * row_bytes) % 65536 == 0:
        r += 32
    if r > r_max:
        r = r_max
        if (r * row_bytes) % 65536 == 0 and r > 32:
            r -= 32
    return r


def segments(lens, K, n_wg, row_bytes, r_min=32, r_max=1 << 30):
    """(w, b, k, t0, t1, slot) for every segment, as the partition passes walk them."""
    B = len(lens)
    total = K * sum(pad32(L) for L in lens)
    R = flat_range(total, n_wg, row_bytes, r_min, r_max)
    starts, run = [], 0
    for L in lens:
        starts.append(run)
        run += K * pad32(L)
    out = []
    for w in range(n_wg):
        pos, end = w * R, min(w * R + R, total)
        if pos >= end:
            continue
        b = next(i for i in range(B) if starts[i] + K * pad32(lens[i]) > pos)
        L, Lp = lens[b], pad32(lens[b])
        k = (pos - starts[b]) // Lp
        base = starts[b] + k * Lp
        while True:
            t0, t1 = pos - base, min(end - base, L)
            if t0 < t1:
                out.append((w, b, k, t0, t1, w + b * K + k))
            pos = base + Lp
            if pos >= end:
                break
            k += 1
            if k == K:
                k = 0
                b += 1
                while b < B and lens[b] == 0:
                    b += 1
                if b >= B:
                    break
                L, Lp = lens[b], pad32(lens[b])
            base = pos
    return out, R, total, starts


def combine_slots(lens, K, b, k, R, starts):
    L = lens[b]
    if L == 0:
        return []
    base = starts[b] + k * pad32(L)
    w0, w1 = base // R, (base + L - 1) // R
    return [w + b * K + k for w in range(w0, w1 + 1)]


CASES = [
    ([8193] * 16, 8, 2048, 256),                 # Llama-3-8B layer
    ([131073] * 4, 8, 2048, 256),                # long context
    ([0, 1, 31, 32, 33, 700, 4095], 4, 64, 128),
    ([0, 0, 0, 5], 2, 3, 256),
    ([1], 1, 512, 256),
    ([300, 45], 8, 2048, 256),
]


def _rand_cases():
    rng = random.Random(7)
    out = []
    for _ in range(40):
        B = rng.randint(1, 80)
        K = rng.choice([1, 2, 4, 8])
        lens = [rng.choice([0, rng.randint(1, 40), rng.randint(1, 5000)]) for _ in range(B)]
        out.append((lens, K, rng.choice([1, 7, 64, 512, 2048, 3072]), rng.choice([64, 128, 256, 512])))
    return out


@pytest.mark.parametrize("lens,K,n_wg,row_bytes", CASES + _rand_cases())
def test_flat_split_covers_each_position_once(lens, K, n_wg, row_bytes):
    segs, R, total, starts = segments(lens, K, n_wg, row_bytes)
    assert R % 32 == 0 and (total == 0 or (total + R - 1) // R <= n_wg)
    cover = {}
    slots = set()
    for w, b, k, t0, t1, slot in segs:
        assert t0 % 32 == 0 and 0 <= t0 < t1 <= lens[b]
        assert t1 - t0 <= R
        assert slot not in slots and slot < n_wg + len(lens) * K
        slots.add(slot)
        cover.setdefault((b, k), []).append((t0, t1, slot))
    for b, L in enumerate(lens):
        for k in range(K):
            got = sorted(cover.get((b, k), []))
            pos = 0
            for t0, t1, _ in got:
                assert t0 == pos
                pos = t1
            assert pos == L
            assert sorted(s for _, _, s in got) == combine_slots(lens, K, b, k, R, starts)


def test_flat_split_paged_cap():
    """With a capped range (paged: block ids of a segment fit one per lane)
    the host's workgroup count still covers the largest total."""
    bs, max_len, B, K = 16, 5000, 3, 2
    r_max = 63 * bs // 32 * 32
    r = r_max - 32
    n_wg = max(64, -(-K * B * pad32(max_len) // r))
    segs, R, total, _ = segments([max_len] * B, K, n_wg, 256, r_max=r_max)
    assert R <= r_max and (total + R - 1) // R <= n_wg
    for _, _, _, t0, t1, _ in segs:
        assert (t1 - 1) // bs - t0 // bs + 1 <= 64  # blocks of a segment fit one per lane
