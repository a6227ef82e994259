"""The arithmetic that shares the cache forward's key tiles among waves (CPU only).

The split kernel lays the valid 32-key tiles of all (b, h) end to end, gives wave w of G
the tiles [w T / G, (w + 1) T / G) with G = min(launched waves, T), and stores the partial
result of each (wave, (b, h)) piece in slot w + bh; the merge kernel finds the waves of a
(b, h) as w(g) = floor(((g + 1) G - 1) / T) for its first and last tile g. These tests
enumerate small configurations by brute force and check what the kernels rely on: no wave
is empty, w(g) is the wave holding tile g, every piece has its own slot, the slots stay
below min(2048, tiles of a full cache) + B H - 1 (the workspace formula), and the merge's
wave range is exactly the set of waves holding tiles of the (b, h).
"""
import random

import pytest

MAX_WAVES = 2048
KT = 32


def _check(lens, H, launched, Nk, slot=lambda w, b, h, H: w + b * H + h):
    tiles = [(L + KT - 1) // KT for L in lens]
    B = len(lens)
    BH = B * H
    T = H * sum(tiles)
    G = min(launched, T)
    if T == 0:
        return
    starts = [w * T // G for w in range(G + 1)]
    assert all(starts[w + 1] > starts[w] for w in range(G)), "a wave without tiles"
    seq = [(b, h) for b in range(B) for h in range(H) for _ in range(tiles[b])]
    pieces = {}
    for w in range(G):
        for g in range(starts[w], starts[w + 1]):
            assert ((g + 1) * G - 1) // T == w
            b, h = seq[g]
            pieces.setdefault((w, b * H + h), 0)
    slots = [slot(w, bh // H, bh % H, H) for (w, bh) in pieces]
    assert len(set(slots)) == len(slots), "two pieces share a slot"
    wave_cap = min(MAX_WAVES, max(B * H * ((Nk + KT - 1) // KT), 1))
    assert launched <= wave_cap
    assert max(slots) < wave_cap + BH - 1
    prefix = [H * sum(tiles[:b]) for b in range(B)]
    for b in range(B):
        for h in range(H):
            bh = b * H + h
            held = sorted(w for (w, x) in pieces if x == bh)
            if tiles[b] == 0:
                assert not held
                continue
            g0 = prefix[b] + h * tiles[b]
            g1 = g0 + tiles[b] - 1
            w0 = ((g0 + 1) * G - 1) // T
            w1 = ((g1 + 1) * G - 1) // T
            assert held == list(range(w0, w1 + 1))


@pytest.mark.parametrize("seed", range(4))
def test_tile_runs_slots_and_merge_ranges(seed):
    rng = random.Random(seed)
    for _ in range(150):
        B, H = rng.randint(1, 9), rng.randint(1, 5)
        Nk = rng.choice([1, 31, 32, 33, 100, 500, 1000])
        lens = [min(rng.choice([0, 1, 31, 32, 33, rng.randint(0, Nk)]), Nk) for _ in range(B)]
        wave_cap = min(MAX_WAVES, B * H * ((Nk + KT - 1) // KT))
        for launched in {1, 2, 3, 7, 64, wave_cap}:
            _check(lens, H, min(launched, wave_cap), Nk)


def test_full_caches_many_heads():
    # 1024 (b, h) of two tiles each over 1024 waves: one piece per wave, slots w + bh
    _check([40] * 64, 16, 1024, 40)


def test_planted_slot_mistake_is_caught():
    # slot w + b (the batch instead of the (b, h) index) gives the pieces of two heads of
    # one batch inside one wave the same slot: 4 batches x 4 heads of 2 tiles over 8 waves,
    # so every wave holds two heads of one batch
    with pytest.raises(AssertionError, match="share a slot"):
        _check([40] * 4, 4, 8, 40, slot=lambda w, b, h, H: w + b)
