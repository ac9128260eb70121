"""The chunk kernel's helper schedule (csrc/fi_chunk.h), replayed on the CPU
with the kernel's own index formulas: during position i the helpers pull, for
target i+1, the lags k = seg + 8m of their first 8 or 16 taps, and (chunks of
256) push the source i-1 along lags 128..255 into its later targets.  Every
pair (s, t) of a chunk with lag t - s >= 2 must be formed exactly once, from a
source already known and before position t; every LDS row touched must be a
slot, or a zero row for the pulled lags that reach before the chunk.  (Lag 1 is
the red-cell lane's own term.)  The gray blocks below G cover exactly these
pairs ([S] "Kachelung-Strategie (Algorithmus 1)")."""
import collections
import os
import re

import pytest

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "long_convolution_sequence_amd",
                   "csrc", "fi_chunk.h")


def _pull_taps():
    """kChunkPullTaps as the kernel header sets it."""
    return int(re.search(r"constexpr int kChunkPullTaps = (\d+);", open(HDR).read()).group(1))


PULL_TAPS, TAPS, ZERO_ROWS = _pull_taps(), 32, 64


def _schedule(G):
    cov = collections.Counter()
    when = {}
    for i in range(G):
        if i + 1 < G:
            nt = 8 * (min((i + 2) >> 6, PULL_TAPS // 8 - 1) + 1)
            for seg in range(8):
                for m in range(nt):
                    k = seg + 8 * m
                    if k < 2 or k >= G:
                        continue                              # tap register zeroed
                    row = G - 2 - i + seg + 8 * m
                    assert row <= G + ZERO_ROWS - 1
                    s = i + 1 - k
                    if s < 0:
                        assert row >= G                       # a zero row
                        continue
                    cov[(s, i + 1)] += 1
                    when[(s, i + 1)] = i
        if G > 8 * PULL_TAPS and 1 <= i <= G - 8 * PULL_TAPS:
            c = min(TAPS - PULL_TAPS, max(0, ((G - i - 7) >> 3) - PULL_TAPS + 1))
            for seg in range(8):
                row16 = G - i - seg - 8 * PULL_TAPS
                ms = list(range(PULL_TAPS, PULL_TAPS + c))
                if PULL_TAPS + c < TAPS and row16 - 8 * c >= 0:
                    ms.append(PULL_TAPS + c)
                for m in range(PULL_TAPS, TAPS):
                    t = i - 1 + seg + 8 * m
                    assert (t <= G - 1) == (m in ms)          # exactly the lane's targets in the chunk
                for m in ms:
                    t = i - 1 + seg + 8 * m
                    row = row16 - 8 * (m - PULL_TAPS)
                    assert row == G - 1 - t and 0 <= row <= G - 1
                    cov[(i - 1, t)] += 1
                    when[(i - 1, t)] = i
    return cov, when


@pytest.mark.parametrize("G", [4, 8, 16, 32, 64, 128, 256])
def test_chunk_helpers_form_every_pair_once_in_time(G):
    cov, when = _schedule(G)
    for t in range(G):
        for s in range(t - 1):
            assert cov[(s, t)] == 1, (s, t)
            assert s + 1 <= when[(s, t)] <= t - 1, (s, t)
    assert all(t - s >= 2 for (s, t) in cov)


def test_pulled_and_pushed_work_per_position():
    """Pulling every lag would give position i of a chunk of 256 i pulled pairs
    per row (255 at the end); the split caps the pulled pairs at K - 2 and the
    pushed ones at 256 - K."""
    K = 8 * PULL_TAPS
    cov, when = _schedule(256)
    pulled = collections.Counter(i for (s, t), i in when.items() if t == i + 1)
    pushed = collections.Counter(i for (s, t), i in when.items() if t != i + 1)
    assert max(pulled.values()) == K - 2
    assert max(pushed.values(), default=0) == 256 - K
