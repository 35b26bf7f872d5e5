"""Plain restatement of the adaptive draft-length policies (test infrastructure only).

From the page "投機的デコーディングとは：同時リクエストが多いと遅くなる理由", section
vLLM は利用者が書く表で、SGLang は実行中に観測した受理の長さで先読み数を変える, and the
page "LLM推測デコーディング最適化実踐", section 動的推測戦略.  Readings where the pages
are silent (recorded in the design notes): the accepted length of a step is the
batch mean of accepted_count; the moving-average weight is 0.2; batch buckets
have upper bounds 1, 2, 4, 8, 16, 31; a bucket with no data uses the largest
candidate; rounding is half away from zero; the windowed acceptance rate of a
step is its mean accepted count divided by the draft length used.
"""
import math
from collections import deque


def _round_half_away(x):
    return int(math.floor(x + 0.5)) if x >= 0 else -int(math.floor(-x + 0.5))


class ByBatch:
    """A table of (largest batch size, gamma); past the table its last entry."""

    def __init__(self, table=((64, 3), (128, 1), (512, 0))):
        self.table = list(table)

    def next(self, batch):
        for top, g in self.table:
            if batch <= top:
                return g
        return self.table[-1][1]

    def observe(self, counts, gamma_used):
        pass


class Ema:
    def __init__(self, buckets=(1, 2, 4, 8, 16, 31), weight=0.2, candidates=(1, 3, 7), fixed_from=32, fixed=1):
        self.buckets = list(buckets)
        self.weight = weight
        self.lo, self.hi = min(candidates), max(candidates)
        self.fixed_from, self.fixed = fixed_from, fixed
        self.avg = {}

    def _bucket(self, batch):
        for i, top in enumerate(self.buckets):
            if batch <= top:
                return i
        return None

    def next(self, batch):
        if batch >= self.fixed_from:
            return self.fixed
        k = self._bucket(batch)
        if k is None or k not in self.avg:
            return self.hi
        return min(max(_round_half_away(self.avg[k]) + 1, self.lo), self.hi)

    def observe(self, counts, gamma_used):
        batch = len(counts)
        if batch >= self.fixed_from:
            return
        k = self._bucket(batch)
        if k is None:
            return
        mean = sum(int(c) for c in counts) / batch
        self.avg[k] = mean if k not in self.avg else (1 - self.weight) * self.avg[k] + self.weight * mean


class RateWindow:
    """Windowed acceptance rate.  The rule as stated: keep the acceptance rates of
    the most recent `window` steps; when their mean exceeds `raise_above` the draft
    length grows by one, when it falls below `lower_below` it shrinks by one, and
    it never leaves [lo, hi]."""

    def __init__(self, window=100, raise_above=0.85, lower_below=0.65, lo=2, hi=8, start=5):
        self.rates = deque(maxlen=window)          # the most recent rates, oldest first
        self.raise_above, self.lower_below = raise_above, lower_below
        self.lo, self.hi, self.gamma = lo, hi, start

    def next(self, batch):
        return self.gamma

    def _mean_rate(self):
        total = 0.0
        for r in self.rates:                       # oldest first
            total += r
        return total / len(self.rates)

    def observe(self, counts, gamma_used):
        if gamma_used == 0:                        # no drafts: no rate to record
            return
        step_rate = sum(int(c) for c in counts) / len(counts) / gamma_used
        self.rates.append(step_rate)
        m = self._mean_rate()
        step = 1 if m > self.raise_above else (-1 if m < self.lower_below else 0)
        self.gamma = min(max(self.gamma + step, self.lo), self.hi)
