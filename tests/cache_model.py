"""Plain Python statement of the tiered-residency replacement rule (test reference)."""


class Model:
    """LFU with recency: hits add a use; a miss takes an empty slot (lowest index), else the
    slot not used by the call with the fewest uses, then the oldest last use, then the lowest
    index, and starts at one use."""

    def __init__(self, E, S):
        self.where = [-1] * E
        self.expert = [-1] * S
        self.count = [0] * S
        self.last = [0] * S
        self.tick = 0
        self.hits = self.misses = 0

    def plan(self, ids):
        distinct = list(dict.fromkeys(int(i) for i in ids))
        assert len(distinct) <= len(self.expert)
        self.tick += 1
        used = set()
        for e in distinct:
            if self.where[e] >= 0:
                s = self.where[e]
                self.count[s] += 1
                self.last[s] = self.tick
                used.add(s)
                self.hits += 1
        fills = []
        for e in distinct:
            if self.where[e] >= 0:
                continue
            empty = [s for s in range(len(self.expert)) if self.expert[s] < 0]
            if empty:
                v = empty[0]
            else:
                v = min((s for s in range(len(self.expert)) if s not in used),
                        key=lambda s: (self.count[s], self.last[s], s))
            if self.expert[v] >= 0:
                self.where[self.expert[v]] = -1
            self.expert[v] = e
            self.where[e] = v
            self.count[v] = 1
            self.last[v] = self.tick
            used.add(v)
            self.misses += 1
            fills.append((e, v))
        return [self.where[int(i)] for i in ids], fills
