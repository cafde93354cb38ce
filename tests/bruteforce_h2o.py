"""Pure-Python brute force of the H2O chunk step, for tiny inputs only.

Written with lists, ``math.exp`` and ``sorted`` on (score, index) tuples -- no
numpy -- so that it shares no routine with the fp64 oracle it pins.  It follows
the same page definitions (softmax attention over the occupied slots plus the
chunk's own keys causally, summed weights over queries and the heads of each KV
group, cumulative H2O scores, bottom-T eviction with ties to the lower slot
index, left-to-right fill, seeding new slots with their own sums).
"""

import math


def _dot(a, b):
    s = 0.0
    for x, y in zip(a, b):
        s += x * y
    return s


class BruteCache:
    """policy: "h2o" (rank by the score), "h2o_norm" (score divided by the
    number of queries that have seen the slot so far) or "h2o_orig" (score
    summed over the batch rows; every row evicts the same slots)."""

    def __init__(self, B, Hq, Hkv, D, C, scale, policy="h2o"):
        self.policy = policy
        self.B, self.Hq, self.Hkv, self.D, self.C = B, Hq, Hkv, D, C
        self.qg = Hq // Hkv
        self.scale = scale
        self.k = [[[[0.0] * D for _ in range(C)] for _ in range(Hkv)] for _ in range(B)]
        self.v = [[[[0.0] * D for _ in range(C)] for _ in range(Hkv)] for _ in range(B)]
        self.phi = [[[0.0] * C for _ in range(Hkv)] for _ in range(B)]
        self.tpos = [[[-1] * C for _ in range(Hkv)] for _ in range(B)]
        self.n_occ = 0
        self.pos = 0

    def step(self, q, kn, vn):
        """q[b][h][i][d], kn[b][g][t][d], vn[b][g][t][d] as nested lists of floats."""
        B, Hq, D, C = self.B, self.Hq, self.D, self.C
        T = len(q[0][0])
        n = self.n_occ
        out = [[[[0.0] * D for _ in range(T)] for _ in range(Hq)] for _ in range(B)]
        w = [[[0.0] * (n + T) for _ in range(self.Hkv)] for _ in range(B)]
        for b in range(B):
            for h in range(Hq):
                g = h // self.qg
                for i in range(T):
                    keys = [self.k[b][g][j] for j in range(n)] + [kn[b][g][t] for t in range(i + 1)]
                    vals = [self.v[b][g][j] for j in range(n)] + [vn[b][g][t] for t in range(i + 1)]
                    logits = [self.scale * _dot(q[b][h][i], kk) for kk in keys]
                    mx = max(logits)
                    e = [math.exp(x - mx) for x in logits]
                    tot = sum(e)
                    for jj in range(len(e)):
                        p = e[jj] / tot
                        w[b][g][jj] += p
                        for d in range(D):
                            out[b][h][i][d] += p * vals[jj][d]
        for b in range(B):
            for g in range(self.Hkv):
                for j in range(n):
                    self.phi[b][g][j] += w[b][g][j]
        slots = []
        for b in range(B):
            srow = []
            for g in range(self.Hkv):
                if n + T <= C:
                    chosen = list(range(n, n + T))
                else:
                    def rank(j):
                        if self.policy == "h2o_orig":
                            return sum(self.phi[bb][g][j] for bb in range(B))
                        if self.policy == "h2o_norm":
                            seen = self.pos + T - self.tpos[b][g][j]  # queries that have attended slot j
                            return self.phi[b][g][j] / seen
                        return self.phi[b][g][j]
                    ranked = sorted((rank(j), j) for j in range(C))
                    chosen = sorted(j for _, j in ranked[:T])
                srow.append(chosen)
            slots.append(srow)
        for b in range(B):
            for g in range(self.Hkv):
                chosen = slots[b][g]
                for t, j in enumerate(chosen):
                    self.k[b][g][j] = list(kn[b][g][t])
                    self.v[b][g][j] = list(vn[b][g][t])
                    self.phi[b][g][j] = w[b][g][n + t]
                    self.tpos[b][g][j] = self.pos + t
        self.n_occ = min(n + T, C)
        self.pos += T
        return out, w, slots
