"""A seeded walk over prefix sharing: sequences start fresh or as a fork of a
live sequence's first n tokens, append a few tokens at a time (copy on write
of shared blocks), and end.  The library's host calls keep the table, the
free list and the counts; the walk keeps every live sequence's own tokens
(its dense history) and a CPU model of the pools built from oracle
operations only, so that after each step

  * the bookkeeping satisfies oracle.paging.refcount_problems, and
  * every live row gathers its own history from the model pools.

Each step returns what a device copy of the cache needs to follow it: table
patches, block copies (before the step's append) and the appended tokens."""
import numpy as np

import paged_kv_attention_17_amd as pkv
from paged_kv_attention_17_amd import workloads as W
from oracle import paging


class SharingWalk:
    def __init__(self, seed, n_slots=8, max_blocks=12, num_blocks=160, n_kv=8):
        self.rng = np.random.default_rng(seed)
        self.n_kv = n_kv
        self.bt = np.full((n_slots, max_blocks), -1, np.int32)
        self.refcount = np.zeros(num_blocks, np.int32)
        self.free = self.rng.permutation(num_blocks).astype(np.int32)
        self.n_free = num_blocks
        self.k_pool = np.full((num_blocks, 16, n_kv, 64), W.BF16_POISON, np.uint16)
        self.v_pool = self.k_pool.copy()
        self.hist = {}          # slot -> (K rows, V rows), each [n][n_kv][64] bits
        self.max_tokens = max_blocks * 16
        self.n_forks = 0        # sequences started as a fork
        self.n_copies = 0       # copy-on-write block copies

    def live(self):
        return sorted(self.hist)

    def check(self):
        problems = paging.refcount_problems([self.bt], self.refcount, self.free[:self.n_free])
        assert problems == [], problems
        for s, (K, V) in self.hist.items():
            n = len(K)
            np.testing.assert_array_equal(paging.gather(self.k_pool, self.bt[s], n), K)
            np.testing.assert_array_equal(paging.gather(self.v_pool, self.bt[s], n), V)
            nb = -(-n // 16)
            assert (self.bt[s, nb:] == -1).all()

    def step(self):
        """One step: maybe end a sequence, maybe start one (fresh or forked),
        then let some live sequences append 1..3 tokens each.  Returns a dict
        with 'patches' (offsets, values), 'copies' (src, dst) and the append
        ('slots', 'positions', 'k', 'v'), in the order a device must apply
        them: patches of the release and fork, copies, then the append's
        patches and the append itself (all patches may be applied together,
        before the copies: a copy reads and writes blocks, not the table)."""
        rng = self.rng
        offs, vals = [], []
        live = self.live()
        if live and rng.random() < 0.25:
            s = int(rng.choice(live))
            self.n_free, o, v = pkv.pkv_blocks_release_shared(self.bt, s, self.free, self.n_free, self.refcount)
            offs += list(o)
            vals += list(v)
            del self.hist[s]
        idle = [s for s in range(self.bt.shape[0]) if s not in self.hist]
        if idle and rng.random() < 0.6:
            d = int(rng.choice(idle))
            donors = [s for s in self.live() if len(self.hist[s][0]) > 0]
            if donors and rng.random() < 0.75:
                src = int(rng.choice(donors))
                n = int(rng.integers(1, len(self.hist[src][0]) + 1))
                o, v = pkv.pkv_blocks_share(self.bt, src, d, n, self.refcount)
                offs += list(o)
                vals += list(v)
                K, V = self.hist[src]
                self.hist[d] = (K[:n].copy(), V[:n].copy())
                self.n_forks += 1
            else:
                self.hist[d] = (np.zeros((0, self.n_kv, 64), np.uint16), np.zeros((0, self.n_kv, 64), np.uint16))
        slots, positions = [], []
        for s in self.live():
            n = len(self.hist[s][0])
            if rng.random() < 0.7:
                m = int(min(rng.integers(1, 4), self.max_tokens - n))
                slots += [s] * m
                positions += list(range(n, n + m))
        slots = np.array(slots, np.int32)
        positions = np.array(positions, np.int32)
        T = len(slots)
        k_new = W.randn_bf16(rng, (T, self.n_kv, 64))
        v_new = W.randn_bf16(rng, (T, self.n_kv, 64))
        cs = cd = np.zeros(0, np.int32)
        if T:
            self.n_free, o, v, cs, cd = pkv.pkv_blocks_assign_shared(self.bt, self.free, self.n_free, self.refcount,
                                                                     slots, positions)
            offs += list(o)
            vals += list(v)
            self.n_copies += len(cs)
            self.k_pool, self.v_pool = paging.copy_blocks(self.k_pool, self.v_pool, cs, cd)
            self.k_pool, self.v_pool = paging.append(self.k_pool, self.v_pool, k_new, v_new, self.bt, slots, positions)
            for t, s in enumerate(slots):
                K, V = self.hist[int(s)]
                self.hist[int(s)] = (np.concatenate([K, k_new[t:t + 1]]), np.concatenate([V, v_new[t:t + 1]]))
        return dict(patches=(np.array(offs, np.int32), np.array(vals, np.int32)), copies=(cs, cd),
                    slots=slots, positions=positions, k=k_new, v=v_new)
