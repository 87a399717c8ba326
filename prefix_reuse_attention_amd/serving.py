"""A stream of recommendation queries served through the prefix-mode choice,
the paged caches and the prefill, all on the library's entry points.

The Bat page ("The idea", "Why it works") has a hotness-aware scheduler pick
each query's prefix (the user's history or the query's items) under memory
limits, with user-prefix and item-prefix caches in separate pools.  Per
query, in arrival order:

1. bat_sched_step chooses the mode and updates its pools (which users and
   items are resident, and the item-pool slot of each resident item);
2. this module keeps the physical places of what the pools hold -- the
   user-pool blocks of each resident user (a free list over the pool's
   blocks: a user is given ceil(n_u / block) of them when admitted and
   gives them back when evicted), the slot the scheduler named for each item
   -- and a transient region of each pool for prefixes that are computed but
   not kept;
3. every prefix the query computes is written into its place with
   bat_kv_build, its prefix rows are computed (bat_attn_prefix_rows for a
   user, bat_attn_item_local for items: the next layer's keys/values come
   from them), and bat_attn_prefill runs the query's suffix over its prefix,
   read from the pools through the block table.

Queries are grouped into sub-batches, each one launch of the prefill after
its cache writes.  A sub-batch ends before any write into a block or slot
that one of its queries reads (an eviction in the same window), so every
query reads exactly the cache the scheduler's order implies.

Only host bookkeeping lives here; every step on the data runs in the HIP
kernels behind the C ABI.  Token activations are synthetic
(workloads.entity_tokens): an entity has the same tokens in every query.
"""
from dataclasses import dataclass, field

import numpy as np

from . import api
from . import workloads as W


@dataclass
class Query:
    r: int                 # position in the stream
    mode: int              # W.USER or W.ITEM
    user: int
    items: np.ndarray      # the query's item ids, in order
    prefix_places: list    # user-pool blocks (user mode) or item-pool slots (item mode)
    prefix_len: int
    suffix_len: int


@dataclass
class SubBatch:
    user_writes: list = field(default_factory=list)   # (user, blocks)
    item_writes: list = field(default_factory=list)   # (item, slot)
    queries: list = field(default_factory=list)


class Placement:
    """Physical places of the scheduler's pools, and the plan of a stream of
    queries as sub-batches of cache writes and one prefill each."""

    def __init__(self, sched, user_len, T, user_block, user_capacity_blocks, item_capacity,
                 transient_user_blocks, transient_item_slots):
        self.sched = sched
        self.user_len = np.asarray(user_len)
        self.T, self.bs = int(T), int(user_block)
        self.ucap, self.icap = int(user_capacity_blocks), int(item_capacity)
        self.tu, self.ti = int(transient_user_blocks), int(transient_item_slots)
        self.free = list(range(self.ucap - 1, -1, -1))   # pop() hands out the lowest block
        self.blocks_of = {}                              # resident user -> its blocks
        res, slot_item = sched.pools()
        self.resident = [int(u) for u in res]
        self.slot_item = np.asarray(slot_item).copy()
        for u in self.resident:                          # residents already in the pools
            self.blocks_of[u] = [self.free.pop() for _ in range(self._nb(u))]

    def _nb(self, u):
        return -(-int(self.user_len[u]) // self.bs)

    @property
    def user_pool_blocks(self):
        return self.ucap + self.tu

    @property
    def item_pool_slots(self):
        return self.icap + self.ti

    def plan(self, users, items, first_r=0):
        """Serve the queries (users [R], items [R, m]) in order; returns the
        sub-batches and the scheduler's per-query outputs."""
        users = np.asarray(users, np.int32)
        items = np.asarray(items, np.int32)
        subs = [SubBatch()]
        reads_u, reads_i = set(), set()
        t_user, t_item = [self.ucap], [self.icap]        # transient cursors
        outs = []

        def flush():
            subs.append(SubBatch())
            reads_u.clear()
            reads_i.clear()
            t_user[0], t_item[0] = self.ucap, self.icap

        for r in range(len(users)):
            u, its = int(users[r]), items[r]
            o = self.sched.step(users[r:r + 1], items[r:r + 1])
            outs.append(o)
            res, slot_item = self.sched.pools()
            res = [int(x) for x in res]
            mode = int(o["mode"][0])
            n_u = int(self.user_len[u])
            m = len(its)
            if mode == W.USER:
                for v in set(self.resident) - set(res):          # evicted: blocks free
                    self.free.extend(self.blocks_of.pop(v))
                    self.free.sort(reverse=True)
                if o["user_hit"][0]:
                    places = self.blocks_of[u]
                else:
                    if u in res:                                  # admitted
                        places = [self.free.pop() for _ in range(self._nb(u))]
                        self.blocks_of[u] = places
                    else:                                         # computed, not kept
                        assert self._nb(u) <= self.tu, "transient user region too small"
                        if t_user[0] + self._nb(u) > self.ucap + self.tu:
                            flush()
                        places = list(range(t_user[0], t_user[0] + self._nb(u)))
                        t_user[0] += self._nb(u)
                    if reads_u.intersection(places):
                        flush()
                    subs[-1].user_writes.append((u, places))
                q = Query(first_r + r, mode, u, its.copy(), places, n_u, m * self.T)
                reads_u.update(places)
            else:
                slots = [int(x) for x in o["item_slot"][0]]
                admitted = {s_ for s_, i in zip(slots, its) if s_ >= 0 and self.slot_item[s_] != i}
                n_t = sum(1 for s_ in slots if s_ < 0)
                assert n_t <= self.ti, "transient item region too small"
                if reads_i.intersection(admitted) or t_item[0] + n_t > self.icap + self.ti:
                    flush()
                places = []
                for s_, i in zip(slots, its):
                    if s_ < 0:                                    # computed, not kept
                        s_ = t_item[0]
                        t_item[0] += 1
                        subs[-1].item_writes.append((int(i), s_))
                    elif s_ in admitted:                          # admitted into slot s_
                        subs[-1].item_writes.append((int(i), s_))
                    places.append(s_)
                q = Query(first_r + r, mode, u, its.copy(), places, m * self.T, n_u)
                reads_i.update(places)
            self.resident = res
            self.slot_item = np.asarray(slot_item).copy()
            subs[-1].queries.append(q)
        return [s for s in subs if s.queries or s.user_writes or s.item_writes], outs


class DeviceWindow:
    """The device buffers of planned sub-batches; run() is one pass over
    them: per sub-batch, the cache writes, the prefix rows of what the
    queries compute, then the prefill."""

    def __init__(self, placement, subs, user_pool, item_pool, seed, H, D, scale,
                 prefix_rows=True):
        import torch
        from .device import to_device
        self.p, self.subs = placement, subs
        self.user_pool, self.item_pool = user_pool, item_pool
        self.H, self.D, self.scale = H, D, float(scale)
        T = placement.T
        cache = {}

        def toks(kind, ident):
            key = (kind, ident)
            if key not in cache:
                n = int(placement.user_len[ident]) if kind == W.USER_STREAM else T
                cache[key] = W.entity_tokens(seed, kind, ident, n, H, D)
            return cache[key]

        def dev(a):
            return to_device(np.ascontiguousarray(a), "bf16")

        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()
        self.calls = []
        self.prefills = []    # (queries, prefill arguments) per sub-batch
        for sb in subs:
            calls = []
            if sb.user_writes:
                ks = [toks(W.USER_STREAM, u) for u, _ in sb.user_writes]
                lens = [len(k[1]) for k in ks]
                nb = max(len(b) for _, b in sb.user_writes)
                bt = np.full((len(ks), nb), -1, np.int32)
                for j, (_, b) in enumerate(sb.user_writes):
                    bt[j, :len(b)] = b
                k, v = dev(np.concatenate([x[1] for x in ks])), dev(np.concatenate([x[2] for x in ks]))
                cu = i32(np.concatenate([[0], np.cumsum(lens)]))
                calls.append(("kv_build", (k, v, cu, i32(bt), "user")))
                if prefix_rows:
                    q = dev(np.concatenate([x[0] for x in ks]))
                    ws = torch.empty(max(1, api.workspace_size(len(ks), H, D, api.BAT_BF16,
                                                               sum(lens), max(lens), 0)),
                                     dtype=torch.uint8, device="cuda")
                    calls.append(("prefix_rows", (q, k, v, cu, max(lens), torch.empty_like(q), ws)))
            if sb.item_writes:
                xs = [toks(W.ITEM_STREAM, i) for i, _ in sb.item_writes]
                k, v = dev(np.concatenate([x[1] for x in xs])), dev(np.concatenate([x[2] for x in xs]))
                cu = i32(np.arange(0, (len(xs) + 1) * T, T))
                bt = i32(np.array([[s] for _, s in sb.item_writes]))
                calls.append(("kv_build", (k, v, cu, bt, "item")))
                if prefix_rows:
                    q = dev(np.concatenate([x[0] for x in xs]))
                    calls.append(("item_local", (q, k, v, torch.empty_like(q))))
            if sb.queries:
                sq, sk, sv, n_s, n_p, mode = [], [], [], [], [], []
                nb = max(len(q.prefix_places) for q in sb.queries)
                bt = np.full((len(sb.queries), nb), -1, np.int32)
                for j, q in enumerate(sb.queries):
                    if q.mode == W.USER:
                        parts = [toks(W.ITEM_STREAM, int(i)) for i in q.items]
                        x = tuple(np.concatenate([p[c] for p in parts]) for c in range(3))
                    else:
                        x = toks(W.USER_STREAM, q.user)
                    sq.append(x[0]); sk.append(x[1]); sv.append(x[2])
                    n_s.append(q.suffix_len)
                    n_p.append(q.prefix_len)
                    mode.append(q.mode)
                    bt[j, :len(q.prefix_places)] = q.prefix_places
                total = int(sum(n_s))
                Q, K, V = dev(np.concatenate(sq)), dev(np.concatenate(sk)), dev(np.concatenate(sv))
                args = dict(q=Q, k=K, v=V, cu=i32(np.concatenate([[0], np.cumsum(n_s)])),
                            plen=i32(n_p),
                            mode=torch.from_numpy(np.asarray(mode, np.uint8)).cuda(),
                            bt=i32(bt), max_s=int(max(n_s)), max_p=int(max(n_p)),
                            out=torch.empty_like(Q),
                            lse=torch.empty((H, total), dtype=torch.float32, device="cuda"))
                args["ws"] = torch.empty(max(1, api.workspace_size(
                    len(n_s), H, D, api.BAT_BF16, total, args["max_s"], args["max_p"])),
                    dtype=torch.uint8, device="cuda")
                calls.append(("prefill", args))
                self.prefills.append((sb.queries, args))
            self.calls.append(calls)

    def run(self):
        for calls in self.calls:
            for kind, a in calls:
                if kind == "kv_build":
                    k, v, cu, bt, which = a
                    api.kv_build(k, v, cu, bt, self.user_pool if which == "user" else self.item_pool)
                elif kind == "prefix_rows":
                    q, k, v, cu, mx, out, ws = a
                    api.attn_prefix_rows(q, k, v, cu, softmax_scale=self.scale, max_prefix_len=mx,
                                         out=out, workspace=ws)
                elif kind == "item_local":
                    q, k, v, out = a
                    api.attn_item_local(q, k, v, self.p.T, softmax_scale=self.scale, out=out)
                else:
                    api.attn_prefill(a["q"], a["k"], a["v"], a["cu"], a["plen"], a["mode"],
                                     a["bt"], self.user_pool, self.item_pool, self.scale,
                                     a["max_s"], a["max_p"], out=a["out"], lse=a["lse"],
                                     workspace=a["ws"])

    def prefill_outputs(self):
        """[(queries, out [rows, H, D], lse [H, rows])] per sub-batch, on the device."""
        return [(qs, a["out"], a["lse"]) for qs, a in self.prefills]
