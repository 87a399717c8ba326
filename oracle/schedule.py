"""Oracle for the hotness-aware prefix-mode choice -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.

The Bat page (sections "The idea" and "Why it works") has a scheduler choose,
per query and under memory limits, whether the user history or the query's
items is the cached prefix, favouring prefixes whose caches are hot and
resident; user-prefix and item-prefix caches live in separate pools with
their own management.  The page gives no policy in detail, so this module
writes out one plain reading of it, step by step, in the order the queries
arrive:

1. Reuse now.  The user's cache is resident or not (user pool); each of the
   query's m items is resident or not (item pool).
2. Choice.  Each mode scores the prefix tokens that are hot: resident now,
   or asked for by an earlier query (hotness: the number of earlier queries
   naming them is above zero) and able to stay resident:
       user mode: n_u if the user is resident, or if it was asked for before
                  and its blocks fit in the user pool at all; else 0;
       item mode: T for each of the query's items that is resident, or was
                  asked for before while the item pool has slots.
   Item mode is chosen when its score is larger; a tie keeps the user as
   the prefix (the conventional choice).  The user-as-prefix policy always
   chooses user mode.
3. Cache update, only for the chosen mode's prefix (the other group's tokens
   are this query's suffix: they see the prefix, so their keys/values are
   not reusable on their own).
   * User mode: a resident user becomes the most recently used; a missing
     one is computed and admitted, evicting least recently used users until
     its ceil(n_u / block) blocks fit (never admitted if they exceed the
     pool).
   * Item mode: resident items are marked used by this query; each missing
     item, in the query's order, takes the lowest free slot, else replaces
     the resident item (not one of this query's) with the fewest earlier
     requests, then the least recent use, then the lowest id -- only when
     that victim was asked for strictly fewer times before than the new
     item; otherwise the item is computed but not kept.
4. Hotness.  The user's and every listed item's counts grow by one, whatever
   the mode.

Accounting per query (n_u user tokens, m items of T tokens, h item hits):
    user mode: prefix tokens computed = 0 on a hit else n_u; suffix = m*T;
               query-key pairs = (0 on a hit else n_u^2) + m*T*(n_u + m*T)
    item mode: prefix tokens computed = T*(m - h); suffix = n_u;
               pairs = (m - h)*T^2 + n_u*(n_u + m*T)
(prefix rows see the prefix only -- per item for items -- and suffix rows
see the prefix and the suffix, as in the attention itself).

Everything is pure Python over lists and dicts, linear scans for the victim
and the LRU end, so each step can be read against the list above.  Pins:
``tests/test_schedule.py``.
"""
import numpy as np

POLICY_USER_PREFIX, POLICY_HOTNESS = 0, 1
MODE_USER, MODE_ITEM = 0, 1


def schedule(user, user_len, items, item_tokens, user_block, user_capacity_blocks,
             item_capacity, policy, num_items=None):
    """Run the choice over a query stream; returns a dict of per-query arrays
    (mode, user_hit, item_hits, prefix_tokens, suffix_tokens, pairs,
    item_slot [R, m], -1 where an item holds no slot for this query) and the
    final pool contents (resident_users in recency order, most recent first;
    slot_item [item_capacity], -1 for a free slot)."""
    user = [int(u) for u in np.asarray(user)]
    user_len = [int(x) for x in np.asarray(user_len)]
    items = np.asarray(items)
    R, m = items.shape
    T = int(item_tokens)
    if num_items is None:
        num_items = int(items.max()) + 1 if items.size else 0

    lru = []                     # resident users, most recent first
    used_blocks = 0
    slot_item = [-1] * item_capacity
    item_slot = {}               # resident item -> slot
    last_use = {}                # resident item -> last query that used it
    count_u = [0] * len(user_len)
    count_i = [0] * num_items

    out = {k: [] for k in ("mode", "user_hit", "item_hits", "prefix_tokens",
                           "suffix_tokens", "pairs")}
    slots = np.full((R, m), -1, np.int32)

    def blocks(n):
        return -(-n // user_block)

    for r in range(R):
        u, n_u = user[r], user_len[user[r]]
        its = [int(i) for i in items[r]]
        # 1) reuse now
        u_hit = u in lru
        resident = [i in item_slot for i in its]
        h = sum(resident)
        # 2) choice
        if policy == POLICY_USER_PREFIX:
            mode = MODE_USER
        else:
            hot_user = u_hit or (count_u[u] > 0 and blocks(n_u) <= user_capacity_blocks)
            s_user = n_u if hot_user else 0
            s_item = 0
            for i, res in zip(its, resident):
                if res or (count_i[i] > 0 and item_capacity > 0):
                    s_item += T
            mode = MODE_ITEM if s_item > s_user else MODE_USER
        # 3) cache update and accounting
        if mode == MODE_USER:
            if u_hit:
                lru.remove(u)
                lru.insert(0, u)
            elif blocks(n_u) <= user_capacity_blocks:
                while used_blocks + blocks(n_u) > user_capacity_blocks:
                    victim = lru.pop()
                    used_blocks -= blocks(user_len[victim])
                lru.insert(0, u)
                used_blocks += blocks(n_u)
            prefix = 0 if u_hit else n_u
            suffix = m * T
            pairs = (0 if u_hit else n_u * n_u) + m * T * (n_u + m * T)
        else:
            for j, (i, res) in enumerate(zip(its, resident)):
                if res:
                    last_use[i] = r
                    slots[r, j] = item_slot[i]
            for j, (i, res) in enumerate(zip(its, resident)):
                if res:
                    continue
                free = [s for s in range(item_capacity) if slot_item[s] < 0]
                if free:
                    s = free[0]
                else:
                    cands = [v for v in item_slot if v not in its]
                    if not cands:
                        continue
                    victim = min(cands, key=lambda v: (count_i[v], last_use[v], v))
                    if not count_i[victim] < count_i[i]:
                        continue
                    s = item_slot.pop(victim)
                    del last_use[victim]
                slot_item[s] = i
                item_slot[i] = s
                last_use[i] = r
                slots[r, j] = s
            prefix = T * (m - h)
            suffix = n_u
            pairs = (m - h) * T * T + n_u * (n_u + m * T)
        # 4) hotness
        count_u[u] += 1
        for i in its:
            count_i[i] += 1
        out["mode"].append(mode)
        out["user_hit"].append(int(u_hit))
        out["item_hits"].append(h)
        out["prefix_tokens"].append(prefix)
        out["suffix_tokens"].append(suffix)
        out["pairs"].append(pairs)

    res = {
        "mode": np.asarray(out["mode"], np.uint8),
        "user_hit": np.asarray(out["user_hit"], np.uint8),
        "item_hits": np.asarray(out["item_hits"], np.int32),
        "prefix_tokens": np.asarray(out["prefix_tokens"], np.int64),
        "suffix_tokens": np.asarray(out["suffix_tokens"], np.int64),
        "pairs": np.asarray(out["pairs"], np.int64),
        "item_slot": slots,
        "resident_users": np.asarray(lru, np.int32),
        "slot_item": np.asarray(slot_item, np.int32),
    }
    return res
