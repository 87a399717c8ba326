"""The prefix-mode choice: the oracle against its pins, then the library's
native scheduler (bat_scheduler_*) against the oracle, bit for bit.

Both run on the host; nothing here needs a GPU.

Pins of the oracle (oracle/schedule.py), each independent of its code:
* a trace of eight queries worked by hand (tests/golden/hand_schedule.json);
* user-as-prefix hits against the LRU stack property (a user is resident
  exactly when the distinct users asked for since its last request, itself
  included, fit in the pool), checked on random traces;
* closed forms: no user pool (every query misses), an unbounded pool
  (misses = first requests of each user), an unbounded item pool with a user
  too large to cache (hits = items named by earlier item-mode queries);
* the hotness-aware policy with no item slots equals user-as-prefix;
* accounting: for every query, computed prefix + suffix + reused tokens is
  the query's size, and the query-key pairs equal a brute-force count over
  the attention mask (prefix rows see the prefix -- one item for item
  prefixes -- suffix rows see everything; only computed rows count).
"""
import json
import os

import numpy as np
import pytest

from oracle import prefix_only_mask
from oracle import schedule as S
from prefix_reuse_attention_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_schedule.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _run_oracle(g, policy):
    return S.schedule(g["user"], g["user_len"], np.asarray(g["items"], np.int32),
                      g["item_tokens"], g["user_block"], g["user_capacity_blocks"],
                      g["item_capacity"], policy, num_items=g["num_items"])


def test_oracle_hand_trace_hotness():
    g = _golden()
    res = _run_oracle(g, S.POLICY_HOTNESS)
    for key, want in g["hotness"].items():
        assert np.asarray(res[key]).tolist() == want, key


def test_oracle_hand_trace_user_prefix():
    g = _golden()
    res = _run_oracle(g, S.POLICY_USER_PREFIX)
    for key, want in g["user_prefix"].items():
        assert np.asarray(res[key]).tolist() == want, key
    assert int(res["pairs"].sum()) == 640
    assert int(_run_oracle(g, S.POLICY_HOTNESS)["pairs"].sum()) == 596


def _small_traffic(seed, R=300, users=40, items=60, m=6):
    return W.make_traffic(seed, R, users, num_items=items, items_per_request=m,
                          user_len_range=(64, 640), user_len_step=64)


@pytest.mark.parametrize("seed,cap", [(1, 8), (2, 30), (3, 100)])
def test_oracle_user_prefix_lru_stack_property(seed, cap):
    tr = _small_traffic(seed)
    blocks = -(-tr.user_len // 64)
    assert blocks.max() <= cap or cap == 8  # cap 8 leaves some users too large
    res = S.schedule(tr.user, tr.user_len, tr.items, 4, 64, cap, 0, S.POLICY_USER_PREFIX)
    last = {}
    for r, u in enumerate(tr.user.tolist()):
        if u in last and blocks[u] <= cap:
            # distinct users since u's last request, each counted once, that
            # can be cached at all (larger ones are never admitted)
            seen = {v for v in tr.user[last[u] + 1:r].tolist() if blocks[v] <= cap}
            seen.discard(u)
            want = int(blocks[u] + sum(int(blocks[v]) for v in seen) <= cap)
        else:
            want = 0
        assert res["user_hit"][r] == want, r
        last[u] = r


def test_oracle_closed_forms_user_pool():
    tr = _small_traffic(4)
    none = S.schedule(tr.user, tr.user_len, tr.items, 4, 64, 0, 0, S.POLICY_USER_PREFIX)
    assert not none["user_hit"].any()
    assert (none["prefix_tokens"] == tr.user_len[tr.user]).all()
    big = S.schedule(tr.user, tr.user_len, tr.items, 4, 64, 10 ** 9, 0, S.POLICY_USER_PREFIX)
    first = np.zeros(tr.R, bool)
    first[np.unique(tr.user, return_index=True)[1]] = True
    assert (big["user_hit"] == ~first).all()
    assert int(big["prefix_tokens"].sum()) == int(tr.user_len[np.unique(tr.user)].sum())
    assert sorted(big["resident_users"].tolist()) == sorted(np.unique(tr.user).tolist())


def test_oracle_item_pool_unbounded_closed_form():
    """One user too large for its pool (user mode never scores): a query
    goes to item mode exactly when one of its items was named before, and
    its hits are its items named by earlier item-mode queries."""
    rng = np.random.default_rng(5)
    R, N, m = 200, 50, 5
    items = np.stack([rng.choice(N, m, replace=False) for _ in range(R)]).astype(np.int32)
    user = np.zeros(R, np.int32)
    res = S.schedule(user, [1000], items, 4, 64, 4, N, S.POLICY_HOTNESS, num_items=N)
    named, cached = set(), set()
    for r in range(R):
        its = set(items[r].tolist())
        want_mode = S.MODE_ITEM if its & named else S.MODE_USER
        assert res["mode"][r] == want_mode, r
        assert res["item_hits"][r] == len(its & cached), r
        if want_mode == S.MODE_ITEM:
            cached |= its
        named |= its
    assert not res["user_hit"].any()


@pytest.mark.parametrize("seed", [6, 7])
def test_oracle_hotness_without_item_slots_is_user_prefix(seed):
    tr = _small_traffic(seed)
    a = S.schedule(tr.user, tr.user_len, tr.items, 4, 64, 20, 0, S.POLICY_HOTNESS)
    b = S.schedule(tr.user, tr.user_len, tr.items, 4, 64, 20, 0, S.POLICY_USER_PREFIX)
    for k in ("mode", "user_hit", "prefix_tokens", "pairs"):
        assert (a[k] == b[k]).all(), k


def _brute_pairs(n_u, m, T, mode, user_hit, item_resident):
    """Query-key pairs of the computed rows, counted over the mask."""
    n = n_u + m * T
    if mode == S.MODE_USER:
        in_prefix = np.arange(n) < n_u
        mask = prefix_only_mask(in_prefix)
        computed = ~in_prefix | (not user_hit)
    else:
        in_prefix = np.arange(n) < m * T
        mask = prefix_only_mask(in_prefix)
        item_of = np.where(in_prefix, np.arange(n) // T, -1)
        same_item = item_of[:, None] == item_of[None, :]
        mask = np.where(in_prefix[:, None], mask & same_item, mask)
        res_tok = np.zeros(n, bool)
        res_tok[:m * T] = np.repeat(np.asarray(item_resident, bool), T)
        computed = ~res_tok
    return int(mask[computed].sum())


@pytest.mark.parametrize("seed,ucap,icap", [(8, 12, 10), (9, 40, 30), (10, 3, 60)])
def test_oracle_accounting(seed, ucap, icap):
    tr = W.make_traffic(seed, 120, 20, num_items=40, items_per_request=4,
                        user_len_range=(4, 40), user_len_step=4)
    T = 3
    res = S.schedule(tr.user, tr.user_len, tr.items, T, 4, ucap, icap, S.POLICY_HOTNESS)
    assert set(res["mode"].tolist()) == {0, 1}, "trace should exercise both modes"
    m = tr.items.shape[1]
    for r in range(tr.R):
        n_u = int(tr.user_len[tr.user[r]])
        mode, uh, h = int(res["mode"][r]), int(res["user_hit"][r]), int(res["item_hits"][r])
        reused = n_u * uh if mode == S.MODE_USER else T * h
        assert res["prefix_tokens"][r] + res["suffix_tokens"][r] + reused == n_u + m * T
        resident = [True] * h + [False] * (m - h)  # the count matters, not which
        assert res["pairs"][r] == _brute_pairs(n_u, m, T, mode, uh, resident), r


def test_oracle_item_slots_valid():
    tr = _small_traffic(11, R=400, items=80, m=8)
    icap = 25
    res = S.schedule(tr.user, tr.user_len, tr.items, 4, 64, 10, icap, S.POLICY_HOTNESS)
    slot_item = [-1] * icap
    for r in range(tr.R):
        s = res["item_slot"][r]
        if res["mode"][r] == S.MODE_USER:
            assert (s == -1).all()
            continue
        held = s[s >= 0]
        assert len(set(held.tolist())) == len(held), "two items in one slot"
        hits = 0
        for i, sl in zip(tr.items[r].tolist(), s.tolist()):
            if sl < 0:
                assert i not in slot_item
                continue
            assert 0 <= sl < icap
            if slot_item[sl] == i:
                hits += 1
            slot_item[sl] = i
        assert hits == res["item_hits"][r]
    assert slot_item == res["slot_item"].tolist()


def test_oracle_admission_needs_strictly_fewer_requests():
    """Worked by hand: one item slot, T = 1, a user too large to cache.
    q0 [0] and q1 [1]: nothing named before, scores tie at 0 -> user mode.
    q2 [0]: item 0 named once -> item mode, takes the free slot.
    q3 [1]: item 1 named once; the victim (item 0, two requests) is not
    asked for less -> not kept.  q4 [1]: item 1 named twice, item 0 twice ->
    equal, still not kept.  q5 [1]: three against two -> item 1 replaces 0."""
    items = np.array([[0], [1], [0], [1], [1], [1]], np.int32)
    res = S.schedule(np.zeros(6, np.int32), [100], items, 1, 1, 10, 1, S.POLICY_HOTNESS,
                     num_items=2)
    assert res["mode"].tolist() == [0, 0, 1, 1, 1, 1]
    assert res["item_slot"][:, 0].tolist() == [-1, -1, 0, -1, -1, 0]
    assert res["item_hits"].tolist() == [0, 0, 0, 0, 0, 0]
    assert res["slot_item"].tolist() == [1]


# ---- the library's scheduler against the oracle ------------------------

def _native(tr_user, user_len, items, T, block, ucap, icap, policy, num_items, chunks=(1,)):
    from prefix_reuse_attention_amd import api
    sch = api.Scheduler(policy, T, block, ucap, icap, user_len, num_items)
    R = len(tr_user)
    parts = []
    cuts = sorted({0, R, *[int(R * c) for c in chunks]})
    for a, b in zip(cuts, cuts[1:]):
        parts.append(sch.step(tr_user[a:b], items[a:b]))
    res = {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}
    res["resident_users"], res["slot_item"] = sch.pools()
    return res


KEYS = ("mode", "user_hit", "item_hits", "prefix_tokens", "suffix_tokens", "pairs",
        "item_slot", "resident_users", "slot_item")


def _same(a, b):
    for k in KEYS:
        assert np.array_equal(np.asarray(a[k]), np.asarray(b[k])), k


@pytest.mark.parametrize("policy", [S.POLICY_HOTNESS, S.POLICY_USER_PREFIX])
def test_native_hand_trace(policy):
    g = _golden()
    ref = _run_oracle(g, policy)
    got = _native(np.asarray(g["user"], np.int32), g["user_len"],
                  np.asarray(g["items"], np.int32), g["item_tokens"], g["user_block"],
                  g["user_capacity_blocks"], g["item_capacity"], policy, g["num_items"],
                  chunks=(0.5,))
    _same(got, ref)


@pytest.mark.parametrize("seed,ucap,icap,policy", [
    (20, 0, 0, 1), (21, 10, 0, 1), (22, 30, 16, 1), (23, 60, 60, 1), (24, 200, 1, 1),
    (25, 30, 16, 0), (26, 12, 40, 1), (27, 10 ** 9, 10 ** 4, 1)])
def test_native_matches_oracle(seed, ucap, icap, policy):
    tr = _small_traffic(seed, R=600, users=50, items=120, m=9)
    ref = S.schedule(tr.user, tr.user_len, tr.items, 4, 64, ucap, icap, policy,
                     num_items=tr.num_items)
    got = _native(tr.user, tr.user_len, tr.items, 4, 64, ucap, icap, policy, tr.num_items,
                  chunks=(0.13, 0.5, 0.51))
    _same(got, ref)
    if policy == S.POLICY_HOTNESS and 0 < icap < 10 ** 4:
        assert 0 < got["mode"].sum() < tr.R


def test_native_zipf_traffic_against_oracle():
    """Traffic shaped like the measured one (Zipf users and items, 64-token
    user blocks, 4-token items), sized for the oracle."""
    tr = W.make_traffic(28, 2000, 400, num_items=2000, items_per_request=32,
                        user_len_range=(256, 4096))
    ref = S.schedule(tr.user, tr.user_len, tr.items, 4, 64, 2000, 300, S.POLICY_HOTNESS,
                     num_items=tr.num_items)
    got = _native(tr.user, tr.user_len, tr.items, 4, 64, 2000, 300, S.POLICY_HOTNESS,
                  tr.num_items, chunks=(0.25, 0.75))
    _same(got, ref)


def test_native_rejects_bad_queries():
    from prefix_reuse_attention_amd import api
    sch = api.Scheduler(1, 4, 64, 10, 4, [100, 200], 10)
    for user, items in (([0, 2], [[1, 2], [3, 4]]),      # user id out of range
                        ([0, 1], [[1, 2], [3, 10]]),     # item id out of range
                        ([0, 1], [[1, 2], [3, 3]]),      # repeated item
                        ([0, -1], [[1, 2], [3, 4]])):
        with pytest.raises(api.BatError):
            sch.step(np.asarray(user), np.asarray(items))
    # the argument check stamps items but serves no query
    got = sch.step(np.asarray([0]), np.asarray([[1, 2]]))
    assert got["mode"].tolist() == [0] and got["user_hit"].tolist() == [0]
    with pytest.raises(api.BatError):
        api.Scheduler(7, 4, 64, 10, 4, [100], 10)       # unknown policy
    with pytest.raises(api.BatError):
        api.Scheduler(1, 0, 64, 10, 4, [100], 10)       # T = 0


def test_native_matches_oracle_under_eviction_pressure():
    """Small pools against many users and items: user evictions, item
    replacements and rejected admissions all happen (checked), T = 2."""
    tr = W.make_traffic(29, 1500, 80, num_items=150, items_per_request=12,
                        user_len_range=(64, 1024), user_zipf_s=0.6, item_zipf_s=0.8)
    args = (tr.user, tr.user_len, tr.items, 2, 64, 20, 24, S.POLICY_HOTNESS)
    ref = S.schedule(*args, num_items=tr.num_items)
    got = _native(*args, tr.num_items, chunks=(0.3, 0.6))
    _same(got, ref)
    item_q = got["mode"] == S.MODE_ITEM
    missing = tr.items.shape[1] - got["item_hits"][item_q]
    kept = (got["item_slot"][item_q] >= 0).sum(axis=1) - got["item_hits"][item_q]
    assert (kept > 0).any() and (kept < missing).any(), "no admissions or no rejections"
    ever = set(tr.user[(got["mode"] == S.MODE_USER) & (got["user_hit"] == 0)].tolist())
    assert len(got["resident_users"]) < len(ever), "no user evictions"


def test_native_scheduler_under_host_sanitizers(tmp_path):
    """The scheduler's C++ built for the host with AddressSanitizer and
    UBSan, driven over random configurations and traces
    (tests/sched_sanitize_driver.cpp): no out-of-bounds access, no undefined
    behaviour, bad queries rejected."""
    import shutil
    import subprocess
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    exe = str(tmp_path / "drv")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-I", os.path.join(root, "include"),
                    os.path.join(root, "tests", "sched_sanitize_driver.cpp"),
                    os.path.join(root, "prefix_reuse_attention_amd", "csrc", "schedule.cpp"),
                    "-o", exe], check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "asan driver ok" in r.stdout


def test_native_matches_oracle_on_measured_traffic_prefix():
    """The measured traffic's shape and budget (20000 users Zipf(0.9) with
    U[256, 4096]-token histories, 128 of 20000 items Zipf(1.1), 2^21 cache
    tokens of which 8192 item slots), on the first 1000 queries of the same
    seeded stream: the oracle's pace bounds the sample."""
    n = 1000
    tr = W.make_traffic(7, n, 20000, num_items=20000, items_per_request=128,
                        user_len_range=(256, 4096), user_zipf_s=0.9, item_zipf_s=1.1)
    T, bs, budget, slots = 4, 64, 1 << 21, 8192
    for policy, ucap, icap in ((S.POLICY_HOTNESS, (budget - slots * T) // bs, slots),
                               (S.POLICY_USER_PREFIX, budget // bs, 0)):
        ref = S.schedule(tr.user, tr.user_len, tr.items, T, bs, ucap, icap, policy,
                         num_items=tr.num_items)
        got = _native(tr.user, tr.user_len, tr.items, T, bs, ucap, icap, policy,
                      tr.num_items, chunks=(0.5,))
        _same(got, ref)
