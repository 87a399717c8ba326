"""Seeded synthetic inputs for prefix-reuse attention.

This module only draws random inputs and block tables: it holds none of the
attention arithmetic and imports nothing from the rest of the package, so the
HIP path and the CPU oracle can both be fed from it.

The pages run Bat on unnamed recommendation datasets, so every workload here
is synthetic and shaped like the five configurations the library is measured
on: activations N(0, 1) (rounded to bfloat16 for the bf16 configurations),
user prefixes paged into shuffled physical blocks, and item prefixes drawn
from a 20 000-item pool with Zipf(1.1) popularity (hot items recur across
users, which is the reuse the Bat page credits to item-as-prefix in section
"Why it works").

Storage convention: float32 arrays for fp32 workloads, uint16 bit patterns for
bfloat16 workloads (`bf16_to_f32` widens them exactly).
"""
from dataclasses import dataclass, field
import math

import numpy as np

USER, ITEM = 0, 1
ITEM_TOKENS = 4          # tokens per cached item (one item per item-pool block)
NUM_ITEMS = 20000        # item-pool size of configurations 3 and 5
ZIPF_S = 1.1


def f32_to_bf16(x):
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_to_f32(b):
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Workload:
    name: str
    seed: int
    dtype: str                 # "f32" or "bf16"
    B: int
    H: int
    D: int
    n_s: np.ndarray            # int32 [B] suffix (fresh) tokens per request
    n_p: np.ndarray            # int32 [B] prefix tokens per request
    mode: np.ndarray           # uint8 [B] USER or ITEM
    cu_s: np.ndarray           # int32 [B+1]
    q: np.ndarray              # [sum n_s, H, D]
    k_s: np.ndarray
    v_s: np.ndarray
    user_block_size: int
    user_num_blocks: int
    cu_user: np.ndarray        # int32 [B+1]; item-mode requests own 0 user tokens
    user_k: np.ndarray         # [sum of user-mode n_p, H, D], logical order
    user_v: np.ndarray
    num_items: int
    item_k: np.ndarray         # [num_items * ITEM_TOKENS, H, D]; item i owns rows 4i..4i+3
    item_v: np.ndarray
    block_table: np.ndarray    # int32 [B, bt_stride]; user rows: physical user blocks,
                               # item rows: item ids (= item-pool block ids); unused = -1
    scale: float
    notes: dict = field(default_factory=dict)

    @property
    def total_s(self) -> int:
        return int(self.cu_s[-1])

    @property
    def bt_stride(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def flops(self) -> float:
        """Algorithmic flops: QK^T and PV over the pairs a suffix row sees."""
        ns = self.n_s.astype(np.float64)
        npf = self.n_p.astype(np.float64)
        return float(np.sum(4.0 * self.D * ns * (npf + ns)) * self.H)

    def alg_bytes(self) -> float:
        """Algorithmic HBM bytes: prefix K+V once, suffix Q/K/V, O, and lse."""
        e = self.elem_bytes
        ns = self.n_s.astype(np.float64)
        npf = self.n_p.astype(np.float64)
        per_h = 2 * npf * self.D * e + 3 * ns * self.D * e + ns * self.D * e + 4 * ns
        return float(np.sum(per_h) * self.H)


def _normal(rng, shape, dtype, value_scale=1.0, chunk=1 << 24):
    """N(0, value_scale^2) values in the storage dtype, generated in chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = rng.standard_normal(e - s, dtype=np.float32)
        if value_scale != 1.0:
            x *= np.float32(value_scale)
        out[s:e] = x if dtype == "f32" else f32_to_bf16(x)
    return out.reshape(shape)


def zipf_items(rng, n_req_items, num_items=NUM_ITEMS, s=ZIPF_S):
    """Per request, distinct item ids drawn with p(rank k) ~ k^-s.

    Draws without replacement by exponential keys (weighted sampling without
    replacement, Efraimidis and Spirakis): key = E / p, keep the smallest.
    Ranks map to ids through one seeded permutation so hot items are spread
    over the pool.
    """
    ranks = np.arange(1, num_items + 1, dtype=np.float64)
    p = ranks ** (-s)
    p /= p.sum()
    rank_to_id = rng.permutation(num_items).astype(np.int32)
    out = []
    for n in n_req_items:
        keys = rng.exponential(size=num_items) / p
        chosen = np.argpartition(keys, n - 1)[:n] if n < num_items else np.arange(num_items)
        chosen = chosen[np.argsort(keys[chosen])]       # draw order
        out.append(rank_to_id[chosen])
    return out


def make_custom(*, dtype, H, D, n_s, n_p, mode, seed, user_block_size=64,
                extra_user_blocks=0, num_items=None, value_scale=1.0,
                q_scale=1.0, name="custom", scale=None, materialize=True):
    """A workload with explicit per-request lengths and modes.

    For item-mode requests n_p must be a multiple of ITEM_TOKENS; the items are
    drawn Zipf(1.1) without replacement from a pool of num_items items.
    With materialize=False only lengths, modes and block tables are drawn (the
    tensors are None); those match the materialized workload of the same seed.
    """
    rng = np.random.default_rng(seed)
    n_s = np.asarray(n_s, dtype=np.int32)
    n_p = np.asarray(n_p, dtype=np.int32)
    mode = np.asarray(mode, dtype=np.uint8)
    B = len(n_s)
    assert len(n_p) == B and len(mode) == B
    bs = int(user_block_size)
    item_req = mode == ITEM
    if np.any(n_p[item_req] % ITEM_TOKENS):
        raise ValueError("item-mode prefix lengths must be multiples of 4")
    n_items_req = np.where(item_req, n_p // ITEM_TOKENS, 0)
    if num_items is None:
        num_items = NUM_ITEMS if item_req.any() else 0
    if item_req.any() and n_items_req.max() > num_items:
        raise ValueError("a request asks for more distinct items than the pool has")

    # block tables
    user_blocks = np.where(item_req, 0, (n_p + bs - 1) // bs)
    user_num_blocks = int(user_blocks.sum()) + int(extra_user_blocks)
    phys = rng.permutation(max(user_num_blocks, 1)).astype(np.int32)
    items = zipf_items(rng, [int(x) for x in n_items_req[item_req]], num_items) if item_req.any() else []
    stride = int(max(1, user_blocks.max(initial=0), n_items_req.max(initial=0)))
    bt = np.full((B, stride), -1, dtype=np.int32)
    pos, it = 0, iter(items)
    for r in range(B):
        if item_req[r]:
            ids = next(it)
            bt[r, :len(ids)] = ids
        else:
            nb = int(user_blocks[r])
            bt[r, :nb] = phys[pos:pos + nb]
            pos += nb

    cu_s = np.zeros(B + 1, np.int32)
    cu_s[1:] = np.cumsum(n_s)
    cu_user = np.zeros(B + 1, np.int32)
    cu_user[1:] = np.cumsum(np.where(item_req, 0, n_p))
    total_s, total_u = int(cu_s[-1]), int(cu_user[-1])

    if materialize:
        q = _normal(rng, (total_s, H, D), dtype, value_scale * q_scale)
        k_s = _normal(rng, (total_s, H, D), dtype, value_scale)
        v_s = _normal(rng, (total_s, H, D), dtype, value_scale)
        user_k = _normal(rng, (total_u, H, D), dtype, value_scale)
        user_v = _normal(rng, (total_u, H, D), dtype, value_scale)
        item_k = _normal(rng, (num_items * ITEM_TOKENS, H, D), dtype, value_scale)
        item_v = _normal(rng, (num_items * ITEM_TOKENS, H, D), dtype, value_scale)
    else:
        q = k_s = v_s = user_k = user_v = item_k = item_v = None
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(D)))
    return Workload(name=name, seed=seed, dtype=dtype, B=B, H=H, D=D, n_s=n_s,
                    n_p=n_p, mode=mode, cu_s=cu_s, q=q, k_s=k_s, v_s=v_s,
                    user_block_size=bs, user_num_blocks=max(user_num_blocks, 1),
                    cu_user=cu_user, user_k=user_k, user_v=user_v,
                    num_items=num_items, item_k=item_k, item_v=item_v,
                    block_table=bt, scale=scale)


CONFIG_DESCRIPTIONS = {
    1: "fp32, B=1, H=4, D=32, user prefix 64 (16-token pages), suffix 8",
    2: "bf16, B=32, H=8, D=64, user prefix 1024 (64-token pages), suffix 256",
    3: "bf16, B=64, H=8, D=64, item prefix 128 Zipf(1.1) items x 4 tokens from 20000, suffix 512",
    4: "bf16, B=16, H=16, D=128, user prefix 8192 (64-token pages), suffix 512",
    5: "bf16, B=128, H=8, D=128, mixed user/item prefix U[256,16384], suffix U[64,1024], varlen",
}


def make_config(k: int, seed=None, materialize=True) -> Workload:
    """The five measured configurations; seed defaults to 100 + k."""
    seed = 100 + k if seed is None else seed
    kw = dict(seed=seed, name=f"config{k}", materialize=materialize)
    if k == 1:
        wl = make_custom(dtype="f32", H=4, D=32, n_s=[8], n_p=[64], mode=[USER],
                         user_block_size=16, extra_user_blocks=4, **kw)
    elif k == 2:
        B = 32
        wl = make_custom(dtype="bf16", H=8, D=64, n_s=[256] * B, n_p=[1024] * B,
                         mode=[USER] * B, **kw)
    elif k == 3:
        B = 64
        wl = make_custom(dtype="bf16", H=8, D=64, n_s=[512] * B,
                         n_p=[128 * ITEM_TOKENS] * B, mode=[ITEM] * B, **kw)
    elif k == 4:
        B = 16
        wl = make_custom(dtype="bf16", H=16, D=128, n_s=[512] * B, n_p=[8192] * B,
                         mode=[USER] * B, **kw)
    elif k == 5:
        B = 128
        rng = np.random.default_rng(seed + 1000)
        n_p = rng.integers(256, 16384, endpoint=True, size=B)
        n_s = rng.integers(64, 1024, endpoint=True, size=B)
        mode = rng.integers(0, 2, size=B).astype(np.uint8)
        n_p = np.where(mode == ITEM, (n_p // ITEM_TOKENS) * ITEM_TOKENS, n_p)
        wl = make_custom(dtype="bf16", H=8, D=128, n_s=n_s, n_p=n_p, mode=mode,
                         **kw)
    else:
        raise ValueError(f"unknown configuration {k}")
    wl.notes["description"] = CONFIG_DESCRIPTIONS[k]
    return wl


USER_STREAM, ITEM_STREAM = 1, 2


def entity_tokens(seed, kind, ident, n, H, D, dtype="bf16"):
    """(q, k, v), each [n, H, D], of one entity's tokens: user `ident`'s
    history (kind USER_STREAM) or item `ident` (kind ITEM_STREAM).  Drawn
    N(0, 1) from a generator seeded by (seed, kind, ident), so an entity has
    the same tokens whichever query names it and whichever group (prefix or
    suffix) they fall in."""
    rng = np.random.default_rng([int(seed), int(kind), int(ident)])
    return tuple(_normal(rng, (n, H, D), dtype) for _ in range(3))


@dataclass
class Traffic:
    """A seeded stream of generative-recommender queries: query r comes from
    user `user[r]` (history of `user_len[user[r]]` tokens) and scores the
    `items.shape[1]` distinct candidate items `items[r]` of ITEM_TOKENS tokens
    each."""
    seed: int
    user: np.ndarray       # [R] int32 user ids
    user_len: np.ndarray   # [num_users] int32 history tokens per user
    items: np.ndarray      # [R, m] int32 item ids, distinct within a row
    num_items: int
    item_tokens: int = ITEM_TOKENS

    @property
    def num_users(self) -> int:
        return len(self.user_len)

    @property
    def R(self) -> int:
        return len(self.user)


def _zipf_ranks(rng, n, s, size):
    """`size` ranks (0-based) with p(rank k) ~ (k+1)^-s, with replacement."""
    cdf = np.cumsum(np.arange(1, n + 1, dtype=np.float64) ** (-s))
    cdf /= cdf[-1]
    return np.minimum(np.searchsorted(cdf, rng.random(size), side="right"), n - 1)


def make_traffic(seed, n_requests, num_users, num_items=NUM_ITEMS, items_per_request=128,
                 user_len_range=(256, 4096), user_len_step=64, user_zipf_s=0.9,
                 item_zipf_s=ZIPF_S):
    """Synthetic Zipf traffic for the prefix-mode choice.

    Users recur with Zipf(user_zipf_s) popularity; each user's history length
    is fixed, a multiple of user_len_step drawn uniformly from user_len_range.
    Each query's items are Zipf(item_zipf_s) draws without replacement (the
    first items_per_request distinct ids of a stream of independent draws,
    which is successive weighted sampling without replacement).  Ranks map to
    ids through seeded permutations so hot users and items are spread over
    the id space.
    """
    rng = np.random.default_rng(seed)
    lo, hi = user_len_range
    user_len = (rng.integers(lo // user_len_step, hi // user_len_step, endpoint=True,
                             size=num_users) * user_len_step).astype(np.int32)
    user_perm = rng.permutation(num_users).astype(np.int32)
    user = user_perm[_zipf_ranks(rng, num_users, user_zipf_s, n_requests)]
    item_perm = rng.permutation(num_items).astype(np.int32)
    m = int(items_per_request)
    if m > num_items:
        raise ValueError("more items per request than the pool has")
    items = np.empty((n_requests, m), np.int32)
    K = 4 * m + 16  # draws per query; a query short of m distinct ids draws more
    for r0 in range(0, n_requests, 4096):
        r1 = min(n_requests, r0 + 4096)
        draws = _zipf_ranks(rng, num_items, item_zipf_s, (r1 - r0, K))
        # first occurrence of each id in its row's draw order
        order = np.argsort(draws, axis=1, kind="stable")
        srt = np.take_along_axis(draws, order, axis=1)
        first_sorted = np.ones_like(srt, dtype=bool)
        first_sorted[:, 1:] = srt[:, 1:] != srt[:, :-1]
        first = np.zeros_like(first_sorted)
        np.put_along_axis(first, order, first_sorted, axis=1)
        take = first & (np.cumsum(first, axis=1) <= m)
        full = take.sum(axis=1) == m
        items[r0:r1][full] = item_perm[draws[full][take[full]].reshape(-1, m)]
        for i in np.nonzero(~full)[0]:
            got = [int(x) for x in draws[i][take[i]]]
            seen = set(got)
            while len(got) < m:
                for k in _zipf_ranks(rng, num_items, item_zipf_s, 2 * (m - len(got)) + 8):
                    k = int(k)
                    if k not in seen:
                        seen.add(k)
                        got.append(k)
                        if len(got) == m:
                            break
            items[r0 + i] = item_perm[np.asarray(got)]
    return Traffic(seed=seed, user=user.astype(np.int32), user_len=user_len, items=items,
                   num_items=num_items)
