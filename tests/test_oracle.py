"""Pins for the CPU oracle (no GPU).

Each test ties the oracle to something other than itself: a hand-worked
example, an independent brute-force loop, torch's scaled-dot-product
attention on the CPU, closed forms, invariances and merge identities.  The
method is the Bat page's prefix-reuse attention (sections "This paper's idea"
and "Why it works"); the mask reading is prefix rows see only the prefix,
suffix rows see every token of their request.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from prefix_reuse_attention_amd import workloads as W
from helpers import assemble_prefix

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _sym(x):
    table = {"ln2": math.log(2), "ln3": math.log(3), "ln5": math.log(5),
             "ln8": math.log(8), "8/3": 8 / 3, "16/3": 16 / 3}
    if isinstance(x, list):
        return [_sym(e) for e in x]
    return table[x] if isinstance(x, str) else float(x)


def brute_force(q, k, v, in_prefix, scale):
    """Independent reference: explicit loops and math.exp, no vectorisation."""
    n, D = q.shape
    out = np.zeros((n, D))
    lse = np.zeros(n)
    for i in range(n):
        vis = [j for j in range(n) if in_prefix[j] or (not in_prefix[i] and not in_prefix[j])]
        s = {j: scale * sum(float(q[i, d]) * float(k[j, d]) for d in range(D)) for j in vis}
        z = sum(math.exp(s[j]) for j in vis)
        lse[i] = math.log(z)
        for j in vis:
            w = math.exp(s[j]) / z
            for d in range(D):
                out[i, d] += w * float(v[j, d])
    return out, lse


def rand_seq(rng, n_p, n_s, D, scale_q=1.0):
    n = n_p + n_s
    q = rng.standard_normal((n, D)) * scale_q
    k = rng.standard_normal((n, D))
    v = rng.standard_normal((n, D))
    in_prefix = np.array([True] * n_p + [False] * n_s)
    return q, k, v, in_prefix


# ---------------------------------------------------------------- hand-worked
def test_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_bipartite.json")))
    q, k, v = (np.array(_sym(g[x])) for x in ("q", "k", "v"))
    out, lse = oracle.bipartite_attention(q, k, v, g["in_prefix"], g["scale"])
    np.testing.assert_allclose(out, np.array(_sym(g["out"])), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(_sym(g["lse"])), rtol=0, atol=1e-12)


def test_hand_kv_scatter():
    g = json.load(open(os.path.join(GOLDEN, "hand_kv_scatter.json")))
    x = np.array(g["tokens"], dtype=np.int32).reshape(-1, 1, 1)
    pool = oracle.kv_scatter(x, g["cu_lens"], np.array(g["block_table"]),
                             g["num_blocks"], g["block_size"], g["fill"])
    assert pool.shape == (g["num_blocks"], 1, g["block_size"], 1)
    np.testing.assert_array_equal(pool[:, 0, :, 0], np.array(g["pool"]))


def test_hand_item_prefix():
    """The item-mode prefix of two requests worked by hand, both from the
    item-major token array and from a pool whose items sit at permuted
    physical slots (read slot by slot through the slot-valued table row)."""
    g = json.load(open(os.path.join(GOLDEN, "hand_item_prefix.json")))
    T = g["tokens_per_item"]
    x = np.array(g["item_tokens"], dtype=np.int32).reshape(-1, 1, 1)
    for ids, want in zip(g["requests"], g["prefixes"]):
        got = oracle.gather_item_prefix(x, ids, T)
        assert got.shape == (len(want), 1, 1)
        np.testing.assert_array_equal(got[:, 0, 0], want)
    n_items = len(g["slot_of_item"])
    cu = np.arange(0, (n_items + 1) * T, T)
    pool = oracle.kv_scatter(x, cu, np.array(g["slot_of_item"]).reshape(-1, 1), n_items, T, -1)
    np.testing.assert_array_equal(pool[:, 0, :, 0], np.array(g["pool_slots"]))
    for slots, want in zip(g["requests_as_slots"], g["prefixes"]):
        np.testing.assert_array_equal(np.concatenate([pool[s, 0, :, 0] for s in slots]), want)


def test_item_prefix_equals_reading_the_scattered_pool():
    """gather_item_prefix over item-major tokens equals reading, head by head,
    the pool kv_scatter builds with the items at permuted physical slots,
    through those items' slots (distinct ids, a repeated id, every id)."""
    rng = np.random.default_rng(41)
    n_items, T, H, D = 9, 4, 3, 5
    tok = rng.standard_normal((n_items * T, H, D))
    slot = rng.permutation(n_items)
    cu = np.arange(0, (n_items + 1) * T, T)
    pool = oracle.kv_scatter(tok, cu, slot.reshape(-1, 1), n_items, T, np.nan)
    for ids in (rng.choice(n_items, 5, replace=False), np.array([3, 3, 0]), np.arange(n_items)):
        want = oracle.gather_item_prefix(tok, ids, T)
        assert want.shape == (len(ids) * T, H, D)
        for h in range(H):
            got = np.concatenate([pool[slot[i], h] for i in ids])
            np.testing.assert_array_equal(got, want[:, h])


def test_bf16_widening_worked_values():
    """bfloat16 bit patterns worked by hand (sign, 8-bit exponent biased by
    127, 7 stored mantissa bits) widen to these exact values in both oracle
    paths: the numpy widening of the isolated rows and the C loader (through
    a one-key attention, whose output is that key's value)."""
    bits = np.array([0x3F80, 0xC000, 0x3E80, 0x4049, 0x0000, 0xBF40, 0x4300], np.uint16)
    want = np.array([1.0, -2.0, 0.25, 3.140625, 0.0, -0.75, 128.0])
    np.testing.assert_array_equal(oracle._widen(bits), want)
    v = bits.reshape(1, -1)
    out, _ = oracle.attention_masked(np.zeros_like(v), np.zeros_like(v), v,
                                     np.ones((1, 1), bool), 1.0)
    np.testing.assert_array_equal(out[0], want)


def test_isolated_bf16_inputs_brute_force():
    """prefill_isolated on bfloat16 bit patterns against explicit loops over
    the values those patterns hold.  The values are multiples of 1/8 in
    [-2, 2], exact in bfloat16, so their bits are the float32 bits' upper
    half and the loops take the values themselves (no bf16 conversion code
    on the reference side)."""
    rng = np.random.default_rng(36)
    T, H, D, scale = 2, 2, 4, 0.4
    lens_p, lens_s = [3, 0, 4], [4, 2, 2]
    vals = {n: rng.integers(-16, 17, size=(sum(lens_p if n in ("kp", "vp") else lens_s), H, D)) / 8.0
            for n in ("q", "ks", "vs", "kp", "vp")}
    bits = {n: (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
            for n, a in vals.items()}
    cu_p = np.concatenate([[0], np.cumsum(lens_p)]).astype(np.int32)
    cu_s = np.concatenate([[0], np.cumsum(lens_s)]).astype(np.int32)
    out, lse = oracle.prefill_isolated(bits["q"], bits["ks"], bits["vs"], cu_s, bits["kp"],
                                       bits["vp"], cu_p, T, scale)
    for r in range(len(lens_s)):
        for i in range(cu_s[r], cu_s[r + 1]):
            c0 = cu_s[r] + ((i - cu_s[r]) // T) * T
            for h in range(H):
                keys = [vals["kp"][j, h] for j in range(cu_p[r], cu_p[r + 1])] + \
                       [vals["ks"][j, h] for j in range(c0, c0 + T)]
                vv = [vals["vp"][j, h] for j in range(cu_p[r], cu_p[r + 1])] + \
                     [vals["vs"][j, h] for j in range(c0, c0 + T)]
                sc = [scale * sum(float(vals["q"][i, h, d]) * float(kk[d]) for d in range(D))
                      for kk in keys]
                z = sum(math.exp(x) for x in sc)
                ref = sum(math.exp(x) / z * w for x, w in zip(sc, vv))
                np.testing.assert_allclose(out[i, h], ref, rtol=0, atol=1e-12)
                assert abs(lse[h, i] - math.log(z)) <= 1e-12


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("n_p", [0, 1, 3, 17])
@pytest.mark.parametrize("n_s", [1, 2, 5])
@pytest.mark.parametrize("D", [1, 4, 32])
def test_brute_force_all_rows(n_p, n_s, D):
    rng = np.random.default_rng(1000 * n_p + 10 * n_s + D)
    q, k, v, pre = rand_seq(rng, n_p, n_s, D)
    scale = 1.0 / math.sqrt(D)
    out, lse = oracle.bipartite_attention(q, k, v, pre, scale)
    ref_o, ref_l = brute_force(q, k, v, pre, scale)
    np.testing.assert_allclose(out, ref_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-12)


def test_brute_force_config1():
    """Config 1 (fp32, 4 heads, D=32, 64 prefix + 8 suffix) vs brute force."""
    wl = W.make_config(1)
    out, lse = oracle.prefill_suffix(wl.q, wl.k_s, wl.v_s, wl.cu_s, wl.user_k,
                                     wl.user_v, wl.cu_user, wl.scale)
    for h in range(wl.H):
        q = np.concatenate([np.zeros((64, wl.D), np.float32), wl.q[:, h]])
        k = np.concatenate([wl.user_k[:, h], wl.k_s[:, h]])
        v = np.concatenate([wl.user_v[:, h], wl.v_s[:, h]])
        pre = np.array([True] * 64 + [False] * 8)
        ref_o, ref_l = brute_force(q.astype(np.float64), k.astype(np.float64),
                                   v.astype(np.float64), pre, wl.scale)
        np.testing.assert_allclose(out[:, h], ref_o[64:], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[h], ref_l[64:], rtol=0, atol=1e-12)


def test_prefill_batch_brute_force_and_selection():
    """Batched suffix rows over several requests (bf16 inputs) vs brute force,
    and the sampled-row mode returns the same numbers."""
    wl = W.make_custom(dtype="bf16", H=2, D=8, n_s=[3, 1, 4], n_p=[5, 0, 8],
                       mode=[W.USER, W.USER, W.ITEM], seed=7, num_items=6)
    k_p, v_p, cu_p = assemble_prefix(wl)
    out, lse = oracle.prefill_suffix(wl.q, wl.k_s, wl.v_s, wl.cu_s, k_p, v_p, cu_p, wl.scale)
    qf, ksf, vsf = (W.bf16_to_f32(x).astype(np.float64) for x in (wl.q, wl.k_s, wl.v_s))
    kpf, vpf = (W.bf16_to_f32(x).astype(np.float64) for x in (k_p, v_p))
    for r in range(wl.B):
        s0, s1, p0, p1 = wl.cu_s[r], wl.cu_s[r + 1], cu_p[r], cu_p[r + 1]
        for h in range(wl.H):
            q = np.concatenate([np.zeros((p1 - p0, wl.D)), qf[s0:s1, h]])
            k = np.concatenate([kpf[p0:p1, h], ksf[s0:s1, h]])
            v = np.concatenate([vpf[p0:p1, h], vsf[s0:s1, h]])
            pre = np.array([True] * (p1 - p0) + [False] * (s1 - s0))
            ro, rl = brute_force(q, k, v, pre, wl.scale)
            np.testing.assert_allclose(out[s0:s1, h], ro[p1 - p0:], rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[h, s0:s1], rl[p1 - p0:], rtol=0, atol=1e-12)
    rows = np.array([0, 3, 7, 5], np.int32)
    heads = np.array([1, 0, 1, 0], np.int32)
    so, sl = oracle.prefill_suffix(wl.q, wl.k_s, wl.v_s, wl.cu_s, k_p, v_p, cu_p,
                                   wl.scale, rows=rows, heads=heads)
    np.testing.assert_array_equal(so, out[rows, heads])
    np.testing.assert_array_equal(sl, lse[heads, rows])


# ------------------------------------------------------- library routine (SDPA)
def test_library_sdpa():
    """Suffix rows equal unmasked SDPA over all tokens; prefix rows equal
    unmasked SDPA over the prefix alone (torch, float64, CPU)."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    rng = np.random.default_rng(3)
    for n_p, n_s, D in [(0, 4, 16), (9, 5, 16), (33, 7, 64), (64, 8, 32)]:
        q, k, v, pre = rand_seq(rng, n_p, n_s, D)
        scale = 1.0 / math.sqrt(D)
        out, _ = oracle.bipartite_attention(q, k, v, pre, scale)
        t = lambda x: torch.from_numpy(np.ascontiguousarray(x))[None, None]
        ref_u = F.scaled_dot_product_attention(t(q[n_p:]), t(k), t(v), scale=scale)[0, 0]
        np.testing.assert_allclose(out[n_p:], ref_u.numpy(), rtol=0, atol=1e-12)
        if n_p:
            ref_p = F.scaled_dot_product_attention(t(q[:n_p]), t(k[:n_p]), t(v[:n_p]),
                                                   scale=scale)[0, 0]
            np.testing.assert_allclose(out[:n_p], ref_p.numpy(), rtol=0, atol=1e-12)


# ------------------------------------------------------------- closed forms
def test_single_token_returns_its_value():
    rng = np.random.default_rng(0)
    q, k, v, pre = rand_seq(rng, 0, 1, 8)
    out, lse = oracle.bipartite_attention(q, k, v, pre, 0.3)
    np.testing.assert_allclose(out, v, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, 0.3 * q @ k.T[:, 0], rtol=0, atol=1e-14)


def test_constant_values():
    rng = np.random.default_rng(1)
    q, k, v, pre = rand_seq(rng, 11, 6, 8)
    v[:] = np.arange(8) * 0.5 - 1.0
    out, _ = oracle.bipartite_attention(q, k, v, pre, 0.5)
    np.testing.assert_allclose(out, np.broadcast_to(v[0], out.shape), rtol=0, atol=1e-13)


def test_zero_query_gives_mean_of_visible_values():
    rng = np.random.default_rng(2)
    n_p, n_s = 7, 5
    q, k, v, pre = rand_seq(rng, n_p, n_s, 4)
    q[:] = 0
    out, lse = oracle.bipartite_attention(q, k, v, pre, 1.0)
    np.testing.assert_allclose(out[:n_p], np.broadcast_to(v[:n_p].mean(0), (n_p, 4)), atol=1e-14)
    np.testing.assert_allclose(out[n_p:], np.broadcast_to(v.mean(0), (n_s, 4)), atol=1e-14)
    np.testing.assert_allclose(lse[:n_p], math.log(n_p), atol=1e-14)
    np.testing.assert_allclose(lse[n_p:], math.log(n_p + n_s), atol=1e-14)


def test_equal_keys_give_mean_and_log_count():
    rng = np.random.default_rng(4)
    n_p, n_s, D = 6, 3, 5
    q, k, v, pre = rand_seq(rng, n_p, n_s, D)
    k[:] = k[0]
    out, lse = oracle.bipartite_attention(q, k, v, pre, 0.7)
    s = 0.7 * q @ k[0]
    np.testing.assert_allclose(out[:n_p], np.broadcast_to(v[:n_p].mean(0), (n_p, D)), atol=1e-13)
    np.testing.assert_allclose(out[n_p:], np.broadcast_to(v.mean(0), (n_s, D)), atol=1e-13)
    np.testing.assert_allclose(lse[:n_p], s[:n_p] + math.log(n_p), atol=1e-13)
    np.testing.assert_allclose(lse[n_p:], s[n_p:] + math.log(n_p + n_s), atol=1e-13)


def test_dominant_score_selects_its_value():
    """One score 60 above the rest: weight of the others is below e^-60 * n."""
    D, n_p, n_s = 4, 5, 3
    q = np.zeros((n_p + n_s, D)); q[:, 0] = 1.0
    k = np.zeros((n_p + n_s, D)); k[2, 0] = 60.0          # prefix token 2 dominates
    rng = np.random.default_rng(5)
    v = rng.standard_normal((n_p + n_s, D))
    pre = np.array([True] * n_p + [False] * n_s)
    out, lse = oracle.bipartite_attention(q, k, v, pre, 1.0)
    np.testing.assert_allclose(out, np.broadcast_to(v[2], out.shape), rtol=0, atol=1e-24 * 10)
    np.testing.assert_allclose(lse[n_p:], 60.0 + math.log1p((n_p + n_s - 1) * math.exp(-60)), atol=1e-13)


def test_duplicate_key_equals_ln2_shift():
    """A (k, v) pair present twice weighs as if its score were raised by ln 2."""
    rng = np.random.default_rng(6)
    D = 6
    q0 = rng.standard_normal(D)
    ks = rng.standard_normal((4, D)); vs = rng.standard_normal((4, D))
    scale = 0.4
    # duplicated key 1
    k_dup = np.vstack([ks, ks[1:2]]); v_dup = np.vstack([vs, vs[1:2]])
    o1, l1 = oracle.attention_masked(q0[None], k_dup, v_dup, np.ones((1, 5)), scale)
    # key 1 moved along q so that its score grows by exactly ln 2
    k_sh = ks.copy(); k_sh[1] += (math.log(2) / scale) * q0 / (q0 @ q0)
    o2, l2 = oracle.attention_masked(q0[None], k_sh, vs, np.ones((1, 4)), scale)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- invariances
def test_permuting_prefix_leaves_suffix_rows():
    rng = np.random.default_rng(8)
    n_p, n_s, D = 13, 6, 16
    q, k, v, pre = rand_seq(rng, n_p, n_s, D)
    out, lse = oracle.bipartite_attention(q, k, v, pre, 0.25)
    perm = np.concatenate([rng.permutation(n_p), np.arange(n_p, n_p + n_s)])
    o2, l2 = oracle.bipartite_attention(q[perm], k[perm], v[perm], pre, 0.25)
    np.testing.assert_allclose(o2[n_p:], out[n_p:], rtol=0, atol=1e-13)
    np.testing.assert_allclose(o2[:n_p], out[perm[:n_p]], rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, lse[perm], rtol=0, atol=1e-13)


def test_permuting_suffix_permutes_rows():
    rng = np.random.default_rng(9)
    n_p, n_s, D = 10, 7, 8
    q, k, v, pre = rand_seq(rng, n_p, n_s, D)
    out, lse = oracle.bipartite_attention(q, k, v, pre, 0.3)
    perm = np.concatenate([np.arange(n_p), n_p + rng.permutation(n_s)])
    o2, l2 = oracle.bipartite_attention(q[perm], k[perm], v[perm], pre, 0.3)
    np.testing.assert_allclose(o2, out[perm], rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, lse[perm], rtol=0, atol=1e-13)


def test_group_order_is_irrelevant():
    """[P; U] and [U; P] (mask carried by membership, not position) agree, and
    so does any interleaving: the order-agnostic view of user and item tokens."""
    rng = np.random.default_rng(10)
    n_p, n_s, D = 9, 5, 8
    q, k, v, pre = rand_seq(rng, n_p, n_s, D)
    out, lse = oracle.bipartite_attention(q, k, v, pre, 0.35)
    for perm in (np.concatenate([np.arange(n_p, n_p + n_s), np.arange(n_p)]),
                 rng.permutation(n_p + n_s)):
        o2, l2 = oracle.bipartite_attention(q[perm], k[perm], v[perm], pre[perm], 0.35)
        np.testing.assert_allclose(o2, out[perm], rtol=0, atol=1e-13)
        np.testing.assert_allclose(l2, lse[perm], rtol=0, atol=1e-13)


def test_item_order_in_block_table_is_irrelevant():
    wl = W.make_custom(dtype="bf16", H=2, D=16, n_s=[5, 3], n_p=[24, 12],
                       mode=[W.ITEM, W.ITEM], seed=11, num_items=40)
    k_p, v_p, cu_p = assemble_prefix(wl)
    out, lse = oracle.prefill_suffix(wl.q, wl.k_s, wl.v_s, wl.cu_s, k_p, v_p, cu_p, wl.scale)
    rng = np.random.default_rng(12)
    for r in range(wl.B):
        n = wl.n_p[r] // W.ITEM_TOKENS
        wl.block_table[r, :n] = wl.block_table[r, rng.permutation(n)]
    k2, v2, cu2 = assemble_prefix(wl)
    o2, l2 = oracle.prefill_suffix(wl.q, wl.k_s, wl.v_s, wl.cu_s, k2, v2, cu2, wl.scale)
    np.testing.assert_allclose(o2, out, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, lse, rtol=0, atol=1e-13)


# ----------------------------------------------------------- merge identities
def _partial(q, k, v, rows, keys, scale):
    mask = np.zeros((len(q), len(k)), bool)
    mask[np.ix_(rows, keys)] = True
    o, l = oracle.attention_masked(q, k, v, mask, scale)
    return o[rows], l[rows]


def test_merge_of_prefix_and_suffix_partials_is_full():
    rng = np.random.default_rng(13)
    n_p, n_s, D = 21, 9, 16
    q, k, v, pre = rand_seq(rng, n_p, n_s, D)
    out, lse = oracle.bipartite_attention(q, k, v, pre, 0.25)
    U = np.arange(n_p, n_p + n_s)
    pp = _partial(q, k, v, U, np.arange(n_p), 0.25)
    pu = _partial(q, k, v, U, U, 0.25)
    mo, ml = oracle.lse_merge([pp, pu])
    np.testing.assert_allclose(mo, out[U], rtol=0, atol=1e-13)
    np.testing.assert_allclose(ml, lse[U], rtol=0, atol=1e-13)
    # commutative
    mo2, ml2 = oracle.lse_merge([pu, pp])
    np.testing.assert_allclose(mo2, mo, rtol=0, atol=1e-14)
    # any chunking of the prefix, merged in any grouping
    cuts = [0, 4, 5, 13, n_p]
    chunks = [_partial(q, k, v, U, np.arange(a, b), 0.25) for a, b in zip(cuts, cuts[1:])]
    left = oracle.lse_merge([oracle.lse_merge(chunks[:2]), oracle.lse_merge(chunks[2:] + [pu])])
    np.testing.assert_allclose(left[0], out[U], rtol=0, atol=1e-13)
    np.testing.assert_allclose(left[1], lse[U], rtol=0, atol=1e-13)


def test_merge_with_empty_partial_is_identity():
    rng = np.random.default_rng(14)
    q, k, v, pre = rand_seq(rng, 0, 6, 8)
    U = np.arange(6)
    pu = _partial(q, k, v, U, U, 0.5)
    empty = _partial(q, k, v, U, np.array([], int), 0.5)
    assert np.all(np.isneginf(empty[1])) and np.all(empty[0] == 0)
    mo, ml = oracle.lse_merge([empty, pu])
    np.testing.assert_array_equal(ml, pu[1])
    np.testing.assert_allclose(mo, pu[0], rtol=0, atol=0)


def test_planted_mistake_is_caught():
    """A plausible oracle bug (prefix rows allowed to see the suffix) changes
    the prefix rows enough for the brute-force pin to fail."""
    rng = np.random.default_rng(15)
    q, k, v, pre = rand_seq(rng, 5, 4, 8)
    good, _ = oracle.bipartite_attention(q, k, v, pre, 0.35)
    wrong, _ = oracle.attention_masked(q, k, v, np.ones((9, 9)), 0.35)
    ref, _ = brute_force(q, k, v, pre, 0.35)
    assert np.abs(wrong[:5] - ref[:5]).max() > 1e-3
    np.testing.assert_allclose(good, ref, atol=1e-12)


# ----------------------------------------------- prefix rows and per-item rows
def _packed_requests(rng, lens, H, D):
    n = int(sum(lens))
    q = rng.standard_normal((n, H, D))
    k = rng.standard_normal((n, H, D))
    v = rng.standard_normal((n, H, D))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return q, k, v, cu


def test_prefix_rows_brute_force_and_suffix_invisible():
    """Each prefix row matches the explicit-loop definition over its own
    request's prefix, and equals the prefix rows of the full bipartite
    attention with a suffix appended (prefix rows never see the suffix)."""
    rng = np.random.default_rng(21)
    lens, H, D, scale = [1, 4, 9], 2, 4, 0.37
    q, k, v, cu = _packed_requests(rng, lens, H, D)
    out, lse = oracle.prefix_rows(q, k, v, cu, scale)
    for r, n_p in enumerate(lens):
        sl = slice(cu[r], cu[r + 1])
        for h in range(H):
            bo, bl = brute_force(q[sl, h], k[sl, h], v[sl, h], np.ones(n_p, bool), scale)
            np.testing.assert_allclose(out[sl, h], bo, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[h, sl], bl, rtol=0, atol=1e-12)
            # the same request with a random suffix behind its prefix
            qs, ks, vs, pre = rand_seq(rng, n_p, 3, D)
            qs[:n_p], ks[:n_p], vs[:n_p] = q[sl, h], k[sl, h], v[sl, h]
            fo, fl = oracle.bipartite_attention(qs, ks, vs, pre, scale)
            np.testing.assert_allclose(out[sl, h], fo[:n_p], rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[h, sl], fl[:n_p], rtol=0, atol=1e-12)


def test_prefix_rows_library_sdpa():
    """Per request, the prefix rows are unmasked SDPA over that prefix alone."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    rng = np.random.default_rng(22)
    lens, H, D = [5, 33, 64], 3, 32
    q, k, v, cu = _packed_requests(rng, lens, H, D)
    scale = 1.0 / math.sqrt(D)
    out, _ = oracle.prefix_rows(q, k, v, cu, scale)
    for r in range(len(lens)):
        sl = slice(cu[r], cu[r + 1])
        t = lambda x: torch.from_numpy(np.ascontiguousarray(x[sl].transpose(1, 0, 2)))[None]
        ref = F.scaled_dot_product_attention(t(q), t(k), t(v), scale=scale)[0]
        np.testing.assert_allclose(out[sl], ref.numpy().transpose(1, 0, 2), rtol=0, atol=1e-12)


def test_item_local_single_token_items():
    """T = 1: every row sees only itself, so out = v and lse = scale * q.k."""
    rng = np.random.default_rng(23)
    q, k, v, _ = _packed_requests(rng, [7], 2, 8)
    out, lse = oracle.item_local(q, k, v, 1, 0.3)
    np.testing.assert_allclose(out, v, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, 0.3 * np.einsum("thd,thd->ht", q, k), rtol=0, atol=1e-14)


def test_item_local_equal_keys_give_item_mean():
    """Equal keys inside an item: each row returns the mean of its item's
    values, and lse = scale * q.k + ln T."""
    rng = np.random.default_rng(24)
    T, n_items, H, D, scale = 4, 3, 2, 8, 0.5
    q = rng.standard_normal((n_items * T, H, D))
    v = rng.standard_normal((n_items * T, H, D))
    kk = rng.standard_normal((n_items, 1, H, D))
    k = np.repeat(kk, T, axis=1).reshape(n_items * T, H, D)
    out, lse = oracle.item_local(q, k, v, T, scale)
    mean = v.reshape(n_items, T, H, D).mean(axis=1)
    np.testing.assert_allclose(out.reshape(n_items, T, H, D), np.repeat(mean[:, None], T, 1),
                               rtol=0, atol=1e-14)
    ref_lse = scale * np.einsum("thd,thd->ht", q, k) + math.log(T)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-13)


def test_item_local_brute_force_and_isolation():
    """Each item matches the explicit-loop definition over its own tokens,
    and changing every other item leaves it unchanged."""
    rng = np.random.default_rng(25)
    T, n_items, H, D, scale = 4, 5, 2, 6, 0.41
    q, k, v, _ = _packed_requests(rng, [n_items * T], H, D)
    out, lse = oracle.item_local(q, k, v, T, scale)
    for i in range(n_items):
        sl = slice(i * T, (i + 1) * T)
        for h in range(H):
            bo, bl = brute_force(q[sl, h], k[sl, h], v[sl, h], np.ones(T, bool), scale)
            np.testing.assert_allclose(out[sl, h], bo, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[h, sl], bl, rtol=0, atol=1e-12)
    q2, k2, v2 = (x.copy() for x in (q, k, v))
    for x in (q2, k2, v2):
        x[T:] = rng.standard_normal(x[T:].shape)
    out2, lse2 = oracle.item_local(q2, k2, v2, T, scale)
    np.testing.assert_array_equal(out2[:T], out[:T])
    np.testing.assert_array_equal(lse2[:, :T], lse[:, :T])


# ------------------------------------------------ candidate-isolated suffix rows
def _iso_case(rng, lens_p, lens_s, H, D):
    k_p = rng.standard_normal((sum(lens_p), H, D))
    v_p = rng.standard_normal((sum(lens_p), H, D))
    q = rng.standard_normal((sum(lens_s), H, D))
    k_s = rng.standard_normal((sum(lens_s), H, D))
    v_s = rng.standard_normal((sum(lens_s), H, D))
    cu_p = np.concatenate([[0], np.cumsum(lens_p)]).astype(np.int32)
    cu_s = np.concatenate([[0], np.cumsum(lens_s)]).astype(np.int32)
    return q, k_s, v_s, cu_s, k_p, v_p, cu_p


def test_isolated_brute_force():
    """Explicit visible sets: the request's prefix plus the row's own
    candidate of T tokens."""
    rng = np.random.default_rng(31)
    T, H, D, scale = 2, 2, 3, 0.45
    lens_p, lens_s = [3, 0, 5], [4, 2, 6]
    q, k_s, v_s, cu_s, k_p, v_p, cu_p = _iso_case(rng, lens_p, lens_s, H, D)
    out, lse = oracle.prefill_isolated(q, k_s, v_s, cu_s, k_p, v_p, cu_p, T, scale)
    for r in range(3):
        for i in range(cu_s[r], cu_s[r + 1]):
            c0 = cu_s[r] + ((i - cu_s[r]) // T) * T
            for h in range(H):
                vis = [("p", j) for j in range(cu_p[r], cu_p[r + 1])] + \
                      [("s", j) for j in range(c0, c0 + T)]
                kk = lambda t, j: (k_p if t == "p" else k_s)[j, h]
                vv = lambda t, j: (v_p if t == "p" else v_s)[j, h]
                sc = [scale * sum(float(q[i, h, d]) * float(kk(t, j)[d]) for d in range(D))
                      for t, j in vis]
                z = sum(math.exp(x) for x in sc)
                ref = sum(math.exp(x) / z * vv(t, j) for x, (t, j) in zip(sc, vis))
                np.testing.assert_allclose(out[i, h], ref, rtol=0, atol=1e-12)
                assert abs(lse[h, i] - math.log(z)) <= 1e-12


def test_isolated_one_candidate_is_the_plain_prefill():
    """T = n_s (one candidate per request): the ordinary suffix prefill."""
    rng = np.random.default_rng(32)
    lens_p, lens_s, H, D = [7, 0, 12], [4, 4, 4], 2, 8
    q, k_s, v_s, cu_s, k_p, v_p, cu_p = _iso_case(rng, lens_p, lens_s, H, D)
    out, lse = oracle.prefill_isolated(q, k_s, v_s, cu_s, k_p, v_p, cu_p, 4, 0.3)
    ref, ref_lse = oracle.prefill_suffix(q, k_s, v_s, cu_s, k_p, v_p, cu_p, 0.3)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


def test_isolated_is_merge_of_prefix_and_candidate_parts():
    """Prefix part (rows over the prefix alone, masked attention) merged with
    the candidate part (per-item rows) gives the isolated rows; with no
    prefix the isolated rows are the per-item rows themselves."""
    rng = np.random.default_rng(33)
    T, H, D, scale = 4, 2, 8, 0.35
    lens_p, lens_s = [9, 0], [8, 12]
    q, k_s, v_s, cu_s, k_p, v_p, cu_p = _iso_case(rng, lens_p, lens_s, H, D)
    out, lse = oracle.prefill_isolated(q, k_s, v_s, cu_s, k_p, v_p, cu_p, T, scale)
    cand, cand_lse = oracle.item_local(q, k_s, v_s, T, scale)
    # request 0: prefix part by masked attention of its suffix rows over its prefix
    sl = slice(cu_s[0], cu_s[1])
    for h in range(H):
        po, pl = oracle.attention_masked(q[sl, h], k_p[:9, h], v_p[:9, h],
                                         np.ones((8, 9), bool), scale)
        mo, ml = oracle.lse_merge([(po, pl), (cand[sl, h], cand_lse[h, sl])])
        np.testing.assert_allclose(out[sl, h], mo, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[h, sl], ml, rtol=0, atol=1e-12)
    # request 1: no prefix
    sl = slice(cu_s[1], cu_s[2])
    np.testing.assert_allclose(out[sl], cand[sl], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[:, sl], cand_lse[:, sl], rtol=0, atol=1e-12)


def test_isolated_single_token_candidates_without_prefix():
    """T = 1 and no prefix: each row sees only itself (out = v)."""
    rng = np.random.default_rng(34)
    q, k_s, v_s, cu_s, k_p, v_p, cu_p = _iso_case(rng, [0, 0], [3, 5], 2, 4)
    out, lse = oracle.prefill_isolated(q, k_s, v_s, cu_s, k_p, v_p, cu_p, 1, 0.7)
    np.testing.assert_allclose(out, v_s, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, 0.7 * np.einsum("thd,thd->ht", q, k_s), rtol=0, atol=1e-14)


def test_isolated_selected_rows_match_full():
    rng = np.random.default_rng(35)
    q, k_s, v_s, cu_s, k_p, v_p, cu_p = _iso_case(rng, [5, 3], [4, 8], 3, 4)
    out, lse = oracle.prefill_isolated(q, k_s, v_s, cu_s, k_p, v_p, cu_p, 2, 0.5)
    rows = np.array([0, 3, 4, 11], np.int32)
    heads = np.array([2, 0, 1, 2], np.int32)
    so, sl = oracle.prefill_isolated(q, k_s, v_s, cu_s, k_p, v_p, cu_p, 2, 0.5, rows=rows,
                                     heads=heads)
    np.testing.assert_array_equal(so, out[rows, heads])
    np.testing.assert_array_equal(sl, lse[heads, rows])


# ------------------------------------------------------ grouped key/value heads
def test_gqa_library_sdpa():
    """Grouped heads equal torch SDPA with enable_gqa (one request: suffix rows
    over prefix + suffix keys, no mask)."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    rng = np.random.default_rng(41)
    n_p, n_s, H, H_kv, D = 13, 6, 8, 2, 16
    q = rng.standard_normal((n_s, H, D))
    k_s, v_s = rng.standard_normal((n_s, H_kv, D)), rng.standard_normal((n_s, H_kv, D))
    k_p, v_p = rng.standard_normal((n_p, H_kv, D)), rng.standard_normal((n_p, H_kv, D))
    scale = 1.0 / math.sqrt(D)
    out, _ = oracle.prefill_suffix_gqa(q, k_s, v_s, np.array([0, n_s], np.int32), k_p, v_p,
                                       np.array([0, n_p], np.int32), scale)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x.transpose(1, 0, 2)))[None]
    kk, vv = np.concatenate([k_p, k_s]), np.concatenate([v_p, v_s])
    ref = F.scaled_dot_product_attention(t(q), t(kk), t(vv), scale=scale, enable_gqa=True)[0]
    np.testing.assert_allclose(out, ref.numpy().transpose(1, 0, 2), rtol=0, atol=1e-12)


def test_gqa_brute_force_head_mapping():
    """Explicit loops: query head h uses key/value head h // (H // H_kv)."""
    rng = np.random.default_rng(42)
    n_p, n_s, H, H_kv, D, scale = 3, 2, 4, 2, 3, 0.6
    q = rng.standard_normal((n_s, H, D))
    k_s, v_s = rng.standard_normal((n_s, H_kv, D)), rng.standard_normal((n_s, H_kv, D))
    k_p, v_p = rng.standard_normal((n_p, H_kv, D)), rng.standard_normal((n_p, H_kv, D))
    out, lse = oracle.prefill_suffix_gqa(q, k_s, v_s, np.array([0, n_s], np.int32), k_p, v_p,
                                         np.array([0, n_p], np.int32), scale)
    for h in range(H):
        g = h // (H // H_kv)
        kk = np.concatenate([k_p[:, g], k_s[:, g]])
        vv = np.concatenate([v_p[:, g], v_s[:, g]])
        bo, bl = brute_force(np.concatenate([np.zeros((n_p, D)), q[:, h]]), kk, vv,
                             np.array([True] * n_p + [False] * n_s), scale)
        np.testing.assert_allclose(out[:, h], bo[n_p:], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[h], bl[n_p:], rtol=0, atol=1e-12)


# ------------------------------------------------------------- fp8 key/value pool
def test_e4m3_values_worked_and_library():
    """The E4M3 value table: values worked by hand, and torch's float8_e4m3fn
    reading of every code (a library decoder)."""
    import torch
    v = oracle.e4m3_values()
    assert len(v) == 127 and np.all(np.diff(v) > 0)
    for code, want in [(0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
                       (0x38, 1.0), (0x39, 1.125), (0x40, 2.0), (0x7E, 448.0)]:
        assert v[code] == want, hex(code)
    codes = torch.arange(0, 256, dtype=torch.int32).to(torch.uint8)
    lib = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = oracle.e4m3_decode(np.arange(256))
    finite = (np.arange(256) & 0x7F) != 0x7F
    np.testing.assert_array_equal(mine[finite], lib[finite])


def test_e4m3_encode_against_library_and_ties():
    """Nearest code with ties to the even code, against torch's conversion
    (round to nearest even) on float32 values, on every exact value, and on
    every midpoint between neighbours."""
    import torch
    rng = np.random.default_rng(51)
    y = np.concatenate([rng.uniform(-448, 448, 20000), rng.normal(0, 0.01, 20000),
                        rng.normal(0, 1e-3, 5000)]).astype(np.float32)
    lib = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.e4m3_encode(y.astype(np.float64)), lib)
    v = oracle.e4m3_values()
    np.testing.assert_array_equal(oracle.e4m3_encode(v), np.arange(127))
    np.testing.assert_array_equal(oracle.e4m3_encode(-v[1:]), np.arange(1, 127) | 0x80)
    mid = (v[:-1] + v[1:]) / 2
    want = np.where(np.arange(126) % 2 == 0, np.arange(126), np.arange(1, 127))
    np.testing.assert_array_equal(oracle.e4m3_encode(mid), want)
    with pytest.raises(ValueError):
        oracle.e4m3_encode([449.0])


def test_fp8_scale_exponent_closed_forms():
    assert oracle.fp8_scale_exponent(0.0) == 0
    for k in range(-20, 21):
        a = 448.0 * 2.0 ** k
        assert oracle.fp8_scale_exponent(a) == k
        assert oracle.fp8_scale_exponent(a * (1 + 2 ** -20)) == k + 1
        assert oracle.fp8_scale_exponent(a * (1 - 2 ** -20)) == k
    assert oracle.fp8_scale_exponent(100.0) == -2


def test_hand_fp8_block():
    g = json.load(open(os.path.join(GOLDEN, "hand_fp8_block.json")))
    x = np.array(g["x"]).reshape(4, 1, 1)
    codes, exps, back = oracle.fp8_quantize_blocks(x, [0, 4], 4)
    assert exps[0].tolist() == [[g["exponent"]]]
    np.testing.assert_array_equal(codes[:, 0, 0], g["codes"])
    np.testing.assert_array_equal(back[:, 0, 0], g["read_back"])


def test_fp8_blocks_per_block_scale_and_round_trip_bound():
    """Blocks of one request at very different magnitudes each get their own
    scale; every read-back value is within half an E4M3 step (at the block's
    scale) of the stored one."""
    rng = np.random.default_rng(52)
    H, D, bs = 2, 8, 4
    lens = [10, 3, 4]
    x = rng.standard_normal((sum(lens), H, D))
    x[4:8] *= 1e4                      # request 0, block 1
    x[8:10] *= 1e-3                    # request 0, block 2 (partial)
    cu = np.concatenate([[0], np.cumsum(lens)])
    codes, exps, back = oracle.fp8_quantize_blocks(x, cu, bs)
    assert [e.shape for e in exps] == [(3, H), (1, H), (1, H)]
    for r in range(len(lens)):
        for j in range(exps[r].shape[0]):
            t0, t1 = cu[r] + j * bs, min(cu[r + 1], cu[r] + (j + 1) * bs)
            for h in range(H):
                e = exps[r][j, h]
                blk = x[t0:t1, h]
                assert np.abs(blk).max() <= 448 * 2.0 ** e < 2 * np.abs(blk).max()
                y = np.abs(blk) / 2.0 ** e
                step = np.where(y >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(y, 1e-300))) - 3),
                                2.0 ** -9) * 2.0 ** e
                assert np.all(np.abs(back[t0:t1, h] - blk) <= step / 2)
    rel = np.abs(back[8:10] - x[8:10]) / np.abs(x[8:10])
    assert np.median(rel) < 0.05       # the small block kept its precision


def test_kv_scatter_fp8_layout():
    """The fp8 pool holds each request's codes where kv_scatter puts values,
    and each (block, head) scale at the block its table row names."""
    rng = np.random.default_rng(53)
    H, D, bs, nb = 2, 4, 4, 7
    lens = [6, 4]
    x = rng.standard_normal((10, H, D))
    cu = np.array([0, 6, 10])
    bt = np.array([[5, 2], [0, -1]])
    pool, scales = oracle.kv_scatter_fp8(x, cu, bt, nb, bs, 0xFF, -1.0)
    codes, exps, back = oracle.fp8_quantize_blocks(x, cu, bs)
    np.testing.assert_array_equal(pool[5, :, :, :].transpose(1, 0, 2), codes[0:4])
    np.testing.assert_array_equal(pool[2, :, :2, :].transpose(1, 0, 2), codes[4:6])
    np.testing.assert_array_equal(pool[0, :, :, :].transpose(1, 0, 2), codes[6:10])
    assert np.all(pool[2, :, 2:] == 0xFF) and np.all(pool[1] == 0xFF)
    np.testing.assert_array_equal(scales[5], 2.0 ** exps[0][0])
    np.testing.assert_array_equal(scales[2], 2.0 ** exps[0][1])
    np.testing.assert_array_equal(scales[0], 2.0 ** exps[1][0])
    assert np.all(scales[[1, 3, 4, 6]] == -1.0)
    dec = oracle.e4m3_decode(pool[5]) * scales[5][:, None, None]
    np.testing.assert_array_equal(dec.transpose(1, 0, 2), back[0:4])
