"""Oracle for prefix-reuse ("bipartite") attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path never does: it runs
the HIP library and fails loudly when that library is missing.

The definitions below follow the Bat page ("Bat: Efficient Generative
Recommender Serving with Bipartite Attention"):

* sections "This paper's idea" and "Why it works" (permutation invariance of
  user and item tokens): no positional encoding, no causal mask, and either
  the user history or a set of items may be the cached prefix;
* sections "Problem" and "Why this problem is worth solving": the prefix's
  key/value cache is built once and reused across queries;
* the UG-Separation page's abstract: tokens that stay purely user-side are
  the reusable ones, hence prefix rows attend within the prefix only;
* the GBLA page's abstract: encoder attention is bidirectional.

Every function is float64 and plain: the masked attention and the batched
suffix-row prefill live in ``oracle.c`` (two-pass softmax per row), the rest
(mask construction, item-prefix gather, paged-pool scatter, log-sum-exp merge)
is a few lines of numpy each.  Pins: ``tests/test_oracle.py``.
"""
import ctypes
import math
import os

import numpy as np

from .build import ensure_built

_lib = None

F32, BF16, F64 = 0, 1, 2


def _load():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(ensure_built())
        p = ctypes.c_void_p
        i = ctypes.c_int
        _lib.oracle_attention_masked.argtypes = [i, i, i, i, p, p, p, p,
                                                 ctypes.c_double, p, p]
        _lib.oracle_attention_masked.restype = None
        _lib.oracle_prefill_suffix.argtypes = [i, i, i, i, p, p, p, p, p, p, p,
                                               ctypes.c_double, i, p, p, p, p]
        _lib.oracle_prefill_suffix.restype = ctypes.c_int
        _lib.oracle_num_threads.argtypes = []
        _lib.oracle_num_threads.restype = ctypes.c_int
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _as_input(x):
    """Return (contiguous array, dtype code).  uint16 arrays are bf16 bits."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return x, BF16
    if x.dtype == np.float32:
        return x, F32
    return np.ascontiguousarray(x, dtype=np.float64), F64


def num_threads() -> int:
    return _load().oracle_num_threads()


def default_scale(D: int) -> float:
    """Softmax scale 1/sqrt(D), rounded once to float32 (the value both sides use)."""
    return float(np.float32(1.0 / math.sqrt(D)))


def attention_masked(q, k, v, mask, scale):
    """Masked softmax attention for one head, float64.

    q [n_q, D], k/v [n_k, D], mask [n_q, n_k] (True = visible).
    Returns (out [n_q, D] float64, lse [n_q] float64, natural log).
    """
    q, dt = _as_input(q)
    k, dk = _as_input(k)
    v, dv = _as_input(v)
    if not (dt == dk == dv):
        q, k, v = (np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v))
        dt = F64
    n_q, D = q.shape
    n_k = k.shape[0]
    m = np.ascontiguousarray(mask, dtype=np.uint8).reshape(n_q, n_k)
    out = np.zeros((n_q, D), np.float64)
    lse = np.zeros((n_q,), np.float64)
    _load().oracle_attention_masked(n_q, n_k, D, dt, _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(m), float(scale), _ptr(out), _ptr(lse))
    return out, lse


def prefix_only_mask(in_prefix):
    """The bipartite mask over one request's tokens.

    in_prefix[j] is True for prefix tokens.  Query i may see key j iff j is a
    prefix token, or both i and j are suffix tokens: prefix rows see only the
    prefix, suffix rows see every token.  Token order plays no role.
    """
    p = np.asarray(in_prefix, dtype=bool)
    return p[None, :] | (~p[:, None] & ~p[None, :])


def bipartite_attention(q, k, v, in_prefix, scale):
    """All rows (prefix and suffix) of one request and head, float64."""
    return attention_masked(q, k, v, prefix_only_mask(in_prefix), scale)


def prefill_suffix(q, k_s, v_s, cu_s, k_p, v_p, cu_p, scale, rows=None,
                   heads=None):
    """Batched suffix-row prefill over packed [tokens, H, D] inputs, float64.

    Request r's suffix is rows cu_s[r]:cu_s[r+1] of q/k_s/v_s and its prefix
    (in the order it sees it) is rows cu_p[r]:cu_p[r+1] of k_p/v_p.  With
    rows/heads None the result is out [total_s, H, D] and lse [H, total_s];
    otherwise out [n, D] and lse [n] for the (rows[i], heads[i]) pairs.
    """
    q, dt = _as_input(q)
    arrs = [q]
    for x in (k_s, v_s, k_p, v_p):
        x, d2 = _as_input(x)
        if d2 != dt:
            raise TypeError("all inputs must share one dtype")
        arrs.append(x)
    q, k_s, v_s, k_p, v_p = arrs
    total_s, H, D = q.shape
    cu_s = np.ascontiguousarray(cu_s, dtype=np.int32)
    cu_p = np.ascontiguousarray(cu_p, dtype=np.int32)
    B = cu_s.shape[0] - 1
    if cu_p.shape[0] != B + 1 or cu_s[-1] != total_s:
        raise ValueError("cu_seqlens do not match the packed inputs")
    if rows is None:
        n_sel = -1
        sr = sh = np.zeros(1, np.int32)
        out = np.zeros((total_s, H, D), np.float64)
        lse = np.zeros((H, total_s), np.float64)
    else:
        sr = np.ascontiguousarray(rows, dtype=np.int32)
        sh = np.ascontiguousarray(heads, dtype=np.int32)
        n_sel = sr.shape[0]
        out = np.zeros((n_sel, D), np.float64)
        lse = np.zeros((n_sel,), np.float64)
    rc = _load().oracle_prefill_suffix(B, H, D, dt, _ptr(q), _ptr(k_s), _ptr(v_s),
                                       _ptr(cu_s), _ptr(k_p), _ptr(v_p), _ptr(cu_p),
                                       float(scale), n_sel, _ptr(sr), _ptr(sh),
                                       _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("selected row or head out of range")
    return out, lse


def _no_prefix(q, B):
    """An empty cached prefix for every request: zero key rows, zero lengths."""
    x = np.ascontiguousarray(q)
    empty = np.zeros((0,) + x.shape[1:], dtype=x.dtype if x.dtype in (np.uint16, np.float32)
                     else np.float64)
    return empty, np.zeros(B + 1, np.int32)


def prefix_rows(q_p, k_p, v_p, cu_p, scale, rows=None, heads=None):
    """Prefix rows of the bipartite mask, batched over packed [tokens, H, D].

    Request r's prefix tokens are rows cu_p[r]:cu_p[r+1]; each such row sees
    exactly the prefix tokens of its own request (never the suffix).  That is
    a row group attending to itself with nothing cached before it, so the
    batched prefill above with an empty prefix computes it.  Returns
    (out, lse) shaped as prefill_suffix's.
    """
    cu_p = np.ascontiguousarray(cu_p, dtype=np.int32)
    empty, zeros = _no_prefix(q_p, cu_p.shape[0] - 1)
    return prefill_suffix(q_p, k_p, v_p, cu_p, empty, empty, zeros, scale, rows, heads)


def item_local(q, k, v, tokens_per_item, scale, rows=None, heads=None):
    """Per-item prefix rows: item i owns rows i*T .. i*T+T-1 (T =
    tokens_per_item) of packed [n_items*T, H, D], and each of them sees only
    its own item's T tokens (the block-diagonal form).  Returns (out, lse)
    shaped as prefill_suffix's.
    """
    n = np.asarray(q).shape[0]
    T = int(tokens_per_item)
    if T <= 0 or n % T:
        raise ValueError("rows must be a whole number of items")
    cu = np.arange(0, n + 1, T, dtype=np.int32)
    empty, zeros = _no_prefix(q, n // T)
    return prefill_suffix(q, k, v, cu, empty, empty, zeros, scale, rows, heads)


def prefill_suffix_gqa(q, k_s, v_s, cu_s, k_p, v_p, cu_p, scale, rows=None, heads=None):
    """prefill_suffix with grouped key/value heads, float64.

    q is [total_s, H, D]; k_s/v_s and k_p/v_p carry H_kv heads, H a multiple
    of H_kv.  Query head h attends with key/value head h // (H // H_kv):
    that is the plain prefill over key/value heads repeated H // H_kv times
    each, which is how it is computed here.
    """
    H = np.asarray(q).shape[1]
    H_kv = np.asarray(k_s).shape[1]
    if H % H_kv:
        raise ValueError("query heads must be a multiple of key/value heads")
    g = H // H_kv
    rep = lambda x: np.repeat(np.asarray(x), g, axis=1)
    return prefill_suffix(q, rep(k_s), rep(v_s), cu_s, rep(k_p), rep(v_p), cu_p, scale,
                          rows, heads)


def _widen(x):
    """float64 values of a float32 or bf16-bits (uint16) array, exactly."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def prefill_isolated(q, k_s, v_s, cu_s, k_p, v_p, cu_p, tokens_per_candidate, scale,
                     rows=None, heads=None):
    """Candidate-isolated suffix rows, float64, written out plainly.

    Request r's suffix rows cu_s[r]:cu_s[r+1] form candidates of T =
    tokens_per_candidate consecutive tokens; a row sees every prefix token of
    its request (rows cu_p[r]:cu_p[r+1] of k_p/v_p) and the T tokens of its own
    candidate, nothing else.  Per visible set: max, exp-sum, normalised sum.
    Returns (out, lse) shaped as prefill_suffix's.
    """
    cu_s = np.asarray(cu_s, np.int64)
    cu_p = np.asarray(cu_p, np.int64)
    T = int(tokens_per_candidate)
    total_s, H, D = np.asarray(q).shape
    if rows is None:
        sel_r = np.repeat(np.arange(total_s), H)
        sel_h = np.tile(np.arange(H), total_s)
    else:
        sel_r, sel_h = np.asarray(rows, np.int64), np.asarray(heads, np.int64)
    out = np.zeros((len(sel_r), D))
    lse = np.zeros(len(sel_r))
    for n, (i, h) in enumerate(zip(sel_r, sel_h)):
        r = int(np.searchsorted(cu_s, i, side="right") - 1)
        c0 = cu_s[r] + ((i - cu_s[r]) // T) * T
        keys = np.concatenate([_widen(k_p[cu_p[r]:cu_p[r + 1], h]), _widen(k_s[c0:c0 + T, h])])
        vals = np.concatenate([_widen(v_p[cu_p[r]:cu_p[r + 1], h]), _widen(v_s[c0:c0 + T, h])])
        sc = scale * (keys @ _widen(q[i, h]))
        m = sc.max()
        w = np.exp(sc - m)
        z = w.sum()
        lse[n] = m + math.log(z)
        out[n] = (w / z) @ vals
    if rows is None:
        return out.reshape(total_s, H, D), lse.reshape(total_s, H).T.copy()
    return out, lse


def gather_item_prefix(item_tokens, item_ids, tokens_per_item):
    """An item-mode prefix: the listed items' tokens, in list order.

    item_tokens is [num_items * tokens_per_item, ...] (item i owns rows
    i*tpi .. i*tpi+tpi-1); item_ids lists the request's items.
    """
    ids = np.asarray(item_ids, dtype=np.int64)
    rows = (ids[:, None] * tokens_per_item + np.arange(tokens_per_item)[None, :]).reshape(-1)
    return item_tokens[rows]


def kv_scatter(x, cu_lens, block_table, num_blocks, block_size, fill):
    """The paged pool the prefix build must produce.

    x is packed [tokens, H, D]; token t of request r lands in block
    block_table[r][t // block_size], slot t % block_size, giving a pool laid
    out [num_blocks, H, block_size, D].  Slots no token maps to keep `fill`.
    """
    x = np.asarray(x)
    _, H, D = x.shape
    pool = np.empty((num_blocks, H, block_size, D), dtype=x.dtype)
    pool[...] = fill
    bt = np.asarray(block_table)
    for r in range(len(cu_lens) - 1):
        for t in range(int(cu_lens[r + 1] - cu_lens[r])):
            blk = int(bt[r, t // block_size])
            pool[blk, :, t % block_size, :] = x[cu_lens[r] + t]
    return pool


def lse_merge(parts):
    """Log-sum-exp merge of attention partials over disjoint key sets.

    parts is a list of (out [..., D], lse [...]) with out normalised over its
    own keys.  lse = log sum_i exp(lse_i); out = sum_i exp(lse_i - lse) out_i.
    An empty partial (lse = -inf) contributes nothing.
    """
    lses = np.stack([np.asarray(l, np.float64) for _, l in parts])
    lse = np.logaddexp.reduce(lses, axis=0)
    out = np.zeros_like(np.asarray(parts[0][0], np.float64))
    for o, l in parts:
        w = np.where(np.isneginf(l), 0.0, np.exp(np.asarray(l) - np.where(np.isneginf(lse), 0.0, lse)))
        out = out + w[..., None] * np.asarray(o, np.float64)
    return out, lse


# ------------------------------------------------------------- fp8 key/value pool
#
# Reading taken (the pages do not describe a compressed cache; an fp8 pool
# only trades precision for pool capacity, which the Bat page's "What it
# costs" counts against item caches): each block of a prefix's keys (and,
# separately, values), per head, is stored as OCP FP8 E4M3 codes with one
# power-of-two scale 2^e per (block, head), e being the smallest integer with
# amax <= 448 * 2^e (amax: the block's largest magnitude; e = 0 for an all-zero
# block).  A value x is stored as the E4M3 code nearest to x / 2^e (ties to the
# even code, sign kept) and read back as code value * 2^e.  The attention over
# such a pool is the plain attention above with the prefix keys/values
# replaced by their read-back values.

E4M3_MAX = 448.0


def e4m3_values():
    """The finite non-negative values of OCP FP8 E4M3, indexed by code
    0x00 .. 0x7E: exponent field E (4 bits, bias 7) and mantissa M (3 bits);
    E = 0 holds M * 2^-9, E >= 1 holds 2^(E - 7) * (1 + M / 8).  Code 0x7F
    is NaN and has no value."""
    vals = []
    for code in range(0x7F):
        E, M = code >> 3, code & 7
        vals.append(M * 2.0 ** -9 if E == 0 else 2.0 ** (E - 7) * (1 + M / 8))
    return np.array(vals)


def e4m3_decode(codes):
    """float64 values of uint8 E4M3 codes (sign bit 0x80; 0x7F and 0xFF are NaN)."""
    codes = np.asarray(codes, np.uint8)
    mag = np.append(e4m3_values(), np.nan)[codes & 0x7F]
    return np.where(codes & 0x80, -mag, mag)


def e4m3_encode(y):
    """uint8 E4M3 codes of float64 values |y| <= 448: the nearest finite
    magnitude, ties to the even code; the sign bit is the sign of y."""
    y = np.asarray(y, np.float64)
    a = np.abs(y)
    if np.any(a > E4M3_MAX):
        raise ValueError("E4M3 holds magnitudes up to 448")
    table = e4m3_values()
    hi = np.minimum(np.searchsorted(table, a), len(table) - 1)   # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - table[lo], table[hi] - a
    code = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(table[hi] == a, hi, code)                    # exact hits
    return (code | (np.signbit(y).astype(np.int64) << 7)).astype(np.uint8)


def fp8_scale_exponent(amax):
    """The smallest integer e with amax <= 448 * 2^e (0 for amax = 0)."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    e = math.frexp(amax)[1] - 9          # 2^(e+9) > amax >= 448 * 2^(e-1) fails below
    while amax > E4M3_MAX * 2.0 ** e:
        e += 1
    while amax <= E4M3_MAX * 2.0 ** (e - 1):
        e -= 1
    return e


def fp8_quantize_blocks(x, cu_lens, block_size):
    """Per request r, per block j of its tokens (tokens j*bs .. of the
    request, the last block possibly partial) and per head: the scale
    exponent of the block and its tokens' E4M3 codes.  x is packed
    [tokens, H, D] (bf16 bits, float32 or float64).  Returns (codes
    [tokens, H, D] uint8, exps: list over requests of [blocks, H] int,
    read-back values [tokens, H, D] float64)."""
    xv = _widen(x)
    cu = np.asarray(cu_lens, np.int64)
    codes = np.zeros(xv.shape, np.uint8)
    back = np.zeros(xv.shape, np.float64)
    exps = []
    H = xv.shape[1]
    for r in range(len(cu) - 1):
        n = int(cu[r + 1] - cu[r])
        nb = -(-n // block_size)
        er = np.zeros((nb, H), np.int64)
        for j in range(nb):
            t0 = int(cu[r]) + j * block_size
            t1 = int(cu[r]) + min(n, (j + 1) * block_size)
            for h in range(H):
                blk = xv[t0:t1, h]
                e = fp8_scale_exponent(np.abs(blk).max())
                er[j, h] = e
                c = e4m3_encode(blk / 2.0 ** e)
                codes[t0:t1, h] = c
                back[t0:t1, h] = e4m3_decode(c) * 2.0 ** e
        exps.append(er)
    return codes, exps, back


def kv_scatter_fp8(x, cu_lens, block_table, num_blocks, block_size, fill_code, fill_scale):
    """The fp8 pool the fp8 prefix build must produce: the codes laid out as
    kv_scatter lays out values ([num_blocks, H, block_size, D], untouched
    slots keep fill_code) and the scales 2^e at [block_table[r][j], h]
    (untouched blocks keep fill_scale)."""
    codes, exps, _ = fp8_quantize_blocks(x, cu_lens, block_size)
    pool = kv_scatter(codes, cu_lens, block_table, num_blocks, block_size, fill_code)
    H = codes.shape[1]
    scales = np.full((num_blocks, H), fill_scale, np.float64)
    bt = np.asarray(block_table)
    for r, er in enumerate(exps):
        for j in range(er.shape[0]):
            scales[int(bt[r, j])] = 2.0 ** er[j]
    return pool, scales
