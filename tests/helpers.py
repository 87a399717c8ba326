"""Shared test helpers: oracle-side assembly of each request's prefix and
sampled-row comparisons.  Only oracle functions compute expected values."""
import numpy as np

import oracle
from prefix_reuse_attention_amd import workloads as W


def assemble_prefix(wl, requests=None):
    """Each request's prefix in the order it sees it (item mode: its listed
    items' tokens).  With `requests`, other requests get an empty prefix."""
    ks, vs, cu = [], [], [0]
    want = set(range(wl.B)) if requests is None else set(int(r) for r in requests)
    for r in range(wl.B):
        if r not in want:
            cu.append(cu[-1])
            continue
        if wl.mode[r] == W.ITEM:
            ids = wl.block_table[r, : wl.n_p[r] // W.ITEM_TOKENS]
            ks.append(oracle.gather_item_prefix(wl.item_k, ids, W.ITEM_TOKENS))
            vs.append(oracle.gather_item_prefix(wl.item_v, ids, W.ITEM_TOKENS))
        else:
            ks.append(wl.user_k[wl.cu_user[r]:wl.cu_user[r + 1]])
            vs.append(wl.user_v[wl.cu_user[r]:wl.cu_user[r + 1]])
        cu.append(cu[-1] + len(ks[-1]))
    shape = (0, wl.H, wl.D)
    dt = np.uint16 if wl.dtype == "bf16" else np.float32
    k = np.concatenate(ks) if ks else np.zeros(shape, dt)
    v = np.concatenate(vs) if vs else np.zeros(shape, dt)
    return k, v, np.array(cu, np.int32)


def oracle_full(wl):
    k_p, v_p, cu_p = assemble_prefix(wl)
    return oracle.prefill_suffix(wl.q, wl.k_s, wl.v_s, wl.cu_s, k_p, v_p, cu_p, wl.scale)


def sample_pairs(wl, n, seed):
    """n (row, head) pairs: random rows plus the first and last row of the
    batch and of the longest request."""
    rng = np.random.default_rng(seed)
    rows = rng.integers(0, wl.total_s, size=n).astype(np.int32)
    r_long = int(np.argmax(wl.n_s))
    extra = [0, wl.total_s - 1, int(wl.cu_s[r_long]), int(wl.cu_s[r_long + 1]) - 1]
    rows = np.concatenate([rows, np.array(extra, np.int32)])
    heads = rng.integers(0, wl.H, size=len(rows)).astype(np.int32)
    return rows, heads


def oracle_sampled(wl, rows, heads):
    req = np.searchsorted(wl.cu_s, rows, side="right") - 1
    k_p, v_p, cu_p = assemble_prefix(wl, np.unique(req))
    return oracle.prefill_suffix(wl.q, wl.k_s, wl.v_s, wl.cu_s, k_p, v_p, cu_p, wl.scale,
                                 rows=rows, heads=heads)


def as_f64(a, dtype_name):
    return (W.bf16_to_f32(a) if dtype_name == "bf16" else a).astype(np.float64)


def check_close(got, ref, dtype_name, strict_abs=None, what="out"):
    """The graded bar (max-abs 1e-5 fp32, 2e-2 bf16) plus, for bf16, a
    relative-RMS gate of 1e-2 and an optional tighter max-abs gate."""
    d = np.abs(got - ref)
    mx = float(d.max()) if d.size else 0.0
    if dtype_name == "f32":
        assert mx <= 1e-5, f"{what}: max-abs {mx:.3e} > 1e-5"
        return mx
    assert mx <= 2e-2, f"{what}: max-abs {mx:.3e} > 2e-2"
    den = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    if den > 0:
        rel = float(np.sqrt(np.mean((got - ref) ** 2))) / den
        assert rel <= 1e-2, f"{what}: relative RMS {rel:.3e} > 1e-2"
    if strict_abs is not None:
        assert mx <= strict_abs, f"{what}: max-abs {mx:.3e} > {strict_abs}"
    return mx
