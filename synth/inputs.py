"""Seeded host-side input generators and the workload shapes.

Model shapes follow the pages' four model classes (TokenSwift summary, §1 and
§4.1: 1.5B, 7B, 8B and 14B, MHA and GQA); head counts, context lengths, tree
sizes, budgets and vocabularies are those of the workloads this repository
measures (see ``CONFIGS``). Penalty and sampling defaults are the TokenSwift
reproducibility checklist's Table 11 values.
"""

import numpy as np

# Table 11 of the TokenSwift reproducibility checklist (LLaMA3.1-8b row).
TABLE11 = dict(k=20, temperature=1.0, top_p=0.9, min_p=0.05, penalty=1.2, penalty_len=1024)

CONFIGS = {
    "tiny": dict(Hq=8, Hkv=2, d=64, n_ctx=2048, T=8, tree="tiny8", budget=256,
                 n_sink=4, n_recent=64, V=1024, W=256, layers=1, seed=0, sigma=2.0),
    "1.5b": dict(Hq=12, Hkv=2, d=128, n_ctx=100_000, T=24, tree="tokenswift", budget=4096,
                 n_sink=4, n_recent=64, V=151936, W=1024, layers=28, seed=1, sigma=2.0,
                 k_scale=(0.5, 2.0)),
    "7b": dict(Hq=32, Hkv=32, d=128, n_ctx=100_000, T=24, tree="tokenswift", budget=4096,
               n_sink=4, n_recent=64, V=32000, W=1024, layers=32, seed=2, sigma=2.0),
    "8b": dict(Hq=32, Hkv=8, d=128, n_ctx=100_000, T=24, tree="tokenswift", budget=4096,
               n_sink=4, n_recent=64, V=128256, W=1024, layers=32, seed=3, sigma=2.0),
    "14b": dict(Hq=40, Hkv=8, d=128, n_ctx=100_000, T=64, tree="tokenswift", budget=8192,
                n_sink=4, n_recent=64, V=152064, W=1024, layers=48, seed=4, sigma=2.0, reselect=64),
}


def bf16_round(x):
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    rounding = ((u >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    out = ((u + rounding) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


BF16_NAN = np.uint16(0x7FC0)


def tree_parent(kind, T=None):
    """Token-tree shapes as parent arrays (parent[0] = -1, parent[i] < i).

    * "tiny8": a root, a chain of depth 3 under it and 4 more children of the
      root: [-1, 0, 1, 2, 0, 0, 0, 0].
    * "chain": T nodes in a line (plain causal decode of T tokens).
    * "wide": the same with the [1,9,9,9] head part (nodes 1-9, 10-18 under
      node 1, 19-27 under node 10), then chains; 88 nodes hold 20 chains.
    * "tokenswift": the [1,3,3,3] head part along the top-1 path (nodes 1-3
      under the root, 4-6 under node 1, 7-9 under node 4), then reused
      4-gram continuations as chains of 3 nodes under the root until T nodes
      exist (the last chain truncated).
    """
    if kind == "tiny8":
        return [-1, 0, 1, 2, 0, 0, 0, 0]
    if kind == "chain":
        return [-1] + list(range(T - 1))
    if kind == "wide":
        # [1,9,9,9]: nodes 1-9 under the root, 10-18 under node 1, 19-27 under
        # node 10, then 4-gram chains of 3 under the root until T nodes
        par = [-1] + [0] * 9 + [1] * 9 + [10] * 9
        if T <= len(par):
            return par[:T]
        while len(par) < T:
            prev = 0
            for _ in range(3):
                if len(par) >= T:
                    break
                par.append(prev)
                prev = len(par) - 1
        return par
    if kind == "tokenswift":
        head = [-1, 0, 0, 0, 1, 1, 1, 4, 4, 4]
        if T <= len(head):
            return head[:T]
        par = list(head)
        while len(par) < T:
            prev = 0
            for _ in range(3):
                if len(par) >= T:
                    break
                par.append(prev)
                prev = len(par) - 1
        return par
    raise ValueError(f"unknown tree kind {kind!r}")


def attention_inputs(seed, Hq, Hkv, d, n_ctx, T, cap=None, k_scale=None, poison_tail=False):
    """Q [Hq][T][d] and K/V caches [Hkv][cap][d] as bfloat16 bits.

    Rows 0..n_ctx-1 are the committed context, rows n_ctx..n_ctx+T-1 the
    tree nodes' own keys/values. Rows past n_ctx+T (if cap is larger) are
    random, or bfloat16 NaN with ``poison_tail`` so that any read of them
    shows up in the result.
    """
    rows = n_ctx + T
    cap = rows if cap is None else cap
    if cap < rows:
        raise ValueError("cap must be at least n_ctx + T")
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((Hq, T, d), dtype=np.float32)
    k = rng.standard_normal((Hkv, cap, d), dtype=np.float32)
    v = rng.standard_normal((Hkv, cap, d), dtype=np.float32)
    if k_scale is not None:
        lo, hi = k_scale
        s = rng.uniform(lo, hi, size=(Hkv, 1, d)).astype(np.float32)
        k *= s
    qb, kb, vb = bf16_round(q), bf16_round(k), bf16_round(v)
    if poison_tail and cap > rows:
        kb[:, rows:, :] = BF16_NAN
        vb[:, rows:, :] = BF16_NAN
    return dict(q=qb, k=kb, v=vb)


def penalty_inputs(seed, rows, V, W, sigma=2.0, shared_window=False, dup_window=False):
    """Logits N(0, sigma^2) fp32 [rows][V], window ids int32, and u in [0,1)."""
    rng = np.random.default_rng(seed)
    logits = (rng.standard_normal((rows, V), dtype=np.float32) * np.float32(sigma)).astype(np.float32)
    nwin = 1 if shared_window else rows
    window = rng.integers(0, V, size=(nwin, W), dtype=np.int64).astype(np.int32)
    if dup_window and W >= 4:
        window[:, W // 2:W // 2 + 2] = window[:, :2]
    u = rng.random(rows).astype(np.float32)
    return dict(logits=logits, window=window[0] if shared_window else window, u=u)


def random_parent(seed, T):
    """A random tree of T nodes in parents-first order: parent[i] ~ U[0, i)."""
    rng = np.random.default_rng(seed)
    return [-1] + [int(rng.integers(0, i)) for i in range(1, T)]


def accept_inputs(seed, parent, vocab=50, p_match=0.5):
    """Node tokens and target tokens (int32) of one verified tree.

    target[i] is uniform over [0, vocab). Each non-root node copies its
    parent's target token with probability p_match (a planted match) and
    otherwise draws a uniform token, so accepted paths of every length occur.
    """
    rng = np.random.default_rng(seed)
    T = len(parent)
    target = rng.integers(0, vocab, size=T).astype(np.int32)
    node = rng.integers(0, vocab, size=T).astype(np.int32)
    plant = rng.random(T) < p_match
    for i in range(1, T):
        if plant[i]:
            node[i] = target[parent[i]]
    return dict(node_token=node, target=target)


def ngram_window(seed, W, vocab, repeat=0.5, n_phrases=6):
    """A token window (int32 [W]) with repeated phrases, as generated text has.

    Tokens are uniform over [0, vocab) except that, with probability
    `repeat` at each position, one of `n_phrases` fixed 4-token phrases is
    copied in; the last token is the root, drawn like the others.
    """
    rng = np.random.default_rng(seed)
    phrases = rng.integers(0, vocab, size=(n_phrases, 4))
    out = []
    while len(out) < W:
        if rng.random() < repeat:
            out.extend(int(t) for t in phrases[rng.integers(0, n_phrases)])
        else:
            out.append(int(rng.integers(0, vocab)))
    return np.asarray(out[:W], dtype=np.int32)
