"""Oracle for token reutilisation: n-gram retrieval, random n-gram choice and
the draft tree built from head candidates and n-grams.

Test infrastructure only (see the package docstring).

What the pages fix (TokenSwift summary §3.2 "Multi-token Generation and
Token Reutilization", §3.4 "Contextual Penalty and Random N-gram Selection",
§4.4.1 "Tree Configuration", Appendix B.2): frequent 4-grams of the generated
text are reused as extra draft candidates, at most k of them are retrieved
(k = 20 in the checklist's Table 11), a random choice among several valid
n-grams keeps the output diverse, and the tree is a simple ternary
[1,3,3,3] tree of the heads' candidates merged with the n-grams.

Readings taken where the pages are silent:

* The table is the multiset of 4-grams (t_i, t_i+1, t_i+2, t_i+3) lying in the
  last W committed tokens (the workloads draw the n-grams from the penalty
  window, W = 1024); it changes only by the window sliding as tokens are
  committed, so it is recomputed from the window each step.
* Root = the last committed token (the tree's node 0). A 4-gram is valid iff
  its first token is the root token; it offers its last three tokens as a
  draft chain. Valid 4-grams are counted per distinct continuation, and the
  distinct ones are numbered q = 0, 1, ... in order of first occurrence.
* Random choice: when more than k distinct continuations are valid, the k
  with the smallest (rho_q, q) are kept, rho_q being output q of SplitMix64
  seeded with the caller's seed (Steele, Lea and Flood, "Fast Splittable
  Pseudorandom Number Generators", OOPSLA 2014): a uniformly random subset.
* The kept chains are ordered by count (descending), then first occurrence.
* Tree: node 0 is the root; level l = 1..L of the head part holds the three
  candidates of level l (node ids 3(l-1)+1 .. 3l) under the root for l = 1
  and under the first node of level l-1 otherwise (the top-1 path); then each
  kept chain (a, b, c) hangs off the root as three nodes in a line. Nodes
  past T_max are cut off (the last chain may be cut short).
"""

MASK64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15


def splitmix64(seed, j):
    """Output j (0-based) of SplitMix64 started from state `seed`."""
    z = (int(seed) + (int(j) + 1) * GOLDEN_GAMMA) & MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def ngram_candidates(window, k, seed):
    """Kept 4-gram continuations of the window's last token.

    Returns (chosen, n_distinct, n_occurrences); chosen is a list of
    (continuation (a, b, c), count, first position) in tree order.
    """
    w = [int(t) for t in window]
    if not w:
        return [], 0, 0
    root = w[-1]
    distinct = {}                      # continuation -> [first position, count]; insertion order = first occurrence
    occurrences = 0
    for i in range(len(w) - 3):
        if w[i] == root:
            occurrences += 1
            key = (w[i + 1], w[i + 2], w[i + 3])
            if key in distinct:
                distinct[key][1] += 1
            else:
                distinct[key] = [i, 1]
    items = [(key, fc[1], fc[0]) for key, fc in distinct.items()]
    if len(items) > k:
        order = sorted(range(len(items)), key=lambda q: (splitmix64(seed, q), q))
        keep = set(order[:k])
        items = [it for q, it in enumerate(items) if q in keep]
    items.sort(key=lambda it: (-it[1], it[2]))
    return items, len(distinct), occurrences


def build_tree(root_token, head_cand, chains, T_max):
    """(parent, node_token) of the draft tree, at most T_max nodes."""
    parent, token = [-1], [int(root_token)]
    prev_first = 0
    for level, cands in enumerate(head_cand):
        first = len(parent)
        for c in cands:
            parent.append(0 if level == 0 else prev_first)
            token.append(int(c))
        prev_first = first
    for (a, b, c) in chains:
        at = 0
        for t in (a, b, c):
            parent.append(at)
            token.append(int(t))
            at = len(parent) - 1
    return parent[:T_max], token[:T_max]


def ngram_tree(window, k, seed, head_cand, T_max):
    """The whole step: retrieval, choice and tree.

    Returns dict(parent, node_token, T, chains, distinct, occurrences), where
    chains counts the kept chains with at least one node in the tree.
    """
    if len(window) < 1:
        raise ValueError("the window holds at least the root token")
    if any(len(c) != 3 for c in head_cand):
        raise ValueError("each head level offers three candidates (ternary tree)")
    chosen, n_distinct, n_occ = ngram_candidates(window, k, seed)
    L = len(head_cand)
    parent, token = build_tree(window[-1], head_cand, [c[0] for c in chosen], T_max)
    placed = 0
    for j in range(len(chosen)):
        if 1 + 3 * L + 3 * j < T_max:
            placed += 1
    return dict(parent=parent, node_token=token, T=len(parent), chains=placed, distinct=n_distinct,
                occurrences=n_occ, chosen=chosen)
