"""Brute-force grouped top-k routing and a textbook dense layer, for pinning the oracle.

Written independently of ``oracle/``: instead of greedy selection it enumerates
every admissible choice and keeps the best one, so a slip in the oracle's
ordering, indexing or tie handling shows up as a disagreement.

Routing rule (baseRT issue "Requesting converter + runtime support for the
Nemotron-H architecture", section "Architecture (config.json)", with the
sigmoid score, top-2 group score, selection-only bias and lowest-index tie
break read as in the oracle):

* group score of g = the largest c_a + c_b over pairs a < b of experts in g
  (c_e itself for one-expert groups);
* the chosen groups are the size-tg subset of largest total group score;
* the chosen experts are the size-k subset, inside the chosen groups, of
  largest total c;
* among equal totals the lexicographically smallest sorted tuple wins.
"""

from __future__ import annotations

import itertools

import numpy as np


def sigmoid(v):
    return 1.0 / (1.0 + np.exp(-np.asarray(v, np.float64)))


def _best_subset(items, size, score):
    best, best_key = None, None
    for sub in itertools.combinations(sorted(items), size):
        key = score(sub)
        if best is None or key > best_key:  # combinations come in lexicographic order
            best, best_key = sub, key
    return best


def route_token(logits, bias, n_group, topk_group, top_k, scale=2.5, norm=True):
    logits = np.asarray(logits, np.float64)
    E = logits.size
    Eg = E // n_group
    s = sigmoid(logits)
    c = s + np.asarray(bias, np.float64)
    gscore = []
    for g in range(n_group):
        members = range(g * Eg, (g + 1) * Eg)
        if Eg == 1:
            gscore.append(c[g])
        else:
            gscore.append(max(c[a] + c[b] for a, b in itertools.combinations(members, 2)))
    groups = _best_subset(range(n_group), topk_group, lambda sub: sum(gscore[g] for g in sub))
    eligible = [e for g in groups for e in range(g * Eg, (g + 1) * Eg)]
    experts = _best_subset(eligible, top_k, lambda sub: sum(c[e] for e in sub))
    experts = np.array(sorted(experts), np.int32)
    sv = s[experts]
    w = scale * sv / sv.sum() if norm else scale * sv
    return experts, w


def relu2_mlp(x, w_up, w_down):
    """Textbook dense relu^2 MLP in fp64: w_down @ relu(w_up @ x)^2."""
    u = np.asarray(w_up, np.float64) @ np.asarray(x, np.float64).T
    return (np.asarray(w_down, np.float64) @ (np.maximum(u, 0.0) ** 2)).T
