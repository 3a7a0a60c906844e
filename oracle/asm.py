"""Attention-state memory (ASM), fp64 reference -- TEST INFRASTRUCTURE ONLY.

[ASM] Method: a prefix is moved out of attention into a lookup memory of precomputed
attention states (a, Z).  Offline, the attention states of calibration queries over the
prefix are collected, the queries are clustered into K centroids, and each cluster keeps
the mean of its queries plus one state merged from its members' states with the
online-softmax rule.  Online, a query retrieves the state of its nearest centroid by cosine
similarity and merges it with its own attention over the tokens after the prefix.

Readings (the page leaves these open):
  - per query head h: head h's memory is built from head h's calibration queries over the
    prefix keys of its KV head h // G;
  - K-means is Lloyd's iteration with squared Euclidean assignment (ties: the lowest
    centroid index), given initial centroids and a fixed iteration count; a centroid with
    no members keeps its position;
  - a cluster's state: the online-softmax merge of its members' states gives
    a = sum Z_i a_i / sum Z_i; its partition is the members' mean, Z = sum Z_i / n, so a
    centroid weighs in the final merge like one query of the cluster
    (lse = logsumexp(lse_i) - log n); a cluster without members holds Z = 0;
  - retrieval takes the largest cosine similarity (ties: the lowest index), without the
    optional whitening or RoPE handling.
"""
import math

import numpy as np

from . import indexmem as im


def prefix_states(Q, K, V, scale):
    """Attention states of calibration queries over the prefix.  Q [N, H_q, d],
    K, V [L, H_kv, d] -> a [N, H_q, d], lse [N, H_q]."""
    Q = np.asarray(Q, np.float64)
    N, H_q, d = Q.shape
    G = H_q // K.shape[1]
    a = np.zeros((N, H_q, d))
    lse = np.zeros((N, H_q))
    for i in range(N):
        for h in range(H_q):
            a[i, h], lse[i, h] = im.attention_state(Q[i, h], K[:, h // G], V[:, h // G], scale)
    return a, lse


def kmeans_assign(X, C):
    """Nearest centroid by squared Euclidean distance (ties: the lowest index).
    X [N, d], C [K, d] -> idx [N], dist2 [N, K]."""
    X = np.asarray(X, np.float64)
    C = np.asarray(C, np.float64)
    dist2 = ((X[:, None, :] - C[None, :, :]) ** 2).sum(-1)
    return np.argmin(dist2, axis=1), dist2


def kmeans_update(X, idx, C):
    """Each centroid becomes the mean of its members; one without members stays."""
    X = np.asarray(X, np.float64)
    out = np.array(C, np.float64)
    for k in range(out.shape[0]):
        members = X[idx == k]
        if len(members):
            out[k] = members.mean(0)
    return out


def kmeans(X, C0, iters):
    """Lloyd's iteration from C0 for `iters` rounds; returns (centroids, last assignment)."""
    C = np.array(C0, np.float64)
    idx = kmeans_assign(X, C)[0]
    for _ in range(iters):
        C = kmeans_update(X, idx, C)
        idx = kmeans_assign(X, C)[0]
    return C, idx


def aggregate(a, lse, idx, K):
    """Per cluster: (a_k, lse_k) from its members' states (reading above).
    a [N, d], lse [N], idx [N] -> a_bar [K, d], lse_bar [K]."""
    a = np.asarray(a, np.float64)
    d = a.shape[1]
    a_bar = np.zeros((K, d))
    lse_bar = np.full(K, -np.inf)
    for k in range(K):
        members = np.nonzero(idx == k)[0]
        if len(members) == 0:
            continue
        a_bar[k], l = im.merge_states([(a[i], float(lse[i])) for i in members])
        lse_bar[k] = l - math.log(len(members))
    return a_bar, lse_bar


def lookup(q, C):
    """Index of the centroid with the largest cosine similarity to q (ties: the lowest)."""
    q = np.asarray(q, np.float64)
    C = np.asarray(C, np.float64)
    cos = (C @ q) / (np.linalg.norm(C, axis=1) * np.linalg.norm(q))
    return int(np.argmax(cos))


def output(q, C, a_bar, lse_bar, a_loc, lse_loc):
    """A query's output: its attention state over the tokens after the prefix, merged with
    the retrieved prefix state [ASM, online phase]."""
    k = lookup(q, C)
    return im.merge_states([(np.asarray(a_loc, np.float64), float(lse_loc)), (a_bar[k], float(lse_bar[k]))]), k
