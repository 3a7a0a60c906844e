"""Seeded input generation.

Every tensor is drawn in fp64 from its own stream
``PCG64(SeedSequence([cfg_id, layer, tensor_id, batch_index]))`` and rounded once to
the workload's storage type (fp32, or bf16 with round-to-nearest-even).  bf16 tensors
are returned as ``uint16`` bit patterns; both the oracle and the GPU side read the
same bytes.

Only the frozen base model's projections (Q/K/V = X W^T for the small workloads)
and the needle planting (a minimum-norm linear solve on the inputs) are computed
here; both are input construction, outside the method.
"""
import numpy as np

from .configs import Config

# tensor ids of the seed streams
T_X, T_WQ, T_WK, T_WV, T_WKI, T_WQI, T_WG, T_WGM = 1, 2, 3, 4, 5, 6, 7, 8
T_QWIN, T_K, T_V, T_NEEDLE, T_OUTLIER = 9, 10, 11, 12, 13
T_DEC_X, T_DEC_Q, T_DEC_K, T_DEC_V, T_SCORES = 20, 21, 22, 23, 24


def rng(cfg_id: int, layer: int, tensor_id: int, batch_index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([cfg_id, layer, tensor_id, batch_index])))


# ----------------------------------------------------------------------------- formats

def bf16_round(x) -> np.ndarray:
    """Round float64 values to bf16 (round-to-nearest-even), returned as uint16 bits.

    The rounding is done in one step from fp64 (no double rounding through fp32):
    x is scaled to an integer grid of 2^(e-7) and rounded half-to-even.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    _, e = np.frexp(xf)                    # xf = m * 2^e with 0.5 <= |m| < 1
    e = np.maximum(e - 1, -126)            # unbiased exponent, subnormals share 2^-126
    ulp = np.ldexp(1.0, e - 7)
    r = np.round(xf / ulp) * ulp           # np.round is half-to-even; exact in fp64
    r = np.where(np.abs(r) > 3.3895313892515355e38, np.copysign(np.inf, r), r)
    out[...] = np.where(finite, r, x)
    bits = out.astype(np.float32).view(np.uint32)   # exact: r has <= 8 significant bits
    return (bits >> 16).astype(np.uint16)


def bf16_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_storage(x64: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_round(x64)
    if dtype == "f32":
        return np.asarray(x64, dtype=np.float64).astype(np.float32)
    raise ValueError(dtype)


def from_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage -> float64 (exact)."""
    if dtype == "bf16":
        return bf16_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------- helpers

def _normal(cfg, layer, tid, bi, shape, std=1.0):
    return rng(cfg.cfg_id, layer, tid, bi).standard_normal(shape) * std


def needle_positions(cfg: Config) -> np.ndarray:
    """Needles at uniformly spaced depths 0%..100% of the non-window prefix."""
    n = cfg.needles
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    if n == 1:
        return np.zeros(1, dtype=np.int64)
    span = cfg.L - cfg.W - 1
    return np.array([int(np.floor(i * span / (n - 1) + 0.5)) for i in range(n)], dtype=np.int64)


def outlier_channels(cfg: Config, layer: int) -> np.ndarray:
    """[H_kv, c] channel indices scaled as key outliers (same for prefill and decode)."""
    r = rng(cfg.cfg_id, layer, T_OUTLIER, 0)
    return np.stack([np.sort(r.permutation(cfg.d)[:cfg.outlier_channels])
                     for _ in range(cfg.H_kv)]) if cfg.outlier_channels else np.zeros((cfg.H_kv, 0), np.int64)


def _aligned(target_dir, current, cos=0.95):
    """Vector of |current|'s norm at cosine `cos` with target_dir, in the plane of both."""
    u = target_dir / np.linalg.norm(target_dir)
    perp = current - (current @ u) * u
    pn = np.linalg.norm(perp)
    if pn < 1e-12:
        perp = np.roll(u, 1) - (np.roll(u, 1) @ u) * u
        pn = np.linalg.norm(perp)
    return np.linalg.norm(current) * (cos * u + np.sqrt(1 - cos * cos) * perp / pn)


def _cos(a, b):
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


# ----------------------------------------------------------------------------- weights

def make_weights(cfg: Config, layer: int = 0) -> dict:
    """Random-init weights ~ N(0, 1/fan_in) of the base projections (small workloads),
    the indexer and the memory gate, in storage format.  gamma (QK-norm) = 1, fp32."""
    L, st = layer, cfg.dtype
    w = {}
    if cfg.qkv_from_hidden:
        w["W_q"] = _normal(cfg, L, T_WQ, 0, (cfg.H_q * cfg.d, cfg.D), cfg.D ** -0.5)
        w["W_k"] = _normal(cfg, L, T_WK, 0, (cfg.H_kv * cfg.d, cfg.D), cfg.D ** -0.5)
        w["W_v"] = _normal(cfg, L, T_WV, 0, (cfg.H_kv * cfg.d, cfg.D), cfg.D ** -0.5)
    if cfg.H_I:
        w["W_kI"] = to_storage(_normal(cfg, L, T_WKI, 0, (cfg.d_I, cfg.D), cfg.D ** -0.5), st)
        w["W_qI"] = to_storage(_normal(cfg, L, T_WQI, 0, (cfg.H_I, cfg.d_I, cfg.d), cfg.d ** -0.5), st)
        w["W_g"] = to_storage(_normal(cfg, L, T_WG, 0, (cfg.H_I, cfg.D), cfg.D ** -0.5), st)
        w["gamma_k"] = np.ones(cfg.d_I, np.float32)
        w["gamma_q"] = np.ones(cfg.d_I, np.float32)
    if not cfg.momentkv:
        w["w_g"] = to_storage(_normal(cfg, L, T_WGM, 0, (cfg.H_q, cfg.d), cfg.d ** -0.5), st)
    return w


# ----------------------------------------------------------------------------- prefill

def make_prefill(cfg: Config, layer: int = 0, batches=None, weights=None) -> dict:
    """Prefill inputs of one layer for the listed batch elements.

    Returns storage-format arrays: X [b,L,D], Qwin [b,W,H_q,d] (queries of positions
    L-W..L-1), K, V [b,L,H_kv,d], plus the weights and the needle positions.
    """
    if batches is None:
        batches = list(range(cfg.b))
    w = make_weights(cfg, layer) if weights is None else weights
    st = cfg.dtype
    Xs, Qs, Ks, Vs = [], [], [], []
    pos = needle_positions(cfg)
    out_ch = outlier_channels(cfg, layer)
    for bi in batches:
        X = None
        if cfg.D:
            X = to_storage(_normal(cfg, layer, T_X, bi, (cfg.L, cfg.D)), st)
        if cfg.qkv_from_hidden:
            Xd = from_storage(X, st)
            if len(pos):
                Xd = _plant_needles_hidden(cfg, w, Xd, pos)
                X = to_storage(Xd, st)
                Xd = from_storage(X, st)
            Q = to_storage((Xd[cfg.L - cfg.W:] @ w["W_q"].T).reshape(cfg.W, cfg.H_q, cfg.d), st)
            K = to_storage((Xd @ w["W_k"].T).reshape(cfg.L, cfg.H_kv, cfg.d), st)
            V = to_storage((Xd @ w["W_v"].T).reshape(cfg.L, cfg.H_kv, cfg.d), st)
            if len(pos):
                _check_needles(cfg, w, X, Q, K, pos)
        else:
            Q = to_storage(_normal(cfg, layer, T_QWIN, bi, (cfg.W, cfg.H_q, cfg.d)), st)
            Kd = _normal(cfg, layer, T_K, bi, (cfg.L, cfg.H_kv, cfg.d))
            if cfg.outlier_channels:
                for g in range(cfg.H_kv):
                    Kd[:, g, out_ch[g]] *= cfg.outlier_scale
            V = to_storage(_normal(cfg, layer, T_V, bi, (cfg.L, cfg.H_kv, cfg.d)), st)
            if len(pos):
                Kd, X = _plant_needles_direct(cfg, w, X, from_storage(Q, st), Kd, pos)
            K = to_storage(Kd, st)
            if len(pos):
                _check_needles(cfg, w, X, Q, K, pos)
        Xs.append(X)
        Qs.append(Q)
        Ks.append(K)
        Vs.append(V)
    out = dict(w)
    if cfg.D:
        out["X"] = np.stack(Xs)
    out["Qwin"] = np.stack(Qs)
    out["K"] = np.stack(Ks)
    out["V"] = np.stack(Vs)
    out["needles"] = pos
    return out


def _indexer_query_direction(cfg, w, q_last):
    """Sum over indexer heads of the down-projected last query (ungated, unnormalised):
    the direction a needle's indexer key is aligned with."""
    WqI = from_storage(w["W_qI"], cfg.dtype)
    c = [(h * cfg.H_q) // cfg.H_I for h in range(cfg.H_I)]
    return sum(WqI[h] @ q_last[c[h]] for h in range(cfg.H_I))


def _plant_needles_hidden(cfg, w, Xd, pos):
    """Min-norm correction of each needle's hidden row so that its model key (every KV
    head) and its indexer key point at the last query at cosine 0.95."""
    q_last = (Xd[cfg.L - 1] @ w["W_q"].T).reshape(cfg.H_q, cfg.d)
    WkI = from_storage(w["W_kI"], cfg.dtype)
    A = np.concatenate([w["W_k"], WkI], axis=0)
    Ap = np.linalg.pinv(A)
    dirI = _indexer_query_direction(cfg, w, q_last)
    for p in pos:
        k0 = (w["W_k"] @ Xd[p]).reshape(cfg.H_kv, cfg.d)
        kt = np.stack([_aligned(q_last[g * cfg.G:(g + 1) * cfg.G].mean(0), k0[g])
                       for g in range(cfg.H_kv)]).reshape(-1)
        kI0 = WkI @ Xd[p]
        kIt = _aligned(dirI, kI0)
        rhs = np.concatenate([kt - k0.reshape(-1), kIt - kI0])
        Xd[p] = Xd[p] + Ap @ rhs
    return Xd


def _plant_needles_direct(cfg, w, X, Qd, Kd, pos):
    q_last = Qd[cfg.W - 1]
    for p in pos:
        for g in range(cfg.H_kv):
            Kd[p, g] = _aligned(q_last[g * cfg.G:(g + 1) * cfg.G].mean(0), Kd[p, g])
    if X is not None and cfg.H_I:
        WkI = from_storage(w["W_kI"], cfg.dtype)
        Ap = np.linalg.pinv(WkI)
        dirI = _indexer_query_direction(cfg, w, q_last)
        Xd = from_storage(X, cfg.dtype)
        for p in pos:
            kI0 = WkI @ Xd[p]
            Xd[p] = Xd[p] + Ap @ (_aligned(dirI, kI0) - kI0)
        X = X.copy()
        X[pos] = to_storage(Xd[pos], cfg.dtype)
    return Kd, X


def _check_needles(cfg, w, X, Q, K, pos):
    Qd = from_storage(Q, cfg.dtype)[cfg.W - 1]
    Kd = from_storage(K, cfg.dtype)
    for p in pos:
        for g in range(cfg.H_kv):
            c = _cos(Kd[p, g], Qd[g * cfg.G:(g + 1) * cfg.G].mean(0))
            assert c > 0.9, f"needle key at {p} head {g}: cos {c}"
    if X is not None and cfg.H_I:
        WkI = from_storage(w["W_kI"], cfg.dtype)
        dirI = _indexer_query_direction(cfg, w, Qd)
        Xd = from_storage(X, cfg.dtype)
        for p in pos:
            c = _cos(WkI @ Xd[p], dirI)
            assert c > 0.9, f"needle indexer key at {p}: cos {c}"


# ----------------------------------------------------------------------------- decode

def make_decode(cfg: Config, layer: int = 0, batches=None, steps=None, weights=None) -> dict:
    """Per-step decode inputs: q [T,b,H_q,d], k_new/v_new [T,b,H_kv,d] and, for the
    streaming workload, x_new [T,b,D] (the new token's hidden state for the indexer)."""
    if batches is None:
        batches = list(range(cfg.b))
    T = cfg.T if steps is None else steps
    st = cfg.dtype
    w = make_weights(cfg, layer) if (weights is None and cfg.qkv_from_hidden) else weights
    out_ch = outlier_channels(cfg, layer)
    qs, ks, vs, xs = [], [], [], []
    for bi in batches:
        if cfg.qkv_from_hidden:
            x = from_storage(to_storage(_normal(cfg, layer, T_DEC_X, bi, (T, cfg.D)), st), st)
            q = (x @ w["W_q"].T).reshape(T, cfg.H_q, cfg.d)
            k = (x @ w["W_k"].T).reshape(T, cfg.H_kv, cfg.d)
            v = (x @ w["W_v"].T).reshape(T, cfg.H_kv, cfg.d)
            xs.append(to_storage(x, st))
        else:
            q = _normal(cfg, layer, T_DEC_Q, bi, (T, cfg.H_q, cfg.d))
            k = _normal(cfg, layer, T_DEC_K, bi, (T, cfg.H_kv, cfg.d))
            v = _normal(cfg, layer, T_DEC_V, bi, (T, cfg.H_kv, cfg.d))
            if cfg.outlier_channels:
                for g in range(cfg.H_kv):
                    k[:, g, out_ch[g]] *= cfg.outlier_scale
            if cfg.streaming:
                xs.append(to_storage(_normal(cfg, layer, T_DEC_X, bi, (T, cfg.D)), st))
        qs.append(to_storage(q, st))
        ks.append(to_storage(k, st))
        vs.append(to_storage(v, st))
    out = {"q": np.stack(qs, 1), "k_new": np.stack(ks, 1), "v_new": np.stack(vs, 1)}
    if xs:
        out["x_new"] = np.stack(xs, 1)
    return out


def make_scores(cfg_id: int, rows: int, L: int, seed: int = 0, ties: int = 0) -> np.ndarray:
    """fp32 importance scores [rows, L] for selection tests; `ties` > 0 quantises the
    values to that many levels so that equal scores occur."""
    r = rng(cfg_id, 0, T_SCORES, seed)
    s = r.standard_normal((rows, L))
    if ties:
        s = np.floor(s * ties) / ties
    return s.astype(np.float32)
