"""Thin torch-facing binding of libkvmem: argument marshalling only.

Each function has the name of the C entry point it calls.  Tensors must be on the
current HIP device; work is enqueued on torch's current stream unless `stream` is
given.  Nothing here computes any part of the method -- every step runs in libkvmem.
"""
import ctypes as C
import math

import torch

from . import _lib as K
from ._lib import check, lib

_DT = {torch.bfloat16: K.KVM_BF16, torch.float32: K.KVM_F32}
_ws_cache = {}


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _dtype(t):
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def workspace(nbytes, device=None, stream=None, tag="default"):
    """A device workspace of at least nbytes, cached per (device, stream, tag); calls on one
    stream use it in stream order."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    s = torch.cuda.current_stream(dev) if stream is None else stream
    key = (dev.index, s.cuda_stream, tag)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=dev)
        _ws_cache[key] = buf
    return buf


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


# ------------------------------------------------------------------------------- decode

def decode_desc(q, Kc, mode, n_split=0, scale=None, eps=1e-6):
    b, H_q, d = q.shape
    _, H_kv, cap, _ = Kc.shape
    return K.DecodeDesc(b=b, H_q=H_q, H_kv=H_kv, d=d, cap=cap, n_split=n_split, dtype=_dtype(q),
                        mode=mode, scale=(1.0 / math.sqrt(d)) if scale is None else scale, eps=eps)


def kvm_decode_attn_mem(q, Kc, Vc, len_, k_new=None, v_new=None, append_slot=None, M=None, bvec=None,
                        w_g=None, moments=None, o=None, lse=None, n_split=0, scale=None, eps=1e-6,
                        stream=None, ws=None, q_mem=None):
    """Decode attention over Kc [b,H_kv,cap,d] / Vc [b,H_kv,d,cap] (appending k_new/v_new), merged split-K
    states, plus the memory read-out (M, bvec, w_g; addressed with q_mem if given, see
    kvm_mem_query) or the MomentKV mix (moments = dict(n_e, s_k, s_v, S)).
    Returns o [b,H_q,d] f32 (and lse [b,H_q] if given)."""
    _contig(q, Kc, Vc, len_, k_new, v_new, append_slot, M, bvec, w_g, q_mem)
    mode = K.KVM_READ_MEMORY if M is not None else (K.KVM_READ_MOMENTS if moments is not None else K.KVM_READ_NONE)
    desc = decode_desc(q, Kc, mode, n_split, scale, eps)
    if o is None:
        o = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    nb = lib().kvm_decode_workspace_size(C.byref(desc))
    if ws is None:
        ws = workspace(nb, q.device, stream, "decode")
    mo = moments or {}
    check(lib().kvm_decode_attn_mem(C.byref(desc), _p(q), _p(k_new), _p(v_new), _p(append_slot), _p(Kc),
                                    _p(Vc), _p(len_), _p(M), _p(bvec), _p(w_g), _p(q_mem), _p(mo.get("n_e")),
                                    _p(mo.get("s_k")), _p(mo.get("s_v")), _p(mo.get("S")), _p(o), _p(lse),
                                    _p(ws), ws.numel(), _stream(stream)))
    return o


def kvm_decode_attn_mem_noalloc(q, Kc, Vc, len_, k_new=None, v_new=None, append_slot=None, M=None, bvec=None,
                                w_g=None, moments=None, o=None, lse=None, n_split=0, scale=None, eps=1e-6,
                                stream=None, q_mem=None):
    """kvm_decode_attn_mem without a workspace: the split states live in the library's own
    per-device scratch array (kvm_decode_noalloc_max_bytes()).  The library call allocates
    nothing; pass `o` (and `lse`) to keep this wrapper from allocating either.  Calls that
    overlap in time on one GPU race on that array."""
    _contig(q, Kc, Vc, len_, k_new, v_new, append_slot, M, bvec, w_g, q_mem, o, lse)
    mode = K.KVM_READ_MEMORY if M is not None else (K.KVM_READ_MOMENTS if moments is not None else K.KVM_READ_NONE)
    desc = decode_desc(q, Kc, mode, n_split, scale, eps)
    if o is None:
        o = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    mo = moments or {}
    check(lib().kvm_decode_attn_mem_noalloc(C.byref(desc), _p(q), _p(k_new), _p(v_new), _p(append_slot), _p(Kc),
                                            _p(Vc), _p(len_), _p(M), _p(bvec), _p(w_g), _p(q_mem),
                                            _p(mo.get("n_e")), _p(mo.get("s_k")), _p(mo.get("s_v")),
                                            _p(mo.get("S")), _p(o), _p(lse), _stream(stream)))
    return o


def kvm_mem_query(q, W_m, q_mem=None, stream=None):
    """q_mem = W_m q per query row (q [..., d], W_m [d, d], same dtype): the projected query
    that the memory read-out addresses M with."""
    _contig(q, W_m, q_mem)
    d = q.shape[-1]
    if q_mem is None:
        q_mem = torch.empty_like(q)
    check(lib().kvm_mem_query(q.numel() // d, d, _dtype(q), _p(q), _p(W_m), _p(q_mem), _stream(stream)))
    return q_mem


def kvm_len_add(len_, delta=1, stream=None):
    check(lib().kvm_len_add(_p(len_), len_.numel(), int(delta), _stream(stream)))
    return len_


# ------------------------------------------------------------------------------- top-k

def kvm_topk_keep(L, B, R=0, recent_inclusive=True, rows=1):
    d = K.TopkDesc(rows=rows, L=L, B=B, R=R, recent_inclusive=int(bool(recent_inclusive)))
    return lib().kvm_topk_keep(C.byref(d))


def kvm_topk_select(I, B, R=0, recent_inclusive=True, idx=None, slot_map=None, stream=None, ws=None,
                    one_block=False):
    """I [rows, L] f32 -> (idx [rows, keep] i32 ascending, slot_map [rows, L] i32).  With the
    workspace (the default) long rows spread over many blocks; one_block=True asks for one
    block per row (no workspace).  Both give the same result."""
    _contig(I)
    if I.dim() == 1:
        I = I[None]
    rows, L = I.shape
    d = K.TopkDesc(rows=rows, L=L, B=B, R=R, recent_inclusive=int(bool(recent_inclusive)))
    keep = lib().kvm_topk_keep(C.byref(d))
    if idx is None:
        idx = torch.empty((rows, max(keep, 0)), dtype=torch.int32, device=I.device)
    if slot_map is None:
        slot_map = torch.empty((rows, L), dtype=torch.int32, device=I.device)
    if one_block:
        ws, nb = None, 0
    else:
        nb = lib().kvm_topk_workspace_size(C.byref(d))
        if ws is None:
            ws = workspace(nb, I.device, stream, "topk")
        nb = ws.numel()
    check(lib().kvm_topk_select(C.byref(d), _p(I), _p(idx), _p(slot_map), _p(ws), nb, _stream(stream)))
    return idx, slot_map


# ------------------------------------------------------------------------------- compaction

def cache_cap(n):
    """Cache capacity for n slots: the decode kernel needs a multiple of 8; a multiple of 64
    puts every V row (dim-major, cap bf16 values) on a 128-byte line boundary."""
    return (int(n) + 63) // 64 * 64


def kvm_compact_kv(Kt, Vt, slot_map, idx, keep, cap=None, Kc=None, Vc=None, M=None, bvec=None, moments=None,
                   lam=1.0, per_head=False, kv_head_major=False, copy=True, v_row_major=False, stream=None, ws=None):
    """Compact kept rows of K, V ([b,L,H_kv,d], or [b,H_kv,L,d] if kv_head_major) into
    Kc [b,H_kv,cap,d] (slot-major) and Vc [b,H_kv,d,cap] (dim-major); fold evicted rows into
    (M, bvec) or into moments dict(n_e, s_k, s_v, S).  slot_map and idx are the two outputs
    of one kvm_topk_select call (idx may be None when no cache is filled).  Returns (Kc, Vc)."""
    _contig(Kt, Vt, slot_map, idx, Kc, Vc, M, bvec)
    if kv_head_major:
        b, H_kv, L, d = Kt.shape
    else:
        b, L, H_kv, d = Kt.shape
    cap = keep if cap is None else cap
    if copy and Kc is None:
        Kc = torch.zeros((b, H_kv, cap, d), dtype=Kt.dtype, device=Kt.device)
        vshape = (b, H_kv, cap, d) if v_row_major else (b, H_kv, d, cap)
        Vc = torch.zeros(vshape, dtype=Vt.dtype, device=Vt.device)
    flags = K.KVM_FUSE_MEM if M is not None else (K.KVM_FUSE_MOMENTS if moments is not None else 0)
    desc = K.CompactDesc(b=b, L=L, H_kv=H_kv, d=d, cap=cap, keep=keep, dtype=_dtype(Kt), per_head=int(per_head),
                         kv_head_major=int(kv_head_major), flags=flags, lam=lam, v_row_major=int(v_row_major))
    nb = lib().kvm_compact_workspace_size(C.byref(desc))
    if ws is None:
        ws = workspace(nb, Kt.device, stream, "compact")
    mo = moments or {}
    check(lib().kvm_compact_kv(C.byref(desc), _p(Kt), _p(Vt), _p(slot_map), _p(idx), _p(Kc), _p(Vc), _p(M), _p(bvec),
                               _p(mo.get("n_e")), _p(mo.get("s_k")), _p(mo.get("s_v")), _p(mo.get("S")),
                               _p(ws), ws.numel(), _stream(stream)))
    return Kc, Vc


def kvm_gather_rows(src, slot_map, cap, dst=None, stream=None):
    """src [rows, L, ...] -> dst [rows, cap, ...] following slot_map [rows, L]."""
    _contig(src, slot_map)
    rows, L = slot_map.shape
    eb = src[0, 0].numel() * src.element_size()
    if dst is None:
        dst = torch.zeros((rows, cap, *src.shape[2:]), dtype=src.dtype, device=src.device)
    check(lib().kvm_gather_rows(rows, L, cap, eb, _p(src), _p(slot_map), _p(dst), _stream(stream)))
    return dst


def kvm_mem_update(K_rows, V_rows, M, bvec, lam, row_slot=None, stream=None):
    """Rank-r decayed update of M [b,H_kv,d,d], bvec [b,H_kv,d] with rows K_rows/V_rows
    [b,r,H_kv,d]; with row_slot [b] i32 the (single) row comes from the caches
    (K_rows = Kc [b,H_kv,cap,d], V_rows = Vc [b,H_kv,d,cap])."""
    _contig(K_rows, V_rows, M, bvec, row_slot)
    if row_slot is not None:
        b, H_kv, cap, d = K_rows.shape
        r = 1
    else:
        b, r, H_kv, d = K_rows.shape
        cap = 0
    desc = K.MemDesc(b=b, H_kv=H_kv, d=d, r=r, cap=cap, dtype=_dtype(K_rows), lam=lam)
    check(lib().kvm_mem_update(C.byref(desc), _p(K_rows), _p(V_rows), _p(row_slot), _p(M), _p(bvec),
                               _stream(stream)))
    return M, bvec


def kvm_moment_update(K_rows, V_rows, moments, row_slot=None, stream=None):
    """Fold evicted rows into the moment sums moments = dict(n_e [b,H_kv] i32, s_k, s_v
    [b,H_kv,d], S [b,H_kv,d,d] f32); rows as in kvm_mem_update."""
    _contig(K_rows, V_rows, row_slot, *moments.values())
    if row_slot is not None:
        b, H_kv, cap, d = K_rows.shape
        r = 1
    else:
        b, r, H_kv, d = K_rows.shape
        cap = 0
    desc = K.MemDesc(b=b, H_kv=H_kv, d=d, r=r, cap=cap, dtype=_dtype(K_rows), lam=1.0)
    check(lib().kvm_moment_update(C.byref(desc), _p(K_rows), _p(V_rows), _p(row_slot), _p(moments["n_e"]),
                                  _p(moments["s_k"]), _p(moments["s_v"]), _p(moments["S"]), _stream(stream)))
    return moments


# ------------------------------------------------------------------------------- indexer

def kvm_index_score(X, Qwin, W_kI, gamma_k, W_qI, gamma_q, W_g, I=None, khat=None, eps=1e-6, stream=None,
                    ws=None):
    """Indexer importance I [b, L] f32 from hidden states X [b,L,D] and the window's model
    queries Qwin [b,W,H_q,d]; optionally the normalised keys khat [b,L,d_I] f32."""
    _contig(X, Qwin, W_kI, gamma_k, W_qI, gamma_q, W_g, I, khat)
    b, L, D = X.shape
    _, W, H_q, d = Qwin.shape
    H_I, d_I, _ = W_qI.shape
    desc = K.IndexDesc(b=b, L=L, D=D, H_q=H_q, d=d, H_I=H_I, d_I=d_I, W=W, dtype=_dtype(X), eps_rms=eps)
    if I is None:
        I = torch.empty((b, L), dtype=torch.float32, device=X.device)
    nb = lib().kvm_index_workspace_size(C.byref(desc))
    if ws is None:
        ws = workspace(nb, X.device, stream, "index")
    check(lib().kvm_index_score(C.byref(desc), _p(X), _p(Qwin), _p(W_kI), _p(gamma_k), _p(W_qI), _p(gamma_q),
                                _p(W_g), _p(I), _p(khat), _p(ws), ws.numel(), _stream(stream)))
    return I


# ------------------------------------------------------------------------------- streaming

def kvm_stream_evict(x_new, q_new, W_kI, gamma_k, W_qI, gamma_q, W_g, khat_pool, I_pool, slot_pos, next_pos,
                     Kc, Vc, M, bvec, lam, R, evict_slot=None, eps=1e-6, stream=None, ws=None):
    """One streaming eviction step: pool scoring with the new token's indexer query,
    running-max importance, eviction of the weakest non-recent slot into (M, bvec) and the
    slot's hand-over to the new token.  Returns evict_slot [b] i32 (the slot that the next
    kvm_decode_attn_mem call, with append_slot = evict_slot, fills with the new K/V)."""
    _contig(x_new, q_new, W_kI, gamma_k, W_qI, gamma_q, W_g, khat_pool, I_pool, slot_pos, next_pos, Kc, Vc, M,
            bvec, evict_slot)
    b, D = x_new.shape
    _, H_q, d = q_new.shape
    H_I, d_I, _ = W_qI.shape
    _, P = I_pool.shape
    _, H_kv, cap, _ = Kc.shape
    desc = K.StreamDesc(b=b, D=D, H_q=H_q, H_kv=H_kv, d=d, H_I=H_I, d_I=d_I, P=P, cap=cap, R=R,
                        dtype=_dtype(x_new), lam=lam, eps_rms=eps)
    if evict_slot is None:
        evict_slot = torch.empty((b,), dtype=torch.int32, device=x_new.device)
    nb = lib().kvm_stream_workspace_size(C.byref(desc))
    if ws is None:
        ws = workspace(nb, x_new.device, stream, "stream")
    check(lib().kvm_stream_evict(C.byref(desc), _p(x_new), _p(q_new), _p(W_kI), _p(gamma_k), _p(W_qI), _p(gamma_q),
                                 _p(W_g), _p(khat_pool), _p(I_pool), _p(slot_pos), _p(next_pos), _p(Kc), _p(Vc),
                                 _p(M), _p(bvec), _p(evict_slot), _p(ws), ws.numel(), _stream(stream)))
    return evict_slot


# ------------------------------------------------------------------------------- MomentKV

def _moment_desc(K_, H_q, W, kv_head_major, scale):
    if kv_head_major:
        b, H_kv, L, d = K_.shape
    else:
        b, L, H_kv, d = K_.shape
    return K.MomentDesc(b=b, L=L, H_q=H_q, H_kv=H_kv, d=d, W=W, dtype=_dtype(K_), kv_head_major=int(kv_head_major),
                        scale=(1.0 / math.sqrt(d)) if scale is None else scale)


def kvm_moment_alpha(Qwin, K_, kv_head_major=False, alpha=None, scale=None, stream=None, ws=None):
    """alpha [b, H_kv, L] f32: the causal softmax weight of each key averaged over the window
    queries Qwin [b, W, H_q, d] (positions L-W..L-1) and the query heads of its KV group."""
    _contig(Qwin, K_, alpha)
    _, W, H_q, _ = Qwin.shape
    desc = _moment_desc(K_, H_q, W, kv_head_major, scale)
    if alpha is None:
        alpha = torch.empty((desc.b, desc.H_kv, desc.L), dtype=torch.float32, device=K_.device)
    nb = lib().kvm_moment_workspace_size(C.byref(desc))
    if ws is None:
        ws = workspace(nb, K_.device, stream, "moment")
    check(lib().kvm_moment_alpha(C.byref(desc), _p(Qwin), _p(K_), _p(alpha), _p(ws), ws.numel(), _stream(stream)))
    return alpha


def kvm_moment_score(K_, V_, alpha, moments, kv_head_major=False, score=None, stream=None):
    """score [b, H_kv, L] = alpha * ||v - v_bar - S~ k / (n_e sqrt d)|| with moments
    dict(n_e, s_k, s_v, S)."""
    _contig(K_, V_, alpha, score)
    desc = _moment_desc(K_, 1, 1, kv_head_major, None)
    if score is None:
        score = torch.empty((desc.b, desc.H_kv, desc.L), dtype=torch.float32, device=K_.device)
    check(lib().kvm_moment_score(C.byref(desc), _p(K_), _p(V_), _p(alpha), _p(moments["n_e"]), _p(moments["s_k"]),
                                 _p(moments["s_v"]), _p(moments["S"]), _p(score), _stream(stream)))
    return score


def kvm_moment_readout(q, o_R, lse_R, moments, o=None, scale=None, stream=None):
    """Normalization-corrected mix of the retained output o_R [b,H_q,d] (log-partition
    lse_R [b,H_q]) with the moments' first-order estimate of the evicted output."""
    _contig(q, o_R, lse_R, o)
    b, H_q, d = q.shape
    H_kv = moments["n_e"].shape[1]
    desc = K.MReadDesc(b=b, H_q=H_q, H_kv=H_kv, d=d, dtype=_dtype(q),
                       scale=(1.0 / math.sqrt(d)) if scale is None else scale)
    if o is None:
        o = torch.empty((b, H_q, d), dtype=torch.float32, device=q.device)
    check(lib().kvm_moment_readout(C.byref(desc), _p(q), _p(o_R), _p(lse_R), _p(moments["n_e"]), _p(moments["s_k"]),
                                   _p(moments["s_v"]), _p(moments["S"]), _p(o), _stream(stream)))
    return o


def kvm_moment_stream_evict(q, k_new, v_new, Kc, Vc, slot_pos, next_pos, moments, R, evict_slot=None,
                            stream=None, ws=None):
    """One MomentKV eviction step during decode, per (sequence, KV head): alpha of the new
    query over the pool, score alpha*||r||, eviction of the lowest non-recent slot into the
    moments dict(n_e, s_k, s_v, S), and the new token's K/V written into the freed slot.
    Returns evict_slot [b, H_kv] i32.  Follow with kvm_decode_attn_mem(q, Kc, Vc, len=P,
    moments=moments) for the step's output."""
    _contig(q, k_new, v_new, Kc, Vc, slot_pos, next_pos, evict_slot, *moments.values())
    b, H_q, d = q.shape
    _, H_kv, cap, _ = Kc.shape
    P = slot_pos.shape[-1]
    desc = K.MStreamDesc(b=b, H_q=H_q, H_kv=H_kv, d=d, P=P, cap=cap, R=R, dtype=_dtype(q))
    if evict_slot is None:
        evict_slot = torch.empty((b, H_kv), dtype=torch.int32, device=q.device)
    nb = lib().kvm_moment_stream_workspace_size(C.byref(desc))
    if ws is None:
        ws = workspace(nb, q.device, stream, "mstream")
    check(lib().kvm_moment_stream_evict(C.byref(desc), _p(q), _p(k_new), _p(v_new), _p(Kc), _p(Vc), _p(slot_pos),
                                        _p(next_pos), _p(moments["n_e"]), _p(moments["s_k"]), _p(moments["s_v"]),
                                        _p(moments["S"]), _p(evict_slot), _p(ws), ws.numel(), _stream(stream)))
    return evict_slot


# ------------------------------------------------------------------------------- ASM

def asm_desc(Q, K_, K_centroids, kv_head_major=False):
    N, H_q, d = Q.shape
    if kv_head_major:
        H_kv, L, _ = K_.shape
    else:
        L, H_kv, _ = K_.shape
    return K.AsmDesc(N=N, H_q=H_q, H_kv=H_kv, d=d, L=L, K=K_centroids, dtype=_dtype(Q),
                     kv_head_major=int(kv_head_major))


def kvm_asm_prefix_states(Q, K_, V, kv_head_major=False, a=None, lse=None, accumulate=False, stream=None):
    """Attention states (a [N, H_q, d] f32, lse [N, H_q] f32) of calibration queries
    Q [N, H_q, d] over the prefix K, V ([L, H_kv, d], or [H_kv, L, d] if kv_head_major).
    accumulate=True merges this chunk of the prefix into the states already in a, lse."""
    _contig(Q, K_, V, a, lse)
    if accumulate and (a is None or lse is None):
        raise ValueError("accumulate needs the states of the earlier chunks in a and lse")
    desc = asm_desc(Q, K_, 1, kv_head_major)
    if a is None:
        a = torch.empty(Q.shape, dtype=torch.float32, device=Q.device)
    if lse is None:
        lse = torch.empty(Q.shape[:2], dtype=torch.float32, device=Q.device)
    check(lib().kvm_asm_prefix_states(C.byref(desc), _p(Q), _p(K_), _p(V), _p(a), _p(lse), int(bool(accumulate)),
                                      _stream(stream)))
    return a, lse


def _asm_ws(desc, device, stream, ws):
    nb = lib().kvm_asm_workspace_size(C.byref(desc))
    return workspace(nb, device, stream, "asm") if ws is None else ws


def kvm_asm_kmeans(Q, C_, iters, idx=None, stream=None, ws=None):
    """Lloyd's K-means per head on Q [N, H_q, d] from centroids C_ [H_q, K, d] f32
    (updated in place).  Returns idx [H_q, N] i32, the final assignment."""
    _contig(Q, C_, idx)
    N, H_q, d = Q.shape
    desc = K.AsmDesc(N=N, H_q=H_q, H_kv=1, d=d, L=1, K=C_.shape[1], dtype=_dtype(Q), kv_head_major=0)
    if idx is None:
        idx = torch.empty((H_q, N), dtype=torch.int32, device=Q.device)
    ws = _asm_ws(desc, Q.device, stream, ws)
    check(lib().kvm_asm_kmeans(C.byref(desc), _p(Q), _p(C_), _p(idx), int(iters), _p(ws), ws.numel(),
                               _stream(stream)))
    return idx


def kvm_asm_cluster_states(a, lse, idx, n_centroids, a_bar=None, lse_bar=None, stream=None, ws=None):
    """Per-cluster attention states from the members' (a [N, H_q, d], lse [N, H_q]) and the
    assignment idx [H_q, N]: a_bar [H_q, K, d], lse_bar [H_q, K] (f32)."""
    _contig(a, lse, idx, a_bar, lse_bar)
    N, H_q, d = a.shape
    desc = K.AsmDesc(N=N, H_q=H_q, H_kv=1, d=d, L=1, K=n_centroids, dtype=K.KVM_BF16, kv_head_major=0)
    if a_bar is None:
        a_bar = torch.empty((H_q, n_centroids, d), dtype=torch.float32, device=a.device)
    if lse_bar is None:
        lse_bar = torch.empty((H_q, n_centroids), dtype=torch.float32, device=a.device)
    ws = _asm_ws(desc, a.device, stream, ws)
    check(lib().kvm_asm_cluster_states(C.byref(desc), _p(a), _p(lse), _p(idx), _p(a_bar), _p(lse_bar), _p(ws),
                                       ws.numel(), _stream(stream)))
    return a_bar, lse_bar


def kvm_asm_lookup(q, C_, a_bar, lse_bar, o_loc, lse_loc, o=None, lse_out=None, idx_out=None, stream=None):
    """Retrieval by cosine similarity and the merge with the local state: returns
    (o [b, H_q, d] f32, idx_out [b, H_q] i32); lse_out [b, H_q] is filled if given."""
    _contig(q, C_, a_bar, lse_bar, o_loc, lse_loc, o, lse_out, idx_out)
    b, H_q, d = q.shape
    desc = K.AsmDesc(N=1, H_q=H_q, H_kv=1, d=d, L=1, K=C_.shape[1], dtype=_dtype(q), kv_head_major=0)
    if o is None:
        o = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if idx_out is None:
        idx_out = torch.empty((b, H_q), dtype=torch.int32, device=q.device)
    check(lib().kvm_asm_lookup(C.byref(desc), b, _p(q), _p(C_), _p(a_bar), _p(lse_bar), _p(o_loc), _p(lse_loc),
                               _p(o), _p(lse_out), _p(idx_out), _stream(stream)))
    return o, idx_out


# ------------------------------------------------------------------------------- chunked prefill

def kvm_index_evict_chunk(X, Qwin, K_, V, W_kI, gamma_k, W_qI, gamma_q, W_g, pool, P, start, B, R, lam, cap_out,
                          final, M, bvec, recent_inclusive=True, eps=1e-6, stream=None, ws=None):
    """One chunk of a chunked pre-eviction (X [b, C, D], Qwin [b, W, H_q, d], K, V [b, C, H_kv, d],
    or K = V = None when rows P .. P+C-1 of pool K, V already hold the chunk).
    pool = dict(K, V [b, H_kv, P + C, d], khat [b, P + C, d_I], I [b, P + C], pos [b, P + C]) with
    rows 0 .. P-1 holding the pool.  Returns (next pool dict with row capacity cap_out, keep);
    with final=True its V is dim-major [b, H_kv, d, cap_out] (the decode caches)."""
    _contig(X, Qwin, K_, V, W_kI, gamma_k, W_qI, gamma_q, W_g, M, bvec, *pool.values())
    b, C_, D = X.shape
    _, W, H_q, d = Qwin.shape
    H_kv = pool["K"].shape[1]
    H_I, d_I, _ = W_qI.shape
    # the library addresses every pool array with a row stride of exactly P + C
    rows = P + C_
    want = dict(K=(b, H_kv, rows, d), V=(b, H_kv, rows, d), khat=(b, rows, d_I), I=(b, rows), pos=(b, rows))
    for k, shape in want.items():
        if tuple(pool[k].shape) != shape:
            raise ValueError(f"pool[{k!r}] has shape {tuple(pool[k].shape)}, expected {shape} (P + C = {rows} rows)")
    if pool["khat"].dtype != torch.float32 or pool["I"].dtype != torch.float32 or pool["pos"].dtype != torch.int32:
        raise ValueError("pool khat and I must be float32, pos int32")
    if pool["K"].dtype != X.dtype or pool["V"].dtype != X.dtype:
        raise ValueError(f"pool K/V dtype {pool['K'].dtype} differs from X's {X.dtype}")
    if (K_ is None) != (V is None):
        raise ValueError("K and V must both be given or both be None (in-place mode)")
    if K_ is not None:
        if tuple(K_.shape) != (b, C_, H_kv, d) or tuple(V.shape) != (b, C_, H_kv, d):
            raise ValueError(f"chunk K/V must be {(b, C_, H_kv, d)}")
        if K_.dtype != X.dtype or V.dtype != X.dtype:
            raise ValueError("chunk K/V dtype differs from X's")
    desc = K.ChunkDesc(b=b, D=D, H_q=H_q, H_kv=H_kv, d=d, H_I=H_I, d_I=d_I, W=W, B=B, R=R,
                       recent_inclusive=int(bool(recent_inclusive)), P=P, C=C_, start=start, cap_out=cap_out,
                       final=int(bool(final)), dtype=_dtype(X), lam=lam, eps_rms=eps)
    keep = lib().kvm_chunk_keep(C.byref(desc))
    dev = X.device
    kdt = pool["K"].dtype
    nxt = dict(K=torch.empty((b, H_kv, cap_out, d), dtype=kdt, device=dev),
               V=torch.empty((b, H_kv, d, cap_out) if final else (b, H_kv, cap_out, d), dtype=kdt, device=dev),
               khat=torch.empty((b, cap_out, d_I), dtype=torch.float32, device=dev),
               I=torch.empty((b, cap_out), dtype=torch.float32, device=dev),
               pos=torch.empty((b, cap_out), dtype=torch.int32, device=dev))
    nb = lib().kvm_chunk_workspace_size(C.byref(desc))
    if ws is None:
        ws = workspace(nb, dev, stream, "chunk")
    check(lib().kvm_index_evict_chunk(C.byref(desc), _p(X), _p(Qwin), _p(K_), _p(V), _p(W_kI), _p(gamma_k),
                                      _p(W_qI), _p(gamma_q), _p(W_g), _p(pool["K"]), _p(pool["V"]), _p(pool["khat"]),
                                      _p(pool["I"]), _p(pool["pos"]), _p(nxt["K"]), _p(nxt["V"]), _p(nxt["khat"]),
                                      _p(nxt["I"]), _p(nxt["pos"]), _p(M), _p(bvec), _p(ws), ws.numel(),
                                      _stream(stream)))
    return nxt, keep


def index_evict_chunked(X, Q, K_, V, W_kI, gamma_k, W_qI, gamma_q, W_g, B, R, lam, C_, W, M, bvec, cap,
                        recent_inclusive=True, eps=1e-6, stream=None):
    """The prefill X [b, L, D], Q [b, L, H_q, d] (only each chunk's last W rows are read),
    K, V [b, L, H_kv, d] taken in chunks of C_ tokens through kvm_index_evict_chunk.  The
    pool buffers of every step hold exactly pool + chunk rows.  Returns the final pool
    (K [b, H_kv, cap, d], V dim-major [b, H_kv, d, cap], khat, I, pos) and its size."""
    b, L, D = X.shape
    H_kv, d, d_I = K_.shape[2], K_.shape[3], W_qI.shape[1]
    starts = list(range(0, L, C_))
    dev = X.device
    P, pool = 0, None
    for i, s0 in enumerate(starts):
        e = min(L, s0 + C_)
        n = e - s0
        if pool is None:
            pool = dict(K=torch.empty((b, H_kv, n, d), dtype=K_.dtype, device=dev),
                        V=torch.empty((b, H_kv, n, d), dtype=V.dtype, device=dev),
                        khat=torch.empty((b, n, d_I), dtype=torch.float32, device=dev),
                        I=torch.empty((b, n), dtype=torch.float32, device=dev),
                        pos=torch.empty((b, n), dtype=torch.int32, device=dev))
        last = i == len(starts) - 1
        if last:
            cap_out = cap
        else:
            keep_next = lib().kvm_chunk_keep(C.byref(K.ChunkDesc(b=b, P=P, C=n, B=B, R=R,
                                                                 recent_inclusive=int(bool(recent_inclusive)))))
            cap_out = keep_next + (min(L, starts[i + 1] + C_) - starts[i + 1])
        pool, P = kvm_index_evict_chunk(X[:, s0:e].contiguous(), Q[:, e - W:e].contiguous(), K_[:, s0:e].contiguous(),
                                        V[:, s0:e].contiguous(), W_kI, gamma_k, W_qI, gamma_q, W_g, pool, P, s0, B, R,
                                        lam, cap_out, last, M, bvec, recent_inclusive, eps, stream)
    return pool, P
