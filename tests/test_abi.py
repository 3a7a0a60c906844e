"""The C ABI on the CPU: the library loads, exports every entry point include/kvm.h
declares, and rejects bad arguments before any HIP call (so no GPU is needed)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "kvm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvm_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    from learned_kv_cache_mqa_amd import _lib
    return _lib.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 10
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    from learned_kv_cache_mqa_amd import _lib
    assert set(names) <= set(_lib.SIGNATURES), set(names) - set(_lib.SIGNATURES)


def test_version_and_strings(L):
    assert L.kvm_abi_version() == 3
    assert L.kvm_status_string(6) == b"workspace too small"


FAKE = 0x7f0000000000      # never dereferenced: validation fails before any HIP call


def _decode(L, **kw):
    from learned_kv_cache_mqa_amd import _lib as K
    d = K.DecodeDesc(b=1, H_q=32, H_kv=8, d=128, cap=64, n_split=0, dtype=K.KVM_BF16,
                     mode=K.KVM_READ_MEMORY, scale=0.088, eps=1e-6)
    for k, v in kw.pop("desc", {}).items():
        setattr(d, k, v)
    p = dict(q=FAKE, kn=FAKE, vn=FAKE, app=None, Kc=FAKE, Vc=FAKE, len=FAKE, M=FAKE, b=FAKE, wg=FAKE, qm=None,
             ne=None, sk=None, sv=None, S=None, o=FAKE, lse=None, ws=FAKE, wsb=1 << 30)
    p.update(kw)
    return L.kvm_decode_attn_mem(C.byref(d), *[None if p[k] is None else C.c_void_p(p[k]) if k != "wsb" else p[k]
                                               for k in ["q", "kn", "vn", "app", "Kc", "Vc", "len", "M", "b", "wg",
                                                         "qm", "ne", "sk", "sv", "S", "o", "lse", "ws", "wsb"]], None)


def test_decode_validation(L):
    assert _decode(L, desc=dict(d=96)) == 2
    assert _decode(L, desc=dict(H_q=24)) == 2           # G = 3
    assert _decode(L, desc=dict(dtype=7)) == 3
    assert _decode(L, q=None) == 1
    assert _decode(L, M=None) == 1                       # memory mode needs M
    assert _decode(L, kn=None) == 1                      # k_new without v_new
    assert _decode(L, Kc=FAKE + 4) == 4
    assert _decode(L, wsb=16) == 6
    assert b"workspace" in L.kvm_last_error()
    assert _decode(L, desc=dict(mode=2)) == 1            # moments mode needs the moments
    assert _decode(L, qm=FAKE + 8) == 4                  # projected query misaligned
    assert _decode(L, desc=dict(mode=0), M=None, qm=FAKE) == 5   # q_mem only with the memory read-out


def test_mem_query_validation(L):
    from learned_kv_cache_mqa_amd import _lib as K
    f = lambda rows=4, d=128, dt=K.KVM_BF16, q=FAKE, w=FAKE, o=FAKE + 4096: L.kvm_mem_query(
        rows, d, dt, None if q is None else C.c_void_p(q), C.c_void_p(w), C.c_void_p(o), None)
    assert f(rows=0) == 2
    assert f(d=96) == 2
    assert f(dt=9) == 3
    assert f(q=None) == 1
    assert f(o=FAKE) == 5                                # q_mem aliases q


def _mstream(L, **kw):
    from learned_kv_cache_mqa_amd import _lib as K
    d = K.MStreamDesc(b=2, H_q=32, H_kv=8, d=128, P=1024, cap=1024, R=16, dtype=K.KVM_BF16)
    for k, v in kw.pop("desc", {}).items():
        setattr(d, k, v)
    names = ["q", "kn", "vn", "Kc", "Vc", "pos", "next", "ne", "sk", "sv", "S", "ev", "ws"]
    p = {n: FAKE for n in names}
    p["wsb"] = 1 << 30
    p.update(kw)
    args = [None if p[n] is None else C.c_void_p(p[n]) for n in names] + [p["wsb"], None]
    return L.kvm_moment_stream_evict(C.byref(d), *args)


def test_moment_stream_validation(L):
    from learned_kv_cache_mqa_amd import _lib as K
    assert _mstream(L, desc=dict(d=96)) == 2
    assert _mstream(L, desc=dict(H_q=36)) == 2          # not a multiple of H_kv
    assert _mstream(L, desc=dict(H_q=8 * 16)) == 2      # group of 16
    assert _mstream(L, desc=dict(H_q=8 * 3)) == 2       # group of 3
    assert _mstream(L, desc=dict(dtype=K.KVM_F32)) == 3
    assert _mstream(L, desc=dict(R=1024)) == 5          # no candidate could exist
    assert _mstream(L, desc=dict(cap=512)) == 5
    assert _mstream(L, S=None) == 1
    assert _mstream(L, Vc=FAKE + 2) == 4
    assert _mstream(L, wsb=64) == 6
    d = K.MStreamDesc(b=2, H_q=32, H_kv=8, d=128, P=1024, cap=1024, R=16, dtype=K.KVM_BF16)
    # logits [pairs, G, P] and norms [pairs, P], f32, each 256-byte aligned
    assert L.kvm_moment_stream_workspace_size(C.byref(d)) == 16 * 4 * 1024 * 4 + 16 * 1024 * 4


def test_asm_validation(L):
    from learned_kv_cache_mqa_amd import _lib as K

    def desc(**kw):
        d = K.AsmDesc(N=4096, H_q=32, H_kv=8, d=128, L=16384, K=256, dtype=K.KVM_BF16, kv_head_major=0)
        for k, v in kw.items():
            setattr(d, k, v)
        return d
    P = lambda *xs: [C.c_void_p(FAKE + 1024 * i) for i in range(len(xs))]
    f = lambda d, **kw: L.kvm_asm_prefix_states(C.byref(d), *P(1, 2, 3, 4, 5), 0, None)
    assert f(desc(d=96)) == 2
    assert f(desc(H_q=36)) == 2
    assert f(desc(dtype=K.KVM_F32)) == 3
    assert f(desc(K=257)) == 5
    assert f(desc(L=0)) == 2
    assert L.kvm_asm_kmeans(C.byref(desc()), *P(1, 2, 3), -1, C.c_void_p(FAKE), 1 << 30, None) == 5
    assert L.kvm_asm_kmeans(C.byref(desc()), *P(1, 2, 3), 3, C.c_void_p(FAKE), 16, None) == 6
    assert L.kvm_asm_lookup(C.byref(desc()), 0, *P(1, 2, 3, 4, 5, 6, 7, 8, 9), None) == 2
    # split centroid planes [H, 3, K, d] bf16, norms [H, K] f32, partial rows
    # [H, chunks of 512 queries, K, d + 4] f32, each 256-byte aligned
    assert L.kvm_asm_workspace_size(C.byref(desc())) == 32 * 3 * 256 * 128 * 2 + 32 * 256 * 4 + 32 * 8 * 256 * 132 * 4


def _chunk(L, **kw):
    from learned_kv_cache_mqa_amd import _lib as K
    d = K.ChunkDesc(b=1, D=4096, H_q=32, H_kv=8, d=128, H_I=4, d_I=64, W=64, B=2048, R=64, recent_inclusive=1,
                    P=2048, C=4096, start=4096, cap_out=2048, final=1, dtype=K.KVM_BF16, lam=0.99, eps_rms=1e-6)
    for k, v in kw.pop("desc", {}).items():
        setattr(d, k, v)
    names = ["X", "Qw", "K", "V", "WkI", "gk", "WqI", "gq", "Wg", "Kp", "Vp", "khp", "Ip", "posp", "Kn", "Vn",
             "khn", "In", "posn", "M", "b", "ws"]
    p = {n: FAKE + 4096 * i for i, n in enumerate(names)}
    p["wsb"] = 1 << 34
    p.update(kw)
    args = [None if p[n] is None else C.c_void_p(p[n]) for n in names] + [p["wsb"], None]
    return L.kvm_index_evict_chunk(C.byref(d), *args), d


def test_chunk_validation(L):
    from learned_kv_cache_mqa_amd import _lib as K
    f = lambda **kw: _chunk(L, **kw)[0]
    assert f(desc=dict(d=96)) == 2
    assert f(desc=dict(d_I=48)) == 2
    assert f(desc=dict(H_q=36)) == 2                    # not a multiple of H_kv
    assert f(desc=dict(P=-1)) == 2
    assert f(desc=dict(dtype=5)) == 3
    assert f(desc=dict(W=4097)) == 5                    # window longer than the chunk
    assert f(desc=dict(R=4097)) == 5
    assert f(desc=dict(B=32)) == 5                      # budget below the recent window
    assert f(desc=dict(cap_out=2047)) == 5              # output pool below the kept count
    assert f(desc=dict(lam=1.5)) == 5
    assert f(X=None) == 1
    assert f(K=None) == 1                                # K and V: both given, or both NULL (in place)
    assert f(K=None, V=None) not in (1, 4)               # in place: accepted by the checks
    assert f(khn=None, In=None, posn=None) != 1          # the new pool's side data is optional
    assert f(Vp=FAKE + 8) == 4
    assert f(wsb=256) == 6
    assert b"workspace" in L.kvm_last_error()
    _, d = _chunk(L)
    # the pool keeps min(P + C, B) tokens; a chunk shorter than the budget keeps all
    assert L.kvm_chunk_keep(C.byref(d)) == 2048
    d.P, d.C = 0, 1000
    assert L.kvm_chunk_keep(C.byref(d)) == 1000
    d.B, d.R = 32, 64
    assert L.kvm_chunk_keep(C.byref(d)) == -1
    assert L.kvm_chunk_workspace_size(C.byref(d)) == 0


def test_moment_update_validation(L):
    from learned_kv_cache_mqa_amd import _lib as K
    P = lambda *xs: [C.c_void_p(FAKE + 4096 * i) for i in range(len(xs))]

    def f(row_slot=None, **kw):
        d = K.MemDesc(b=2, H_kv=8, d=128, r=4, cap=0, dtype=K.KVM_BF16, lam=1.0)
        for k, v in kw.items():
            setattr(d, k, v)
        return L.kvm_moment_update(C.byref(d), *P(1, 2), row_slot, *P(3, 4, 5, 6), None)
    assert f(d=96) == 2
    assert f(b=0) == 2
    assert f(dtype=9) == 3
    assert f(row_slot=C.c_void_p(FAKE)) == 5          # a cache slot needs r == 1 and cap > 0
    assert f(row_slot=C.c_void_p(FAKE + 4), r=1, cap=8) == 4
    d = K.MemDesc(b=2, H_kv=8, d=128, r=4, cap=0, dtype=K.KVM_BF16, lam=1.0)
    assert L.kvm_moment_update(C.byref(d), *P(1, 2), None, None, *P(4, 5, 6), None) == 1


def test_header_is_c99_and_links(tmp_path):
    """include/kvm.h compiles as strict C99, and a C program linked against libkvmem.so calls
    the library directly: version, status strings, and argument validation that fails before
    any HIP call (so no GPU is needed)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    libdir = os.path.join(ROOT, "learned_kv_cache_mqa_amd")
    src = tmp_path / "abi.c"
    src.write_text(r'''
#include <stdio.h>
#include "kvm.h"
int main(void) {
  kvm_topk_desc d = {1, 64, 80, 0, 1};      /* budget above L: keep everything */
  kvm_topk_desc bad = {1, 64, 8, 16, 1};    /* budget below the recent window */
  int st;
  printf("abi %d\n", (int)kvm_abi_version());
  printf("keep %d bad %d\n", (int)kvm_topk_keep(&d), (int)kvm_topk_keep(&bad));
  st = (int)kvm_topk_select(NULL, NULL, NULL, NULL, NULL, 0, NULL);
  printf("null %d %s\n", st, kvm_status_string(st));
  return 0;
}
''')
    exe = tmp_path / "abi"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           str(src), "-L", libdir, "-lkvmem", f"-Wl,-rpath,{libdir}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    lines = r.stdout.split("\n")
    assert lines[0] == "abi 3"
    assert lines[1] == "keep 64 bad -1"
    assert lines[2].startswith("null 1 ")


def test_chunk_wrapper_rejects_mismatched_pool():
    """The chunked pre-eviction addresses every pool array with a row stride of P + C, so the
    binding refuses pools of any other row count or dtype before calling the library."""
    import torch
    from learned_kv_cache_mqa_amd import api
    b, C_, D, W, H_q, H_kv, d, H_I, d_I, P = 1, 64, 32, 16, 4, 2, 8, 4, 8, 40
    X = torch.zeros((b, C_, D), dtype=torch.bfloat16)
    Q = torch.zeros((b, W, H_q, d), dtype=torch.bfloat16)
    Kt = torch.zeros((b, C_, H_kv, d), dtype=torch.bfloat16)
    w = [torch.zeros((d_I, D), dtype=torch.bfloat16), torch.ones(d_I), torch.zeros((H_I, d_I, d), dtype=torch.bfloat16),
         torch.ones(d_I), torch.zeros((H_I, D), dtype=torch.bfloat16)]
    M, bv = torch.zeros((b, H_kv, d, d)), torch.zeros((b, H_kv, d))

    def pool(rows, kdt=torch.bfloat16):
        return dict(K=torch.zeros((b, H_kv, rows, d), dtype=kdt), V=torch.zeros((b, H_kv, rows, d), dtype=kdt),
                    khat=torch.zeros((b, rows, d_I)), I=torch.zeros((b, rows)),
                    pos=torch.zeros((b, rows), dtype=torch.int32))

    call = lambda pl, K_=Kt, V_=Kt: api.kvm_index_evict_chunk(X, Q, K_, V_, *w, pl, P, 0, 32, 4, 0.99, 64, False,
                                                              M, bv)
    for bad in (pool(P + C_ + 64), pool(P + C_ - 1), pool(P + C_, torch.float32)):
        with pytest.raises(ValueError):
            call(bad)
    with pytest.raises(ValueError):
        call(pool(P + C_), K_=None)                    # only one of K, V
    with pytest.raises(ValueError):
        call(pool(P + C_), K_=Kt[:, :10].contiguous(), V_=Kt[:, :10].contiguous())


def test_decode_noalloc_rejects_shapes_beyond_its_scratch(L):
    """The no-allocation decode holds its split states in a fixed array; a shape that needs
    more is refused before any HIP call, with a message naming the limit."""
    from learned_kv_cache_mqa_amd import _lib as K
    cap = int(L.kvm_decode_noalloc_max_bytes())
    assert cap == 4 << 20

    def call(**dk):
        d = K.DecodeDesc(b=1, H_q=32, H_kv=8, d=128, cap=2176, n_split=0, dtype=K.KVM_BF16,
                         mode=K.KVM_READ_MEMORY, scale=0.088, eps=1e-6)
        for k, v in dk.items():
            setattr(d, k, v)
        ptr = [C.c_void_p(FAKE)] * 3 + [None] + [C.c_void_p(FAKE)] * 7 + [None] * 4 + [C.c_void_p(FAKE), None]
        return L.kvm_decode_attn_mem_noalloc(C.byref(d), *ptr, None), L.kvm_decode_workspace_size(C.byref(d))

    st, need = call(b=4, H_q=64, n_split=64)
    assert need > cap and st == 6
    assert b"scratch" in L.kvm_last_error()
    st, need = call(d=96)
    assert st == 2
