"""ctypes view of include/kvm.h.  Loads the in-tree libkvmem.so; raises if it is missing.

torch is imported first so that the library binds to the HIP runtime torch has already
loaded (one runtime per process, so torch's stream handles are valid inside libkvmem).
"""
import ctypes as C
import os

import torch  # noqa: F401  (must precede loading libkvmem)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvmem.so")

KVM_OK, KVM_ERR_NULL, KVM_ERR_SHAPE, KVM_ERR_DTYPE, KVM_ERR_ALIGN = 0, 1, 2, 3, 4
KVM_ERR_RANGE, KVM_ERR_WORKSPACE, KVM_ERR_ARCH, KVM_ERR_HIP = 5, 6, 7, 8
KVM_F32, KVM_BF16 = 0, 1
KVM_FUSE_MEM, KVM_FUSE_MOMENTS = 1, 2
KVM_READ_NONE, KVM_READ_MEMORY, KVM_READ_MOMENTS = 0, 1, 2

i32, f32, vp, sz = C.c_int32, C.c_float, C.c_void_p, C.c_size_t


class IndexDesc(C.Structure):
    _fields_ = [("b", i32), ("L", i32), ("D", i32), ("H_q", i32), ("d", i32), ("H_I", i32),
                ("d_I", i32), ("W", i32), ("dtype", i32), ("eps_rms", f32)]


class TopkDesc(C.Structure):
    _fields_ = [("rows", i32), ("L", i32), ("B", i32), ("R", i32), ("recent_inclusive", i32)]


class CompactDesc(C.Structure):
    _fields_ = [("b", i32), ("L", i32), ("H_kv", i32), ("d", i32), ("cap", i32), ("keep", i32),
                ("dtype", i32), ("per_head", i32), ("kv_head_major", i32), ("flags", i32),
                ("lam", f32), ("v_row_major", i32)]


class MemDesc(C.Structure):
    _fields_ = [("b", i32), ("H_kv", i32), ("d", i32), ("r", i32), ("cap", i32), ("dtype", i32),
                ("lam", f32)]


class DecodeDesc(C.Structure):
    _fields_ = [("b", i32), ("H_q", i32), ("H_kv", i32), ("d", i32), ("cap", i32), ("n_split", i32),
                ("dtype", i32), ("mode", i32), ("scale", f32), ("eps", f32)]


class StreamDesc(C.Structure):
    _fields_ = [("b", i32), ("D", i32), ("H_q", i32), ("H_kv", i32), ("d", i32), ("H_I", i32),
                ("d_I", i32), ("P", i32), ("cap", i32), ("R", i32), ("dtype", i32), ("lam", f32),
                ("eps_rms", f32)]


class MomentDesc(C.Structure):
    _fields_ = [("b", i32), ("L", i32), ("H_q", i32), ("H_kv", i32), ("d", i32), ("W", i32),
                ("dtype", i32), ("kv_head_major", i32), ("scale", f32)]


class MReadDesc(C.Structure):
    _fields_ = [("b", i32), ("H_q", i32), ("H_kv", i32), ("d", i32), ("dtype", i32), ("scale", f32)]


class ChunkDesc(C.Structure):
    _fields_ = [("b", i32), ("D", i32), ("H_q", i32), ("H_kv", i32), ("d", i32), ("H_I", i32), ("d_I", i32),
                ("W", i32), ("B", i32), ("R", i32), ("recent_inclusive", i32), ("P", i32), ("C", i32),
                ("start", i32), ("cap_out", i32), ("final", i32), ("dtype", i32), ("lam", f32), ("eps_rms", f32)]


class AsmDesc(C.Structure):
    _fields_ = [("N", i32), ("H_q", i32), ("H_kv", i32), ("d", i32), ("L", i32), ("K", i32), ("dtype", i32),
                ("kv_head_major", i32)]


class MStreamDesc(C.Structure):
    _fields_ = [("b", i32), ("H_q", i32), ("H_kv", i32), ("d", i32), ("P", i32), ("cap", i32), ("R", i32),
                ("dtype", i32)]


# name -> (restype, argtypes); symbols that the header declares
SIGNATURES = {
    "kvm_abi_version": (C.c_int, []),
    "kvm_status_string": (C.c_char_p, [C.c_int]),
    "kvm_last_error": (C.c_char_p, []),
    "kvm_check_device": (C.c_int, []),
    "kvm_index_workspace_size": (sz, [C.POINTER(IndexDesc)]),
    "kvm_index_score": (C.c_int, [C.POINTER(IndexDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
    "kvm_topk_keep": (i32, [C.POINTER(TopkDesc)]),
    "kvm_topk_select": (C.c_int, [C.POINTER(TopkDesc), vp, vp, vp, vp, sz, vp]),
    "kvm_topk_workspace_size": (sz, [C.POINTER(TopkDesc)]),
    "kvm_compact_workspace_size": (sz, [C.POINTER(CompactDesc)]),
    "kvm_compact_kv": (C.c_int, [C.POINTER(CompactDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                 vp, sz, vp]),
    "kvm_gather_rows": (C.c_int, [i32, i32, i32, i32, vp, vp, vp, vp]),
    "kvm_mem_update": (C.c_int, [C.POINTER(MemDesc), vp, vp, vp, vp, vp, vp]),
    "kvm_moment_update": (C.c_int, [C.POINTER(MemDesc), vp, vp, vp, vp, vp, vp, vp, vp]),
    "kvm_decode_workspace_size": (sz, [C.POINTER(DecodeDesc)]),
    "kvm_decode_attn_mem": (C.c_int, [C.POINTER(DecodeDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                      vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
    "kvm_decode_attn_mem_noalloc": (C.c_int, [C.POINTER(DecodeDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                              vp, vp, vp, vp, vp, vp, vp, vp]),
    "kvm_decode_noalloc_max_bytes": (sz, []),
    "kvm_mem_query": (C.c_int, [i32, i32, i32, vp, vp, vp, vp]),
    "kvm_chunk_keep": (i32, [C.POINTER(ChunkDesc)]),
    "kvm_chunk_workspace_size": (sz, [C.POINTER(ChunkDesc)]),
    "kvm_index_evict_chunk": (C.c_int, [C.POINTER(ChunkDesc)] + [vp] * 22 + [sz, vp]),
    "kvm_asm_workspace_size": (sz, [C.POINTER(AsmDesc)]),
    "kvm_asm_prefix_states": (C.c_int, [C.POINTER(AsmDesc), vp, vp, vp, vp, vp, i32, vp]),
    "kvm_asm_kmeans": (C.c_int, [C.POINTER(AsmDesc), vp, vp, vp, i32, vp, sz, vp]),
    "kvm_asm_cluster_states": (C.c_int, [C.POINTER(AsmDesc), vp, vp, vp, vp, vp, vp, sz, vp]),
    "kvm_asm_lookup": (C.c_int, [C.POINTER(AsmDesc), i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
    "kvm_len_add": (C.c_int, [vp, i32, i32, vp]),
    "kvm_stream_workspace_size": (sz, [C.POINTER(StreamDesc)]),
    "kvm_stream_evict": (C.c_int, [C.POINTER(StreamDesc)] + [vp] * 17 + [sz, vp]),
    "kvm_moment_workspace_size": (sz, [C.POINTER(MomentDesc)]),
    "kvm_moment_alpha": (C.c_int, [C.POINTER(MomentDesc), vp, vp, vp, vp, sz, vp]),
    "kvm_moment_score": (C.c_int, [C.POINTER(MomentDesc)] + [vp] * 9),
    "kvm_moment_readout": (C.c_int, [C.POINTER(MReadDesc)] + [vp] * 9),
    "kvm_moment_stream_workspace_size": (sz, [C.POINTER(MStreamDesc)]),
    "kvm_moment_stream_evict": (C.c_int, [C.POINTER(MStreamDesc)] + [vp] * 13 + [sz, vp]),
}


class KvmError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"libkvmem status {status}: {msg}")
        self.status = status


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m learned_kv_cache_mqa_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            if hasattr(L, name):
                f = getattr(L, name)
                f.restype = res
                f.argtypes = args
        _lib = L
    return _lib


def check(status):
    if status != KVM_OK:
        raise KvmError(status, lib().kvm_last_error().decode())
