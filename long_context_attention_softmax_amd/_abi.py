"""ctypes mirror of include/hca.h and the loader of the in-tree HIP library.

Importing this module loads ``lib/libhca.so``; if it has not been built the import
fails with an error naming the build step.  Nothing here computes any part of the
path: it only describes memory to the library.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_double, c_float, c_int, c_int32, c_int64, c_size_t, c_uint32, c_void_p

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libhca.so")

HCA_OK = 0
ERRORS = {-1: "HCA_E_NULL", -2: "HCA_E_SHAPE", -3: "HCA_E_ALIGN", -4: "HCA_E_DTYPE",
          -5: "HCA_E_UNSUPPORTED", -6: "HCA_E_WORKSPACE", -7: "HCA_E_LAUNCH", -8: "HCA_E_VERSION"}
F32, BF16, FP8_E4M3, MXFP4 = 0, 1, 2, 3
MODE_CSA, MODE_HCA, MODE_SWA = 0, 1, 2
OP_KV_COMPRESS, OP_INDEXER_TOPK, OP_ATTN_DECODE, OP_ATTN_PREFILL, OP_QKV_PROLOGUE, OP_OUT_PROJ = 0, 1, 2, 3, 4, 5
OP_DECODE_LAYER = 6
STRUCT_KV_PLANES, STRUCT_IDX_PLANES, STRUCT_PROFILE_EVENTS = 100, 101, 102

EXPORTS = ["hca_abi_version", "hca_last_error", "hca_struct_size", "hca_workspace_bytes", "hca_indexer_query_group",
           "hca_kv_compress", "hca_indexer_topk", "hca_attn_decode", "hca_attn_prefill", "hca_attn_decode_noalloc",
           "hca_qkv_prologue",
           "hca_out_proj", "hca_decode_layer", "hca_profiled"]


class KvPlanes(ctypes.Structure):
    _fields_ = [("fmt", c_int32), ("reserved", c_int32),
                ("f32", c_void_p), ("f32_pitch", c_int64),
                ("nope", c_void_p), ("nope_pitch", c_int64),
                ("rope", c_void_p), ("rope_pitch", c_int64),
                ("scale", c_void_p)]


class IdxPlanes(ctypes.Structure):
    _fields_ = [("fmt", c_int32), ("reserved", c_int32),
                ("data", c_void_p), ("pitch", c_int64),
                ("scales", c_void_p), ("scale_pitch", c_int64)]


class KvCompressDesc(ctypes.Structure):
    _fields_ = [("struct_size", c_uint32), ("m", c_int32), ("D", c_int32), ("D_r", c_int32),
                ("d_I", c_int32), ("n_blocks", c_int32), ("rope_base", c_double),
                ("raw_fmt", c_int32), ("reserved", c_int32),
                ("raw", c_void_p), ("raw_pitch", c_int64),
                ("raw_idx", c_void_p), ("raw_idx_pitch", c_int64),
                ("block_row", c_void_p), ("block_pos", c_void_p), ("out_row", c_void_p),
                ("gate_w", c_void_p), ("gate_b", c_void_p),
                ("out", KvPlanes), ("out_idx", IdxPlanes), ("debug", c_void_p)]


class IndexerTopkDesc(ctypes.Structure):
    _fields_ = [("struct_size", c_uint32), ("Nq", c_int32), ("B", c_int32), ("H_I", c_int32),
                ("d_I", c_int32), ("k", c_int32), ("m", c_int32), ("reserved", c_int32),
                ("max_visible", c_int64), ("q", IdxPlanes), ("w", c_void_p), ("keys", IdxPlanes),
                ("cache_row_start", c_void_p), ("seq_id", c_void_p), ("q_pos", c_void_p),
                ("idx", c_void_p), ("score", c_void_p),
                ("workspace", c_void_p), ("workspace_bytes", c_size_t),
                ("page_table", c_void_p), ("page_table_pitch", c_int64), ("page_rows", c_int32),
                ("reserved_page", c_int32)]


class AttnDesc(ctypes.Structure):
    _fields_ = [("struct_size", c_uint32), ("Nq", c_int32), ("B", c_int32), ("H", c_int32),
                ("D", c_int32), ("D_r", c_int32), ("mode", c_int32), ("m", c_int32), ("k", c_int32),
                ("n_win", c_int32), ("win_cap", c_int32), ("tau", c_float), ("io_fmt", c_int32),
                ("rope_base", c_double), ("max_visible", c_int64),
                ("q", c_void_p), ("cache", KvPlanes), ("cache_row_start", c_void_p),
                ("idx", c_void_p), ("win", c_void_p), ("win_pitch", c_int64), ("sink", c_void_p),
                ("seq_id", c_void_p), ("q_pos", c_void_p), ("o", c_void_p), ("lse", c_void_p),
                ("workspace", c_void_p), ("workspace_bytes", c_size_t),
                ("page_table", c_void_p), ("page_table_pitch", c_int64), ("page_rows", c_int32),
                ("split_chunks", c_int32)]


class DecodeLayerDesc(ctypes.Structure):
    _fields_ = [("struct_size", c_uint32), ("reserved", c_int32),
                ("pool", ctypes.POINTER(KvCompressDesc)), ("indexer", ctypes.POINTER(IndexerTopkDesc)),
                ("attn", ctypes.POINTER(AttnDesc))]


class QkvPrologueDesc(ctypes.Structure):
    _fields_ = [("struct_size", c_uint32), ("io_fmt", c_int32), ("Nq", c_int32), ("H", c_int32),
                ("D", c_int32), ("Nt", c_int32), ("B", c_int32), ("W_cap", c_int32), ("d_I", c_int32),
                ("eps", c_double), ("q_in", c_void_p), ("q_out", c_void_p), ("gamma_q", c_void_p),
                ("kv_in", c_void_p), ("kv_pitch", c_int64), ("gamma_kv", c_void_p),
                ("tok_seq", c_void_p), ("tok_pos", c_void_p), ("win", c_void_p), ("win_pitch", c_int64),
                ("idx_in", c_void_p), ("idx_pitch", c_int64), ("win_idx", c_void_p),
                ("win_idx_pitch", c_int64)]


class OutProjDesc(ctypes.Structure):
    _fields_ = [("struct_size", c_uint32), ("out_fmt", c_int32), ("Nq", c_int32), ("H", c_int32),
                ("D", c_int32), ("G", c_int32), ("d_g", c_int32), ("o", c_void_p), ("o_pitch", c_int64),
                ("w", c_void_p), ("w_pitch", c_int64), ("y", c_void_p), ("y_pitch", c_int64)]


class ProfileEvents(ctypes.Structure):
    _fields_ = [("struct_size", c_uint32), ("reserved", c_int32), ("begin", c_void_p), ("end", c_void_p)]


class HcaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


def _load():
    # PyTorch bundles its own HIP runtime under the same soname as /opt/rocm's; the
    # library must bind to the one PyTorch uses (its streams and device memory come
    # from there), so PyTorch is loaded first.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"HIP library {LIB_PATH} is not built; run "
                          "`python -c 'import __graft_entry__ as g; g.build()'` first")
    lib = ctypes.CDLL(LIB_PATH)
    lib.hca_abi_version.restype = c_int
    lib.hca_last_error.restype = ctypes.c_char_p
    lib.hca_struct_size.restype = c_size_t
    lib.hca_struct_size.argtypes = [c_int]
    lib.hca_workspace_bytes.restype = c_int
    lib.hca_workspace_bytes.argtypes = [c_int, c_void_p, ctypes.POINTER(c_size_t)]
    lib.hca_indexer_query_group.restype = c_int
    lib.hca_indexer_query_group.argtypes = [c_void_p, ctypes.POINTER(c_int32)]
    for name, dt in [("hca_kv_compress", KvCompressDesc), ("hca_indexer_topk", IndexerTopkDesc),
                     ("hca_attn_decode", AttnDesc), ("hca_attn_prefill", AttnDesc),
                     ("hca_attn_decode_noalloc", AttnDesc),
                     ("hca_qkv_prologue", QkvPrologueDesc), ("hca_out_proj", OutProjDesc),
                     ("hca_decode_layer", DecodeLayerDesc)]:
        f = getattr(lib, name)
        f.restype = c_int
        f.argtypes = [ctypes.POINTER(dt), c_void_p]
    lib.hca_profiled.restype = c_int
    lib.hca_profiled.argtypes = [c_int, c_void_p, ctypes.POINTER(ProfileEvents), c_void_p]
    return lib


lib = _load()


def check(rc: int) -> None:
    if rc != HCA_OK:
        raise HcaError(rc, lib.hca_last_error().decode())


def new_desc(cls):
    d = cls()
    d.struct_size = ctypes.sizeof(cls)
    return d


def indexer_query_group(desc) -> int:
    g = c_int32(0)
    check(lib.hca_indexer_query_group(ctypes.byref(desc), ctypes.byref(g)))
    return g.value


def workspace_bytes(op: int, desc) -> int:
    n = c_size_t(0)
    check(lib.hca_workspace_bytes(op, ctypes.byref(desc), ctypes.byref(n)))
    return n.value
