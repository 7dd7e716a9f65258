"""ctypes binding of libcdb.so — argument marshalling only.

Every name mirrors include/cdb.h.  The library must be built in-tree
(``python -m continuous_depth_batching_amd.build``); importing this module
without it raises, so nothing can silently run elsewhere.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcdb.so")

CDB_OK, CDB_EINVAL, CDB_EHIP, CDB_ENOMEM, CDB_ESTATE = 0, -1, -2, -3, -4
CDB_FP32, CDB_BF16 = 0, 1
CDB_KV_DEPTH, CDB_KV_SINGLE, CDB_KV_FIRST_SHARED, CDB_KV_DEPTH_COPY = 0, 1, 2, 3
CDB_GATE_LINEAR, CDB_GATE_CONVERGENCE = 0, 1

I32 = C.c_int32
P = C.c_void_p
PI32 = C.POINTER(C.c_int32)
PF32 = C.POINTER(C.c_float)
PU8 = C.POINTER(C.c_uint8)

# every symbol include/cdb.h declares
EXPORTS = ["cdb_pack_weight", "cdb_workspace_bytes", "cdb_init", "cdb_init_static", "cdb_prefill", "cdb_core_step", "cdb_gate_compact",
           "cdb_boundary", "cdb_profile", "cdb_profile_read", "cdb_graph_begin", "cdb_graph_end",
           "cdb_graph_launch", "cdb_graph_destroy", "cdb_sync", "cdb_destroy", "cdb_strerror",
           "cdb_last_error", "cdb_version"]


class cdb_dims(C.Structure):
    _fields_ = [("vocab", I32), ("hidden", I32), ("n_heads", I32), ("head_dim", I32), ("ffn", I32),
                ("n_prelude", I32), ("n_core", I32), ("n_coda", I32), ("r_max", I32), ("dtype", I32),
                ("kv_layout", I32), ("inject", I32), ("gate_kind", I32), ("rms_eps", C.c_float),
                ("rope_theta", C.c_float), ("gate_bias", C.c_float), ("gate_threshold", C.c_float),
                ("conv_threshold", C.c_float)]


class cdb_layer(C.Structure):
    _fields_ = [("attn_norm", P), ("wqkv", P), ("wo", P), ("mlp_norm", P), ("wgu", P), ("wd", P)]


class cdb_weights(C.Structure):
    _fields_ = [("embed", P), ("prelude", C.POINTER(cdb_layer)), ("core", C.POINTER(cdb_layer)),
                ("coda", C.POINTER(cdb_layer)), ("final_norm", P), ("lm_head", P), ("gate_w", P)]


class cdb_kv(C.Structure):
    _fields_ = [("block_size", I32), ("num_blocks", I32), ("core_k", P), ("core_v", P), ("bnd_k", P),
                ("bnd_v", P), ("exit_depth", P), ("block_table", P), ("max_seqs", I32),
                ("max_blocks_per_seq", I32)]


class cdb_seqs(C.Structure):
    _fields_ = [("tokens_out", P), ("exits_out", P), ("n_gen", P), ("n_out", P), ("max_out", I32)]


class cdb_pools(C.Structure):
    _fields_ = [("state", P), ("inject", P), ("prev_state", P), ("n_slots", I32), ("workspace", P),
                ("workspace_bytes", C.c_size_t),
                ("max_rows", I32), ("max_prefill_tokens", I32), ("max_context", I32)]


class cdb_core_desc(C.Structure):
    _fields_ = [("n_valid", P), ("slot", P), ("seq", P), ("pos", P), ("depth", P), ("exit_at", P), ("cap", I32)]


class cdb_exit_queue(C.Structure):
    _fields_ = [("n", P), ("slot", P), ("seq", P), ("pos", P), ("depth", P), ("cap", I32)]


class cdb_compact_out(C.Structure):
    _fields_ = [("counts", P), ("fired_seq", P), ("host_counts", P), ("host_fired", P), ("event", P)]


class cdb_prefill_desc(C.Structure):
    _fields_ = [("n_seqs", I32), ("n_tokens", I32), ("tokens", P), ("cu_seqlens", P), ("seq", P),
                ("start_pos", P), ("slot", P), ("is_final", P), ("host_cu_seqlens", P),
                ("host_start_pos", P), ("host_is_final", P), ("logits_out", P)]


class cdb_boundary_desc(C.Structure):
    _fields_ = [("rows_pad", I32), ("exit_states_out", P), ("logits_out", P), ("tokens_out_rows", P)]


class CDBError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{msg} (code {code})")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python -m continuous_depth_batching_amd.build")
    lib = C.CDLL(LIB_PATH)
    lib.cdb_pack_weight.argtypes = [I32, P, P, I32, I32, P]
    lib.cdb_pack_weight.restype = C.c_int
    lib.cdb_workspace_bytes.argtypes = [C.POINTER(cdb_dims), I32, I32, I32]
    lib.cdb_workspace_bytes.restype = C.c_size_t
    lib.cdb_init.argtypes = [C.POINTER(cdb_dims), C.POINTER(cdb_weights), C.POINTER(cdb_kv), C.POINTER(cdb_pools),
                             C.POINTER(cdb_seqs), P, C.POINTER(P)]
    lib.cdb_init_static.argtypes = lib.cdb_init.argtypes
    lib.cdb_prefill.argtypes = [P, C.POINTER(cdb_prefill_desc), C.POINTER(cdb_core_desc)]
    lib.cdb_core_step.argtypes = [P, C.POINTER(cdb_core_desc), I32]
    lib.cdb_gate_compact.argtypes = [P, C.POINTER(cdb_core_desc), I32, I32, C.POINTER(cdb_exit_queue),
                                     C.POINTER(cdb_compact_out)]
    lib.cdb_boundary.argtypes = [P, C.POINTER(cdb_exit_queue), C.POINTER(cdb_core_desc), C.POINTER(cdb_boundary_desc)]
    lib.cdb_profile.argtypes = [P, I32]
    lib.cdb_profile_read.argtypes = [P, C.c_char_p, C.POINTER(C.c_double), C.POINTER(C.c_int64)]
    lib.cdb_graph_begin.argtypes = [P]
    lib.cdb_graph_end.argtypes = [P, C.POINTER(P)]
    lib.cdb_graph_launch.argtypes = [P, P]
    lib.cdb_graph_destroy.argtypes = [P]
    lib.cdb_graph_destroy.restype = None
    lib.cdb_sync.argtypes = [P]
    lib.cdb_destroy.argtypes = [P]
    lib.cdb_destroy.restype = None
    lib.cdb_strerror.argtypes = [C.c_int]
    lib.cdb_strerror.restype = C.c_char_p
    lib.cdb_last_error.argtypes = []
    lib.cdb_last_error.restype = C.c_char_p
    lib.cdb_version.restype = C.c_char_p
    for name in ("cdb_init", "cdb_init_static", "cdb_prefill", "cdb_core_step", "cdb_gate_compact", "cdb_boundary", "cdb_sync",
                 "cdb_profile", "cdb_profile_read", "cdb_graph_begin", "cdb_graph_end", "cdb_graph_launch"):
        getattr(lib, name).restype = C.c_int
    return lib


lib = _load()


def check(rc: int):
    if rc != CDB_OK:
        raise CDBError(rc, f"{lib.cdb_strerror(rc).decode()}: {lib.cdb_last_error().decode()}")
    return rc
