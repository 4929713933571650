"""ctypes declarations of libbdr.so (the C ABI in include/bdr.h)."""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libbdr.so")

BDR_F32 = 0
BDR_BF16 = 1
BDR_BF16_PACKED = 2

BDR_OK = 0
BDR_EINVAL = -1
BDR_EUNSUPPORTED = -2
BDR_EWORKSPACE = -3
BDR_EHIP = -4

MAX_TAPS = 8
MAX_K = 16
MAX_RANK = 128

_vp = C.c_void_p
_i64 = C.c_int64
_int = C.c_int
_sz = C.c_size_t
_u64 = C.c_uint64

# name -> (restype, argtypes)
SIGNATURES = {
    "bdr_abi_version": (_int, []),
    "bdr_last_error": (C.c_char_p, []),
    "bdr_set_markov_poll_timeout_us": (None, [C.c_double]),
    "bdr_set_markov_forced_time_out": (None, [C.c_int]),
    "bdr_set_row_split_override": (_int, [_int, _i64, _int]),
    "bdr_packed_weight_bytes": (_sz, [_i64, _i64]),
    "bdr_pack_weight": (_int, [_vp, _i64, _i64, _vp, _vp]),
    "dflash_fuse_fc_workspace_bytes": (_sz, [_i64, _i64, _int, _int]),
    "dflash_fuse_fc": (_int, [C.POINTER(_vp), _int, _i64, _i64, _int, _vp, _vp, _vp, _sz, _vp]),
    "dspark_lm_head": (_int, [_vp, _i64, _i64, _i64, _int, _vp, _vp, _vp]),
    "dflash_fuse_fc_lm_head_workspace_bytes": (_sz, [_i64, _i64, _int, _i64, _i64, _int]),
    "dflash_fuse_fc_lm_head": (_int, [C.POINTER(_vp), _int, _i64, _i64, _int, _vp, _vp, _vp, _i64,
                                      _i64, _vp, _vp, _vp, _sz, _vp]),
    "dflash_hc_average": (_int, [C.POINTER(_vp), _int, _int, _i64, _i64, _i64, _i64, _int,
                                 C.POINTER(_vp), _vp]),
    "dflash_fuse_fc_fp8_workspace_bytes": (_sz, [_i64, _i64, _int]),
    "dflash_fuse_fc_rows_fp8_workspace_bytes": (_sz, [_i64, _i64, _int]),
    "dflash_fuse_fc_rows_fp8": (_int, [C.POINTER(_vp), _int, _i64, _i64, _vp, _vp, _i64, _vp, _vp,
                                       _vp, _vp, _sz, _vp]),
    "dflash_fuse_fc_fp8": (_int, [C.POINTER(_vp), _int, _i64, _i64, _vp, _vp, _vp, _vp, _sz, _vp]),
    "dspark_lm_head_fp8": (_int, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp]),
    "dspark_markov_workspace_bytes": (_sz, [_i64, _int]),
    "dspark_markov_argmax": (_int, [_vp, _i64, _int, _i64, _int, _vp, _vp, _int, _vp, _vp,
                                    _vp, _vp, _sz, _vp]),
    "dspark_draft_workspace_bytes": (_sz, [_i64, _int, _i64, _int]),
    "dspark_draft_block": (_int, [_vp, _i64, _int, _i64, _i64, _int, _vp, _vp, _vp, _int, _vp,
                                  _vp, _vp, _vp, _vp, _sz, _vp]),
    "dspark_draft_block_noalloc": (_int, [_vp, _i64, _int, _i64, _i64, _int, _vp, _vp, _vp, _int,
                                          _vp, _vp, _vp, _vp, _vp]),
    "spec_verify_workspace_bytes": (_sz, [_i64, _int, _i64]),
    "spec_verify_greedy": (_int, [_vp, _int, _i64, _int, _i64, _vp, _vp, C.c_float, _vp, _vp,
                                  _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "dspark_gumbel_noise": (_int, [_i64, _int, _i64, _u64, _int, _vp, _vp]),
    "dspark_markov_sample_workspace_bytes": (_sz, [_i64, _int, _i64]),
    "dspark_markov_sample": (_int, [_vp, _i64, _int, _i64, _int, _vp, _vp, _int, _vp, C.c_float,
                                    _u64, _vp, _vp, _vp, C.c_float, _vp, _vp, _sz, _vp]),
    "spec_verify_sample_workspace_bytes": (_sz, [_i64, _int, _i64]),
    "spec_verify_sample": (_int, [_vp, _int, _i64, _int, _i64, _vp, _vp, _vp, C.c_float,
                                  C.c_float, _u64, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "spec_commit": (_int, [_vp, _vp, _vp, _vp, _i64, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "dflash_fuse_fc_rows_workspace_bytes": (_sz, [_i64, _i64, _int, _int]),
    "dflash_fuse_fc_rows": (_int, [C.POINTER(_vp), _int, _i64, _i64, _int, _vp, _vp, _i64, _vp,
                                   _vp, _vp, _sz, _vp]),
}

_lib = None


class BdrError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed ({code}): {msg}")
        self.code = code


def load(path: str = LIB_PATH) -> C.CDLL:
    """Load libbdr.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
            "(or python block_draft_readout_amd/build.py)")
    lib = C.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(fn: str, rc: int) -> None:
    if rc != BDR_OK:
        msg = load().bdr_last_error()
        raise BdrError(fn, rc, msg.decode() if msg else "")
