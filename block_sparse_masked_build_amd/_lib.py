"""ctypes view of the C ABI declared in include/bsm.h.

Loading fails loudly: there is no fallback path.  If libbsm.so is missing,
importing this module raises ImportError with the command that builds it.
"""
from __future__ import annotations

import ctypes
import os

# libbsm.so links libamdhip64 dynamically.  PyTorch ships its own HIP runtime;
# importing torch first makes the library bind to that one, so that device
# memory and streams from torch and the kernels launched here share a single
# runtime in the process.
import torch  # noqa: F401

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbsm.so")

BSM_OK, BSM_E_INVALID, BSM_E_UNSUPPORTED, BSM_E_WORKSPACE, BSM_E_HIP = range(5)
STATUS_NAMES = {0: "BSM_OK", 1: "BSM_E_INVALID", 2: "BSM_E_UNSUPPORTED",
                3: "BSM_E_WORKSPACE", 4: "BSM_E_HIP"}

BSM_MASK_CAUSAL, BSM_MASK_DOCUMENT, BSM_MASK_WINDOW, BSM_MASK_SINKS, BSM_MASK_PREFIX = 1, 2, 4, 8, 16
BSM_MASK_TABLE = 32
BSM_MOD_ALIBI, BSM_MOD_SOFTCAP, BSM_MOD_BIAS = 1, 2, 4
BSM_BIAS_MAX_RADIUS = 1024
BSM_DTYPE_BF16, BSM_DTYPE_F16 = 0, 1


class BsmMaskSpec(ctypes.Structure):
    _fields_ = [("flags", ctypes.c_uint32), ("seq_len", ctypes.c_int32),
                ("mask_b", ctypes.c_int32), ("doc_ids", ctypes.c_void_p),
                ("window", ctypes.c_void_p), ("num_sinks", ctypes.c_int32),
                ("prefix_len", ctypes.c_int32), ("q_len", ctypes.c_int32),
                ("q_offset", ctypes.c_int32), ("table", ctypes.c_uint32),
                ("kv_block", ctypes.c_int32)]


class BsmBlockMask(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "kv_num_blocks", "kv_indices", "full_kv_num_blocks", "full_kv_indices",
        "q_num_blocks", "q_indices", "full_q_num_blocks", "full_q_indices", "doc_range",
        "kv_order", "q_order")]


class BsmScoreMod(ctypes.Structure):
    _fields_ = [("flags", ctypes.c_uint32), ("alibi_slopes", ctypes.c_void_p),
                ("softcap", ctypes.c_float), ("alibi_slopes_grad", ctypes.c_void_p),
                ("bias", ctypes.c_void_p), ("bias_radius", ctypes.c_int32), ("bias_grad", ctypes.c_void_p)]


class BsmTensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("stride_t", ctypes.c_int64),
                ("dtype", ctypes.c_int32)]


# Every symbol include/bsm.h declares, with its ctypes signature.
_P = ctypes.POINTER
SIGNATURES = {
    "bsm_block_mask_workspace_bytes": (ctypes.c_size_t, [_P(BsmMaskSpec)]),
    "bsm_build_block_mask": (ctypes.c_int, [_P(BsmMaskSpec), _P(BsmBlockMask), ctypes.c_void_p,
                                            ctypes.c_size_t, ctypes.c_void_p]),
    "bsm_flex_attention_fwd": (ctypes.c_int, [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        _P(BsmTensor), _P(BsmTensor), _P(BsmTensor), _P(BsmBlockMask), _P(BsmMaskSpec),
        _P(BsmScoreMod), ctypes.c_float, _P(BsmTensor), ctypes.c_void_p, ctypes.c_void_p]),
    "bsm_bwd_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int32] * 4),
    "bsm_bwd_workspace_bytes_mod": (ctypes.c_size_t, [ctypes.c_int32] * 4 + [_P(BsmScoreMod)]),
    "bsm_flex_attention_bwd": (ctypes.c_int, [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        _P(BsmTensor), _P(BsmTensor), _P(BsmTensor), _P(BsmTensor), ctypes.c_void_p,
        _P(BsmTensor), _P(BsmBlockMask), _P(BsmMaskSpec), _P(BsmScoreMod), ctypes.c_float,
        _P(BsmTensor), _P(BsmTensor), _P(BsmTensor), ctypes.c_void_p, ctypes.c_size_t,
        ctypes.c_void_p]),
    "bsm_decode_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int32] * 4),
    "bsm_flex_attention_decode": (ctypes.c_int, [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
        _P(BsmTensor), _P(BsmTensor), _P(BsmTensor), _P(BsmMaskSpec), _P(BsmBlockMask), _P(BsmScoreMod),
        ctypes.c_float, _P(BsmTensor), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "bsm_flex_attention_decode_paged": (ctypes.c_int, [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
        ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
        _P(BsmTensor), _P(BsmTensor), _P(BsmTensor), _P(BsmMaskSpec), _P(BsmBlockMask), _P(BsmScoreMod),
        ctypes.c_float, _P(BsmTensor), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "bsm_gather_kv_pages": (ctypes.c_int, [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
        ctypes.c_int32, ctypes.c_int32, _P(BsmTensor), _P(BsmTensor), _P(BsmTensor), _P(BsmTensor),
        ctypes.c_void_p]),
    "bsm_decode_static_max_bytes": (ctypes.c_size_t, []),
    "bsm_flex_attention_decode_static": (ctypes.c_int, [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
        _P(BsmTensor), _P(BsmTensor), _P(BsmTensor), _P(BsmMaskSpec), _P(BsmBlockMask), _P(BsmScoreMod),
        ctypes.c_float, _P(BsmTensor), ctypes.c_void_p, ctypes.c_void_p]),
    "bsm_last_error": (ctypes.c_char_p, []),
    "bsm_version": (ctypes.c_char_p, []),
}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m block_sparse_masked_build_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = load()


class BsmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def check(status: int) -> None:
    if status != BSM_OK:
        raise BsmError(status, lib.bsm_last_error().decode())
