"""ctypes declarations for libqam.so (the C ABI in include/qam.h).

Loading fails loudly: if the library has not been built, or cannot be
loaded, an ImportError names the problem.  There is no fallback path.
"""

from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# QAM_LIBRARY names another build of the same library (the host-sanitizer or
# the timeline build)
LIB_PATH = os.environ.get("QAM_LIBRARY") or os.path.join(HERE, "libqam.so")

QAM_OK = 0
ERRORS = {-1: "QAM_ERR_NULL", -2: "QAM_ERR_SHAPE", -3: "QAM_ERR_ARG", -4: "QAM_ERR_LADDER",
          -5: "QAM_ERR_ALIGN", -6: "QAM_ERR_HIP", -7: "QAM_ERR_WORKSPACE", -8: "QAM_ERR_IO"}
QAM_MAX_LENSES = 64
QAM_MAX_STOPS = 15
QAM_MAX_BATCH = 1
QAM_MAX_BATCH_MFMA = 32
QAM_MAX_K = 65536
QAM_X_F32, QAM_X_BF16 = 0, 1
QAM_COMBINE_SUM, QAM_COMBINE_MAX = 0, 1
QAM_OUT_STORE, QAM_OUT_ADD, QAM_OUT_GLU = 0, 1, 2
QAM_RADIUS_LENS, QAM_RADIUS_ZONE = 0, 1
QAM_MAX_BLOCKS = 65536
QAM_MAX_FIELD_BLOCKS = 262144
QAM_WS_STATUS_OFFSET = QAM_MAX_BLOCKS * 4
QAM_WS_COUNTER_BYTES = QAM_MAX_BLOCKS * 4 + 256
QAM_STATUS_BAD_RUNG = 1
QAM_SCRATCH_BYTES = 32 * 1024 * 1024


class QamPacked(C.Structure):
    _fields_ = [("N", C.c_int64), ("K", C.c_int64), ("n_blocks", C.c_int64),
                ("planes", C.c_void_p), ("scales", C.c_void_p)]


QAM_TIMELINE_SLOTS = 8
QAM_TIMELINE_GROUPS = 512
QAM_TIMELINE_POINTS = 8

QAM_STACK_VERSION = 1
QAM_STACK_NAME_BYTES = 32
QAM_STACK_MAX_MATRICES = 65536


class QamStackHeader(C.Structure):
    _fields_ = [("magic", C.c_char * 8), ("version", C.c_uint32), ("n_matrices", C.c_uint32),
                ("n_rungs", C.c_uint32), ("ladder_bits", C.c_uint8 * 16), ("rows_per_block", C.c_uint32),
                ("data_offset", C.c_uint64), ("plane_section_bytes", C.c_uint64), ("scales_offset", C.c_uint64),
                ("scales_bytes", C.c_uint64), ("file_bytes", C.c_uint64), ("reserved", C.c_uint8 * 48)]


class QamStackEntry(C.Structure):
    _fields_ = [("N", C.c_int64), ("K", C.c_int64), ("plane_offset", C.c_uint64), ("scales_offset", C.c_uint64),
                ("name", C.c_char * QAM_STACK_NAME_BYTES)]


class QamLens(C.Structure):
    _fields_ = [("cx", C.c_double), ("cy", C.c_double), ("r", C.c_double)]


class QamLensParams(C.Structure):
    _fields_ = [("f", C.c_double), ("g", C.c_double), ("combine", C.c_int), ("n_stops", C.c_int),
                ("stops", C.c_double * QAM_MAX_STOPS), ("radius_mode", C.c_int), ("reserved", C.c_int),
                ("width", C.c_double)]


QAM_LAYER_THRESHOLD = 0
QAM_LAYER_SHARE = 1


class QamLayerRule(C.Structure):
    _fields_ = [("mode", C.c_int), ("reserved", C.c_int), ("lam", C.c_double), ("share", C.c_double),
                ("g", C.c_double)]


QAM_LAYER_GROUP_MAX = 16


class QamLayerItem(C.Structure):
    _fields_ = [("y_base", C.c_void_p), ("w", QamPacked), ("shat_out", C.c_void_p), ("level_out", C.c_void_p)]


class QamGemvItem(C.Structure):
    _fields_ = [("w", QamPacked), ("x", C.c_void_p), ("y", C.c_void_p), ("level_map", C.c_void_p),
                ("level_stride", C.c_int64), ("coords", C.c_void_p)]


class QamTuning(C.Structure):
    _fields_ = [("target_waves", C.c_int), ("max_chunk_tiles", C.c_int), ("tail_pct", C.c_int),
                ("tail_div", C.c_int), ("ksplit", C.c_int), ("set_max", C.c_int), ("tiles_per_request", C.c_int)]


class QamGroup(C.Structure):
    _fields_ = [("dev_mem", C.c_void_p), ("ksplit", C.c_int), ("n_items", C.c_int), ("B", C.c_int64),
                ("x_dtype", C.c_int), ("n_workgroups", C.c_int64),
                ("lds_bytes", C.c_size_t), ("table", C.c_void_p), ("wg_map", C.c_void_p), ("route", C.c_int),
                ("per_request_maps", C.c_int), ("n_pre_workgroups", C.c_int64), ("pre_map", C.c_void_p),
                ("lens_ready", C.c_int), ("sets", C.c_int), ("set_size", C.c_int), ("col_groups", C.c_int)]


class QamUncertainty(C.Structure):
    _fields_ = [("entropy", C.c_double), ("margin", C.c_double), ("p1", C.c_double), ("p2", C.c_double),
                ("top1", C.c_int64), ("top2", C.c_int64), ("escalate", C.c_int32), ("reserved", C.c_int32)]


class QamEpilogue(C.Structure):
    _fields_ = [("rms_norm", C.c_int), ("out_mode", C.c_int), ("eps", C.c_double)]


class QamDecoderLayer(C.Structure):
    _fields_ = [("qkv", QamPacked), ("o", QamPacked), ("gate_up", QamPacked), ("down", QamPacked)]


class QamDecoderDesc(C.Structure):
    _fields_ = [("n_layers", C.c_int), ("hidden", C.c_int64), ("q_dim", C.c_int64), ("kv_dim", C.c_int64),
                ("ffn", C.c_int64), ("vocab", C.c_int64), ("layers", C.POINTER(QamDecoderLayer)),
                ("lm_head", QamPacked), ("eps", C.c_double), ("target_waves", C.c_int),
                ("waves_per_block", C.c_int), ("max_chunk_tiles", C.c_int)]


class QamSpecStats(C.Structure):
    _fields_ = [("rounds", C.c_int64), ("draft_steps", C.c_int64), ("drafted", C.c_int64), ("accepted", C.c_int64),
                ("emitted", C.c_int64)]


QAM_VER_X, QAM_VER_H, QAM_VER_QKV, QAM_VER_M, QAM_VER_XN, QAM_VER_LOGITS, QAM_VER_Y = range(7)


class QamError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


# (name, restype, argtypes) for every exported function declared in qam.h
_P, _I64, _I, _SZ, _D = C.c_void_p, C.c_int64, C.c_int, C.c_size_t, C.c_double
SIGNATURES = [
    ("qam_packed_bytes", C.c_size_t, [_I64, _I64]),
    ("qam_pack_slices", _I, [_P, _P, _I64, _I64, _P, _SZ, C.POINTER(QamPacked), _P]),
    ("qam_describe_packed", _I, [_P, _I64, _I64, C.POINTER(QamPacked)]),
    ("qam_unpack_codes", _I, [C.POINTER(QamPacked), _P, _P, _P]),
    ("qam_stack_write", _I, [C.c_char_p, C.POINTER(QamPacked), C.POINTER(C.c_char_p), _I, _P]),
    ("qam_stack_info", _I, [C.c_char_p, C.POINTER(QamStackHeader), C.POINTER(QamStackEntry), _I]),
    ("qam_stack_read", _I, [C.c_char_p, _I, _I, _I, C.POINTER(QamPacked), _P, C.POINTER(C.c_uint64)]),
    ("qam_build_level_map", _I, [_P, _I64, C.POINTER(QamLens), _I, C.POINTER(QamLensParams), _P, _I, _I, _P, _P]),
    ("qam_build_rung_map", _I, [_P, _I64, C.POINTER(QamLens), _I, C.POINTER(QamLensParams), _P, _I, _I, _P, _P]),
    ("qam_field_width", _I, [_P, _I64, _P, _SZ, C.POINTER(_D), _P]),
    ("qam_status", _I, [_P, _I, C.POINTER(C.c_uint32), _P]),
    ("qam_build_level_maps", _I, [_P, _I64, C.POINTER(QamLens), _I, C.POINTER(QamLensParams), _P, _I, _I, _I, _P,
                                  _P]),
    ("qam_map_weight_bytes", _I, [_P, _I64, _I64, _P, _I, C.POINTER(_D), C.POINTER(_I64)]),
    ("qam_qmatvec_workspace_bytes", C.c_size_t, [_I64, _I64, _I64]),
    ("qam_qmatvec", _I, [_P, _I, _I64, C.POINTER(QamPacked), _P, _I, _P, _P, _SZ, _P]),
    ("qam_qmatvec_noalloc", _I, [_P, _I, _I64, C.POINTER(QamPacked), _P, _I, _P, _P]),
    ("qam_qmatvec_ep", _I, [_P, _I, _I64, C.POINTER(QamPacked), _P, C.POINTER(QamEpilogue), _P, _P, _SZ, _P]),
    ("qam_decoder_bytes", C.c_size_t, [C.POINTER(QamDecoderDesc)]),
    ("qam_decoder_create", _I, [C.POINTER(QamDecoderDesc), _P, _SZ, C.POINTER(_P), _P]),
    ("qam_decoder_buffer", _P, [_P, _I]),
    ("qam_decoder_step", _I, [_P, _I, _P]),
    ("qam_decoder_run", _I, [_P, _I, _I, _I, _P]),
    ("qam_decoder_capture", _I, [_P, _I, _P]),
    ("qam_decoder_replay", _I, [_P, _I, _P]),
    ("qam_decoder_destroy", None, [_P]),
    ("qam_escalation_schedule", _I, [_P, _I64, _D, _P, C.POINTER(_I64)]),
    ("qam_group_bytes", C.c_size_t, [C.POINTER(QamGemvItem), _I, _I64, _I]),
    ("qam_group_init", _I, [C.POINTER(QamGemvItem), _I, _I64, _I, _I, _P, _SZ, C.POINTER(QamGroup), _P]),
    ("qam_group_bytes_tuned", C.c_size_t, [C.POINTER(QamGemvItem), _I, _I64, _I, C.POINTER(QamTuning)]),
    ("qam_group_init_tuned", _I, [C.POINTER(QamGemvItem), _I, _I64, _I, _I, C.POINTER(QamTuning), _P, _SZ,
                                  C.POINTER(QamGroup), _P]),
    ("qam_qmatvec_group", _I, [C.POINTER(QamGroup), _P]),
    ("qam_qmatvec_group_lens", _I, [C.POINTER(QamGroup), C.POINTER(QamLens), _I, C.POINTER(QamLensParams), _P, _I,
                                    _I, _P]),
    ("qam_layer_levels", _I, [_P, _I64, C.POINTER(QamPacked), C.POINTER(QamLayerRule), _I, _I, _P, _P, _P]),
    ("qam_layer_levels_group", _I, [C.POINTER(QamLayerItem), _I, _I64, C.POINTER(QamLayerRule), _I, _I, _P]),
    ("qam_qmatvec_group_refine", _I, [_P, _I, _P]),
    ("qam_fit_focus_area", _I, [_P, _I64, _P, C.POINTER(QamLens), _I, C.POINTER(QamLensParams), _P, _I, _I, _I64,
                                _I, _P, _P, _SZ, C.POINTER(C.c_double), C.POINTER(C.c_int64), _P]),
    ("qam_decoder_decode_gated", _I, [_P, _P, _I64, _I, _I, C.c_double, C.c_double, _P, _SZ, _P, _P, _P, _P]),
    ("qam_decoder_decode_gated_async", _I, [_P, _P, _I64, _I, _I, C.c_double, C.c_double, _P, _SZ, _P, _P, _P]),
    ("qam_gate_workspace_bytes", C.c_size_t, [_I64]),
    ("qam_gate", _I, [_P, _I64, C.c_double, C.c_double, _P, _P, _SZ, _P]),
    ("qam_verifier_bytes", C.c_size_t, [C.POINTER(QamDecoderDesc), _I]),
    ("qam_verifier_create", _I, [_P, _I, _P, _SZ, C.POINTER(_P), _P]),
    ("qam_verifier_buffer", _P, [_P, _I]),
    ("qam_verifier_run", _I, [_P, _I, _I, _I, _I, _P]),
    ("qam_verifier_step", _I, [_P, _I, _I, _P]),
    ("qam_verifier_capture", _I, [_P, _I, _I, _P]),
    ("qam_verifier_replay", _I, [_P, _I, _I, _P]),
    ("qam_verifier_destroy", None, [_P]),
    ("qam_argmax_rows", _I, [_P, _I64, _I64, _I64, _P, _P, _P]),
    ("qam_decoder_speculate", _I, [_P, _P, _P, C.c_int32, _I, _I, _I, _I, _P, C.POINTER(QamSpecStats), _P]),
    ("qam_timeline_select", _I, [_P, _I]),
    ("qam_timeline_read", _I, [_P, _SZ]),
    ("qam_last_error", C.c_char_p, []),
    ("qam_last_variant", C.c_char_p, []),
    ("qam_version", C.c_char_p, []),
]
# benchmark hooks (kernel-side launch timing), not part of the product ABI contract
EXTRA_SIGNATURES = [
    ("qam_group_launch_times", _I, [C.POINTER(QamGroup), _I, _P, _P]),
    ("qam_group_lens_launch_times", _I, [C.POINTER(QamGroup), C.POINTER(QamLens), _I, C.POINTER(QamLensParams), _P,
                                         _I, _I, _I, _P, _P]),
]


def load(path: str = LIB_PATH) -> C.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"libqam.so not built at {path}: run `python -c 'import __graft_entry__ as g; g.build()'`")
    try:
        lib = C.CDLL(path)
    except OSError as exc:
        raise ImportError(f"cannot load {path}: {exc}") from exc
    for name, res, args in SIGNATURES + EXTRA_SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_LIB = None


def lib() -> C.CDLL:
    global _LIB
    if _LIB is None:
        _LIB = load()
    return _LIB


def check(rc: int) -> None:
    if rc != QAM_OK:
        raise QamError(rc, lib().qam_last_error().decode())
