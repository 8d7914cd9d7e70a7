"""ctypes binding of libsdrl.so (include/er_api.h, include/er_ops.h).

Argument marshalling only: every step of the rollout runs in the library's
gfx950 kernels.  Loading fails loudly when the library has not been built or
cannot be opened; there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsdrl.so")

ER_OK, ER_EINVAL, ER_ENOMEM, ER_EDEVICE, ER_ESTATE = 0, -1, -2, -3, -4
ER_F32, ER_BF16 = 0, 1
ER_W8_PERCH_SYM, ER_W4_G128_ASYM = 0, 1
ER_POLICY_AUTO, ER_POLICY_FORCE_SD, ER_POLICY_FORCE_AR, ER_POLICY_TIMING, ER_POLICY_HISTORY = 0, 1, 2, 3, 4
ER_KPROF_OFF, ER_KPROF_ALL, ER_KPROF_ATTENTION = 0, 1, 2
ER_MODE_AR, ER_MODE_SD, ER_MODE_HISTORY = 0, 1, 3
ER_FMT_F32, ER_FMT_BF16, ER_FMT_W8, ER_FMT_W4 = 0, 1, 2, 3
PURPOSE_DRAFT, PURPOSE_ACCEPT, PURPOSE_RESIDUAL, PURPOSE_AR = 0, 1, 2, 3

_NAMES = {ER_EINVAL: "ER_EINVAL", ER_ENOMEM: "ER_ENOMEM", ER_EDEVICE: "ER_EDEVICE", ER_ESTATE: "ER_ESTATE"}


class ModelDesc(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32), ("vocab", C.c_int32),
                ("dtype", C.c_int32), ("rms_eps", C.c_float), ("rope_theta", C.c_float)]


class DraftDesc(C.Structure):
    _fields_ = [("quant", C.c_int32), ("group_size", C.c_int32), ("quant_lm_head", C.c_int32)]


class RolloutDesc(C.Structure):
    _fields_ = [("seed", C.c_uint64), ("temperature", C.c_float), ("top_p", C.c_float),
                ("gamma_init", C.c_int32), ("gamma_min", C.c_int32), ("gamma_max", C.c_int32),
                ("ema_beta", C.c_float), ("switch_margin", C.c_float), ("alpha_init", C.c_float),
                ("policy", C.c_int32), ("kv_block", C.c_int32), ("max_seqs", C.c_int32), ("max_batch", C.c_int32),
                ("max_ctx", C.c_int32), ("prefill_chunk", C.c_int32), ("kv_pool_blocks", C.c_int64),
                ("hbm_bytes_per_s", C.c_double), ("flops_per_s", C.c_double), ("t_fwd_s", C.c_double)]


class Weights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("final_norm", C.c_void_p), ("lm_head", C.c_void_p),
                ("attn_norm", C.POINTER(C.c_void_p)), ("wqkv", C.POINTER(C.c_void_p)),
                ("wo", C.POINTER(C.c_void_p)), ("mlp_norm", C.POINTER(C.c_void_p)),
                ("wgate_up", C.POINTER(C.c_void_p)), ("wdown", C.POINTER(C.c_void_p))]


class StepInfo(C.Structure):
    _fields_ = [("mode", C.c_int32), ("gamma", C.c_int32), ("batch", C.c_int32), ("accepted", C.c_int32),
                ("emitted", C.c_int32), ("kept", C.c_int32), ("finished", C.c_int32),
                ("alpha_step", C.c_float), ("alpha_ema", C.c_float), ("ms_draft", C.c_float),
                ("ms_verify", C.c_float), ("ms_sample", C.c_float), ("ms_total", C.c_float)]


class Stats(C.Structure):
    _fields_ = [("predict_times", C.c_int64), ("effective_times", C.c_int64), ("total_right_length", C.c_int64),
                ("effective_length", C.c_double), ("effective_percent", C.c_double),
                ("sd_steps", C.c_int64), ("ar_steps", C.c_int64), ("drafted", C.c_int64), ("accepted", C.c_int64),
                ("emitted", C.c_int64), ("bonus", C.c_int64), ("tokens_kept", C.c_int64),
                ("alpha_ema", C.c_double), ("gamma", C.c_int32), ("mode", C.c_int32),
                ("ms_draft", C.c_double), ("ms_verify", C.c_double), ("ms_sample", C.c_double),
                ("ms_ar", C.c_double), ("ms_prefill", C.c_double),
                ("history_steps", C.c_int64), ("history_drafted", C.c_int64), ("history_accepted", C.c_int64)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class GraphStats(C.Structure):
    _fields_ = [("max_batch", C.c_int32), ("cached", C.c_int32), ("captures", C.c_int64), ("replays", C.c_int64),
                ("evictions", C.c_int64)]


class KernelStat(C.Structure):
    _fields_ = [("name", C.c_char * 64), ("launches", C.c_int64), ("ms", C.c_double), ("bytes", C.c_double),
                ("flops", C.c_double)]


class CostModel(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32), ("vocab", C.c_int32),
                ("w_bytes", C.c_double), ("q_bytes", C.c_double), ("kv_bytes_el", C.c_double),
                ("hbm_bytes_per_s", C.c_double), ("flops_per_s", C.c_double), ("t_fwd_s", C.c_double),
                ("t_row_draft_s", C.c_double), ("t_row_target_s", C.c_double)]


class PlanState(C.Structure):
    _fields_ = [("choice", C.c_int32), ("ar_streak", C.c_int32), ("probe_every", C.c_int32)]


ER_GUARD_BUCKETS = 16


class GuardParams(C.Structure):
    _fields_ = [("max_sd_batch", C.c_int32), ("probe_max_batch", C.c_int32), ("compare_after", C.c_int32),
                ("probe_steps", C.c_int32), ("ema_alpha", C.c_double), ("margin", C.c_double),
                ("cooldown", C.c_int64), ("cooldown_max", C.c_int64), ("cooldown_growth", C.c_double),
                ("bad_ratio", C.c_double)]


class GuardState(C.Structure):
    _fields_ = [("p", GuardParams), ("step", C.c_int64),
                ("ema_ar", C.c_double * ER_GUARD_BUCKETS), ("ema_sd", C.c_double * ER_GUARD_BUCKETS),
                ("n_ar", C.c_int64 * ER_GUARD_BUCKETS), ("probe_left", C.c_int32 * ER_GUARD_BUCKETS),
                ("cool_until", C.c_int64 * ER_GUARD_BUCKETS), ("cool_len", C.c_int64 * ER_GUARD_BUCKETS)]


P = C.c_void_p
I32P = C.POINTER(C.c_int32)
I64P = C.POINTER(C.c_int64)

# name -> (restype, argtypes)
class QkvArgs(C.Structure):
    _fields_ = [("hq", C.c_int), ("hkv", C.c_int), ("hd", C.c_int), ("d_pos", C.c_void_p), ("d_slot", C.c_void_p),
                ("d_cos_sin", C.c_void_p), ("d_q_out", C.c_void_p), ("d_kv_pool", C.c_void_p), ("layer", C.c_int),
                ("n_layers", C.c_int)]


EPI_F32, EPI_RESID, EPI_SWIGLU, EPI_QKV = 0, 2, 3, 4

SIGNATURES = {
    # er_api.h
    "er_rollout_init": (C.c_int, [C.POINTER(ModelDesc), C.POINTER(Weights), C.POINTER(DraftDesc),
                                  C.POINTER(RolloutDesc), P, C.c_size_t, P, C.POINTER(P)]),
    "er_arena_bytes": (C.c_int, [C.POINTER(ModelDesc), C.POINTER(DraftDesc), C.POINTER(RolloutDesc), C.c_int64,
                                 C.POINTER(C.c_size_t)]),
    "er_update_weights": (C.c_int, [P, C.POINTER(Weights)]),
    "er_kv_alloc": (C.c_int, [P, C.c_int, I32P, I32P, I32P, I32P]),
    "er_prefill": (C.c_int, [P, C.c_int, I32P, I32P, I64P, I32P]),
    "er_spec_step": (C.c_int, [P, C.c_int, I32P, I32P, I32P, C.POINTER(StepInfo)]),
    "er_ar_step": (C.c_int, [P, C.c_int, I32P, I32P, C.POINTER(StepInfo)]),
    "er_step": (C.c_int, [P, C.c_int, I32P, I32P, I32P, C.POINTER(StepInfo)]),
    "er_rollout": (C.c_int, [P, C.c_int, I32P, C.c_int32, I32P, I32P, C.POINTER(Stats)]),
    "er_set_gamma": (C.c_int, [P, C.c_int]),
    "er_set_policy": (C.c_int, [P, C.c_int]),
    "er_history_create": (C.c_int, [C.c_int, C.POINTER(P)]),
    "er_history_destroy": (C.c_int, [P]),
    "er_history_add": (C.c_int, [P, C.c_int, I32P, C.c_int, I32P, C.c_float]),
    "er_history_propose": (C.c_int, [P, C.c_int, I32P, C.c_int, I32P, C.c_int, I32P, I32P]),
    "er_history_records": (C.c_int, [P, C.POINTER(C.c_int64)]),
    "er_set_history": (C.c_int, [P, P, C.c_int, C.c_int]),
    "er_history_step": (C.c_int, [P, C.c_int, I32P, I32P, I32P, C.POINTER(StepInfo)]),
    "er_kv_fork": (C.c_int, [P, C.c_int32, C.c_int, I32P, I32P]),
    "er_kv_free": (C.c_int, [P, C.c_int, I32P]),
    "er_seq_info": (C.c_int, [P, C.c_int32, I32P, I32P, I32P]),
    "er_get_stats": (C.c_int, [P, C.POINTER(Stats)]),
    "er_reset_stats": (C.c_int, [P]),
    "er_set_timing": (C.c_int, [P, C.c_int, C.c_int]),
    "er_set_fused": (C.c_int, [P, C.c_int]),
    "er_set_persistent": (C.c_int, [P, C.c_int]),
    "er_get_persistent": (C.c_int, [P, C.POINTER(C.c_int)]),
    "er_set_graphs": (C.c_int, [P, C.c_int]),
    "er_set_library_gemm": (C.c_int, [P, C.c_int]),
    "er_get_graph_stats": (C.c_int, [P, C.POINTER(GraphStats)]),
    "er_set_decode_spin_limit": (C.c_int, [P, C.c_int64]),
    "er_set_decode_trace": (C.c_int, [P, C.c_int]),
    "er_get_decode_trace": (C.c_int, [P, C.POINTER(C.c_double), C.POINTER(C.c_double), C.c_int,
                                      C.POINTER(C.c_int)]),
    "er_kv_free_blocks": (C.c_int, [P, I64P, I64P]),
    "er_set_kernel_profile": (C.c_int, [P, C.c_int]),
    "er_get_kernel_profile": (C.c_int, [P, C.POINTER(KernelStat), C.c_int, C.POINTER(C.c_int)]),
    "er_reset_kernel_profile": (C.c_int, [P]),
    "er_debug_logits": (C.c_int, [P, C.c_int, C.c_int, C.POINTER(C.c_float), I32P]),
    "er_debug_drafts": (C.c_int, [P, I32P]),
    "er_controller_choose": (C.c_int, [C.POINTER(CostModel), C.c_int, C.c_double, C.c_double, C.c_int, C.c_int,
                                       C.c_int, C.c_double, C.POINTER(C.c_int)]),
    "er_expected_tokens": (C.c_double, [C.c_double, C.c_int]),
    "er_get_cost_model": (C.c_int, [P, C.POINTER(CostModel)]),
    "er_controller_times": (C.c_int, [C.POINTER(CostModel), C.c_int, C.c_double, C.c_int,
                                      C.POINTER(C.c_double), C.POINTER(C.c_double)]),
    "er_controller_plan": (C.c_int, [C.POINTER(CostModel), C.POINTER(PlanState), C.c_int, C.c_int, C.c_double,
                                     C.c_double, C.c_double, C.c_int, C.c_int, C.c_double, C.POINTER(C.c_int)]),
    "er_get_plan_state": (C.c_int, [P, C.POINTER(PlanState)]),
    "er_guard_default_params": (None, [C.POINTER(GuardParams)]),
    "er_guard_init": (C.c_int, [C.POINTER(GuardState), C.POINTER(GuardParams)]),
    "er_guard_choose": (C.c_int, [C.POINTER(GuardState), C.c_int]),
    "er_guard_observe": (C.c_int, [C.POINTER(GuardState), C.c_int, C.c_int, C.c_double, C.c_double]),
    "er_get_guard": (C.c_int, [P, C.POINTER(GuardState)]),
    "er_last_error": (C.c_char_p, [P]),
    "er_destroy": (None, [P]),
    # er_ops.h
    "er_op_quantize": (C.c_int, [C.c_int, C.c_int, P, C.c_int, C.c_int, P, P, P, P]),
    "er_op_w4_kernel_order": (C.c_int, [P, C.c_int, C.c_int, P, P]),
    "er_op_linear": (C.c_int, [C.c_int, P, C.c_int, C.c_int, C.c_int, P, P, P, C.c_int, C.c_int, P, C.c_int,
                               C.c_int, P]),
    "er_op_linear_fused": (C.c_int, [C.c_int, P, C.c_int, C.c_int, C.c_int, P, P, P, C.c_float, C.c_int, P, P, P,
                                     C.c_int, C.c_int, P, C.c_int, P, P, C.POINTER(QkvArgs), C.c_int, P]),
    "er_op_attention": (C.c_int, [C.c_int, P, P, P, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, P, C.c_int, P, P,
                                  P, P, C.c_int, C.c_int, C.c_int, P]),
    "er_op_attention_noalloc": (C.c_int, [C.c_int, P, P, P, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, P, C.c_int,
                                          P, P, P, P, C.c_int, C.c_int, C.c_int, P]),
    "er_op_stats_bytes": (C.c_size_t, [C.c_int]),
    "er_op_row_stats": (C.c_int, [P, C.c_int, C.c_int, C.c_long, C.c_float, C.c_float, P, P]),
    "er_op_sample_rows": (C.c_int, [P, P, C.c_int, C.c_int, C.c_long, C.c_float, C.c_float, C.c_uint64, P, P, C.c_int,
                                    C.c_int, P, C.c_int, P]),
    "er_op_spec_decide": (C.c_int, [P, P, P, P, P, C.c_int, C.c_int, C.c_int, C.c_float, C.c_float, C.c_uint64, P, P,
                                    P, P, P]),
    "er_op_philox_uniform": (C.c_int, [C.c_uint64, P, C.c_int, P, P]),
}

_lib = None


def lib_path() -> str:
    return LIB_PATH


def load() -> C.CDLL:
    """Open libsdrl.so and declare every exported signature; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run speculative_decoding_rl_amd/build.py (or __graft_entry__.build())")
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class ErError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_NAMES.get(code, code)}: {msg}")
        self.code = code


def check(code: int, ctx=None, what: str = ""):
    if code == ER_OK:
        return
    msg = what
    if ctx:
        m = load().er_last_error(ctx)
        msg = f"{what}: {m.decode() if m else ''}"
    raise ErError(code, msg)
