"""ctypes binding of libdg.so (include/dg.h).  Argument marshalling only.

torch is imported first so that the library's HIP runtime dependency
(libamdhip64.so.7) resolves to the copy torch has already loaded: device
pointers and streams from torch are then valid inside the library.  Loading
fails loudly if libdg.so has not been built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede the CDLL load, see above)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdg.so")

DG_OK = 0
DG_ERR_ARG = -1
DG_ERR_CAPACITY = -2
DG_ERR_HIP = -3
DG_ERR_UNSUPPORTED = -4
DG_DTYPE_F32 = 0
DG_DTYPE_BF16 = 1
DG_DTYPE_FP8_E4M3 = 2
(DG_MODEL_VIEW_EXPERT_GATEUP, DG_MODEL_VIEW_EXPERT_DOWN, DG_MODEL_VIEW_EXPERT_SCALES_GATEUP,
 DG_MODEL_VIEW_EXPERT_SCALES_DOWN, DG_MODEL_VIEW_HEAD_CODES, DG_MODEL_VIEW_HEAD_SCALES) = range(6)
(DG_VIEW_K_CACHE, DG_VIEW_V_CACHE, DG_VIEW_SELF_COND, DG_VIEW_PREV_ARGMAX, DG_VIEW_ROUTE,
 DG_VIEW_HIDDEN, DG_VIEW_ROUTER_LOGITS, DG_VIEW_ATTN_OUT, DG_VIEW_CTX_LENS, DG_VIEW_CANVAS_INDEX) = range(10)
DG_RUN_GRAPH, DG_RUN_EARLY_EXIT, DG_RUN_COMMIT_KV = 1, 2, 4
STAGES = ["embed", "norm", "qkv", "attn", "oproj", "router", "expert_up", "expert_down", "combine",
          "lm_head", "sampler", "selfcond", "commit"]

EXPORTS = [
    "dg_last_error", "dg_weight_count", "dg_model_create", "dg_model_destroy", "dg_model_view", "dg_state_bytes",
    "dg_state_init", "dg_state_destroy", "dg_state_ctx_len", "dg_state_canvas_index", "dg_state_view",
    "dg_init_canvas", "dg_encode_prompt", "dg_denoise_step", "dg_sample_logits", "dg_sample_logits_static",
    "dg_sample_commit",
    "dg_commit_canvas_to_kv", "dg_run_canvas", "dg_corrupt_forward_loss", "dg_profile_enable", "dg_profile_read",
]


class DgConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim", "n_experts", "ffn_hidden",
        "top_k", "vocab", "canvas_len", "dtype", "self_cond")] + [
        ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float), ("expert_dtype", ctypes.c_int32),
        ("head_dtype", ctypes.c_int32)]


class DgSamplerParams(ctypes.Structure):
    _fields_ = [("t_start", ctypes.c_float), ("t_end", ctypes.c_float),
                ("entropy_bound", ctypes.c_float), ("stop_tau", ctypes.c_float),
                ("max_steps", ctypes.c_int32), ("stop_mode", ctypes.c_int32), ("top_k", ctypes.c_int32)]


class DgError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"dg status {status}: {msg}")
        self.status = status


_lib = None
vp = ctypes.c_void_p
i32 = ctypes.c_int32


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m discrete_text_diffusion_dg_amd.build` (no CPU fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.dg_last_error.restype = ctypes.c_char_p
    lib.dg_weight_count.argtypes = [ctypes.POINTER(DgConfig)]
    lib.dg_weight_count.restype = i32
    lib.dg_model_create.argtypes = [ctypes.POINTER(DgConfig), ctypes.POINTER(vp), i32, ctypes.POINTER(vp)]
    lib.dg_model_destroy.argtypes = [vp]
    lib.dg_model_view.argtypes = [vp, i32, i32, ctypes.POINTER(vp), ctypes.POINTER(ctypes.c_size_t)]
    lib.dg_model_destroy.restype = None
    lib.dg_state_bytes.argtypes = [vp, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.dg_state_init.argtypes = [vp, vp, ctypes.c_size_t, i32, i32, ctypes.POINTER(vp)]
    lib.dg_state_destroy.argtypes = [vp]
    lib.dg_state_destroy.restype = None
    lib.dg_state_ctx_len.argtypes = [vp]
    lib.dg_state_ctx_len.restype = i32
    lib.dg_state_canvas_index.argtypes = [vp]
    lib.dg_state_canvas_index.restype = i32
    lib.dg_state_view.argtypes = [vp, i32, ctypes.POINTER(vp), ctypes.POINTER(ctypes.c_size_t)]
    lib.dg_init_canvas.argtypes = [vp, vp, vp, vp]
    lib.dg_encode_prompt.argtypes = [vp, vp, i32, vp]
    lib.dg_denoise_step.argtypes = [vp, vp, i32, ctypes.POINTER(DgSamplerParams), vp, vp, vp, vp, vp, vp,
                                    vp, vp]
    lib.dg_sample_logits.argtypes = [vp, vp, i32, ctypes.POINTER(DgSamplerParams), vp, vp, vp, vp, vp, vp, vp]
    lib.dg_sample_logits_static.argtypes = [vp, i32, i32, i32, i32, i32, ctypes.POINTER(DgSamplerParams), vp, vp,
                                            vp, vp, vp, vp]
    lib.dg_sample_commit.argtypes = [vp, vp, vp, vp, vp, i32, ctypes.POINTER(DgSamplerParams), vp, vp, vp,
                                     vp, vp]
    lib.dg_commit_canvas_to_kv.argtypes = [vp, vp, vp, vp]
    lib.dg_corrupt_forward_loss.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp]
    lib.dg_run_canvas.argtypes = [vp, vp, ctypes.POINTER(DgSamplerParams), vp, vp, vp, vp, vp, vp, vp, vp,
                                  i32, i32, ctypes.c_uint32, ctypes.POINTER(i32), vp]
    lib.dg_profile_enable.argtypes = [vp, ctypes.c_uint32]
    lib.dg_profile_read.argtypes = [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    for name in ("dg_model_create", "dg_model_view", "dg_state_bytes", "dg_state_init", "dg_state_view", "dg_init_canvas",
                 "dg_encode_prompt", "dg_denoise_step", "dg_sample_logits", "dg_sample_logits_static",
                 "dg_sample_commit",
                 "dg_commit_canvas_to_kv", "dg_run_canvas", "dg_corrupt_forward_loss", "dg_profile_enable", "dg_profile_read"):
        getattr(lib, name).restype = i32
    _check_single_hip_runtime()
    _lib = lib
    return lib


def _check_single_hip_runtime() -> None:
    try:
        with open("/proc/self/maps") as f:
            paths = {ln.split()[-1] for ln in f if "libamdhip64" in ln}
    except OSError:
        return
    real = {os.path.realpath(p) for p in paths}
    if len(real) > 1:
        raise ImportError(f"two HIP runtimes are mapped in this process: {sorted(real)}")


def check(status: int) -> None:
    if status != DG_OK:
        raise DgError(status, _lib.dg_last_error().decode())
