"""Engine: torch-owned device buffers around the libdg.so handles.

torch supplies device memory and the stream; every step of the denoise path
runs in the library's HIP kernels.  The generate loop follows the pages'
block-autoregressive sampling: encode the prompt, then per canvas draw random
tokens, run denoise + commit rounds until the request stops or the budget
ends, and append the finished canvas to the KV cache ([chooseai] multi-canvas
paragraph; [bohu] 一; [mlqm] 四).
"""
from __future__ import annotations

import ctypes
from typing import Dict, Optional, Sequence

import numpy as np
import torch

from . import _lib as L


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _copy_to_host(ptr: int, nbytes: int) -> np.ndarray:
    """Bytes of device memory the library owns, copied to the host (hipMemcpy of the HIP runtime torch loaded)."""
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    hip.hipMemcpy.restype = ctypes.c_int
    out = np.empty(nbytes, np.uint8)
    torch.cuda.synchronize()
    rc = hip.hipMemcpy(out.ctypes.data_as(ctypes.c_void_p), ctypes.c_void_p(ptr), nbytes, 2)   # device to host
    if rc != 0:
        raise RuntimeError(f"hipMemcpy failed with {rc}")
    return out


def config_struct(mc) -> L.DgConfig:
    return L.DgConfig(mc.n_layers, mc.d_model, mc.n_q_heads, mc.n_kv_heads, mc.head_dim, mc.n_experts,
                      mc.ffn_hidden, mc.top_k, mc.vocab, mc.canvas_len,
                      L.DG_DTYPE_BF16 if mc.dtype == "bf16" else L.DG_DTYPE_F32,
                      1 if mc.self_cond else 0, mc.rope_theta, mc.rms_eps,
                      L.DG_DTYPE_FP8_E4M3 if getattr(mc, "expert_dtype", "") == "fp8" else 0,
                      L.DG_DTYPE_FP8_E4M3 if getattr(mc, "head_dtype", "") == "fp8" else 0)


def sampler_struct(sp) -> L.DgSamplerParams:
    return L.DgSamplerParams(sp.t_start, sp.t_end, sp.entropy_bound, sp.stop_tau, sp.max_steps,
                             sp.stop_mode, getattr(sp, "top_k", 0))


def upload_weights(weights, names: Sequence[str], device) -> Dict[str, torch.Tensor]:
    """Host arrays (float32, or uint16 bfloat16 bits) -> device tensors, same bytes."""
    out = {}
    for n in names:
        a = np.ascontiguousarray(weights.get(n))
        if a.dtype == np.uint16:
            t = torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
        else:
            t = torch.from_numpy(a).to(device)
        out[n] = t
    return out


class Engine:
    """One model + one state (batch of requests sharing a context length)."""

    def __init__(self, model_cfg, device_weights: Dict[str, torch.Tensor], names: Sequence[str],
                 batch: int, max_ctx: int, device="cuda"):
        self.lib = L.load()
        self.cfg = model_cfg
        self.device = torch.device(device)
        self.B, self.n, self.max_ctx = batch, model_cfg.canvas_len, max_ctx
        self.weights = device_weights                          # keep alive
        self._cfg = config_struct(model_cfg)
        ptrs = (ctypes.c_void_p * len(names))(*[device_weights[n].data_ptr() for n in names])
        self._model = ctypes.c_void_p()
        L.check(self.lib.dg_model_create(ctypes.byref(self._cfg), ptrs, len(names), ctypes.byref(self._model)))
        nbytes = ctypes.c_size_t()
        L.check(self.lib.dg_state_bytes(self._model, batch, max_ctx, ctypes.byref(nbytes)))
        self.state_buf = torch.empty(nbytes.value, dtype=torch.uint8, device=self.device)
        self._state = ctypes.c_void_p()
        L.check(self.lib.dg_state_init(self._model, self.state_buf.data_ptr(), nbytes.value, batch, max_ctx,
                                       ctypes.byref(self._state)))
        B, n, dev = batch, self.n, self.device
        self.canvas = torch.zeros(B, n, dtype=torch.int32, device=dev)
        self.H = torch.zeros(B, n, dtype=torch.float32, device=dev)
        self.y = torch.zeros(B, n, dtype=torch.int32, device=dev)
        self.am = torch.zeros(B, n, dtype=torch.int32, device=dev)
        self.margin = torch.zeros(B, n, dtype=torch.float32, device=dev)
        self.mask = torch.zeros(B, n, dtype=torch.uint8, device=dev)
        self.n_committed = torch.zeros(B, dtype=torch.int32, device=dev)
        self.done = torch.zeros(B, dtype=torch.uint8, device=dev)
        self.seeds = np.zeros(B, np.uint64)

    # ------------------------------------------------------------ lifetime
    def close(self) -> None:
        if getattr(self, "_state", None):
            self.lib.dg_state_destroy(self._state)
            self._state = None
        if getattr(self, "_model", None):
            self.lib.dg_model_destroy(self._model)
            self._model = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------ helpers
    def _stream(self) -> int:
        return torch.cuda.current_stream(self.device).cuda_stream

    def set_seeds(self, seeds: np.ndarray) -> None:
        self.seeds = np.ascontiguousarray(seeds, dtype=np.uint64)
        assert self.seeds.size == self.B

    def _seed_ptr(self):
        return self.seeds.ctypes.data_as(ctypes.c_void_p)

    @property
    def ctx_len(self) -> int:
        return self.lib.dg_state_ctx_len(self._state)

    @property
    def canvas_index(self) -> int:
        return self.lib.dg_state_canvas_index(self._state)

    def view(self, which: int, dtype: torch.dtype, shape) -> torch.Tensor:
        """A torch tensor aliasing part of the state buffer (K/V cache, self-cond, prev argmax)."""
        p = ctypes.c_void_p()
        nb = ctypes.c_size_t()
        L.check(self.lib.dg_state_view(self._state, which, ctypes.byref(p), ctypes.byref(nb)))
        off = p.value - self.state_buf.data_ptr()
        el = torch.tensor([], dtype=dtype).element_size()
        return self.state_buf[off:off + nb.value].view(dtype).view(*shape)

    def kv_views(self):
        """K and V caches as [L][B][Hkv][max_ctx][hd] tensors aliasing the state.

        K is stored row-major per key, V transposed ([hd][ctx] per kv head), each
        with the context capacity rounded up to 64; the V view is a transposed
        (strided) view, so writes through it land in the library's layout."""
        c = self.cfg
        dt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
        ctx_pad = (self.max_ctx + 63) // 64 * 64
        k = self.view(L.DG_VIEW_K_CACHE, dt, (c.n_layers, self.B, c.n_kv_heads, ctx_pad, c.head_dim))
        v = self.view(L.DG_VIEW_V_CACHE, dt, (c.n_layers, self.B, c.n_kv_heads, c.head_dim, ctx_pad))
        return k[:, :, :, :self.max_ctx, :], v.transpose(-1, -2)[:, :, :, :self.max_ctx, :]

    def self_cond_view(self) -> torch.Tensor:
        return self.view(L.DG_VIEW_SELF_COND, torch.float32, (self.B, self.n, self.cfg.d_model))

    def hidden_view(self, rows: int) -> torch.Tensor:
        t = self.view(L.DG_VIEW_HIDDEN, torch.float32, (self.B * self.n, self.cfg.d_model))
        return t[:rows]

    def router_logits_view(self, rows: int) -> torch.Tensor:
        c = self.cfg
        t = self.view(L.DG_VIEW_ROUTER_LOGITS, torch.float32, (c.n_layers, self.B * self.n, c.n_experts))
        return t[:, :rows]

    def attn_out_view(self, rows: int) -> torch.Tensor:
        c = self.cfg
        dt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
        t = self.view(L.DG_VIEW_ATTN_OUT, dt, (self.B * self.n, c.n_q_heads * c.head_dim))
        return t[:rows]

    def route_view(self, rows: int) -> torch.Tensor:
        c = self.cfg
        t = self.view(L.DG_VIEW_ROUTE, torch.int32, (c.n_layers, self.B * self.n, c.top_k))
        return t[:, :rows]

    def model_view(self, which: int, layer: int) -> np.ndarray:
        """Host copy (raw bytes) of one of the model's derived weight copies (dg_model_view)."""
        p = ctypes.c_void_p()
        nb = ctypes.c_size_t()
        L.check(self.lib.dg_model_view(self._model, which, layer, ctypes.byref(p), ctypes.byref(nb)))
        return _copy_to_host(p.value, nb.value)

    # ------------------------------------------------------------ stage timing
    def profile(self, stages) -> None:
        mask = 0
        for st in stages:
            mask |= 1 << L.STAGES.index(st)
        L.check(self.lib.dg_profile_enable(self._state, mask))

    def profile_read(self) -> Dict[str, tuple]:
        ms = (ctypes.c_double * len(L.STAGES))()
        n = (ctypes.c_int64 * len(L.STAGES))()
        L.check(self.lib.dg_profile_read(self._state, ms, n))
        return {st: (ms[i], n[i]) for i, st in enumerate(L.STAGES) if n[i]}

    # ------------------------------------------------------------ the calls
    def init_canvas(self) -> torch.Tensor:
        L.check(self.lib.dg_init_canvas(self._state, self.canvas.data_ptr(), self._seed_ptr(), self._stream()))
        return self.canvas

    def encode_prompt(self, ids: torch.Tensor) -> None:
        ids = ids.to(device=self.device, dtype=torch.int32).contiguous()
        assert ids.shape[0] == self.B
        L.check(self.lib.dg_encode_prompt(self._state, ids.data_ptr(), ids.shape[1], self._stream()))

    def denoise_step(self, step: int, sp, active: Optional[torch.Tensor] = None,
                     logits: Optional[torch.Tensor] = None, canvas: Optional[torch.Tensor] = None) -> None:
        prm = sampler_struct(sp)
        cv = self.canvas if canvas is None else canvas
        L.check(self.lib.dg_denoise_step(self._state, cv.data_ptr(), step, ctypes.byref(prm), self._seed_ptr(),
                                         _ptr(active), self.H.data_ptr(), self.y.data_ptr(), self.am.data_ptr(),
                                         self.margin.data_ptr(), _ptr(logits), self._stream()))

    def sample_logits(self, step: int, sp, logits: torch.Tensor, active: Optional[torch.Tensor] = None) -> None:
        prm = sampler_struct(sp)
        logits = logits.to(device=self.device, dtype=torch.float32).contiguous()
        L.check(self.lib.dg_sample_logits(self._state, logits.data_ptr(), step, ctypes.byref(prm), self._seed_ptr(),
                                          _ptr(active), self.H.data_ptr(), self.y.data_ptr(), self.am.data_ptr(),
                                          self.margin.data_ptr(), self._stream()))

    def sample_commit(self, step: int, sp, H: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                      am: Optional[torch.Tensor] = None) -> None:
        prm = sampler_struct(sp)
        H = self.H if H is None else H
        y = self.y if y is None else y
        am = self.am if am is None else am
        L.check(self.lib.dg_sample_commit(self._state, H.data_ptr(), y.data_ptr(), am.data_ptr(),
                                          self.canvas.data_ptr(), step, ctypes.byref(prm), self._seed_ptr(),
                                          self.mask.data_ptr(), self.n_committed.data_ptr(),
                                          self.done.data_ptr(), self._stream()))

    def commit_canvas_to_kv(self, canvas: Optional[torch.Tensor] = None,
                            which: Optional[torch.Tensor] = None) -> None:
        """Append the canvas of the requests `which` selects (uint8 [B], None = all) to the KV cache."""
        cv = self.canvas if canvas is None else canvas
        L.check(self.lib.dg_commit_canvas_to_kv(self._state, cv.data_ptr(), _ptr(which), self._stream()))

    def corrupt_forward_loss(self, clean: torch.Tensor, rates) -> tuple:
        """Training-side forward pass (dg_corrupt_forward_loss): (corrupted, ce [B, n], loss [B])."""
        clean = clean.to(device=self.device, dtype=torch.int32).contiguous()
        r = np.ascontiguousarray(rates, dtype=np.float32)
        assert clean.shape == (self.B, self.n) and r.size == self.B
        corrupted = torch.empty_like(clean)
        ce = torch.empty(self.B, self.n, dtype=torch.float32, device=self.device)
        loss = torch.empty(self.B, dtype=torch.float32, device=self.device)
        L.check(self.lib.dg_corrupt_forward_loss(self._state, clean.data_ptr(), r.ctypes.data_as(ctypes.c_void_p),
                                                 self._seed_ptr(), corrupted.data_ptr(), ce.data_ptr(),
                                                 loss.data_ptr(), self._stream()))
        return corrupted, ce, loss

    def ctx_lens(self) -> torch.Tensor:
        """Per-request context lengths (device view)."""
        return self.view(L.DG_VIEW_CTX_LENS, torch.int32, (self.B,))

    def canvas_indices(self) -> torch.Tensor:
        """Per-request canvas indices (device view)."""
        return self.view(L.DG_VIEW_CANVAS_INDEX, torch.int32, (self.B,))

    def run_canvas_device(self, sp, first_step: int = 0, n_steps: Optional[int] = None, graph: bool = True,
                          early_exit: bool = False, commit_kv: bool = False):
        """Steps first_step .. first_step + n_steps - 1 of the canvas, driven by the library
        (dg_run_canvas): no host read of device memory.  Returns (steps issued, canvas finished)."""
        prm = sampler_struct(sp)
        if n_steps is None:
            n_steps = sp.max_steps - first_step
        flags = ((L.DG_RUN_GRAPH if graph else 0) | (L.DG_RUN_EARLY_EXIT if early_exit else 0)
                 | (L.DG_RUN_COMMIT_KV if commit_kv else 0))
        res = (ctypes.c_int32 * 2)()
        L.check(self.lib.dg_run_canvas(self._state, self.canvas.data_ptr(), ctypes.byref(prm), self._seed_ptr(),
                                       self.H.data_ptr(), self.y.data_ptr(), self.am.data_ptr(),
                                       self.margin.data_ptr(), self.mask.data_ptr(), self.n_committed.data_ptr(),
                                       self.done.data_ptr(), first_step, n_steps, flags, res, self._stream()))
        return res[0], bool(res[1])

    # ------------------------------------------------------------ loop
    def run_canvas(self, sp, graph: bool = True, commit_kv: bool = False) -> int:
        """Denoise one canvas for all requests on the device (dg_run_canvas).

        The done flags gate every step on the device, the step index and
        temperature stay there, and with a stop rule the library ends the
        canvas once every request is done, learning it from a progress record
        in mapped host memory: no host read of device memory, no torch
        kernel.  Returns the number of steps issued."""
        return self.run_canvas_device(sp, graph=graph, early_exit=sp.stop_mode != 0, commit_kv=commit_kv)[0]
