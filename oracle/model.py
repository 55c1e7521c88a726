"""Oracle model: prompt encode, one denoise step, canvas commit to the KV cache.

Pages followed:
  * [mlqm] 二: the model is the Gemma 4 mixture-of-experts transformer, 128
    expert groups of which 8 serve each token; the prompt is encoded with causal
    attention, the 256-token answer canvas with bidirectional attention; a
    self-conditioning signal (the previous round's prediction) enters each round.
  * [chooseai] architecture paragraph: an autoregressive encoder builds and
    caches the prompt context; the diffusion decoder attends bidirectionally on
    the canvas.  [bohu] 一: a finished canvas enters the KV cache, then the next
    canvas starts (block-autoregressive multi-canvas sampling).
  * [mlqm] 一: all 256 canvas positions are predicted at once in each round.

Readings where the pages are silent (no layer formula is printed):
  * pre-norm block: h += Attn(RMSNorm(h)); h += MoE(RMSNorm(h)); final RMSNorm;
    LM head tied to the embedding (logits = h E^T); no biases, no Gemma extras
    (no embedding scale, QK-norm, soft-cap, sliding window or shared expert);
  * router: logits r = m W_r^T (fp32), top-k by value with ties to the lower
    expert id, weights softmax over the k selected logits, no capacity limit;
  * self-conditioning: s = softmax(z) E (the previous step's tempered
    distribution times the embedding), added as s W_sc^T; s = 0 at step 0;
  * FP8 serving (chooseai.io speed paragraph, bohuyeshan.top 一: the model is
    served in FP8): experts, and optionally the LM head's rows of E, use the
    E4M3 codes of each output channel times its scale (oracle/fp8.py); the
    embedding lookup and the self-conditioning product keep the stored E;
  * canvas queries sit at positions N..N+255 after an N-token context and see
    every cached key and every canvas key; the canvas's own K/V are not kept;
    committing a canvas re-encodes it causally and appends its K/V.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional

import numpy as np

from . import fp8
from . import numerics as nm
from . import sampler as smp


class OracleModel:
    """Plain fp64 model over a batch of independent requests sharing one context length."""

    def __init__(self, cfg, weights, batch: int, max_ctx: int, cache_f64: Optional[bool] = None):
        self.cfg = cfg
        self.w = weights
        self.B = batch
        self.max_ctx = max_ctx
        self.rnd = nm.bf16_round if cfg.dtype == "bf16" else (lambda a: np.asarray(a, np.float64))
        if cache_f64 is None:
            cache_f64 = cfg.n_params() < 1.2e9
        self._cache_f64 = cache_f64
        self._f64: Dict[str, np.ndarray] = {}
        # without the fp64 cache (large models), the stored tensors of the layer
        # in use are held so that a weight set which regenerates on every access
        # is asked for each tensor once per pass
        self._raw: Dict[str, np.ndarray] = {}
        self._raw_layer = None
        self._fp8: Dict[tuple, np.ndarray] = {}      # dequantised FP8 experts of the layer in use
        self._fp8_layer = None
        self.on_layer = None      # optional callback(layer) after each layer (progress of long runs)
        # optional callback(request, layer, router logits r, top-k ids) -> ids: lets a
        # test impose another expert choice on rows whose own top-k is a near tie
        # (the callback decides where; the weights stay the softmax of these logits)
        self.route_override = None
        # optional callback(request, logits [n, V]) -> per-row id sets (None for a row to
        # keep its own): the same for the top-k truncated sampler's vocabulary selection
        self.topk_override = None
        L, Hkv, hd = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim
        self.k_cache = [np.zeros((batch, Hkv, max_ctx, hd)) for _ in range(L)]
        self.v_cache = [np.zeros((batch, Hkv, max_ctx, hd)) for _ in range(L)]
        self.ctx = 0
        self.canvas_index = 0
        self.s = np.zeros((batch, cfg.canvas_len, cfg.d_model))

    # ------------------------------------------------------------ weights
    def _stored(self, name: str) -> np.ndarray:
        layer = name.split(".", 1)[0] if name.startswith("l") and "." in name else None
        if layer is not None and layer != self._raw_layer:
            self._raw = {}
            self._raw_layer = layer
        if name not in self._raw:
            self._raw[name] = self.w.get(name)
        return self._raw[name]

    def W(self, name: str) -> np.ndarray:
        if name in self._f64:
            return self._f64[name]
        if self._cache_f64 or name == "emb":
            a = nm.upcast(self.w.get(name))
            self._f64[name] = a
            return a
        return nm.upcast(self._stored(name))

    def expert(self, layer: int, kind: str, e: int) -> np.ndarray:
        name = f"l{layer}.{kind}"
        if getattr(self.cfg, "expert_dtype", "") == "fp8":
            # FP8 experts: the E4M3 codes of each output channel times its scale
            # (oracle/fp8.py), from the stored bf16 weights
            key = (name, int(e))
            if key not in self._fp8:
                if self._fp8_layer != layer:
                    self._fp8 = {}
                    self._fp8_layer = layer
                w = nm.upcast(self._stored(name)[e] if not self._cache_f64 else self.w.get(name)[e])
                q, s = fp8.quantize_rows(w.astype(np.float32))
                self._fp8[key] = fp8.dequantize_rows(q, s)
            return self._fp8[key]
        if self._cache_f64:
            return self.W(name)[e]
        return nm.upcast(self._stored(name)[e])

    def head_weight(self) -> np.ndarray:
        """Rows of the LM head: E, or (FP8 head) each row's E4M3 codes times its scale."""
        if getattr(self.cfg, "head_dtype", "") != "fp8":
            return self.W("emb")
        if "emb.fp8" not in self._f64:
            E = self.W("emb")
            out = np.empty_like(E)
            # row by row is the definition; blocks of rows only bound the temporaries
            for r0 in range(0, E.shape[0], 8192):
                q, s = fp8.quantize_rows(E[r0:r0 + 8192].astype(np.float32))
                out[r0:r0 + 8192] = fp8.dequantize_rows(q, s)
            self._f64["emb.fp8"] = out
        return self._f64["emb.fp8"]

    # ------------------------------------------------------------ blocks
    def _moe(self, l: int, xm: np.ndarray, trace: Optional[dict], b: int = 0) -> np.ndarray:
        cfg = self.cfg
        n, k = xm.shape[0], cfg.top_k
        r = (xm @ self.W(f"l{l}.w_router").T).astype(np.float32)          # decision in fp32
        order = np.argsort(-r, axis=1, kind="stable")                    # ties -> lower id
        idx = order[:, :k]
        if self.route_override is not None:
            idx = np.asarray(self.route_override(b, l, r, idx))
        rsel = np.take_along_axis(r, idx, axis=1).astype(np.float64)
        wts = nm.softmax(rsel, axis=1)
        contrib = np.zeros((n, k, cfg.d_model))
        experts = np.unique(idx)
        kinds = ("w_gate", "w_up", "w_down")
        if self._cache_f64:
            mats = {(kind, e): self.expert(l, kind, e) for kind in kinds for e in experts}
        else:
            # widen the selected experts' stored matrices to fp64 on several threads
            # (plain element conversions; the products below stay in order)
            for kind in kinds:
                self._stored(f"l{l}.{kind}")
            keys = [(kind, e) for kind in kinds for e in experts]
            with ThreadPoolExecutor(min(len(keys), os.cpu_count() or 1)) as ex:
                mats = dict(zip(keys, ex.map(lambda ke: self.expert(l, ke[0], ke[1]), keys)))
        for e in experts:
            rows, slots = np.nonzero(idx == e)
            m = xm[rows]
            g = m @ mats[("w_gate", e)].T
            u = m @ mats[("w_up", e)].T
            a = self.rnd(nm.silu(g) * u)
            contrib[rows, slots] = a @ mats[("w_down", e)].T
        del mats
        y = np.zeros((n, cfg.d_model))
        for j in range(k):                                               # fixed slot order
            y += wts[:, j:j + 1] * contrib[:, j]
        if trace is not None:
            trace.setdefault("route_idx", []).append(idx.astype(np.int32))
            trace.setdefault("route_w", []).append(wts)
            trace.setdefault("router_logits", []).append(r)
        return y

    def _layer(self, l: int, b: int, h: np.ndarray, pos: np.ndarray, causal: bool,
               store_kv: bool, trace: Optional[dict]) -> np.ndarray:
        cfg = self.cfg
        n = h.shape[0]
        Hq, Hkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
        N = int(pos[0])
        xn = self.rnd(nm.rmsnorm(h, self.W(f"l{l}.attn_norm"), cfg.rms_eps))
        q = self.rnd(nm.rope((xn @ self.W(f"l{l}.wq").T).reshape(n, Hq, hd), pos, cfg.rope_theta))
        k = self.rnd(nm.rope((xn @ self.W(f"l{l}.wk").T).reshape(n, Hkv, hd), pos, cfg.rope_theta))
        v = self.rnd((xn @ self.W(f"l{l}.wv").T).reshape(n, Hkv, hd))
        K = np.concatenate([self.k_cache[l][b, :, :N].transpose(1, 0, 2), k], axis=0)
        V = np.concatenate([self.v_cache[l][b, :, :N].transpose(1, 0, 2), v], axis=0)
        o = nm.attention(q, K, V, pos, np.arange(N + n), causal)
        if store_kv:
            self.k_cache[l][b, :, N:N + n] = k.transpose(1, 0, 2)
            self.v_cache[l][b, :, N:N + n] = v.transpose(1, 0, 2)
        h = h + self.rnd(o.reshape(n, Hq * hd)) @ self.W(f"l{l}.wo").T
        if trace is not None:
            trace.setdefault("q", []).append(q)
            trace.setdefault("k", []).append(k)
            trace.setdefault("v", []).append(v)
            trace.setdefault("attn", []).append(o)
        xm = self.rnd(nm.rmsnorm(h, self.W(f"l{l}.ffn_norm"), self.cfg.rms_eps))
        return h + self._moe(l, xm, trace, b)

    def _stack(self, b: int, ids: np.ndarray, pos: np.ndarray, causal: bool, store_kv: bool,
               h0_extra: Optional[np.ndarray], trace: Optional[dict]) -> np.ndarray:
        h = self.W("emb")[np.asarray(ids)].copy()
        if h0_extra is not None:
            h = h + h0_extra
        if trace is not None:
            trace["h0"] = h.copy()
        for l in range(self.cfg.n_layers):
            h = self._layer(l, b, h, pos, causal, store_kv, trace)
            if self.on_layer is not None:
                self.on_layer(l)
        return h

    # ------------------------------------------------------------ the four calls
    def encode_prompt(self, ids: np.ndarray, traces: Optional[List[dict]] = None) -> None:
        """Causal encode of ids [B, P] at positions ctx..ctx+P-1; K/V appended.

        traces: optional list of B dicts that receive per-layer intermediates."""
        ids = np.asarray(ids)
        P = ids.shape[1]
        assert self.ctx + P <= self.max_ctx
        pos = self.ctx + np.arange(P)
        for b in range(self.B):
            if P:
                self._stack(b, ids[b], pos, True, True, None, traces[b] if traces else None)
        self.ctx += P

    def commit_canvas_to_kv(self, canvas: np.ndarray, traces: Optional[List[dict]] = None) -> None:
        """The finished canvas is encoded causally and appended ([bohu] 一)."""
        self.encode_prompt(canvas, traces)
        self.canvas_index += 1

    def denoise_step(self, canvas: np.ndarray, step: int, sp, seeds: np.ndarray,
                     active: Optional[np.ndarray] = None, want_logits: bool = False,
                     trace_requests: Optional[List[int]] = None) -> Dict[str, np.ndarray]:
        """One denoising round over the [B, 256] canvas.

        sp: dg_inputs.SamplerConfig.  seeds: per-request 64-bit Philox seeds.
        Returns H, y, am, margin (each [B, 256]), optionally logits [B, 256, V],
        and per-request traces; updates the self-conditioning state.
        """
        cfg = self.cfg
        n, V = cfg.canvas_len, cfg.vocab
        T = smp.temperature(step, sp.max_steps, sp.t_start, sp.t_end)
        inv_t = smp.inv_temperature(T)
        canvas = np.asarray(canvas)
        out = {"H": np.zeros((self.B, n), np.float32), "y": np.zeros((self.B, n), np.int32),
               "am": np.zeros((self.B, n), np.int32), "margin": np.zeros((self.B, n), np.float32),
               "T": T, "inv_t": inv_t, "traces": {}}
        if want_logits:
            out["logits"] = np.zeros((self.B, n, V), np.float32)
        pos = self.ctx + np.arange(n)
        s_next = self.s.copy()
        for b in range(self.B):
            if active is not None and not active[b]:
                continue
            trace = {} if (trace_requests is not None and b in trace_requests) else None
            extra = None
            if cfg.self_cond and step > 0:
                extra = self.rnd(self.s[b]) @ self.W("w_sc").T
            h = self._stack(b, canvas[b], pos, False, False, extra, trace)
            xf = self.rnd(nm.rmsnorm(h, self.W("final_norm"), cfg.rms_eps))
            logits = (xf @ self.head_weight().T).astype(np.float32)
            top_k = getattr(sp, "top_k", 0)
            if top_k:
                # the distribution truncated to each position's top_k logits ([mlqm] 九)
                forced = self.topk_override(b, logits) if self.topk_override is not None else None
                st = smp.head_stats_topk(logits, inv_t, top_k, int(seeds[b]), self.canvas_index, step,
                                         np.arange(n), want_probs=cfg.self_cond, forced_ids=forced)
            else:
                st = smp.head_stats(logits, inv_t, int(seeds[b]), self.canvas_index, step,
                                    np.arange(n), want_probs=cfg.self_cond)
            for key in ("H", "y", "am", "margin"):
                out[key][b] = st[key]
            if want_logits:
                out["logits"][b] = logits
            if cfg.self_cond:
                E = self.W("emb")
                if top_k:
                    Ek = E[st["ids"]]                                   # [n, k, d]
                    s_next[b] = np.einsum("nk,nkd->nd", st["p"], Ek)
                else:
                    s_next[b] = st["p"] @ E
                if want_logits:
                    # spread of that sum under independent relative perturbations of its terms (tests):
                    # sqrt(sum_v p_v^2 E_v^2)
                    rms = (np.sqrt(np.einsum("nk,nkd->nd", st["p"] ** 2, Ek * Ek)) if top_k
                           else np.sqrt((st["p"] ** 2) @ (E * E)))
                    out.setdefault("s_rms", np.zeros((self.B, n, cfg.d_model)))[b] = rms
            if trace is not None and not top_k:
                trace["m"], trace["logS"] = st["m"], st["logS"]
            if trace is not None:
                out["traces"][b] = trace
        self.s = s_next
        return out
