"""dg_sample_logits_static (the entry point that allocates nothing) against dg_sample_logits.

Two calls in a row, the second on a smaller input, each compared bit for bit
with the state-based entry point on the same logits; then the capacity check
of the fixed scratch.
"""
import ctypes

import numpy as np
import pytest

import dg_inputs as di

from _util import log, make_engine, micro

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _static_call(torch, eng, logits, rows, vocab, n, canvas_index, step, sp, seeds):
    from discrete_text_diffusion_dg_amd import _lib as L
    from discrete_text_diffusion_dg_amd.runtime import sampler_struct
    H = torch.full((rows,), float("nan"), device="cuda")
    y = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    am = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    mg = torch.full((rows,), float("nan"), device="cuda")
    prm = sampler_struct(sp)
    sd = np.ascontiguousarray(seeds, dtype=np.uint64)
    st = eng.lib.dg_sample_logits_static(logits.data_ptr(), rows, vocab, n, canvas_index, step, ctypes.byref(prm),
                                         sd.ctypes.data_as(ctypes.c_void_p), H.data_ptr(), y.data_ptr(),
                                         am.data_ptr(), mg.data_ptr(), torch.cuda.current_stream().cuda_stream)
    L.check(st)
    torch.cuda.synchronize()
    return H, y, am, mg


def _bits(t):
    import torch
    return t.contiguous().view(-1).view(torch.uint8)


def _case(torch, mc, B, seed, step, S, scale):
    W = di.make_weights(mc, seed)
    eng = make_engine(mc, W, B, 2 * mc.canvas_len)
    seeds = di.request_seeds(seed, B)
    eng.set_seeds(seeds)
    rng = np.random.default_rng(seed)
    n, V = mc.canvas_len, mc.vocab
    logits = torch.from_numpy((rng.standard_normal((B * n, V)) * scale).astype(np.float32)).cuda()
    sp = di.SamplerConfig(max_steps=S, entropy_bound=0.1)
    eng.sample_logits(step, sp, logits.view(B, n, V))
    torch.cuda.synchronize()
    ref = [eng.H.view(-1).clone(), eng.y.view(-1).clone(), eng.am.view(-1).clone(), eng.margin.view(-1).clone()]
    got = _static_call(torch, eng, logits, B * n, V, n, eng.canvas_index, step, sp, seeds)
    for name, a, b in zip(("H", "y", "argmax", "margin"), got, ref):
        assert torch.equal(_bits(a), _bits(b)), f"{name} differs from dg_sample_logits"
    log(f"[no-alloc] {B} x {n} rows, vocabulary {V}, step {step}: identical to dg_sample_logits")
    return eng


def test_static_sampler_matches_state_sampler(torch_cuda):
    torch = torch_cuda
    # first call: two requests, a ragged vocabulary (32.5 chunks of 128 ids)
    e1 = _case(torch, micro(n_layers=1, vocab=4160), 2, 41, 3, 12, 2.0)
    # second call, smaller: one request of a 100-position canvas, 2048 ids
    e2 = _case(torch, micro(n_layers=1, vocab=2048, canvas_len=100), 1, 42, 0, 4, 0.5)
    # beyond the fixed scratch: 512 rows x 2048 chunks of the largest vocabulary
    from discrete_text_diffusion_dg_amd.runtime import sampler_struct
    prm = sampler_struct(di.SamplerConfig(max_steps=4, entropy_bound=0.1))
    seeds = np.zeros(2, np.uint64)
    dummy = torch.zeros(4, device="cuda")
    st = e2.lib.dg_sample_logits_static(dummy.data_ptr(), 512, 262144, 256, 0, 0, ctypes.byref(prm),
                                        seeds.ctypes.data_as(ctypes.c_void_p), dummy.data_ptr(), dummy.data_ptr(),
                                        dummy.data_ptr(), dummy.data_ptr(), None)
    assert st == -2 and "scratch" in e2.lib.dg_last_error().decode()
    e1.close()
    e2.close()
