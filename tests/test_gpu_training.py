"""Training-side forward pass on the GPU against the oracle (oracle/training.py).

The corrupted canvas must match bit for bit (integer Philox draws); the
per-position cross-entropy of the clean tokens within the logits' tolerance
(2e-2 of the row's largest |logit| for bf16 models, 1e-4 for fp32), the pass
teacher-forced at its routing decisions like every parity case.
"""
import numpy as np
import pytest

import dg_inputs as di
from oracle import training as otr
from oracle.model import OracleModel

from _forcing import RouteForcing, gpu_routing
from _util import log, make_engine, micro, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _case(torch, mc, seed, B, P, rates, tag, gain_std=0.1):
    W = di.make_weights(mc, seed, gain_std=gain_std)
    n = mc.canvas_len
    eng = make_engine(mc, W, B, P + 2 * n)
    seeds = di.request_seeds(seed, B)
    eng.set_seeds(seeds)
    reqs = list(range(B))
    om = OracleModel(mc, W, B, P + 2 * n)
    if P:
        prompts = di.make_prompts(mc.vocab, B, P, seed)
        for p0 in range(0, P, n):
            ln = min(n, P - p0)
            eng.encode_prompt(torch.from_numpy(np.ascontiguousarray(prompts[:, p0:p0 + ln])))
            torch.cuda.synchronize()
            rf = RouteForcing(mc, *gpu_routing(mc, eng, B, ln, reqs), f"{tag} prompt {p0}")
            om.route_override = rf
            om.encode_prompt(prompts[:, p0:p0 + ln])
            om.route_override = None
            rf.finish()
        # the oracle's cache stands in for the GPU's, so that the pass itself is compared
        kc, vc = eng.kv_views()
        for l in range(mc.n_layers):
            kc[l, :, :, :P] = torch.from_numpy(om.k_cache[l][:, :, :P]).to(kc.dtype).cuda()
            vc[l, :, :, :P] = torch.from_numpy(om.v_cache[l][:, :, :P]).to(vc.dtype).cuda()
    clean = np.random.default_rng(seed).integers(0, mc.vocab, (B, n)).astype(np.int32)
    corrupted, ce, loss = eng.corrupt_forward_loss(torch.from_numpy(clean), rates)
    torch.cuda.synchronize()
    rf = RouteForcing(mc, *gpu_routing(mc, eng, B, n, reqs), f"{tag} pass")
    om.route_override = rf
    ref = otr.forward_loss(om, clean, rates, seeds, want_logits=True)
    om.route_override = None
    rf.finish()
    got_c = corrupted.cpu().numpy()
    assert np.array_equal(got_c, ref["corrupted"]), f"{tag}: corrupted canvas differs"
    tol = tol_for(mc)
    scale = np.abs(ref["logits"]).max(axis=2)
    e = np.abs(ce.cpu().numpy().astype(np.float64) - ref["ce"]) / scale
    el = np.abs(loss.cpu().numpy().astype(np.float64) - ref["loss"]) / scale.max(axis=1)
    frac = ref["replaced"].mean(axis=1)
    log(f"[{tag}] replaced {np.round(frac, 3).tolist()} at rates {list(rates)}; CE max |diff| / row scale "
        f"{e.max():.2e}; loss {np.round(ref['loss'], 4).tolist()} (rel {el.max():.2e})")
    assert (e <= tol).all() and (el <= tol).all(), f"{tag}: cross-entropy beyond tol"
    eng.close()


def test_corrupt_forward_loss_micro(torch_cuda):
    # rates 0, 0.4 and 1 in one batch, after a ragged prompt
    mc = micro(n_layers=2, vocab=4096)
    _case(torch_cuda, mc, 61, 3, 300, [0.0, 0.4, 1.0], "train-micro")


def test_corrupt_forward_loss_fp32_no_prompt(torch_cuda):
    mc = micro(n_layers=1, dtype="f32", vocab=2048)
    _case(torch_cuda, mc, 62, 2, 0, [0.25, 0.75], "train-f32")


def test_corrupt_forward_loss_small_workload(torch_cuda):
    wl = di.workload("small")
    _case(torch_cuda, wl.model, wl.seed, 1, wl.prompt_len, [0.5], "train-small", gain_std=0.0)


def test_corrupt_forward_loss_fp8_experts(torch_cuda):
    # the pass through the FP8 expert products (grouped: 256 canvas positions per request)
    mc = micro(n_layers=2, d_model=512, ffn_hidden=256, vocab=2048, expert_dtype="fp8")
    _case(torch_cuda, mc, 63, 2, 130, [0.3, 0.9], "train-fp8")


def test_corrupt_forward_loss_fp8_head(torch_cuda):
    # experts and LM head in FP8: the log-sum-exp and the clean token's logit from the E4M3 rows
    mc = micro(n_layers=2, d_model=512, ffn_hidden=256, vocab=4160, expert_dtype="fp8", head_dtype="fp8")
    _case(torch_cuda, mc, 64, 2, 130, [0.3, 0.9], "train-fp8-head")
