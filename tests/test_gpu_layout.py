"""One expert weight layout: after dg_model_create a bf16 model reads only its
fragment-packed expert copy.  A denoising step run again after the caller's
w_gate / w_up / w_down tensors are zeroed gives the same outputs bit for bit,
through the weight-streaming products (few routed rows) and the grouped
128 x 128 products (many)."""
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


@pytest.mark.parametrize("batch,path", [(1, "streaming"), (4, "grouped")])
def test_expert_products_read_only_the_packed_copy(torch_cuda, batch, path):
    torch = torch_cuda
    mc = micro(n_layers=2, vocab=2048)          # 8 experts top-2: 256 rows stream, 1024 rows take the grouped tiles
    W = di.make_weights(mc, 41, gain_std=0.1)
    eng = make_engine(mc, W, batch, 512)
    eng.set_seeds(di.request_seeds(41, batch))
    prompts = di.make_prompts(mc.vocab, batch, 100, 41)
    eng.encode_prompt(torch.from_numpy(prompts).cuda())
    eng.init_canvas()
    sp = di.SamplerConfig(max_steps=12, entropy_bound=0.5)
    eng.denoise_step(0, sp)                     # a self-conditioning vector for step 1
    s0 = eng.self_cond_view().clone()

    def step():
        eng.self_cond_view().copy_(s0)
        logits = torch.empty(batch, mc.canvas_len, mc.vocab, dtype=torch.float32, device="cuda")
        eng.denoise_step(1, sp, logits=logits)
        torch.cuda.synchronize()
        return [logits.clone(), eng.H.clone(), eng.y.clone(), eng.am.clone(), eng.margin.clone(),
                eng.self_cond_view().clone()]

    a = step()
    zeroed = 0
    for name, t in eng.weights.items():
        if name.split(".")[-1] in ("w_gate", "w_up", "w_down"):
            t.zero_()
            zeroed += 1
    torch.cuda.synchronize()
    b = step()
    assert zeroed == 3 * mc.n_layers
    for nm, x, y in zip(["logits", "H", "y", "argmax", "margin", "self-cond"], a, b):
        assert torch.equal(x.view(-1).view(torch.uint8), y.view(-1).view(torch.uint8)), f"{path}: {nm} changed"
    log(f"[layout {path}] {zeroed} caller expert tensors zeroed after create: step outputs bit-identical")
    eng.close()
