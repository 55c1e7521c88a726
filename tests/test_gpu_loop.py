"""The device-driven canvas loop, per-request stop and per-request context, on the GPU.

- dg_run_canvas (with and without the captured step graph) gives bit for bit
  the outputs, state and cache of the explicit dg_denoise_step /
  dg_sample_commit / dg_commit_canvas_to_kv sequence ([mlqm] 五: the host-device
  exchange made asynchronous must not change what a step computes).
- Requests stop independently ([mlqm] 四): a done request takes no part in
  later steps -- its canvas, self-conditioning vector and cached K/V stay as
  they were -- while the others still match the oracle.
- dg_commit_canvas_to_kv with d_which commits only the selected requests;
  each request then runs with its own context length and canvas index, and
  matches an oracle holding that request alone.
"""
import numpy as np
import pytest

import dg_inputs as di
from oracle import sampler as osmp
from oracle.model import OracleModel

from _forcing import RouteForcing, gpu_routing
from _util import log, make_engine, micro, rel_err_rows, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _bits(t):
    return t.contiguous().view(-1).view(__import__("torch").uint8)


def _snapshot(eng):
    kc, vc = eng.kv_views()
    return {"canvas": eng.canvas.clone(), "H": eng.H.clone(), "y": eng.y.clone(), "am": eng.am.clone(),
            "margin": eng.margin.clone(), "mask": eng.mask.clone(), "n_committed": eng.n_committed.clone(),
            "done": eng.done.clone(), "s": eng.self_cond_view().clone(), "k": kc.clone(), "v": vc.clone(),
            "ctx": eng.ctx_lens().clone(), "cidx": eng.canvas_indices().clone()}


def _assert_same(a, b, tag):
    import torch
    for k in a:
        assert torch.equal(_bits(a[k]), _bits(b[k])), f"{tag}: {k} differs"


@pytest.mark.parametrize("graph", [False, True])
def test_device_loop_matches_explicit_calls(torch_cuda, graph):
    torch = torch_cuda
    mc = micro(n_layers=2, vocab=4096)
    W = di.make_weights(mc, 31, gain_std=0.1)
    B, P, S = 2, 300, 5
    prompts = torch.from_numpy(di.make_prompts(mc.vocab, B, P, 31))
    seeds = di.request_seeds(31, B)
    sp = di.SamplerConfig(max_steps=S, entropy_bound=0.5, stop_mode=0)
    # explicit calls
    ea = make_engine(mc, W, B, P + 4 * mc.canvas_len)
    ea.set_seeds(seeds)
    ea.encode_prompt(prompts)
    for c in range(2):
        ea.init_canvas()
        ea.done.zero_()
        for t in range(S):
            ea.denoise_step(t, sp)
            ea.sample_commit(t, sp)
        ea.commit_canvas_to_kv()
    torch.cuda.synchronize()
    ref = _snapshot(ea)
    ea.close()
    # the device loop: two canvases, the first in two calls (steps 0..1, then 2..4)
    eb = make_engine(mc, W, B, P + 4 * mc.canvas_len)
    eb.set_seeds(seeds)
    eb.encode_prompt(prompts)
    n1, f1 = eb.run_canvas_device(sp, first_step=0, n_steps=2, graph=graph, commit_kv=True)
    n2, f2 = eb.run_canvas_device(sp, first_step=2, n_steps=3, graph=graph, commit_kv=True)
    n3, f3 = eb.run_canvas_device(sp, graph=graph, commit_kv=True)
    torch.cuda.synchronize()
    assert (n1, f1, n2, f2, n3, f3) == (2, False, 3, True, S, True)
    _assert_same(ref, _snapshot(eb), f"device loop (graph={graph})")
    assert eb.ctx_len == P + 2 * mc.canvas_len and eb.canvas_index == 2
    log(f"[device loop graph={graph}] two canvases of {S} steps and their commits bit-identical to the explicit calls")
    eb.close()


@pytest.mark.parametrize("variant", ["topk", "fp8", "fp8-topk", "fp8-head", "fp8-head-topk", "streamed-router"])
def test_device_loop_variants_match_explicit_calls(torch_cuda, variant):
    # the captured step with the top-k sampler and / or FP8 experts (and the FP8
    # LM head), or with the streamed norm + router (d 1024, 24 experts): one
    # canvas through the graph, bit-identical to the explicit calls
    torch = torch_cuda
    fp8 = variant.startswith("fp8")
    if variant == "streamed-router":
        mc = micro(n_layers=2, vocab=4096, d_model=1024, n_experts=24, top_k=3, ffn_hidden=128)
    else:
        mc = micro(n_layers=2, vocab=4096, d_model=512, ffn_hidden=256, expert_dtype="fp8" if fp8 else "",
                   head_dtype="fp8" if variant.startswith("fp8-head") else "")
    W = di.make_weights(mc, 33, gain_std=0.1)
    B, P, S = 2, 200, 4
    prompts = torch.from_numpy(di.make_prompts(mc.vocab, B, P, 33))
    seeds = di.request_seeds(33, B)
    sp = di.SamplerConfig(max_steps=S, entropy_bound=0.5, stop_mode=0, top_k=8 if "topk" in variant else 0)
    ea = make_engine(mc, W, B, P + 2 * mc.canvas_len)
    ea.set_seeds(seeds)
    ea.encode_prompt(prompts)
    ea.init_canvas()
    for t in range(S):
        ea.denoise_step(t, sp)
        ea.sample_commit(t, sp)
    ea.commit_canvas_to_kv()
    torch.cuda.synchronize()
    ref = _snapshot(ea)
    ea.close()
    eb = make_engine(mc, W, B, P + 2 * mc.canvas_len)
    eb.set_seeds(seeds)
    eb.encode_prompt(prompts)
    n, f = eb.run_canvas_device(sp, graph=True, commit_kv=True)
    torch.cuda.synchronize()
    assert (n, f) == (S, True)
    _assert_same(ref, _snapshot(eb), f"device loop ({variant})")
    log(f"[device loop {variant}] one canvas of {S} steps and its commit bit-identical to the explicit calls")
    eb.close()


def test_device_loop_early_exit(torch_cuda):
    # a stop threshold above log V stops every request at its first step: the
    # host learns it from the mapped progress record and issues no more steps
    torch = torch_cuda
    mc = micro(n_layers=1, vocab=2048)
    W = di.make_weights(mc, 32)
    B = 3
    eng = make_engine(mc, W, B, 64 + 2 * mc.canvas_len)
    eng.set_seeds(di.request_seeds(32, B))
    eng.encode_prompt(torch.from_numpy(di.make_prompts(mc.vocab, B, 64, 32)))
    sp = di.SamplerConfig(max_steps=48, entropy_bound=0.1, stop_mode=1, stop_tau=100.0)
    for graph in (False, True):
        issued, fin = eng.run_canvas_device(sp, graph=graph, early_exit=True)
        torch.cuda.synchronize()
        assert fin and eng.done.cpu().numpy().all()
        # the host is at most two steps ahead when it sees the flag
        assert 1 <= issued <= 3, issued
        assert (eng.n_committed.cpu().numpy() == mc.canvas_len).all()
        log(f"[early exit graph={graph}] all requests done after step 0; {issued} steps issued of 48")
    eng.close()


@pytest.mark.parametrize("router", ["pieces", "streamed", "hd128"])
def test_requests_stop_independently(torch_cuda, router):
    # four requests; request b is driven to stop at step b (crafted entropies into
    # dg_sample_commit), the others continue with the model's own
    torch = torch_cuda
    if router == "pieces":
        mc = micro(n_layers=2, vocab=4096)
    elif router == "hd128":
        # 128-dim heads on the half-head QKV tiles: 75-row canvases put tile
        # rows across requests, and a finished request's rows are left out
        mc = micro(n_layers=2, d_model=512, n_q_heads=4, n_kv_heads=2, head_dim=128, vocab=4096, canvas_len=75)
    else:
        # the streamed norm + router: 75-row canvases put row pairs across requests
        mc = micro(n_layers=2, d_model=1024, n_experts=24, top_k=3, ffn_hidden=128, vocab=4096, canvas_len=75)
    W = di.make_weights(mc, 33, gain_std=0.1)
    B, P, S = 4, min(100, mc.canvas_len), 6       # the prompt in one pass
    eng = make_engine(mc, W, B, P + 2 * mc.canvas_len)
    seeds = di.request_seeds(33, B)
    eng.set_seeds(seeds)
    prompts = di.make_prompts(mc.vocab, B, P, 33)
    eng.encode_prompt(torch.from_numpy(prompts))
    torch.cuda.synchronize()
    om = OracleModel(mc, W, B, P + 2 * mc.canvas_len)
    rf = RouteForcing(mc, *gpu_routing(mc, eng, B, P, list(range(B))), "independent stop: prompt")
    om.route_override = rf
    om.encode_prompt(prompts)
    om.route_override = None
    rf.finish()
    # the oracle's cache stands in for the GPU's (teacher forcing), so that only the
    # step's own arithmetic is compared
    kc, vc = eng.kv_views()
    for l in range(mc.n_layers):
        kc[l, :, :, :P] = torch.from_numpy(om.k_cache[l][:, :, :P]).to(kc.dtype).cuda()
        vc[l, :, :, :P] = torch.from_numpy(om.v_cache[l][:, :, :P]).to(vc.dtype).cuda()
    sp = di.SamplerConfig(max_steps=S, entropy_bound=0.1, stop_mode=1, stop_tau=0.05)
    eng.init_canvas()
    eng.done.zero_()
    canvas = eng.canvas.cpu().numpy()
    done = np.zeros(B, bool)
    tol = tol_for(mc)
    for t in range(S):
        active = torch.from_numpy((~done).astype(np.uint8)).cuda()
        before = _snapshot(eng)
        if mc.self_cond and t > 0:
            eng.self_cond_view()[torch.from_numpy(~done).cuda()] = torch.from_numpy(
                om.s[~done].astype(np.float32)).cuda()
            before["s"] = eng.self_cond_view().clone()
        logits = torch.full((B, mc.canvas_len, mc.vocab), float("nan"), device="cuda")
        eng.H.fill_(-1.0)
        before["H"] = eng.H.clone()
        eng.denoise_step(t, sp, active=active, logits=logits)
        torch.cuda.synchronize()
        after = _snapshot(eng)
        rf = RouteForcing(mc, *gpu_routing(mc, eng, B, mc.canvas_len, list(range(B))), f"independent stop: step {t}")
        om.route_override = rf
        ref = om.denoise_step(canvas, t, sp, seeds, active=~done, want_logits=True)
        om.route_override = None
        rf.finish()
        for b in range(B):
            if done[b]:
                # nothing of a finished request is touched: outputs, canvas, self-conditioning, K/V
                for key in ("H", "y", "am", "margin", "canvas", "s"):
                    assert torch.equal(_bits(after[key][b]), _bits(before[key][b])), f"step {t} req {b}: {key}"
                assert torch.equal(_bits(after["k"][:, b]), _bits(before["k"][:, b]))
                assert torch.equal(_bits(after["v"][:, b]), _bits(before["v"][:, b]))
                assert torch.isnan(logits[b]).all(), "a finished request's logits were written"
            else:
                e = rel_err_rows(logits[b].cpu().numpy(), ref["logits"][b]).max()
                eH = np.abs(after["H"][b].cpu().numpy() - ref["H"][b]).max() / np.abs(ref["H"][b]).max()
                assert e <= tol and eH <= tol, f"step {t} req {b}: logits {e:.2e} H {eH:.2e}"
        # crafted entropies: request t stops now, the others keep high entropies
        H = eng.H.clone()
        if t < B:
            H[t] = 0.001
        for b in range(B):
            if b != t and not done[b]:
                H[b] = H[b].clamp(min=1.0)
        eng.sample_commit(t, sp, H=H)
        torch.cuda.synchronize()
        gd = eng.done.cpu().numpy().astype(bool)
        Hh, yh, amh = H.cpu().numpy(), eng.y.cpu().numpy(), eng.am.cpu().numpy()
        for b in range(B):
            if done[b]:
                continue
            new, _, _, d = osmp.commit(Hh[b], yh[b], amh[b], None, canvas[b], t, S, sp.entropy_bound,
                                       sp.stop_mode, sp.stop_tau, int(seeds[b]), 0, mc.vocab)
            canvas[b] = new
            assert d == gd[b]
        assert np.array_equal(eng.canvas.cpu().numpy(), canvas)
        expect = np.array([b <= t for b in range(B)])
        assert np.array_equal(gd, expect | (t == S - 1)), (t, gd)
        done = gd
        log(f"[independent stop] step {t}: done {done.astype(int).tolist()}")
    eng.close()


def test_partial_commit_per_request_context(torch_cuda):
    # request 0 commits its canvas, request 1 does not: contexts and canvas
    # indices diverge, and each request matches an oracle holding it alone
    torch = torch_cuda
    mc = micro(n_layers=2, vocab=4096)
    W = di.make_weights(mc, 34, gain_std=0.1)
    B, P = 2, 150
    n = mc.canvas_len
    eng = make_engine(mc, W, B, P + 3 * n)
    seeds = di.request_seeds(34, B)
    eng.set_seeds(seeds)
    prompts = di.make_prompts(mc.vocab, B, P, 34)
    eng.encode_prompt(torch.from_numpy(prompts))
    torch.cuda.synchronize()
    oms = [OracleModel(mc, W, 1, P + 3 * n) for _ in range(B)]

    def forced_pass(b, rows, tag, fn):
        rf = RouteForcing(mc, *gpu_routing(mc, eng, B, rows, [b]), tag)
        oms[b].route_override = rf
        out = fn()
        oms[b].route_override = None
        rf.finish()
        return out

    for b in range(B):
        forced_pass(b, P, f"partial commit: prompt {b}", lambda: oms[b].encode_prompt(prompts[b:b + 1]))
    kc, vc = eng.kv_views()

    def force_cache(b, lo, hi):
        for l in range(mc.n_layers):
            kc[l, b, :, lo:hi] = torch.from_numpy(oms[b].k_cache[l][0, :, lo:hi]).to(kc.dtype).cuda()
            vc[l, b, :, lo:hi] = torch.from_numpy(oms[b].v_cache[l][0, :, lo:hi]).to(vc.dtype).cuda()

    for b in range(B):
        force_cache(b, 0, P)
    canvas = eng.init_canvas().clone()
    k1_before = kc[:, 1].clone()
    v1_before = vc[:, 1].clone()
    which = torch.tensor([1, 0], dtype=torch.uint8, device="cuda")
    eng.commit_canvas_to_kv(canvas, which=which)
    torch.cuda.synchronize()
    assert eng.ctx_lens().cpu().tolist() == [P + n, P]
    assert eng.canvas_indices().cpu().tolist() == [1, 0]
    assert torch.equal(_bits(kc[:, 1]), _bits(k1_before)) and torch.equal(_bits(vc[:, 1]), _bits(v1_before))
    forced_pass(0, n, "partial commit: canvas of request 0",
                lambda: oms[0].commit_canvas_to_kv(canvas[0:1].cpu().numpy()))
    tol = tol_for(mc)
    for l in range(mc.n_layers):
        gk = kc[l, 0, :, P:P + n].float().cpu().numpy()
        rk = oms[0].k_cache[l][0, :, P:P + n]
        assert np.abs(gk - rk).max() / np.abs(rk).max() <= tol
    force_cache(0, P, P + n)
    # each request's next canvas: its own canvas index, its own context
    eng.init_canvas()
    got_canvas = eng.canvas.cpu().numpy()
    sp = di.SamplerConfig(max_steps=4, entropy_bound=0.1)
    for b in range(B):
        ref_c = osmp.init_canvas(int(seeds[b]), oms[b].canvas_index, n, mc.vocab)
        assert np.array_equal(got_canvas[b], ref_c), f"request {b}: initial canvas"
    logits = torch.empty(B, n, mc.vocab, device="cuda")
    eng.denoise_step(0, sp, logits=logits)
    torch.cuda.synchronize()
    for b in range(B):
        ref = forced_pass(b, n, f"partial commit: step of request {b}",
                          lambda: oms[b].denoise_step(got_canvas[b:b + 1], 0, sp, seeds[b:b + 1], want_logits=True))
        e = rel_err_rows(logits[b].cpu().numpy(), ref["logits"][0]).max()
        eH = np.abs(eng.H[b].cpu().numpy() - ref["H"][0]).max() / np.abs(ref["H"][0]).max()
        log(f"[partial commit] request {b} (context {oms[b].ctx}, canvas {oms[b].canvas_index}): "
            f"logits rel {e:.2e}, H rel {eH:.2e}")
        assert e <= tol and eH <= tol
    eng.close()
