"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Integer outputs (canvas draws, sampled tokens, argmax, commit masks) must match
bit-exactly, except sampled tokens whose oracle Gumbel top-2 margin is below
1e-3; logits and entropies must match within 2e-2 relative (bf16 models) or
1e-4 (fp32), relative meaning max|diff| / max|ref| per row.
"""
import numpy as np
import pytest

import dg_inputs as di
from oracle import sampler as osmp
from oracle.model import OracleModel

from _util import log, make_engine, micro, rel_err_rows, replace, tol_for

pytestmark = pytest.mark.gpu

MARGIN_EXEMPT = 1e-3


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _compare_step(mc, got, ref, tag, allow_route_taint=0.0):
    tol = tol_for(mc)
    gl = got["logits"].reshape(-1, mc.vocab)
    rl = ref["logits"].reshape(-1, mc.vocab)
    e_log = rel_err_rows(gl, rl)
    e_H = np.abs(got["H"].astype(np.float64) - ref["H"]) / np.abs(ref["H"]).max()
    exempt = ref["margin"] < MARGIN_EXEMPT
    y_bad = (got["y"] != ref["y"]) & ~exempt
    am_bad = got["am"] != ref["am"]
    log(f"[{tag}] logits rel err max {e_log.max():.3e} median {np.median(e_log):.3e}; "
        f"H rel err max {e_H.max():.3e}; y mismatches {int((got['y'] != ref['y']).sum())} "
        f"(non-exempt {int(y_bad.sum())}); argmax mismatches {int(am_bad.sum())}")
    n_rows = gl.shape[0]
    bad_rows = e_log > tol
    assert bad_rows.sum() <= allow_route_taint * n_rows, f"{tag}: {int(bad_rows.sum())} rows beyond tol {tol}"
    ok = ~bad_rows.reshape(got["y"].shape)
    assert (e_H.reshape(got["H"].shape)[ok] <= tol).all()
    assert not (y_bad & ok).any(), f"{tag}: sampled tokens differ beyond the margin exemption"
    assert not (am_bad & ok).any() or mc.dtype == "bf16", f"{tag}: argmax differs"
    return e_log


def _gpu_step(eng, torch, step, sp, with_logits=True):
    logits = torch.empty(eng.B, eng.n, eng.cfg.vocab, dtype=torch.float32, device="cuda") if with_logits else None
    eng.denoise_step(step, sp, logits=logits)
    torch.cuda.synchronize()
    out = {"H": eng.H.cpu().numpy(), "y": eng.y.cpu().numpy(), "am": eng.am.cpu().numpy(),
           "margin": eng.margin.cpu().numpy()}
    if with_logits:
        out["logits"] = logits.cpu().numpy()
    return out


def test_init_canvas_bit_exact(torch_cuda):
    torch = torch_cuda
    mc = micro(n_layers=1, vocab=2048)
    W = di.make_weights(mc, 1)
    eng = make_engine(mc, W, 3, 512)
    seeds = np.array([5, (1 << 32) | 7, 0xFFFFFFFFFFFFFFFF], np.uint64)
    eng.set_seeds(seeds)
    got = eng.init_canvas().cpu().numpy()
    for b in range(3):
        ref = osmp.init_canvas(int(seeds[b]), 0, mc.canvas_len, mc.vocab)
        assert np.array_equal(got[b], ref)
    log("init canvas bit-exact for 3 requests")
    eng.close()


def _commit_case(torch, eng, mc, H, y, am, prev_am, canvas, step, sp, seeds, done_in):
    B, n = H.shape
    eng.set_seeds(seeds)
    eng.canvas.copy_(torch.from_numpy(canvas))
    eng.done.copy_(torch.from_numpy(done_in.astype(np.uint8)))
    pa = eng.view(3, torch.int32, (B, n))
    pa.copy_(torch.from_numpy(prev_am))
    eng.mask.fill_(7)
    eng.n_committed.fill_(-5)
    Ht = torch.from_numpy(H).cuda()
    yt = torch.from_numpy(y).cuda()
    amt = torch.from_numpy(am).cuda()
    eng.sample_commit(step, sp, H=Ht, y=yt, am=amt)
    torch.cuda.synchronize()
    g_canvas = eng.canvas.cpu().numpy()
    g_mask = eng.mask.cpu().numpy()
    g_n = eng.n_committed.cpu().numpy()
    g_done = eng.done.cpu().numpy()
    for b in range(B):
        if done_in[b]:
            assert np.array_equal(g_canvas[b], canvas[b]) and g_n[b] == -5 and (g_mask[b] == 7).all()
            continue
        new, mask, ncom, done = osmp.commit(H[b], y[b], am[b], prev_am[b], canvas[b], step, sp.max_steps,
                                           sp.entropy_bound, sp.stop_mode, sp.stop_tau, int(seeds[b]),
                                           eng.canvas_index, mc.vocab)
        assert np.array_equal(g_canvas[b], new), f"canvas differs for request {b}"
        assert np.array_equal(g_mask[b], mask)
        assert g_n[b] == ncom and bool(g_done[b]) == done
    return g_n, g_done


def test_commit_bit_exact_on_identical_inputs(torch_cuda):
    torch = torch_cuda
    mc = micro(n_layers=1, vocab=2048)
    W = di.make_weights(mc, 2)
    B = 4
    eng = make_engine(mc, W, B, 512)
    rng = np.random.default_rng(0)
    n = mc.canvas_len
    total_committed = 0
    for trial in range(24):
        kind = trial % 6
        if kind == 0:      # spread of entropies, some tiny
            H = (rng.exponential(0.02, (B, n)) * (rng.random((B, n)) < 0.3) + rng.random((B, n)) * 3 * (rng.random((B, n)) < 0.5)).astype(np.float32)
        elif kind == 1:    # many exact ties
            H = rng.choice(np.float32([0.0, 0.001, 0.01, 0.5]), (B, n)).astype(np.float32)
        elif kind == 2:    # all low: stop rules fire
            H = (rng.random((B, n)) * 0.01).astype(np.float32)
        elif kind == 3:    # all high: nothing commits, everything re-noised
            H = (5 + rng.random((B, n))).astype(np.float32)
        elif kind == 4:    # mixed per request
            H = np.stack([(rng.random(n) * s).astype(np.float32) for s in (0.001, 0.02, 1.0, 10.0)])
        else:
            H = np.abs(rng.standard_normal((B, n)) * 0.05).astype(np.float32)
        y = rng.integers(0, mc.vocab, (B, n)).astype(np.int32)
        am = rng.integers(0, mc.vocab, (B, n)).astype(np.int32)
        prev = am.copy() if trial % 2 else rng.integers(0, mc.vocab, (B, n)).astype(np.int32)
        canvas = rng.integers(0, mc.vocab, (B, n)).astype(np.int32)
        sp = di.SamplerConfig(max_steps=12, entropy_bound=float(rng.choice([0.0, 0.1, 0.5, 2.0])),
                              stop_mode=trial % 3, stop_tau=float(rng.choice([0.005, 0.05])))
        step = int(rng.choice([0, 1, 5, 11]))
        done_in = np.zeros(B, bool)
        if trial % 4 == 3:
            done_in[1] = True
        seeds = rng.integers(0, 2**63, B).astype(np.uint64)
        g_n, _ = _commit_case(torch, eng, mc, H, y, am, prev, canvas, step, sp, seeds, done_in)
        total_committed += int(g_n[~done_in].sum())
    log(f"commit bit-exact over 24 trials; {total_committed} positions committed in total")
    eng.close()


def _run_parity(torch, mc, seed, P, batch, steps, tag, gain_std=0.0, emb_scale=None, check_kv=True,
                route_taint=0.0):
    W = di.make_weights(mc, seed, gain_std=gain_std)
    if emb_scale is not None:
        W._store["emb"] = _scaled(W.get("emb"), mc, emb_scale)
    max_ctx = P + mc.canvas_len * 2
    eng = make_engine(mc, W, batch, max_ctx)
    om = OracleModel(mc, W, batch, max_ctx)
    prompts = di.make_prompts(mc.vocab, batch, P, seed)
    seeds = di.request_seeds(seed, batch)
    eng.set_seeds(seeds)
    om.encode_prompt(prompts)
    eng.encode_prompt(torch.from_numpy(prompts))
    torch.cuda.synchronize()
    assert eng.ctx_len == om.ctx == P
    if check_kv and P > 0:
        kc, vc = eng.kv_views()
        tol = tol_for(mc)
        for l in range(mc.n_layers):
            gk = kc[l, :, :, :P].float().cpu().numpy()
            rk = om.k_cache[l][:, :, :P]
            gv = vc[l, :, :, :P].float().cpu().numpy()
            rv = om.v_cache[l][:, :, :P]
            ek = np.abs(gk - rk).max() / np.abs(rk).max()
            ev = np.abs(gv - rv).max() / np.abs(rv).max()
            log(f"[{tag}] layer {l} prompt K rel {ek:.2e} V rel {ev:.2e}")
            assert ek < tol and ev < tol
    sp = di.SamplerConfig(max_steps=steps, entropy_bound=0.5, stop_mode=0)
    canvas = np.stack([osmp.init_canvas(int(seeds[b]), 0, mc.canvas_len, mc.vocab) for b in range(batch)])
    eng.init_canvas()
    assert np.array_equal(eng.canvas.cpu().numpy(), canvas)
    for t in range(steps):
        ref = om.denoise_step(canvas, t, sp, seeds, want_logits=True)
        got = _gpu_step(eng, torch, t, sp)
        _compare_step(mc, got, ref, f"{tag} step {t}", allow_route_taint=route_taint)
        if mc.self_cond:
            gs = eng.self_cond_view().cpu().numpy()
            es = rel_err_rows(gs.reshape(-1, mc.d_model), om.s.reshape(-1, mc.d_model))
            log(f"[{tag} step {t}] self-cond rel err max {es.max():.3e}")
            assert es.max() < tol_for(mc)
        # commit on the oracle's entropies so both canvases stay identical
        Ht = torch.from_numpy(ref["H"]).cuda()
        yt = torch.from_numpy(ref["y"]).cuda()
        amt = torch.from_numpy(ref["am"]).cuda()
        eng.sample_commit(t, sp, H=Ht, y=yt, am=amt)
        new_canvas = canvas.copy()
        for b in range(batch):
            new_canvas[b], _, _, _ = osmp.commit(ref["H"][b], ref["y"][b], ref["am"][b], None, canvas[b], t,
                                                 sp.max_steps, sp.entropy_bound, sp.stop_mode, sp.stop_tau,
                                                 int(seeds[b]), 0, mc.vocab)
        canvas = new_canvas
        torch.cuda.synchronize()
        assert np.array_equal(eng.canvas.cpu().numpy(), canvas)
    # the finished canvas enters the cache
    om.commit_canvas_to_kv(canvas)
    eng.commit_canvas_to_kv()
    torch.cuda.synchronize()
    assert eng.ctx_len == om.ctx and eng.canvas_index == 1
    if check_kv:
        kc, vc = eng.kv_views()
        l = mc.n_layers - 1
        gk = kc[l, :, :, P:P + mc.canvas_len].float().cpu().numpy()
        rk = om.k_cache[l][:, :, P:P + mc.canvas_len]
        ek = np.abs(gk - rk).max() / np.abs(rk).max()
        log(f"[{tag}] committed canvas K rel {ek:.2e}")
        assert ek < tol_for(mc)
    eng.close()


def _scaled(arr, mc, s):
    from oracle.numerics import upcast
    x = upcast(arr) * s
    if mc.dtype == "bf16":
        return di.f32_to_bf16_bits(x.astype(np.float32))
    return x.astype(np.float32)


def test_tiny_workload_full_canvas(torch_cuda):
    wl = di.workload("tiny")
    _run_parity(torch_cuda, wl.model, wl.seed, wl.prompt_len, 1, wl.sampler.max_steps, "tiny")


def test_micro_bf16_selfcond_ragged_prompt(torch_cuda):
    mc = micro()
    _run_parity(torch_cuda, mc, 11, 300, 2, 3, "micro-bf16", gain_std=0.1, route_taint=0.02)


def test_micro_hd128_gqa(torch_cuda):
    mc = micro(n_layers=1, n_q_heads=4, n_kv_heads=2, head_dim=128, n_experts=16, top_k=4, ffn_hidden=128,
               vocab=2048)
    _run_parity(torch_cuda, mc, 12, 70, 1, 2, "micro-hd128", route_taint=0.02)


def test_micro_f32_no_prompt_dense_moe(torch_cuda):
    # empty prompt, E = k (every expert selected): the MoE is a dense weighted sum
    mc = micro(n_layers=1, dtype="f32", n_experts=4, top_k=4, self_cond=True, vocab=1024)
    _run_parity(torch_cuda, mc, 13, 0, 1, 2, "micro-f32-dense")
