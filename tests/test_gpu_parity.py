"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Integer outputs (canvas draws, sampled tokens, argmax, commit masks, routing)
must match bit-exactly, except sampled tokens whose oracle Gumbel top-2 margin
is below max(1e-3, twice the row's score discrepancy) and routing near-ties
(below); logits and entropies must match within 2e-2 relative (bf16 models)
or 1e-4 (fp32), relative meaning max|diff| / max|ref| per row.

Every pass is teacher-forced at its decisions.  The GPU runs first; the
oracle then runs the same pass and, layer by layer, compares its router
logits with the GPU's (within the value tolerance of the row's largest
|logit|).  Where the two expert sets differ, the oracle's own logits must
show that every swapped pair lies within twice the row's measured logit
discrepancy -- two logits that close can trade places under the rounding
noise the tolerance allows -- and the oracle then continues with the GPU's
experts, so the next layers compare like with like on every row.  At most
MAX_FLIP_FRAC of the rows may take such a swap in any one layer.  Before each
denoise step the GPU state also gets the oracle's self-conditioning vector and
(after their own comparison) the oracle's K/V.
"""
import numpy as np
import pytest

import dg_inputs as di
from oracle import numerics as nm
from oracle import sampler as osmp
from oracle.model import OracleModel

from _forcing import RouteForcing, TopkForcing, gpu_routing
from _util import log, make_engine, micro, rel_err_rows, replace, tol_for

pytestmark = pytest.mark.gpu

MARGIN_EXEMPT = 1e-3
MAX_EXEMPT_TOKEN_FRAC = 0.02   # sampled tokens that differ under the margin exemption, per step


def progress(msg: str) -> None:
    """A progress line on stdout and, when DG_PROGRESS_LOG names a file, appended
    there too (long cases: pytest holds a test's stdout until it ends)."""
    import os
    import time
    log(msg)
    path = os.environ.get("DG_PROGRESS_LOG")
    if not path:
        return
    try:
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        with open(path, "a") as f:
            f.write(f"{time.strftime('%H:%M:%S')} {msg}\n")
    except OSError:
        pass


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _compare_step(mc, got, ref, tag):
    tol = tol_for(mc)
    gl = got["logits"].reshape(-1, mc.vocab)
    rl = ref["logits"].reshape(-1, mc.vocab)
    e_log = rel_err_rows(gl, rl)
    e_H = np.abs(got["H"].astype(np.float64) - ref["H"]) / np.abs(ref["H"]).max()
    # a sampled token may differ only where the oracle's top-2 perturbed-score
    # margin is within 1e-3 or within twice this row's measured score
    # discrepancy (bf16 logits carry ~1e-3 relative noise from the roundings)
    inv_t = float(ref["inv_t"])
    dz = (np.abs(gl.astype(np.float64) - rl) * inv_t).max(axis=1).reshape(got["y"].shape)
    exempt = ref["margin"] < np.maximum(MARGIN_EXEMPT, 2 * dz)
    y_bad = (got["y"] != ref["y"]) & ~exempt
    am_bad = got["am"] != ref["am"]
    n_ex = int(((got["y"] != ref["y"]) & exempt).sum())
    log(f"[{tag}] logits rel err max {e_log.max():.3e} median {np.median(e_log):.3e}; H rel err max "
        f"{e_H.max():.3e}; y mismatches {int((got['y'] != ref['y']).sum())} (non-exempt {int(y_bad.sum())}, "
        f"exempt threshold max {float(np.maximum(MARGIN_EXEMPT, 2 * dz).max()):.1e}); argmax mismatches "
        f"{int(am_bad.sum())}")
    assert (e_log <= tol).all(), f"{tag}: logits beyond tol {tol} (max {e_log.max():.3e})"
    assert (e_H <= tol).all(), f"{tag}: entropies beyond tol {tol}"
    assert not y_bad.any(), f"{tag}: sampled tokens differ beyond the margin exemption"
    assert n_ex <= MAX_EXEMPT_TOKEN_FRAC * got["y"].size, f"{tag}: {n_ex} exempted token differences"
    # the logit argmax is exempt only where the top two logits are within twice
    # the row's measured logit discrepancy
    rl2 = -np.sort(-rl, axis=1)[:, :2]
    dl = np.abs(gl.astype(np.float64) - rl).max(axis=1)
    am_close = ((rl2[:, 0] - rl2[:, 1]) <= 2 * dl).reshape(am_bad.shape)
    assert not (am_bad & ~am_close).any(), f"{tag}: argmax differs"
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


def _run_parity(torch, mc, seed, P, batch, steps, tag, gain_std=0.0, check_kv=True, canvases=1,
                oracle_reqs=None, sp_max_steps=None, determinism=False, top_k=0, v_scale_exp=0):
    """GPU engine over `batch` requests against the oracle on `oracle_reqs` (default: all).

    The prompt is encoded in canvas-length chunks, each compared (routing) and
    teacher-forced at its decisions; per canvas: initial canvas bit-exact,
    `steps` teacher-forced denoise steps, then the canvas is appended to the KV
    cache (early if steps < budget).  determinism: before the first canvas's
    steps, two steps are run twice from the same inputs and every output
    compared bit for bit."""
    W = di.make_weights(mc, seed, gain_std=gain_std)
    if v_scale_exp:
        # V (the cache and the attention output) scaled by 2^e, the output projection by 2^-e:
        # the residual stream keeps its scale while attention sees values outside fp16's range
        for l in range(mc.n_layers):
            W.scale_by_power_of_two(f"l{l}.wv", v_scale_exp)
            W.scale_by_power_of_two(f"l{l}.wo", -v_scale_exp)
    reqs = list(range(batch)) if oracle_reqs is None else list(oracle_reqs)
    nb = len(reqs)
    n = mc.canvas_len
    max_ctx = P + n * (canvases + 1)
    progress(f"[{tag}] weights + engine ({mc.n_layers} layers, d {mc.d_model}, V {mc.vocab})")
    eng = make_engine(mc, W, batch, max_ctx)
    om = OracleModel(mc, W, nb, max_ctx)
    if mc.n_layers >= 8:
        om.on_layer = lambda l: progress(f"[{tag}] oracle layer {l} done") if l % 10 == 9 else None
    prompts = di.make_prompts(mc.vocab, batch, P, seed)
    seeds = di.request_seeds(seed, batch)
    oseeds = seeds[reqs]
    eng.set_seeds(seeds)
    tol = tol_for(mc)
    ridx = torch.tensor(reqs, device="cuda")

    def forced(rows, what):
        gr, gl = gpu_routing(mc, eng, batch, rows, reqs)
        return RouteForcing(mc, gr, gl, f"{tag} {what}")

    # prompt, chunk by chunk: the GPU pass, then the oracle's pass forced at its decisions
    for p0 in range(0, P, n):
        ln = min(n, P - p0)
        eng.encode_prompt(torch.from_numpy(np.ascontiguousarray(prompts[:, p0:p0 + ln])))
        torch.cuda.synchronize()
        rf = forced(ln, f"prompt {p0}..{p0 + ln - 1}")
        om.route_override = rf
        progress(f"[{tag}] oracle prompt chunk {p0}..{p0 + ln - 1}")
        om.encode_prompt(prompts[reqs, p0:p0 + ln])
        om.route_override = None
        rf.finish()
    assert eng.ctx_len == om.ctx == P

    def check_cache(lo, hi, what, teacher=True):
        kc, vc = eng.kv_views()
        for l in range(mc.n_layers):
            gk = kc[l, ridx, :, lo:hi].float().cpu().numpy()
            rk = om.k_cache[l][:, :, lo:hi]
            gv = vc[l, ridx, :, lo:hi].float().cpu().numpy()
            rv = om.v_cache[l][:, :, lo:hi]
            ek = np.abs(gk - rk).max() / np.abs(rk).max()
            ev = np.abs(gv - rv).max() / np.abs(rv).max()
            if l == 0 or l == mc.n_layers - 1 or ek > tol or ev > tol:
                log(f"[{tag}] {what} layer {l} K rel {ek:.2e} V rel {ev:.2e}")
            assert ek <= tol and ev <= tol, f"{tag} {what} layer {l}: K/V beyond tol ({ek:.2e}, {ev:.2e})"
            if teacher:   # later passes start from the oracle's cache
                dt = kc.dtype
                for j, b in enumerate(reqs):
                    kc[l, b, :, lo:hi] = torch.from_numpy(rk[j]).to(dt).cuda()
                    vc[l, b, :, lo:hi] = torch.from_numpy(rv[j]).to(dt).cuda()

    if check_kv and P > 0:
        check_cache(0, P, "prompt")
    S = sp_max_steps or steps
    sp = di.SamplerConfig(max_steps=S, entropy_bound=0.5, stop_mode=0, top_k=top_k)
    for c in range(canvases):
        canvas = np.stack([osmp.init_canvas(int(oseeds[j]), om.canvas_index, n, mc.vocab) for j in range(nb)])
        eng.init_canvas()
        assert np.array_equal(eng.canvas[ridx].cpu().numpy(), canvas), f"{tag}: initial canvas {c}"
        if determinism and c == 0:
            _check_determinism(torch, eng, sp, min(steps, 2), tag)
        for t in range(steps):
            if mc.self_cond and t > 0:
                eng.self_cond_view()[ridx] = torch.from_numpy(om.s.astype(np.float32)).cuda()
            logits = torch.empty(batch, n, mc.vocab, dtype=torch.float32, device="cuda")
            eng.denoise_step(t, sp, logits=logits)
            torch.cuda.synchronize()
            got = {"H": eng.H[ridx].cpu().numpy(), "y": eng.y[ridx].cpu().numpy(),
                   "am": eng.am[ridx].cpu().numpy(), "margin": eng.margin[ridx].cpu().numpy(),
                   "logits": logits[ridx].cpu().numpy()}
            tf = None
            if top_k:
                # the fused head's selection is the top k of the logits it wrote: the GPU sampler
                # run on those logits repeats the step's outputs bit for bit
                fused = {k_: eng_v.clone() for k_, eng_v in (("H", eng.H), ("y", eng.y), ("am", eng.am),
                                                             ("margin", eng.margin))}
                s_fused = eng.self_cond_view().clone() if mc.self_cond else None
                eng.sample_logits(t, sp, logits)
                torch.cuda.synchronize()
                for k_, v_ in fused.items():
                    assert torch.equal(getattr(eng, k_), v_), \
                        f"{tag} canvas {c} step {t}: fused top-k head {k_} differs from the sampler on its logits"
                if s_fused is not None:
                    assert torch.equal(eng.self_cond_view(), s_fused), f"{tag}: fused top-k self-conditioning"
                tf = TopkForcing(got["logits"], top_k, f"{tag} canvas {c} step {t}")
            del logits
            rf = forced(n, f"canvas {c} step {t}")
            om.route_override = rf
            om.topk_override = tf
            ref = om.denoise_step(canvas, t, sp, oseeds, want_logits=True)
            om.route_override = None
            om.topk_override = None
            rf.finish()
            if tf is not None:
                tf.finish()
            _compare_step(mc, got, ref, f"{tag} canvas {c} step {t}")
            if mc.self_cond:
                # s = sum_v p_v E_v.  A logit discrepancy dz (max over the row, z units) perturbs the terms by
                # relative amounts up to ~dz; summed with cancellation that moves s by about dz * sqrt(sum_v p_v^2 E_v^2)
                # per element, which exceeds tol * |s| where p is near uniform (s then cancels to ~1/sqrt(V) of its
                # terms).  Bound: tol * max|s_row| + 4 dz * sqrt(p^2 @ E^2).
                gs = eng.self_cond_view()[ridx].cpu().numpy().astype(np.float64).reshape(-1, mc.d_model)
                rs = om.s.reshape(-1, mc.d_model)
                dz = (np.abs(got["logits"].astype(np.float64) - ref["logits"]) * float(ref["inv_t"])).max(axis=2)
                bound = tol * np.abs(rs).max(axis=1, keepdims=True) + 4.0 * dz.reshape(-1, 1) * ref["s_rms"].reshape(-1, mc.d_model)
                ratio = (np.abs(gs - rs) / bound).max(axis=1)
                es = rel_err_rows(gs, rs)
                log(f"[{tag} canvas {c} step {t}] self-cond: max |ds| / bound {ratio.max():.3f}; "
                    f"rel err max {es.max():.3e}")
                assert ratio.max() <= 1.0
            # commit on the oracle's entropies (GPU's own for requests the oracle does not run)
            Hf, yf, amf = eng.H.clone(), eng.y.clone(), eng.am.clone()
            Hf[ridx] = torch.from_numpy(ref["H"]).cuda()
            yf[ridx] = torch.from_numpy(ref["y"]).cuda()
            amf[ridx] = torch.from_numpy(ref["am"]).cuda()
            eng.sample_commit(t, sp, H=Hf, y=yf, am=amf)
            new_canvas = canvas.copy()
            for j in range(nb):
                new_canvas[j], _, _, _ = osmp.commit(ref["H"][j], ref["y"][j], ref["am"][j], None, canvas[j], t,
                                                     sp.max_steps, sp.entropy_bound, sp.stop_mode, sp.stop_tau,
                                                     int(oseeds[j]), om.canvas_index, mc.vocab)
            canvas = new_canvas
            torch.cuda.synchronize()
            assert np.array_equal(eng.canvas[ridx].cpu().numpy(), canvas)
            del ref
        # the canvas enters the cache: the GPU pass, then the oracle's forced at its decisions
        lo = om.ctx
        eng.commit_canvas_to_kv()
        torch.cuda.synchronize()
        rf = forced(n, f"canvas {c} commit")
        om.route_override = rf
        om.commit_canvas_to_kv(canvas)
        om.route_override = None
        rf.finish()
        assert eng.ctx_len == om.ctx and eng.canvas_index == om.canvas_index == c + 1
        if check_kv:
            check_cache(lo, lo + n, f"canvas {c} commit")
    eng.close()


def _check_determinism(torch, eng, sp, steps, tag):
    """Run `steps` denoise + commit steps twice from the same canvas and state;
    every output and the state the steps write must agree bit for bit."""
    c0 = eng.canvas.clone()
    s0 = eng.self_cond_view().clone()
    runs = []
    for rep in range(2):
        eng.canvas.copy_(c0)
        eng.self_cond_view().copy_(s0)
        eng.done.zero_()
        rec = []
        for t in range(steps):
            logits = torch.empty(eng.B, eng.n, eng.cfg.vocab, dtype=torch.float32, device="cuda")
            eng.denoise_step(t, sp, logits=logits)
            out = [eng.H.clone(), eng.y.clone(), eng.am.clone(), eng.margin.clone(), logits,
                   eng.self_cond_view().clone(), eng.route_view(eng.B * eng.n).clone(),
                   eng.router_logits_view(eng.B * eng.n).clone()]
            eng.sample_commit(t, sp)
            out += [eng.canvas.clone(), eng.mask.clone(), eng.n_committed.clone(), eng.done.clone()]
            rec.append(out)
        torch.cuda.synchronize()
        runs.append(rec)
    names = ["H", "y", "argmax", "margin", "logits", "self-cond", "routing", "router logits", "canvas",
             "commit mask", "n_committed", "done"]
    for t in range(steps):
        for nmx, a, b in zip(names, runs[0][t], runs[1][t]):
            # raw bytes: bit for bit, NaN and -0 included
            ab, bb = a.contiguous().view(-1).view(torch.uint8), b.contiguous().view(-1).view(torch.uint8)
            assert torch.equal(ab, bb), f"{tag}: step {t} {nmx} differs between identical runs"
    log(f"[{tag}] determinism: {steps} denoise + commit steps repeated bit for bit ({len(names)} outputs each)")
    eng.canvas.copy_(c0)
    eng.self_cond_view().copy_(s0)
    eng.done.zero_()


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
    _run_parity(torch_cuda, mc, 11, 300, 2, 3, "micro-bf16", gain_std=0.1)


def test_micro_hd128_gqa(torch_cuda):
    mc = micro(n_layers=1, n_q_heads=4, n_kv_heads=2, head_dim=128, n_experts=16, top_k=4, ffn_hidden=128,
               vocab=2048)
    _run_parity(torch_cuda, mc, 12, 70, 1, 2, "micro-hd128")


def test_micro_many_experts_top8(torch_cuda):
    # 128 experts, top-8 (the proxy's router shape: 4-row router blocks, 8 logit column blocks)
    mc = micro(n_layers=2, n_experts=128, top_k=8, ffn_hidden=128, vocab=2048)
    _run_parity(torch_cuda, mc, 14, 200, 2, 2, "micro-e128", gain_std=0.1)


def test_micro_streamed_router_rank_select(torch_cuda):
    # d 1024 with 24 experts (not a power of two): the fused norm + router streams W_r by whole
    # waves (two kilobyte pieces per row) for two rows a workgroup, ranks the 24 logits, and its
    # last wave has no rows; three 75-row canvases: 225 rows, row pairs across requests, a
    # workgroup of one row at the end
    mc = micro(n_layers=2, d_model=1024, n_experts=24, top_k=3, ffn_hidden=128, vocab=2048, canvas_len=75)
    _run_parity(torch_cuda, mc, 18, 100, 3, 2, "micro-stream-e24", gain_std=0.1)


def test_micro_streamed_router_two_waves(torch_cuda):
    # d 512, 128 experts top-8: two waves per row stream W_r sixteen rows a batch, top-8 by rounds
    mc = micro(n_layers=2, d_model=512, n_experts=128, top_k=8, ffn_hidden=128, vocab=2048)
    _run_parity(torch_cuda, mc, 19, 100, 1, 2, "micro-stream-e128", gain_std=0.1, determinism=True)


@pytest.mark.parametrize("d,E,k,dtype", [(3072, 64, 4, "bf16"), (4096, 128, 8, "bf16"), (1024, 64, 4, "f32")])
def test_micro_streamed_router_wide_rows(torch_cuda, d, E, k, dtype):
    # the streamed norm + router at its other row widths: 3072 (six waves, six pieces
    # per router row, two rows a batch), 4096 (eight waves, two float4 chunks per thread),
    # and fp32 weights (FMAs, four rows a batch)
    mc = micro(n_layers=1, d_model=d, n_experts=E, top_k=k, ffn_hidden=128, vocab=2048, canvas_len=100,
               dtype=dtype)
    _run_parity(torch_cuda, mc, 20 + d // 1024, 60, 1, 2, f"micro-stream-d{d}-{dtype}", gain_std=0.1)


def test_micro_grouped_experts_fused_router(torch_cuda):
    # 4 experts top-2: 512 routed entries over 4 experts take the grouped 128-row tile products
    # (ragged last tiles per expert), routed by the fused norm + router and the one-workgroup sort
    mc = micro(n_layers=2, n_experts=4, top_k=2, vocab=2048)
    _run_parity(torch_cuda, mc, 15, 130, 1, 2, "micro-grouped-e4", determinism=True)


def test_micro_grouped_experts_split_router(torch_cuda):
    # 6 experts top-3 (not a power of two: the three-launch router) on the grouped 128-row tiles,
    # two requests so the 512 canvas rows span several router blocks
    mc = micro(n_layers=1, n_experts=6, top_k=3, vocab=2048)
    _run_parity(torch_cuda, mc, 16, 70, 2, 2, "micro-grouped-e6")


def test_micro_many_requests_wide_attention_bf16(torch_cuda):
    # 16 requests x 16/8 heads x 64: the wide attention kernel with two 16-row query blocks
    # per wave (256 workgroups without key splits); the oracle runs requests 0 and 15
    mc = micro(n_layers=1, n_q_heads=16, n_kv_heads=8, head_dim=64, n_experts=8, top_k=2, vocab=2048)
    _run_parity(torch_cuda, mc, 17, 40, 16, 2, "micro-wide-bf16", oracle_reqs=[0, 15])


def test_micro_many_requests_wide_attention_f32(torch_cuda):
    # the same shape in fp32: the wide kernel's fp32 path (one query block per wave)
    mc = micro(n_layers=1, dtype="f32", n_q_heads=16, n_kv_heads=8, head_dim=64, n_experts=8, top_k=2,
               vocab=2048)
    _run_parity(torch_cuda, mc, 18, 40, 16, 2, "micro-wide-f32", oracle_reqs=[0, 15])


@pytest.mark.parametrize("e", [20, -24])
def test_attention_values_beyond_fp16_range(torch_cuda, e):
    # V ~ 0.3 * 2^e: 2^20 puts |v| near 3e5, past fp16's 65504; 2^-24 puts it near 2e-8, under fp16's
    # smallest subnormal.  One request takes the spread kernel (bf16 V in its products), sixteen take
    # the wide kernel (V staged as fp16, rescaled tile by tile when out of range); both on the oracle.
    mc = micro(n_layers=1, vocab=2048)
    _run_parity(torch_cuda, mc, 31, 300, 1, 2, f"v-2^{e}-spread", v_scale_exp=e)
    mcw = micro(n_layers=1, n_q_heads=16, n_kv_heads=8, head_dim=64, n_experts=8, top_k=2, vocab=2048)
    _run_parity(torch_cuda, mcw, 32, 300, 16, 2, f"v-2^{e}-wide", oracle_reqs=[0, 15], v_scale_exp=e)


def test_micro_ragged_vocabulary_full_step(torch_cuda):
    # vocabulary 4160 = 32.5 chunks of 128: the fused LM-head tiles and the chunk-scaled
    # softmax @ E product both end on a half chunk (one 64-id slice)
    mc = micro(n_layers=1, vocab=4160)
    _run_parity(torch_cuda, mc, 19, 50, 1, 3, "micro-ragged-vocab")


def test_micro_short_canvas_two_requests(torch_cuda):
    # a 100-position canvas: ragged query blocks, head tiles of 100 rows per request
    # (tiles straddling requests), positions past the canvas in the commit sort
    mc = micro(n_layers=1, canvas_len=100, vocab=2048)
    _run_parity(torch_cuda, mc, 20, 37, 2, 2, "micro-canvas100")


def test_micro_f32_no_prompt_dense_moe(torch_cuda):
    # empty prompt, E = k (every expert selected): the MoE is a dense weighted sum
    mc = micro(n_layers=1, dtype="f32", n_experts=4, top_k=4, self_cond=True, vocab=1024)
    _run_parity(torch_cuda, mc, 13, 0, 1, 2, "micro-f32-dense")


def test_proxy_shapes_two_layers(torch_cuda):
    # the 26B-scale proxy's layer, head, expert and vocabulary shapes (d 2048, 16/8 heads x 128, 128 experts
    # top-8, F 768, vocab 262144: 64 sampler chunks) with 2 of its 30 layers and a 256-token prompt
    mc = replace(di.workload("proxy").model, n_layers=2)
    _run_parity(torch_cuda, mc, 2, 256, 1, 2, "proxy-2L")


def test_small_workload_full_canvas(torch_cuda):
    # the 4-layer bf16 model at its full shape: 512-token prompt, self-conditioning,
    # all 24 steps of the canvas (the last one takes y everywhere), then the commit;
    # the first two steps are also repeated and compared bit for bit
    wl = di.workload("small")
    _run_parity(torch_cuda, wl.model, wl.seed, wl.prompt_len, 1, wl.sampler.max_steps, "small",
                determinism=True)


def test_proxy_workload_full_depth(torch_cuda):
    # the 26B-scale proxy at its full shape: 30 layers, d 2048, 16/8 heads x 128, 128 experts
    # top-8, F 768, vocabulary 262144, 2048-token prompt; one teacher-forced step (the
    # routing of all 30 layers and the K/V of the whole prompt compared), repeated bit for bit
    wl = di.workload("proxy")
    _run_parity(torch_cuda, wl.model, wl.seed, wl.prompt_len, 1, 1, "proxy", check_kv=True,
                sp_max_steps=wl.sampler.max_steps, determinism=True)


def test_multicanvas_workload_sampled(torch_cuda):
    # the block-autoregressive shape: 8192-token prompt, four canvases appended to
    # the cache one after the other (2 denoise steps each, then an early commit)
    wl = di.workload("multicanvas")
    _run_parity(torch_cuda, wl.model, wl.seed, wl.prompt_len, 1, 2, "multicanvas", canvases=4,
                sp_max_steps=wl.sampler.max_steps)


def test_batched_workload_sampled(torch_cuda):
    # 32 concurrent requests with 4096-token prompts; the oracle runs requests 0 and 31
    wl = di.workload("batched")
    _run_parity(torch_cuda, wl.model, wl.seed, wl.prompt_len, wl.batch, 2, "batched", oracle_reqs=[0, 31],
                sp_max_steps=wl.sampler.max_steps, determinism=True)


def _crafted_logits(rng, B, n, V, kind):
    if kind == "random":
        return (rng.standard_normal((B, n, V)) * 2.0).astype(np.float32)
    if kind == "peaked":        # one dominant logit per row, margin varying: low entropies
        lg = (rng.standard_normal((B, n, V)) * 0.5).astype(np.float32)
        top = rng.integers(0, V, (B, n))
        bump = rng.uniform(4.0, 30.0, (B, n)).astype(np.float32)
        np.put_along_axis(lg, top[..., None], bump[..., None], axis=2)
        return lg
    if kind == "ties":          # repeated maxima: the lowest id must win
        lg = np.round(rng.standard_normal((B, n, V)) * 2).astype(np.float32)
        return lg
    return np.zeros((B, n, V), np.float32)     # uniform


@pytest.mark.parametrize("kind", ["random", "peaked", "ties", "uniform"])
def test_sampler_stage_on_identical_logits(torch_cuda, kind):
    torch = torch_cuda
    mc = micro(n_layers=1, vocab=4160)          # two vocabulary chunks, the second one ragged
    W = di.make_weights(mc, 21)
    B, n = 2, mc.canvas_len
    eng = make_engine(mc, W, B, 512)
    seeds = di.request_seeds(21, B)
    eng.set_seeds(seeds)
    rng = np.random.default_rng(hash(kind) % 2**32)
    lg = _crafted_logits(rng, B, n, mc.vocab, kind)
    E = nm.upcast(W.get("emb"))
    for t, S in ((0, 12), (11, 12)):
        sp = di.SamplerConfig(max_steps=S, entropy_bound=0.1)
        eng.sample_logits(t, sp, torch.from_numpy(lg).cuda())
        torch.cuda.synchronize()
        T = osmp.temperature(t, S)
        inv_t = osmp.inv_temperature(T)
        for b in range(B):
            st = osmp.head_stats(lg[b], inv_t, int(seeds[b]), 0, t, np.arange(n), want_probs=True)
            gy, gam = eng.y[b].cpu().numpy(), eng.am[b].cpu().numpy()
            gH, gm = eng.H[b].cpu().numpy(), eng.margin[b].cpu().numpy()
            assert np.array_equal(gam, st["am"]), f"{kind} t={t}: argmax differs on identical logits"
            tie = st["margin"] < 1e-4
            assert np.array_equal(gy[~tie], st["y"][~tie]), f"{kind} t={t}: sampled tokens differ"
            eH = np.abs(gH.astype(np.float64) - st["H"]).max() / max(np.abs(st["H"]).max(), 1e-30)
            assert eH < 1e-5 or np.abs(gH - st["H"]).max() < 1e-6, f"{kind}: entropy rel err {eH}"
            assert np.abs(gm[~tie] - st["margin"][~tie]).max() < 1e-4
            s_ref = st["p"] @ E
            es = rel_err_rows(eng.self_cond_view()[b].cpu().numpy(), s_ref)
            assert es.max() < tol_for(mc), f"{kind}: self-conditioning rel err {es.max()}"
            log(f"[sampler {kind} t={t} b={b}] H rel {eH:.1e}, ties {int(tie.sum())}, s rel {es.max():.1e}")


def test_commit_and_stop_from_peaked_logits(torch_cuda):
    # low-entropy logits make positions commit and the mean-entropy stop fire
    torch = torch_cuda
    mc = micro(n_layers=1, vocab=2048)
    W = di.make_weights(mc, 22)
    B, n = 3, mc.canvas_len
    eng = make_engine(mc, W, B, 512)
    seeds = di.request_seeds(22, B)
    eng.set_seeds(seeds)
    rng = np.random.default_rng(5)
    lg = (rng.standard_normal((B, n, mc.vocab)) * 0.3).astype(np.float32)
    top = rng.integers(0, mc.vocab, (B, n))
    # request 0: very peaked everywhere (stops); 1: mixed (partial commit); 2: flat (nothing commits)
    bump = np.stack([np.full(n, 40.0), np.where(rng.random(n) < 0.3, 40.0, 2.0), np.full(n, 0.0)]).astype(np.float32)
    np.put_along_axis(lg, top[..., None], bump[..., None], axis=2)
    sp = di.SamplerConfig(max_steps=48, entropy_bound=0.1, stop_mode=1, stop_tau=0.05)
    canvas0 = eng.init_canvas().cpu().numpy()
    eng.done.zero_()
    eng.sample_logits(3, sp, torch.from_numpy(lg).cuda())
    eng.sample_commit(3, sp)
    torch.cuda.synchronize()
    n_com = eng.n_committed.cpu().numpy()
    done = eng.done.cpu().numpy()
    H = eng.H.cpu().numpy()
    y = eng.y.cpu().numpy()
    am = eng.am.cpu().numpy()
    for b in range(B):
        new, mask, ncom, d = osmp.commit(H[b], y[b], am[b], None, canvas0[b], 3, sp.max_steps, sp.entropy_bound,
                                         sp.stop_mode, sp.stop_tau, int(seeds[b]), 0, mc.vocab)
        assert np.array_equal(eng.canvas[b].cpu().numpy(), new) and n_com[b] == ncom and bool(done[b]) == d
    log(f"[commit/stop] committed {n_com.tolist()}, done {done.tolist()}")
    assert done[0] == 1 and n_com[0] == n          # stopped: every position takes y
    assert 0 < n_com[1] < n and done[1] == 0       # partial commit under the 0.1 nat bound
    assert n_com[2] == 0 and done[2] == 0


# ------------------------------------------------------------------ FP8 experts
def _unpack_fp8(raw, E, N, K, nf):
    """Codes [E][nf][N][K] from the packed layout [E][N/16][K/64][nf][64 lanes][16 bytes]."""
    a = raw.reshape(E, N // 16, K // 64, nf, 4, 16, 2, 8)       # lane = g * 16 + c; bytes = half * 8 + j
    # -> [E][nf][N/16][c][K/64][half][g][j]: row n = nb * 16 + c, k = ks * 64 + half * 32 + g * 8 + j
    a = a.transpose(0, 3, 1, 5, 2, 6, 4, 7)
    return a.reshape(E, nf, N, K)


def test_fp8_expert_quantisation_bit_exact(torch_cuda):
    # the model's E4M3 codes and channel scales equal the oracle's quantisation of the same bf16 weights
    from discrete_text_diffusion_dg_amd import _lib as L
    from oracle import fp8
    mc = micro(n_layers=2, d_model=512, ffn_hidden=256, n_experts=8, top_k=2, vocab=2048, expert_dtype="fp8")
    W = di.make_weights(mc, 51, gain_std=0.1)
    eng = make_engine(mc, W, 1, 512)
    E, F, d = mc.n_experts, mc.ffn_hidden, mc.d_model
    for l in range(mc.n_layers):
        gu = _unpack_fp8(eng.model_view(L.DG_MODEL_VIEW_EXPERT_GATEUP, l), E, F, d, 2)
        dn = _unpack_fp8(eng.model_view(L.DG_MODEL_VIEW_EXPERT_DOWN, l), E, d, F, 1)[:, 0]
        sgu = eng.model_view(L.DG_MODEL_VIEW_EXPERT_SCALES_GATEUP, l).view(np.float32).reshape(E, 2, F)
        sd = eng.model_view(L.DG_MODEL_VIEW_EXPERT_SCALES_DOWN, l).view(np.float32).reshape(E, d)
        for j, name in enumerate(("w_gate", "w_up")):
            q, s = fp8.quantize_rows(nm.upcast(W.get(f"l{l}.{name}")).astype(np.float32))
            assert np.array_equal(sgu[:, j].view(np.uint32), s.view(np.uint32)), f"layer {l} {name} scales"
            assert np.array_equal(gu[:, j], q), f"layer {l} {name} codes ({int((gu[:, j] != q).sum())} differ)"
        q, s = fp8.quantize_rows(nm.upcast(W.get(f"l{l}.w_down")).astype(np.float32))
        assert np.array_equal(sd.view(np.uint32), s.view(np.uint32)), f"layer {l} down scales"
        assert np.array_equal(dn, q), f"layer {l} down codes"
    log(f"[fp8] codes and scales of {mc.n_layers} layers x {E} experts bit-identical to the oracle's quantisation")
    eng.close()


def test_fp8_micro_experts_parity(torch_cuda):
    mc = micro(n_layers=2, d_model=512, ffn_hidden=256, n_experts=8, top_k=2, vocab=2048, expert_dtype="fp8")
    _run_parity(torch_cuda, mc, 52, 300, 2, 2, "fp8-micro", gain_std=0.1, determinism=True)


def test_fp8_small_workload(torch_cuda):
    wl = di.workload("small-fp8")
    _run_parity(torch_cuda, wl.model, wl.seed, wl.prompt_len, 1, 2, "fp8-small")


def test_fp8_proxy_shapes_two_layers(torch_cuda):
    # the proxy's expert shapes (128 experts top-8, d 2048, F 768) in FP8, 2 of its 30 layers
    mc = replace(di.workload("proxy-fp8").model, n_layers=2)
    _run_parity(torch_cuda, mc, 2, 256, 1, 1, "fp8-proxy-2L", sp_max_steps=48)


# ------------------------------------------------------------------ FP8 LM head
def test_fp8_head_quantisation_bit_exact(torch_cuda):
    # the LM head's E4M3 codes and per-id scales equal the oracle's quantisation of the bf16 E
    from discrete_text_diffusion_dg_amd import _lib as L
    from oracle import fp8
    mc = micro(n_layers=1, d_model=512, vocab=4160, head_dtype="fp8")
    W = di.make_weights(mc, 53)
    eng = make_engine(mc, W, 1, 512)
    V, d = mc.vocab, mc.d_model
    codes = _unpack_fp8(eng.model_view(L.DG_MODEL_VIEW_HEAD_CODES, 0), 1, V, d, 1)[0, 0]
    sc = eng.model_view(L.DG_MODEL_VIEW_HEAD_SCALES, 0).view(np.float32)
    q, s = fp8.quantize_rows(nm.upcast(W.get("emb")).astype(np.float32))
    assert np.array_equal(sc.view(np.uint32), s.view(np.uint32)), "head scales"
    assert np.array_equal(codes, q), f"head codes ({int((codes != q).sum())} differ)"
    log(f"[fp8 head] codes and scales of {V} rows bit-identical to the oracle's quantisation")
    eng.close()


def test_fp8_head_micro_parity(torch_cuda):
    # 4160 ids: 32.5 head tiles, the last one 64 wide (the per-id scales of a ragged tile)
    mc = micro(n_layers=2, d_model=512, ffn_hidden=256, n_experts=8, top_k=2, vocab=4160, head_dtype="fp8")
    _run_parity(torch_cuda, mc, 54, 300, 2, 2, "fp8-head-micro", gain_std=0.1, determinism=True)


def test_fp8_head_small_workload(torch_cuda):
    wl = di.workload("small-fp8-head")
    _run_parity(torch_cuda, wl.model, wl.seed, wl.prompt_len, 1, 2, "fp8-head-small")


def test_fp8_head_topk_micro_parity(torch_cuda):
    # top-k truncated sampling from the FP8 head's scaled products (4160 ids: a ragged last segment)
    mc = micro(n_layers=2, d_model=512, ffn_hidden=256, n_experts=8, top_k=2, vocab=4160, head_dtype="fp8")
    _run_parity(torch_cuda, mc, 56, 300, 2, 2, "fp8-head-topk-micro", gain_std=0.1, top_k=8, determinism=True)


def test_fp8_head_proxy_shapes_one_layer(torch_cuda):
    # the proxy's head (262144 ids, d 2048) and experts in FP8, 1 of its 30 layers
    mc = replace(di.workload("proxy-fp8-head").model, n_layers=1)
    _run_parity(torch_cuda, mc, 2, 256, 1, 1, "fp8-head-proxy-1L", sp_max_steps=48)


# ------------------------------------------------------------------ top-k truncated sampler
@pytest.mark.parametrize("kind", ["random", "peaked", "ties", "uniform"])
def test_topk_sampler_on_identical_logits(torch_cuda, kind):
    torch = torch_cuda
    mc = micro(n_layers=1, vocab=4160)          # 32.5 chunks: a ragged last segment
    W = di.make_weights(mc, 23)
    B, n = 2, mc.canvas_len
    eng = make_engine(mc, W, B, 512)
    seeds = di.request_seeds(23, B)
    eng.set_seeds(seeds)
    rng = np.random.default_rng(hash(kind) % 2**32 + 1)
    lg = _crafted_logits(rng, B, n, mc.vocab, kind)
    E = nm.upcast(W.get("emb"))
    for k, (t, S) in ((8, (0, 12)), (3, (11, 12)), (1, (5, 12))):
        sp = di.SamplerConfig(max_steps=S, entropy_bound=0.1, top_k=k)
        eng.sample_logits(t, sp, torch.from_numpy(lg).cuda())
        torch.cuda.synchronize()
        inv_t = osmp.inv_temperature(osmp.temperature(t, S))
        for b in range(B):
            st = osmp.head_stats_topk(lg[b], inv_t, k, int(seeds[b]), 0, t, np.arange(n), want_probs=True)
            gy, gam = eng.y[b].cpu().numpy(), eng.am[b].cpu().numpy()
            gH, gm = eng.H[b].cpu().numpy(), eng.margin[b].cpu().numpy()
            assert np.array_equal(gam, st["am"]), f"{kind} k={k}: argmax differs"
            tie = st["margin"] < 1e-4
            assert np.array_equal(gy[~tie], st["y"][~tie]), f"{kind} k={k}: sampled tokens differ"
            assert np.abs(gH.astype(np.float64) - st["H"]).max() < 1e-5, f"{kind} k={k}: entropy"
            fin = np.isfinite(st["margin"]) & ~tie
            assert np.abs(gm[fin] - st["margin"][fin]).max(initial=0) < 1e-4
            s_ref = np.einsum("nk,nkd->nd", st["p"], E[st["ids"]])
            es = rel_err_rows(eng.self_cond_view()[b].cpu().numpy(), s_ref)
            assert es.max() < tol_for(mc), f"{kind} k={k}: self-conditioning rel err {es.max()}"
            log(f"[top-k sampler {kind} k={k} b={b}] ties {int(tie.sum())}, s rel {es.max():.1e}")


def test_topk_denoise_steps_micro(torch_cuda):
    mc = micro(n_layers=2, vocab=4096)
    _run_parity(torch_cuda, mc, 24, 300, 2, 3, "topk-micro", gain_std=0.1, top_k=8, determinism=True)


def test_topk_small_workload(torch_cuda):
    wl = di.workload("small")
    _run_parity(torch_cuda, wl.model, wl.seed, wl.prompt_len, 1, 2, "topk-small", top_k=8)


def test_topk_batched_workload_sampled(torch_cuda):
    # the high-batch shape the truncation is for: 32 requests x 4096-token prompts, requests 0 and 31 checked
    wl = di.workload("batched")
    _run_parity(torch_cuda, wl.model, wl.seed, wl.prompt_len, wl.batch, 2, "topk-batched", oracle_reqs=[0, 31],
                sp_max_steps=wl.sampler.max_steps, top_k=8)
