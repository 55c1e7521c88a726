"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Integer outputs (canvas draws, sampled tokens, argmax, commit masks, routing)
must match bit-exactly, except sampled tokens whose oracle Gumbel top-2 margin
is below 1e-3 and rows with a router near-tie; logits and entropies must match
within 2e-2 relative (bf16 models) or 1e-4 (fp32), relative meaning
max|diff| / max|ref| per row.

Each denoise step is compared teacher-forced: before it the GPU state gets the
oracle's self-conditioning vector and (after their own comparison) the
oracle's prompt K/V, so a routing flip on a near-tie row in one step cannot
leak into the next step's inputs.
"""
import numpy as np
import pytest

import dg_inputs as di
from oracle import numerics as nm
from oracle import sampler as osmp
from oracle.model import OracleModel

from _util import log, make_engine, micro, rel_err_rows, replace, tol_for

pytestmark = pytest.mark.gpu

MARGIN_EXEMPT = 1e-3
# Routing may differ from the oracle only where the oracle's k-th and (k+1)-th
# router logits are closer than GAP_REL * max|r| of the row.  Both sides round
# the same activations to bf16, but fp32 sums (whose error near-cancelling
# attention outputs amplify to ~1e-5) against fp64 ones flip ~1% of those
# roundings by one ulp, and the flips carry through the residual stream to a
# router-logit drift of up to ~1% of the logit scale (the tests print the
# measured drift).  2e-2 is the bf16 value tolerance; fp32 operands drift ~1e-6.
GAP_REL = {"bf16": 2e-2, "f32": 1e-4}
MAX_FLIP_FRAC = 0.25     # sanity bound on rows with an (explained) routing flip
MAX_KV_OFF_FRAC = 0.10   # cached K/V positions beyond the value tolerance (all at router near-ties)


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def router_gap(r: np.ndarray, k: int) -> np.ndarray:
    """Gap between the k-th and (k+1)-th largest router logits per row (inf if k = E)."""
    if r.shape[1] <= k:
        return np.full(r.shape[0], np.inf)
    srt = -np.sort(-r.astype(np.float64), axis=1)
    return srt[:, k - 1] - srt[:, k]


def near_tie(r: np.ndarray, mc) -> np.ndarray:
    return router_gap(r, mc.top_k) < GAP_REL[mc.dtype] * np.abs(r).max(axis=1)


def _routing_core(mc, groute, glog, traces, tag):
    """Routing of one pass (groute / glog: [L][requests][rows][...]) against the oracle traces.

    A row's expert set may differ from the oracle's only where the oracle's gap
    between its k-th and (k+1)-th router logits is at most twice the row's
    measured logit discrepancy (the largest |GPU - oracle| over its experts):
    an expert swap needs the two logits to move past each other, and each moved
    by at most that much.  A row that flipped in an earlier layer carries other
    values from then on and is not checked again.  Returns the flipped rows."""
    nreq, n = groute.shape[1], groute.shape[2]
    flipped = np.zeros((nreq, n), bool)
    drift_max, drift_med, n_flip = 0.0, [], 0
    for l in range(mc.n_layers):
        for j in range(nreq):
            r = traces[j]["router_logits"][l]
            rr = traces[j]["route_idx"][l]
            gap = router_gap(r, mc.top_k)
            drift_row = np.abs(glog[l, j].astype(np.float64) - r).max(axis=1)
            flip = np.array([set(groute[l, j, i]) != set(rr[i]) for i in range(n)])
            bad = flip & (gap > 2.0 * drift_row * (1 + 1e-6)) & ~flipped[j]
            assert not bad.any(), (f"{tag} layer {l}: routing differs where the oracle gap {gap[bad][:5]} exceeds "
                                   f"twice the measured drift {drift_row[bad][:5]} (rows {np.nonzero(bad)[0][:5]})")
            clean = ~flipped[j] & ~flip
            if clean.any():
                drift_max = max(drift_max, float(drift_row[clean].max()))
                drift_med.append(float(np.median(drift_row[clean])))
            n_flip += int(flip.sum())
            flipped[j] |= flip
    log(f"[{tag}] routing flips {n_flip} (rows {int(flipped.sum())}), each within twice its row's measured "
        f"drift; router drift max {drift_max:.2e} median {np.median(drift_med):.2e}")
    assert flipped.mean() <= MAX_FLIP_FRAC, f"{tag}: too many routing flips"
    return flipped


def check_routing(mc, eng, traces, rows_per_req, tag):
    """Per-layer routing of the last pass against the oracle traces (see _routing_core)."""
    B = len(traces)
    groute = eng.route_view(B * rows_per_req).cpu().numpy().reshape(mc.n_layers, B, rows_per_req, -1)
    glog = eng.router_logits_view(B * rows_per_req).cpu().numpy().reshape(mc.n_layers, B, rows_per_req, -1)
    return _routing_core(mc, groute, glog, traces, tag)


def _compare_step(mc, got, ref, tag, taint):
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
    ok = ~taint
    y_bad = (got["y"] != ref["y"]) & ~exempt
    am_bad = got["am"] != ref["am"]
    log(f"[{tag}] logits rel err max {e_log[ok.ravel()].max():.3e} (all rows {e_log.max():.3e}) "
        f"median {np.median(e_log):.3e}; H rel err max {e_H[ok].max():.3e}; y mismatches "
        f"{int((got['y'] != ref['y']).sum())} (non-exempt {int((y_bad & ok).sum())}, exempt margin "
        f"max {float(np.maximum(MARGIN_EXEMPT, 2 * dz).max()):.1e}); argmax mismatches "
        f"{int(am_bad.sum())}; rows with a routing flip {int(taint.sum())}")
    assert (e_log[ok.ravel()] <= tol).all(), f"{tag}: logits beyond tol {tol}"
    assert (e_H[ok] <= tol).all(), f"{tag}: entropies beyond tol {tol}"
    assert not (y_bad & ok).any(), f"{tag}: sampled tokens differ beyond the margin exemption"
    # the logit argmax is exempt only where the top two logits are within twice
    # the row's measured logit discrepancy
    rl2 = -np.sort(-rl, axis=1)[:, :2]
    dl = np.abs(gl.astype(np.float64) - rl).max(axis=1)
    am_close = ((rl2[:, 0] - rl2[:, 1]) <= 2 * dl).reshape(am_bad.shape)
    assert not (am_bad & ok & ~am_close).any(), f"{tag}: argmax differs"
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
                oracle_reqs=None, sp_max_steps=None):
    """GPU engine over `batch` requests against the oracle on `oracle_reqs` (default: all).

    Per canvas: initial canvas bit-exact, `steps` teacher-forced denoise steps,
    then the canvas is appended to the KV cache (early if steps < budget)."""
    W = di.make_weights(mc, seed, gain_std=gain_std)
    reqs = list(range(batch)) if oracle_reqs is None else list(oracle_reqs)
    nb = len(reqs)
    max_ctx = P + mc.canvas_len * (canvases + 1)
    eng = make_engine(mc, W, batch, max_ctx)
    om = OracleModel(mc, W, nb, max_ctx)
    prompts = di.make_prompts(mc.vocab, batch, P, seed)
    seeds = di.request_seeds(seed, batch)
    oseeds = seeds[reqs]
    eng.set_seeds(seeds)
    ptr = [dict() for _ in range(nb)]
    om.encode_prompt(prompts[reqs], ptr)
    eng.encode_prompt(torch.from_numpy(prompts))
    torch.cuda.synchronize()
    assert eng.ctx_len == om.ctx == P
    tol = tol_for(mc)
    ridx = torch.tensor(reqs, device="cuda")

    def check_cache(lo, hi, traces, what, teacher=True):
        kc, vc = eng.kv_views()
        near = np.zeros((nb, hi - lo), bool)
        for l in range(mc.n_layers):
            gk = kc[l, ridx, :, lo:hi].float().cpu().numpy()
            rk = om.k_cache[l][:, :, lo:hi]
            gv = vc[l, ridx, :, lo:hi].float().cpu().numpy()
            rv = om.v_cache[l][:, :, lo:hi]
            ek = np.abs(gk - rk).max(axis=(1, 3)) / np.abs(rk).max()
            ev = np.abs(gv - rv).max(axis=(1, 3)) / np.abs(rv).max()
            off = (ek >= tol) | (ev >= tol)
            log(f"[{tag}] {what} layer {l} K rel {ek[~off].max():.2e} V rel {ev[~off].max():.2e}; "
                f"positions beyond tol {int(off.sum())}")
            assert not (off & ~near).any(), f"{tag} {what} layer {l}: K/V differ away from router near-ties"
            assert off.mean() <= MAX_KV_OFF_FRAC
            near |= np.stack([near_tie(traces[b]["router_logits"][l], mc) for b in range(nb)])
            if teacher:   # later passes start from the oracle's cache
                dt = kc.dtype
                for j, b in enumerate(reqs):
                    kc[l, b, :, lo:hi] = torch.from_numpy(rk[j]).to(dt).cuda()
                    vc[l, b, :, lo:hi] = torch.from_numpy(rv[j]).to(dt).cuda()

    if check_kv and P > 0:
        check_cache(0, P, ptr, "prompt")
    S = sp_max_steps or steps
    sp = di.SamplerConfig(max_steps=S, entropy_bound=0.5, stop_mode=0)
    for c in range(canvases):
        canvas = np.stack([osmp.init_canvas(int(oseeds[j]), om.canvas_index, mc.canvas_len, mc.vocab)
                           for j in range(nb)])
        eng.init_canvas()
        assert np.array_equal(eng.canvas[ridx].cpu().numpy(), canvas), f"{tag}: initial canvas {c}"
        full_canvas = eng.canvas.clone()
        for t in range(steps):
            if mc.self_cond and t > 0:
                eng.self_cond_view()[ridx] = torch.from_numpy(om.s.astype(np.float32)).cuda()
            ref = om.denoise_step(canvas, t, sp, oseeds, want_logits=True, trace_requests=list(range(nb)))
            logits = torch.empty(batch, mc.canvas_len, mc.vocab, dtype=torch.float32, device="cuda")
            eng.denoise_step(t, sp, logits=logits)
            torch.cuda.synchronize()
            got = {"H": eng.H[ridx].cpu().numpy(), "y": eng.y[ridx].cpu().numpy(),
                   "am": eng.am[ridx].cpu().numpy(), "margin": eng.margin[ridx].cpu().numpy(),
                   "logits": logits[ridx].cpu().numpy()}
            traces = [ref["traces"][j] for j in range(nb)]
            taint = check_routing_subset(mc, eng, traces, reqs, batch, f"{tag} canvas {c} step {t}")
            _compare_step(mc, got, ref, f"{tag} canvas {c} step {t}", taint)
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
                log(f"[{tag} canvas {c} step {t}] self-cond: max |ds| / bound {ratio[~taint.ravel()].max():.3f}; "
                    f"rel err max {es[~taint.ravel()].max():.3e}")
                assert ratio[~taint.ravel()].max() <= 1.0
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
        # the canvas enters the cache
        lo = om.ctx
        ctr = [dict() for _ in range(nb)]
        om.commit_canvas_to_kv(canvas, ctr)
        eng.commit_canvas_to_kv()
        torch.cuda.synchronize()
        assert eng.ctx_len == om.ctx and eng.canvas_index == om.canvas_index == c + 1
        if check_kv:
            check_routing_subset(mc, eng, ctr, reqs, batch, f"{tag} canvas {c} commit")
            check_cache(lo, lo + mc.canvas_len, ctr, f"canvas {c} commit")
    eng.close()


def check_routing_subset(mc, eng, traces, reqs, batch, tag):
    """check_routing for an oracle that runs a subset of the GPU's requests."""
    n = mc.canvas_len
    groute = eng.route_view(batch * n).cpu().numpy().reshape(mc.n_layers, batch, n, -1)[:, reqs]
    glog = eng.router_logits_view(batch * n).cpu().numpy().reshape(mc.n_layers, batch, n, -1)[:, reqs]
    return _routing_core(mc, groute, glog, traces, tag)


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


def test_micro_grouped_experts_fused_router(torch_cuda):
    # 4 experts top-2: 512 routed entries over 4 experts take the grouped 128-row tile products
    # (ragged last tiles per expert), routed by the fused norm + router and the one-workgroup sort
    mc = micro(n_layers=2, n_experts=4, top_k=2, vocab=2048)
    _run_parity(torch_cuda, mc, 15, 130, 1, 2, "micro-grouped-e4")


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


def test_small_workload_full_size(torch_cuda):
    # the 4-layer bf16 model at its full shape: 512-token prompt, self-conditioning, 2 steps
    wl = di.workload("small")
    _run_parity(torch_cuda, wl.model, wl.seed, wl.prompt_len, 1, 2, "small")


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
                sp_max_steps=wl.sampler.max_steps)


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
