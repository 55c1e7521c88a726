"""Decision-level teacher forcing of the oracle by a GPU pass (test helper).

The GPU runs a pass first; the oracle then runs the same pass and, layer by
layer, compares its router logits with the GPU's (within the value tolerance
of the row's largest |logit|: 2e-2 for bf16 operands, 1e-4 for fp32).  Where
the two expert sets differ, the oracle's own logits must show that every
swapped pair lies within twice the row's measured logit discrepancy -- two
logits that close can trade places under the rounding noise that tolerance
allows -- and the oracle then continues with the GPU's experts, so later
layers compare like with like on every row.  At most MAX_FLIP_FRAC of the
rows may take such a swap in any one layer of a pass.

The top-k truncated sampler's vocabulary selection is forced the same way
(TopkForcing): the GPU's selection is the top k of the logits it wrote (the
fused head computes the same values; the test checks that by re-running the
GPU sampler on those logits), and where it differs from the oracle's, the
swapped ids must be within twice the row's measured logit discrepancy in the
oracle's logits.
"""
import numpy as np

from _util import log

ROUTER_TOL = {"bf16": 2e-2, "f32": 1e-4}
MAX_FLIP_FRAC = 0.10
MAX_TOPK_SWAP_FRAC = 0.10


class RouteForcing:
    """Decision-level teacher forcing of one pass (see the module docstring).

    groute / glog: the GPU's expert ids [L][requests][rows][k] and router
    logits [L][requests][rows][E] of the pass, for the oracle's requests."""

    def __init__(self, mc, groute, glog, tag):
        self.mc, self.groute, self.glog, self.tag = mc, groute, glog, tag
        self.flips = np.zeros(mc.n_layers, np.int64)
        self.rows = np.zeros(mc.n_layers, np.int64)
        self.drift_max = 0.0
        self.drift_rel_max = 0.0

    def __call__(self, b, l, r, idx):
        mc = self.mc
        g = self.groute[l, b]
        gl = self.glog[l, b].astype(np.float64)
        r64 = r.astype(np.float64)
        drift = np.abs(gl - r64).max(axis=1)
        scale = np.maximum(np.abs(r64).max(axis=1), 1e-30)
        rel = drift / scale
        tol = ROUTER_TOL[mc.dtype]
        assert (rel <= tol).all(), (f"{self.tag} layer {l}: router logits beyond {tol} of the row scale "
                                    f"(max {rel.max():.3e} at rows {np.nonzero(rel > tol)[0][:5]})")
        self.drift_max = max(self.drift_max, float(drift.max()))
        self.drift_rel_max = max(self.drift_rel_max, float(rel.max()))
        out = idx.copy()
        n_flip = 0
        for i in range(idx.shape[0]):
            gs = set(int(e) for e in g[i])
            if gs == set(int(e) for e in idx[i]):
                continue
            assert len(gs) == mc.top_k and all(0 <= e < mc.n_experts for e in gs), \
                f"{self.tag} layer {l} row {i}: invalid GPU expert set {sorted(gs)}"
            inside = np.array(sorted(gs))
            outside = np.setdiff1d(np.arange(mc.n_experts), inside)
            swap = (r64[i, outside].max() - r64[i, inside].min()) if outside.size else -np.inf
            assert swap <= 2.0 * drift[i] * (1 + 1e-6), (
                f"{self.tag} layer {l} row {i}: GPU experts {sorted(gs)} vs oracle {sorted(idx[i].tolist())}: "
                f"a swapped pair is {swap:.3e} apart in the oracle's logits, beyond twice the row's "
                f"measured discrepancy {drift[i]:.3e}")
            out[i] = g[i]
            n_flip += 1
        self.flips[l] += n_flip
        self.rows[l] += idx.shape[0]
        return out

    def finish(self):
        frac = self.flips / np.maximum(self.rows, 1)
        log(f"[{self.tag}] near-tie expert swaps per layer {self.flips.tolist()} (max {frac.max():.3f} of the rows); "
            f"router drift max {self.drift_max:.2e} ({self.drift_rel_max:.2e} of the row scale)")
        assert frac.max() <= MAX_FLIP_FRAC, f"{self.tag}: {frac.max():.3f} of a layer's rows took expert swaps"


class TopkForcing:
    """The top-k sampler's selection, forced from the GPU's logits gl [requests][n][V]."""

    def __init__(self, gl, k, tag):
        self.gl, self.k, self.tag = gl, k, tag
        self.swaps = 0
        self.rows = 0

    def __call__(self, b, logits):
        k = self.k
        g = self.gl[b].astype(np.float32)
        r = np.asarray(logits, np.float32)
        dl = np.abs(g.astype(np.float64) - r).max(axis=1)
        out = [None] * r.shape[0]
        for i in range(r.shape[0]):
            gs = np.sort(np.argsort(-g[i], kind="stable")[:k])
            os_ = np.sort(np.argsort(-r[i], kind="stable")[:k])
            if np.array_equal(gs, os_):
                continue
            gin = np.setdiff1d(gs, os_)          # taken by the GPU only
            oin = np.setdiff1d(os_, gs)          # taken by the oracle only
            gap = float(r[i, oin].astype(np.float64).max() - r[i, gin].astype(np.float64).min())
            assert gap <= 2.0 * dl[i] * (1 + 1e-6), (
                f"{self.tag} row {i}: GPU top-{k} ids {gs.tolist()} vs oracle {os_.tolist()}: the swapped ids "
                f"are {gap:.3e} apart in the oracle's logits, beyond twice the row's discrepancy {dl[i]:.3e}")
            out[i] = gs
            self.swaps += 1
        self.rows += r.shape[0]
        return out

    def finish(self):
        frac = self.swaps / max(self.rows, 1)
        log(f"[{self.tag}] near-tie top-{self.k} selection swaps {self.swaps} of {self.rows} rows ({frac:.3f})")
        assert frac <= MAX_TOPK_SWAP_FRAC, f"{self.tag}: {frac:.3f} of the rows took top-k selection swaps"


def gpu_routing(mc, eng, batch, rows, reqs):
    """GPU expert ids and router logits of the last pass, [L][len(reqs)][rows][.]."""
    gr = eng.route_view(batch * rows).cpu().numpy().reshape(mc.n_layers, batch, rows, -1)[:, reqs]
    gl = eng.router_logits_view(batch * rows).cpu().numpy().reshape(mc.n_layers, batch, rows, -1)[:, reqs]
    return gr, gl


