"""The C ABI library loads and exports what include/dg.h declares (no GPU needed).

Only calls that fail argument validation before touching the device are made.
"""
import ctypes
import os
import re

import pytest

import dg_inputs as di

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    from discrete_text_diffusion_dg_amd import _lib
    return _lib.load()


def _declared():
    src = open(os.path.join(ROOT, "include", "dg.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z_]+)\s*\(", src)))


def test_header_symbols_exported(lib):
    names = _declared()
    assert len(names) >= 15
    from discrete_text_diffusion_dg_amd import _lib
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/dg.h but not exported"
        assert n in _lib.EXPORTS, f"{n} not bound in the Python binding"


def test_weight_count(lib):
    from discrete_text_diffusion_dg_amd.runtime import config_struct
    for name in ("tiny", "small", "proxy"):
        mc = di.workload(name).model
        c = config_struct(mc)
        assert lib.dg_weight_count(ctypes.byref(c)) == len(di.tensor_list(mc))


def _create(lib, **kw):
    from discrete_text_diffusion_dg_amd import _lib
    from discrete_text_diffusion_dg_amd.runtime import config_struct
    mc = di.workload("tiny").model
    c = config_struct(mc)
    for k, v in kw.items():
        setattr(c, k, v)
    n = lib.dg_weight_count(ctypes.byref(c))
    ptrs = (ctypes.c_void_p * max(n, 1))(*([None] * max(n, 1)))
    out = ctypes.c_void_p()
    st = lib.dg_model_create(ctypes.byref(c), ptrs, n, ctypes.byref(out))
    return st, lib.dg_last_error().decode(), out


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 96, -4), ("d_model", 100, -4), ("d_model", 1280, -4), ("d_model", 1536, -4),
    ("n_kv_heads", 3, -1), ("n_experts", 200, -4),
    ("top_k", 9, -4), ("vocab", 1000, -4), ("vocab", 262208, -4), ("canvas_len", 300, -4), ("dtype", 5, -1),
    ("ffn_hidden", 100, -4), ("n_layers", 0, -1),
    ("expert_dtype", 5, -1), ("head_dtype", 5, -1),
    ("head_dtype", 2, -4),          # an FP8 LM head needs a bf16 model (this one is fp32)
])
def test_model_create_rejects_bad_config(lib, field, value, code):
    st, msg, out = _create(lib, **{field: value})
    assert st == code and msg and out.value is None


def test_model_create_rejects_null_weights(lib):
    st, msg, out = _create(lib)
    assert st == -1 and "null" in msg


def test_null_handles(lib):
    assert lib.dg_encode_prompt(None, None, 4, None) == -1
    assert "null" in lib.dg_last_error().decode()
    assert lib.dg_denoise_step(None, None, 0, None, None, None, None, None, None, None, None, None) == -1
    assert lib.dg_sample_commit(None, None, None, None, None, 0, None, None, None, None, None, None) == -1
    assert lib.dg_commit_canvas_to_kv(None, None, None, None) == -1
    assert lib.dg_corrupt_forward_loss(None, None, None, None, None, None, None, None) == -1
    assert lib.dg_model_view(None, 0, 0, None, None) == -1
    assert lib.dg_run_canvas(None, None, None, None, None, None, None, None, None, None, None, 0, 1, 0, None, None) == -1
    assert lib.dg_state_ctx_len(None) == -1
    sz = ctypes.c_size_t()
    assert lib.dg_state_bytes(None, 1, 512, ctypes.byref(sz)) == -1


def test_product_path_fails_loudly_without_library(tmp_path, monkeypatch):
    from discrete_text_diffusion_dg_amd import _lib
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        _lib.load()


def test_product_path_does_not_import_oracle():
    pkg = os.path.join(ROOT, "discrete_text_diffusion_dg_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in txt and "from oracle" not in txt, f


def test_static_sampler_argument_checks(lib):
    # the checks run before any device work, so they hold on a host without a GPU
    from discrete_text_diffusion_dg_amd import _lib as L
    fake = ctypes.c_void_p(16)                 # never dereferenced: every case fails its checks first
    seeds = (ctypes.c_uint64 * 1)(1)

    def call(rows=256, vocab=4096, canvas=256, cidx=0, step=0, **kw):
        sp = L.DgSamplerParams(0.8, 0.4, 0.1, 0.05, kw.get("max_steps", 12), 0, kw.get("top_k", 0))
        return lib.dg_sample_logits_static(fake, rows, vocab, canvas, cidx, step, ctypes.byref(sp), seeds, fake,
                                           fake, fake, fake, None)
    assert call(top_k=8) == -4 and "top_k" in lib.dg_last_error().decode()
    assert call(step=12) == -1
    assert call(rows=100) == -1                # not a multiple of the canvas length
    assert call(vocab=1000) == -4
    assert call(rows=256 * 129) == -4          # more than 128 requests
    assert call(rows=512, vocab=262144) == -2  # the records would not fit the fixed scratch
    assert call(cidx=-1) == -1
    assert lib.dg_sample_logits_static(None, 256, 4096, 256, 0, 0, None, None, None, None, None, None, None) == -1


def test_bench_refuses_more_than_one_gpu():
    # one GPU only: N > 1 ends at once with the reason, before any device work
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""
