"""CPU oracle for the DiffusionGemma denoise-step hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its
Python binding) may import, call or link anything in this package; only the
tests, ``__graft_entry__.smoke()`` and the CPU baseline leg of the benchmark do.

The oracle is a plain, slow numpy implementation of what one denoising step
computes, written from the pages that describe the method and shares no code
with the HIP path.  Floating point is fp64 except where a decision is taken in
the kernel's precision (fp32 router logits, fp32 Gumbel-perturbed scores); the
bf16 rounding points of the bf16 models are written out explicitly (``rnd``).

Pages cited (all are secondary summaries of the DiffusionGemma technical report):
  [mlqm]     mlqm.cn/news/993655, Chinese summary of the report (sections 一..九)
  [chooseai] chooseai.io/news/4338, news article on the release
  [rebas]    rebasdaily.com explainer on DiffusionGemma
  [bohu]     bohuyeshan.top blog post, sections 一 and 二
"""
from . import philox, numerics, sampler, model, loop  # noqa: F401
from .model import OracleModel  # noqa: F401
