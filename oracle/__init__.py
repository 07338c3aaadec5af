"""CPU oracle for the Mixture-of-Experts layer (top-k routing, schedule, dispatch,
expert-grouped SwiGLU FFN, weighted combine, and the backward).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here.  The
product path (``mixture_experts_layer_dispatch_amd``) never imports it, and this
package never imports the product path; the two share no code beyond the
seeded input generators in ``synth_inputs``.

Everything is plain NumPy in float64 (float32 inputs are widened), written as
the textbook definition of each step, one step per function, with no blocking,
fusion or reordering beyond what the definition states.

Sources (the pages describing the method):
  [AREX]  arex-research.com, "Cursor 放出 MoK：NVL72 训练提速 2.37 倍", section
          "pull 代替 push，ring buffer 踢掉 CPU：三个决定性的设计选择"
          (three design decisions; the closing paragraph lists the precision
          modes and the fused router-weight gradient).
  [AIGWX] aigwx.org, "Cursor 开源 MoK：面向 GB300 NVL72 的确定性 MoE 训练内核",
          section "详细发生了什么".
  [ALPHA] alphalab.site, "Mixture-of-Kittens" review, sections 一 (what was
          published), 二 (one megakernel is not one GPU), 三 (what the 2.37x
          measured), 四 (README vs API).

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
brute force, closed forms, special cases, invariants or finite differences.
No function is "parity unpinned".
"""
from .routing import route
from .schedule import schedule
from .ffn import forward, backward, swiglu, swiglu_grad
from .router import router_logits, router_backward
from .mx import (mx_quantize, mx_dequantize, mx_roundtrip, e4m3_round, e4m3_encode,
                 e4m3_decode, E4M3_MAX, MX_BLOCK, mxfp4_quantize, mxfp4_dequantize,
                 mxfp4_roundtrip, e2m1_round, e2m1_encode, e2m1_decode)

__all__ = ["route", "schedule", "forward", "backward", "swiglu", "swiglu_grad",
           "router_logits", "router_backward",
           "mx_quantize", "mx_dequantize", "mx_roundtrip", "e4m3_round", "e4m3_encode",
           "e4m3_decode", "E4M3_MAX", "MX_BLOCK", "mxfp4_quantize", "mxfp4_dequantize",
           "mxfp4_roundtrip", "e2m1_round", "e2m1_encode", "e2m1_decode"]
