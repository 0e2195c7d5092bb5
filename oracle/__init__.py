"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import, call or execute anything in this package.  The product path (the HIP
library ``libfa.so`` and its Python binding ``exact_tiled_attention_forward_amd``)
never imports it, and this package imports nothing from the product path: the two
share no kernels, headers, helpers, tables or pre/post-processing.  Inputs reach both
sides from the seeded generators in ``exact_tiled_attention_forward_amd.workloads``,
which hold none of the method's arithmetic.

Sources, cited by page title and section (the pages are web pages on one subject):

* [FA-ch]  "Flash Attention" -- chapter 4 deep-dive at mlx.void.app
           (sections: intro; 地基：流式 softmax (streaming softmax);
           FlashAttention——把整件事分块塞进 SRAM; FlashAttention-2——让每个核心都忙起来).
* [FA-nips] "【NeurIPS 2022】FlashAttention：IO 感知的快速内存高效精确注意力" -- paper
           summary at trdm.cn (sections: 基准/方法设计 (method design); 方法细节 (method
           details); 常见问题 FAQ).
* [FA-blog] practitioner article at cf-1.com/news/4497868 (sections 1.1 经典自注意力的那笔
           “天价账单”; 2.2 online softmax; 3.1 naive attention 到 flash kernel 的替换路径;
           4.2 长上下文训练/推理的避坑要点).
* [FA-17]  "大模型数学速成（17）：Flash Attention——不物化注意力矩阵" at shiguol.github.io
           (sections 二、数学不变，变的是计算路径; 三、分块 + 在线 Softmax 直觉, with its
           worked two-block example).

Modules:

* ``naive``     -- the definition written out: S = scale*Q K^T, P = softmax(S), O = P V,
                   per (batch, head), materialising S and P in fp64; the backward pass by
                   plain calculus of that definition (the pages give no gradient formulas).
* ``fp8``       -- E4M3 quantization with block scales (the format decoded from its
                   definition, nearest-even rounding, 128-row block and per-channel
                   scales, a random rotation) and the FP8 kernel's tiled recurrence with
                   P rounded to E4M3 ([FA-ch] FlashAttention-3, the FP8 lever).
* ``tiled_ref`` -- the tiled online-softmax recurrence in the pages' order (query block
                   outer, key/value blocks inner, running max m, running sum l,
                   unnormalised o, one division at the end).  Used only to pin the
                   worked examples and the tiled == untiled identity on tiny inputs.

Every function here is pinned by ``tests/test_oracle_*.py`` against values the pages
print, closed forms, library routines (torch SDPA on CPU fp64, autograd), finite
differences and invariants.  Nothing here is "parity unpinned".
"""

from . import naive, tiled_ref  # noqa: F401

__all__ = ["naive", "tiled_ref"]
