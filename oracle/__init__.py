"""CPU oracle for the block-scaled MXFP8 publishing GEMM and its Lamport mailbox.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call, link or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library (``mxfp8_decode_gemm_amd``) and imports nothing from it.

It is a plain, slow, obviously correct restatement of what the hot path
computes, in float64 / exact integer arithmetic:

* ``codecs``    -- e4m3fn and E8M0 decoding, BF16 round-to-nearest-even from
                   float64, negative-zero clearing of BF16 bits.
* ``quant``     -- the per-32 MXFP8 quantizer (scale = smallest power of two that
                   brings the block into e4m3 range), used to pin the input
                   generator, and its BF16-input form for the activation
                   quantizer in front of the GEMM.
* ``gemm``      -- C[t, n] = sum_k dec(W[n,k]) 2^(Ws-127) dec(x[t,k]) 2^(xs-127)
                   in float64, its absolute-value sum, and the BF16 result.
* ``mailbox``   -- the three-generation Lamport mailbox: publish, collect,
                   reset, generation advance, and the invariant checker; the
                   word publish and fused all-gather; the all-reduce collect.
* ``tolerance`` -- the BF16 acceptance bound used by every parity test.

Page citations in this package name the four API pages by module:
  "all_gather page"      = vllm.models.deepseek_v41.nvidia.ops.cute_dsl.all_gather
  "publishing_gemm page" = vllm.models.deepseek_v41.nvidia.specialized_decode.
                           boundary.publishing_gemm
  "sync page"            = vllm.models.deepseek_v41.amd.mono.common.sync
"""

from . import codecs, gemm, mailbox, quant, tolerance  # noqa: F401

__all__ = ["codecs", "gemm", "mailbox", "quant", "tolerance"]
