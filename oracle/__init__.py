"""Plain, slow, float64 CPU oracle for paged split-KV decode attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute anything in this package: only the test suite, the package smoke
check and the benchmark's CPU-baseline leg use it. It shares no code with the
HIP library or its Python binding, and imports neither.

Sources (cited by page title and section, in every function):
  [cascade-PR]  mlxcel pull request "perf(core): compute shared prompt
                prefixes once per decode batch" (issue 903 / PR 1004).
  [DCP-PR]      ROCm/ATOM pull request "[feat][DCP] Optimize MLA DCP (Enable
                Prefix Cache / Chunked Prefill + FP8 KVCache)".
  [OCP-FP8]     OCP 8-bit floating point specification, E4M3 encoding.

What each module computes:
  codecs     bf16 and OCP E4M3FN decode, bf16 round-to-nearest-even encode,
             the fp8 -> bf16 dequant with a per-tensor scale.
  attention  full softmax attention for one query token per request over a
             paged KV range (the plain definition), the same definition on a
             partition of the range (a normalized partial and its log2 LSE),
             and the log2-LSE merge of such states.
  planner    shared-prefix detection and the two-level cascade plan.
  cascade    the cascade composition (stacked level 0, level 1, pair merge).
  mla        the chunked cached-prefix / new-suffix composition.
  nested     spans inside spans (system prompt, tenant sub-prefix, private
             suffix) and their composition.
  multitoken T query tokens per request in one step (causal over the new
             tokens, non-causal over a cached prefix), their partials and
             merges, and the chunked split with T query tokens.

Every parity claim against the HIP path rests on these functions, which are in
turn pinned by the not-GPU tests to closed forms, library routines, brute force
and the invariants the pages state.
"""
from . import codecs, attention, planner, cascade, mla, multitoken, nested  # noqa: F401
