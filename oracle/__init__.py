"""CPU oracle for DFlash2 q-token verification attention over a paged E4M3 KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link or
execute anything in this package: only the test suite, the smoke check of the
package entry file and the ``cpu_baseline`` leg of the benchmark use it.  It shares
no code with the HIP library (no kernels, headers, helpers, tables or constants).

Everything is plain numpy in float64.  The pages it follows (three pull-request
pages of a vLLM fork) are cited by PR number and section:

* [#556] "[Perf] Add opt-in DFlash2 schedules and numerical audits"
* [#587] "[Perf] Reduce DFlash2 long-context verification decay"
* [#589] "[Perf] Reduce DFlash2 attention cost and screen exact QK reuse"

Modules:

* :mod:`oracle.e4m3`      -- OCP E4M3 decode table built from the format's formula.
* :mod:`oracle.attention` -- unsplit softmax attention, the 80 per-split FP64
  (max, sum, numerator) states and their merge.
* :mod:`oracle.qk`        -- the QK stage on its own: every FP32 tiled score with
  its masks and the untouched guard region ([#589] Purpose, Test Plan).
* :mod:`oracle.kv_append` -- E4M3 encoding (nearest, ties to even, saturating) of
  new FP16 key/value rows and their write into the paged cache by slot.
* :mod:`oracle.brute`     -- a pure-Python brute force for tiny inputs, used to pin
  :mod:`oracle.attention` and :mod:`oracle.qk`.

Pins (all in ``tests/``, CPU only): the decode table against torch's
``float8_e4m3fn`` cast and OCP spec values; the attention against the brute
force, split-count invariance, closed forms (equal keys, equal values, one key)
and paging invariance; the split-size rule against the pages' split of 3296
tokens at the 261888-token capacity boundary; the tiled scores against the
brute force, a closed form, the attention oracle and paging invariance; the
E4M3 encoder against torch's float8_e4m3fn cast wherever that cast is finite,
an exhaustive round trip through the decode table, midpoint ties and the
saturation reading.  No function here is
"parity unpinned".
"""
