"""Divergence localisation over tensor fingerprints.

Reading notes "Bitwise-Deterministic Pretraining at Scale: How Megatron Core
Finds and Removes Every Flipped Bit":
  * section "5. Fingerprinting Tensors on the GPU": a record is the shape, the
    dtype, the element count and a bit-pattern digest computed in GPU memory
    (here ``det_fingerprint``, include/det_fingerprint.h);
  * section "Trace without synchronizing": each run (rank) keeps its own log;
    events of two runs are matched afterwards by run-independent identifiers:
    operation name, module scope and invocation count;
  * section "Reading the first mismatch": the origin is the first event whose
    input digests agree between the runs and whose output digests differ; an
    event whose inputs already differ is a downstream receiver.

Host logic only; the digests come from the library's kernels.
"""
from dataclasses import dataclass

from . import det_fingerprint, digest_value


def record(t):
    """The fingerprint record of a contiguous GPU tensor."""
    return {"shape": tuple(t.shape), "dtype": str(t.dtype), "numel": t.numel(),
            "digest": digest_value(det_fingerprint(t))}


class Trace:
    """One run's event log.  Inputs and outputs may be GPU tensors (fingerprinted
    here) or records already computed."""

    def __init__(self):
        self.events = []
        self._count = {}

    def log(self, op, scope, inputs, outputs):
        key = (scope, op)
        n = self._count.get(key, 0)
        self._count[key] = n + 1
        def rec(x):
            return x if isinstance(x, dict) else record(x)

        self.events.append({"op": op, "scope": scope, "count": n,
                            "inputs": [rec(x) for x in inputs],
                            "outputs": [rec(x) for x in outputs]})
        return outputs


def _key(ev):
    return (ev["scope"], ev["op"], ev["count"])


@dataclass
class Divergence:
    kind: str            # "origin", "downstream" or "identical"
    event: dict = None   # run A's event of the first output mismatch
    origin: dict = None  # first event whose inputs agree and outputs differ


def first_divergence(run_a, run_b):
    """Align two event lists by (scope, op, invocation count) and read the
    first mismatch in run A's order: "origin" when its inputs agree (the
    candidate origin), "downstream" when they already differ (keep looking
    upstream: the origin lies outside the traced events), "identical" when no
    aligned event's outputs differ.  ``origin`` is the first event meeting the
    origin condition, wherever it lies."""
    b = {_key(ev): ev for ev in run_b}
    first, origin = None, None
    for ev in run_a:
        other = b.get(_key(ev))
        if other is None:
            continue
        if ev["outputs"] == other["outputs"]:
            continue
        same_in = ev["inputs"] == other["inputs"]
        if first is None:
            first = (ev, same_in)
        if same_in and origin is None:
            origin = ev
        if first is not None and origin is not None:
            break
    if first is None:
        return Divergence("identical")
    return Divergence("origin" if first[1] else "downstream", first[0], origin)
