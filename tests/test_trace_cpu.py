"""Host logic of the divergence localiser (reading notes "Bitwise-Deterministic
Pretraining at Scale", sections "Trace without synchronizing" and "Reading the
first mismatch"): events matched by (scope, op, invocation count), the first
output mismatch classified by its inputs."""
from invariant_deterministic_gemm_det_amd.trace import Trace, first_divergence


def rec(d):
    return {"shape": (4,), "dtype": "torch.bfloat16", "numel": 4, "digest": d}


def run(values):
    """A chain x -> op_k -> ... ; values[k] is the digest of op k's output."""
    t = Trace()
    prev = rec(1)
    for k, v in enumerate(values):
        out = rec(v)
        t.log("matmul" if k % 2 == 0 else "add", f"layer{k // 2}", [prev], [out])
        prev = out
    return t.events


def test_identical_runs():
    assert first_divergence(run([10, 11, 12]), run([10, 11, 12])).kind == "identical"


def test_origin_is_first_event_with_equal_inputs_and_different_outputs():
    d = first_divergence(run([10, 11, 12, 13]), run([10, 99, 98, 97]))
    assert d.kind == "origin"
    assert (d.event["scope"], d.event["op"]) == ("layer0", "add")
    assert d.origin is d.event


def test_downstream_when_inputs_already_differ():
    a, b = run([10, 11]), run([10, 11])
    b[0]["inputs"] = [rec(2)]          # the data entered the traced region already different
    b[0]["outputs"] = [rec(55)]
    b[1]["inputs"] = [rec(55)]
    b[1]["outputs"] = [rec(56)]
    d = first_divergence(a, b)
    assert d.kind == "downstream" and d.origin is None
    assert d.event["op"] == "matmul"


def test_alignment_by_identifiers_not_position():
    a = run([10, 11, 12])
    b = [dict(ev) for ev in reversed(run([10, 11, 12]))]   # logged in another order
    assert first_divergence(a, b).kind == "identical"
    # invocation counts tell repeated calls of one op in one scope apart
    t = Trace()
    t.log("matmul", "blk", [rec(1)], [rec(2)])
    t.log("matmul", "blk", [rec(2)], [rec(3)])
    assert [e["count"] for e in t.events] == [0, 1]


def test_events_missing_from_the_other_run_are_skipped():
    a, b = run([10, 11, 12]), run([10, 11, 12])
    del b[1]
    a[2]["outputs"] = [rec(77)]
    d = first_divergence(a, b)
    assert d.kind == "origin" and d.event["scope"] == "layer1"
