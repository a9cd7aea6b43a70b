"""Calls from two host threads on two streams at once (the entry points keep no state between calls
and take the caller's stream): every result equals, bitwise, the same call made alone."""
import threading

import numpy as np
import pytest
import torch

from synth import gen_qkv

pytestmark = pytest.mark.gpu


def _fa():
    import exact_tiled_attention_22_amd as fa

    return fa


def test_two_threads_two_streams_match_serial_bitwise():
    fa = _fa()
    dev = torch.device("cuda")
    qa, ka, va = (t.to(dev) for t in gen_qkv(2, 4, 1000, 128, "bf16", seed=51))
    qb, kb, vb = (t.to(dev) for t in gen_qkv(1, 4, 700, 64, "f16", seed=52))
    gb = gen_qkv(1, 4, 700, 64, "f16", seed=53)[0].to(dev)
    qc, kc, vc = (t.to(dev) for t in gen_qkv(2, 8, 3000, 256, "bf16", seed=54))
    qc1 = qc[:, :, -1:, :].contiguous()
    ob, lb = fa.fwd(qb, kb, vb, causal=True)

    def job_a():  # causal forward, bf16 d128
        return fa.fwd(qa, ka, va, causal=True)

    def job_b():  # backward, fp16 d64
        return fa.bwd(qb, kb, vb, ob, lb, gb, causal=True)

    def job_c():  # one-query decode against a 3000-key cache, bf16 d256, then a non-causal forward
        return (*fa.fwd_decode(qc1, kc, vc, causal=True), *fa.fwd(qc, kc, vc, causal=False))

    serial = {}
    for name, job in (("a", job_a), ("b", job_b), ("c", job_c)):
        serial[name] = [t.clone() for t in job()]
    torch.cuda.synchronize()

    got, errors = {}, []

    def run(name, job, reps):
        try:
            s = torch.cuda.Stream(device=dev)  # default priority
            with torch.cuda.stream(s):
                for _ in range(reps):
                    out = job()
                s.synchronize()
            got[name] = [t.clone() for t in out]
            torch.cuda.synchronize()
        except Exception as e:  # pragma: no cover - reported below
            errors.append(f"{name}: {e!r}")

    threads = [threading.Thread(target=run, args=(n, j, r)) for n, j, r in (("a", job_a, 12), ("b", job_b, 8),
                                                                              ("c", job_c, 6))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=100)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    for name in ("a", "b", "c"):
        for i, (g, w) in enumerate(zip(got[name], serial[name])):
            assert torch.equal(g, w), f"job {name} output {i} differs from the serial call"
    print("three concurrent jobs on three streams: all outputs bitwise equal to the serial calls", flush=True)
