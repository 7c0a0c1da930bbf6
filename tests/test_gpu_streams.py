"""GPU: the entry points from several host threads on several streams at once.

The library keeps no state: every call validates its arguments, enqueues its
kernels on the stream it is given and returns.  Four host threads each run
one INT8 linear layer with GELU forward and backward, residual add,
LayerNorm and the bfloat16 dequantization (the sequence of
test_gpu_graph.py) on their own inputs and their own stream, concurrently
(ctypes releases the interpreter lock for the calls); every output must
equal, bit for bit, the same sequence run alone on the default stream.
Streams are created at the default priority.
"""
import threading

import pytest
import torch

from gpu_util import note
from test_gpu_graph import layer, make_inputs, same

pytestmark = pytest.mark.gpu

SEEDS = (31, 32, 33, 34)


def test_threads_on_their_own_streams_match_sequential():
    want = []
    for seed in SEEDS:
        outs = layer(make_inputs(seed))
        torch.cuda.synchronize()
        want.append([o.clone() for o in outs])
    got = [None] * len(SEEDS)
    errors = []

    def worker(i):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                for _ in range(3):                 # several rounds, so the threads' launches interleave
                    outs = layer(make_inputs(SEEDS[i]))
                stream.synchronize()
                got[i] = [o.clone() for o in outs]
                stream.synchronize()
        except Exception as e:                     # reported in the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(SEEDS))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i, (g, w) in enumerate(zip(got, want)):
        bad = [k for k, (a, b) in enumerate(zip(g, w)) if not same(a, b)]
        assert not bad, f"thread {i}: outputs {bad} differ from the sequential run"
    note(f"{len(SEEDS)} threads x 3 rounds on their own streams: {len(want[0])} outputs each bit-identical")
