"""Calls in flight on several HIP streams at once, and from several host
threads (needs an MI355X).

Every call takes its scratch from its own workspace (a caller buffer, or the
library's stream-ordered allocation), and the only state the library keeps
across calls is the per-thread record of the last plan.  So calls enqueued on
two streams with no synchronisation between them, or made from two host
threads each on its own stream, must give exactly the bits each call gives on
its own, and each thread must read back the plan of its own last call.
"""
import threading

import pytest
import torch

import oracle
import parity
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the -m gpu tests need an MI355X")
    import split_kv_decode_amd as mx
    mx.lib()
    oracle.build()


WORKLOADS = [
    # the 64-row matrix-core kernel with its merge
    wl.Workload("st1", B=16, qLen=8, Hq=64, Hkv=8, D=128, kv_cap=1100, dtype="bf16",
                causal=True, sigma=0.5, seed=111, len_range=(1, 1100)),
    # the vector-ALU kernel, 4 heads per workgroup
    wl.Workload("st2", B=2, qLen=1, Hq=32, Hkv=32, D=128, kv_cap=2500, dtype="fp16",
                causal=False, sigma=1.0, seed=112, len_range=(0, 2500)),
    # the 16-row matrix-core variant, head dim 64
    wl.Workload("st3", B=4, qLen=2, Hq=32, Hkv=4, D=64, kv_cap=1800, dtype="bf16",
                causal=True, sigma=1.0, seed=113, len_range=(0, 1800)),
]


class Case:
    """A workload's inputs on the GPU, its own output buffers and scratch,
    and the bits its call gives on its own."""

    def __init__(self, w, copy):
        import split_kv_decode_amd as mx
        self.w = w
        self.inp = wl.make_inputs(w, seed=w.seed + copy)
        self.g = self.inp.to("cuda")
        dt = 1 if w.dtype == "bf16" else 0
        need = mx.workspace_size(w.B, w.Hq, w.Hkv, w.D, w.qLen, w.kv_cap, w.causal, dt, 0)
        self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        self.out = torch.empty_like(self.g.q)
        self.lse = torch.empty((w.B, w.Hq, w.qLen), dtype=torch.float32, device="cuda")
        self.ref = None

    def call(self, own_scratch: bool):
        import split_kv_decode_amd as mx
        self.out.fill_(float("nan"))
        self.lse.fill_(float("nan"))
        mx.fwd_kvcache(self.g.q, self.g.k_cache, self.g.v_cache, self.g.cache_seqlens,
                       self.w.causal, out=self.out, lse=self.lse,
                       workspace=None if own_scratch else self.ws)

    def record(self):
        torch.cuda.synchronize()
        self.call(False)
        torch.cuda.synchronize()
        self.ref = (self.out.clone(), self.lse.clone())

    def same(self):
        return torch.equal(self.out.view(torch.int16), self.ref[0].view(torch.int16)) and \
            torch.equal(self.lse, self.ref[1])


def test_calls_on_two_streams_without_synchronisation():
    import split_kv_decode_amd as mx
    cases = [Case(w, c) for w in WORKLOADS for c in range(2)]
    for c in cases:
        c.record()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        print(f"case two streams rep {rep}", flush=True)
        torch.cuda.synchronize()
        # half the calls on each stream, interleaved on the host; library
        # scratch for some, caller workspaces for the others
        for i, c in enumerate(cases):
            with torch.cuda.stream(s1 if i % 2 == 0 else s2):
                c.call(own_scratch=(i + rep) % 2 == 0)
        torch.cuda.synchronize()
        for c in cases:
            assert c.same(), (c.w.name, rep)
    # and the concurrent results still match the oracle
    c = cases[0]
    ro, rl = parity.oracle_full(c.inp)
    print(parity.compare(parity.to_f64(c.out), c.lse.cpu().double().numpy(), ro, rl,
                         c.w.dtype), mx.last_plan().as_dict(), flush=True)


def test_calls_from_two_host_threads():
    import split_kv_decode_amd as mx
    per_thread = [[Case(WORKLOADS[0], 7), Case(WORKLOADS[1], 7)],
                  [Case(WORKLOADS[2], 7), Case(WORKLOADS[1], 8)]]
    plans = {}
    for cs in per_thread:
        for c in cs:
            c.record()
            plans[id(c)] = mx.last_plan().as_dict()
    errors = []
    start = threading.Barrier(2)

    def worker(t):
        try:
            stream = torch.cuda.Stream()
            start.wait(timeout=60)
            with torch.cuda.stream(stream):
                for rep in range(20):
                    for c in per_thread[t]:
                        c.call(own_scratch=rep % 2 == 1)
                        # the plan record is per thread: it describes this
                        # thread's call, whatever the other thread ran meanwhile
                        got = mx.last_plan().as_dict()
                        if got != plans[id(c)]:
                            errors.append((t, rep, c.w.name, got))
                        stream.synchronize()
                        if not c.same():
                            errors.append((t, rep, c.w.name, "output differs"))
        except Exception as e:  # surfaced in the main thread
            errors.append((t, repr(e)))

    print("case two host threads", flush=True)
    threads = [threading.Thread(target=worker, args=(t,), daemon=True) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=100)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    assert not errors, errors[:5]
