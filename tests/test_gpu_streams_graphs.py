"""The library on several streams and inside HIP graphs.

The entry points keep no state and allocate nothing, so two problems may run
at once on two streams, and a captured graph may be replayed: both must give
exactly the results of plain sequential calls (the kernels are
deterministic, so the comparison is bitwise). Each graph replay is checked on
its own inputs, with eager work and synchronisations between replays.
"""

import pytest
import torch

import dynamic_block_sparse_rr_amd as rr
from synthetic.gen import Workload, make_inputs
from tests.gpu_cases import say

pytestmark = pytest.mark.gpu


class Job:
    def __init__(self, w):
        self.w = w
        q, k, v = make_inputs(w)
        self.q, self.k, self.v = q.cuda(), k.cuda(), v.cuda()
        self.p = rr.problem(w.L, w.Hq, w.Hkv, w.d, w.S, w.B, 0.9, True, w.dtype)
        self.ws = torch.empty(rr.rr_workspace_bytes(self.p), dtype=torch.uint8, device="cuda")
        self.out = torch.empty_like(self.q)
        self.rc = torch.empty((w.Hq, w.nb), dtype=torch.int32, device="cuda")
        self.ci = torch.empty((w.Hq, w.nb, w.nb), dtype=torch.int32, device="cuda")

    def run(self, stream=None):
        rr.rr_prefill(self.p, self.q, self.k, self.v, self.out, self.rc, self.ci, self.ws, stream=stream)

    def result(self):
        return self.out.clone(), self.rc.clone(), self.ci.clone()


def same(a, b):
    return all(torch.equal(x, y) for x, y in zip(a, b))


def test_two_streams_at_once_match_sequential_calls():
    a = Job(Workload("sa", 8192, 16, 4, 128, "bf16", 128, 16, (0.9,), 31, "llm", 8))
    b = Job(Workload("sb", 5000, 8, 2, 64, "bf16", 64, 8, (0.9,), 32, "gauss", 8))
    a.run()
    torch.cuda.synchronize()
    ra = a.result()
    b.run()
    torch.cuda.synchronize()
    rb = b.result()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        a.run(stream=s1.cuda_stream)
        b.run(stream=s2.cuda_stream)
    torch.cuda.synchronize()
    assert same(a.result(), ra) and same(b.result(), rb)
    say("  two streams: both results bitwise equal to sequential calls")


@pytest.mark.parametrize("L,hq,hkv", [(4096, 8, 2), (4096, 6, 2), (40960, 32, 8)],
                         ids=["group4", "group3_odd", "claimed_items"])
def test_prefill_graph_replays_match_eager_calls(L, hq, hkv):
    # group3_odd: the lone head of each group runs paired with itself over two query
    # blocks; claimed_items: 5,120 head-pair items, enough per CU on a 256-CU GPU that
    # the attention's workgroups claim up to two items each from the per-XCD queues
    # (counters zeroed inside the captured work at every replay)
    w = Workload("g", L, hq, hkv, 128, "bf16", 128, 16, (0.9,), 33, "llm", 8)
    job = Job(w)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        job.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        job.run()
    torch.cuda.synchronize()
    for rep in range(3):
        # new inputs in the captured buffers, then the replay, then the eager call on the same inputs
        q, k, v = make_inputs(Workload("g", L, hq, hkv, 128, "bf16", 128, 16, (0.9,), 40 + rep, "llm", 8))
        job.q.copy_(q.cuda())
        job.k.copy_(k.cuda())
        job.v.copy_(v.cuda())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = job.result()
        job.out.fill_(0)
        job.rc.fill_(-1)
        torch.cuda.synchronize()
        job.run()
        torch.cuda.synchronize()
        want = job.result()
        assert same(got, want), rep
    say("  prefill graph: 3 replays on new inputs, each bitwise equal to the eager call")


def test_decode_graph_replays_match_eager_calls():
    w = Workload("gd", 20000, 8, 2, 128, "bf16", 128, 16, (0.9,), 34, "llm", 8)
    Q, K, V = make_inputs(w)
    p = rr.problem(w.L, w.Hq, w.Hkv, w.d, w.S, w.B, 0.9, True, "bf16")
    q, k, v = Q[w.L - 1].contiguous().cuda(), K.cuda(), V.cuda()
    out = torch.empty_like(q)
    rc = torch.empty((w.Hq,), dtype=torch.int32, device="cuda")
    ci = torch.empty((w.Hq, w.nb), dtype=torch.int32, device="cuda")
    ws = torch.empty(rr.rr_decode_workspace_bytes(p), dtype=torch.uint8, device="cuda")

    def run():
        rr.rr_decode(p, q, k, v, out, rc, ci, None, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        q.copy_(Q[w.L - 1 - 7 * (rep + 1)].cuda())  # another query each time
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (out.clone(), rc.clone(), ci.clone())
        out.fill_(0)
        torch.cuda.synchronize()
        run()
        torch.cuda.synchronize()
        assert torch.equal(got[0], out) and torch.equal(got[1], rc)
        for h in range(w.Hq):
            n = int(rc[h])
            assert torch.equal(got[2][h, :n], ci[h, :n])
    say("  decode graph: 3 replays on new queries, each bitwise equal to the eager call")


def test_varlen_graph_replays_match_eager_calls():
    # 17,000 tokens at the 8B shape: a sequence searched and attended in launches of its own;
    # the three short ones searched and attended together
    lens = [17000, 3000, 999, 500]
    shape = dict(Hq=32, Hkv=8)

    def inputs(seed):
        parts = [make_inputs(Workload(f"vg{b}", L, 32, 8, 128, "bf16", 128, 16, (0.9,), seed + b, "llm", 8))
                 for b, L in enumerate(lens)]
        return [torch.cat([x[i] for x in parts]).cuda() for i in range(3)]

    q, k, v = inputs(50)
    p = rr.problem(sum(lens), shape["Hq"], shape["Hkv"], 128, 16, 128, 0.9, True, "bf16")
    nbs = [-(-L // 128) for L in lens]
    rc = torch.empty((sum(32 * n for n in nbs),), dtype=torch.int32, device="cuda")
    ci = torch.empty((sum(32 * n * n for n in nbs),), dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    ws = torch.empty(rr.rr_workspace_bytes_varlen(p, lens), dtype=torch.uint8, device="cuda")

    def run():
        rr.rr_prefill_varlen(p, lens, q, k, v, out, rc, ci, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        nq, nk, nv = inputs(60 + 10 * rep)
        q.copy_(nq)
        k.copy_(nk)
        v.copy_(nv)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (out.clone(), rc.clone(), ci.clone())
        out.fill_(0)
        rc.fill_(-1)
        torch.cuda.synchronize()
        run()
        torch.cuda.synchronize()
        assert same(got, (out, rc, ci)), rep
    say("  varlen graph: 3 replays on new inputs, each bitwise equal to the eager call")
