"""Two properties the C ABI states for every entry point, checked on the GPU:

* calls on different streams may run at the same time when their buffers do
  not overlap (the library keeps no device state between calls, apart from
  the allocation-free entry point's own array);
* a sequence of calls can be captured into a HIP graph and replayed: the
  library enqueues only kernel launches (no memory sets, copies, allocations
  or host synchronisation), so each replay gives the eager results again.

Both compare bit for bit with the same calls run one after another (every
kernel here takes its decisions in a fixed order, so reruns are bitwise
equal). Workloads: 8B-class heads (32 query / 8 KV heads, d = 128) over a
20,000-row cache with the 24-node tree, the draft over a 4,164-row partial
cache, the selection at budget 2,000, and the logit pass over 8 rows of a
32,000-token vocabulary.
"""

import pytest
import torch

import long_kv_attention_amd as ts
from synth import attention_inputs, penalty_inputs, tree_parent
from tests.gpu_util import banner, dev_bf16

pytestmark = pytest.mark.gpu

HQ, HKV, D, N_CTX, T = 32, 8, 128, 20_000, 24
N_PART, TQ = 4164, 4
BUDGET, N_SINK, N_RECENT = 2000, 4, 64


class _Work:
    """Inputs and preallocated outputs and workspaces of one set of calls."""

    def __init__(self, seed):
        dev = torch.device("cuda:0")
        x = attention_inputs(seed, HQ, HKV, D, N_CTX, T)
        self.q, self.k, self.v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
        xd = attention_inputs(seed + 1, HQ, HKV, D, N_PART, TQ)
        self.qd, self.kp, self.vp = dev_bf16(xd["q"]), dev_bf16(xd["k"]), dev_bf16(xd["v"])
        px = penalty_inputs(seed + 2, 8, 32_000, 256)
        self.logits = torch.from_numpy(px["logits"]).to(dev)
        self.window = torch.from_numpy(px["window"]).to(dev)
        self.u = torch.from_numpy(px["u"]).to(dev)
        self.parent = tree_parent("tokenswift", T)
        L = ts.lib()
        self.out = torch.empty((HQ, T, D), dtype=torch.float32, device=dev)
        self.outd = torch.empty((HQ, TQ, D), dtype=torch.float32, device=dev)
        self.ws_v = torch.zeros(max(1, L.ts_verify_attn_workspace_size(N_CTX, T, HQ, HKV, D, 0)), dtype=torch.uint8,
                                device=dev)
        self.ws_d = torch.zeros(max(1, L.ts_draft_attn_workspace_size(N_PART, TQ, HQ, HKV, D, 0)), dtype=torch.uint8,
                                device=dev)
        self.ws_s = torch.zeros(L.ts_partial_kv_select_workspace_size(N_CTX, T, HQ, HKV, D, BUDGET),
                                dtype=torch.uint8, device=dev)
        self.ws_p = torch.zeros(max(1, L.ts_penalty_sample_workspace_size(8, 32_000)), dtype=torch.uint8, device=dev)
        rows = N_SINK + BUDGET + N_RECENT
        self.k_part = torch.empty((HKV, rows, D), dtype=torch.bfloat16, device=dev)
        self.v_part = torch.empty_like(self.k_part)
        self.sel = torch.empty((HKV, BUDGET), dtype=torch.int32, device=dev)
        self.z = torch.empty_like(self.logits)
        self.tok = torch.empty(8, dtype=torch.int32, device=dev)
        self.keep = self.probs = None   # allocated by the call (inside a capture: by the graph's pool)

    def attention(self, stream=None):
        ts.verify_attn(self.q, self.k, self.v, N_CTX, self.parent, out=self.out, ws=self.ws_v, stream=stream)

    def draft_and_select(self, stream=None):
        ts.draft_attn(self.qd, self.kp, self.vp, N_PART, out=self.outd, ws=self.ws_d, stream=stream)
        ts.partial_kv_select(self.q, self.k, self.v, N_CTX, N_SINK, BUDGET, N_RECENT, k_part=self.k_part,
                             v_part=self.v_part, sel_idx=self.sel, ws=self.ws_s, stream=stream)
        _, self.keep, self.probs, _ = ts.penalty_sample(self.logits, self.window, 1.2, 1.0, 0.9, 0.05, u=self.u,
                                                        out=self.z, token_out=self.tok, ws=self.ws_p, stream=stream)

    def results(self, attention=True, rest=True):
        """Copies of the outputs of the calls that ran (verification, then the
        draft, selection and logit pass)."""
        torch.cuda.synchronize()
        outs = ((self.out,) if attention else ()) + \
               ((self.outd, self.k_part, self.v_part, self.sel, self.z, self.keep, self.probs, self.tok) if rest else ())
        return [t.clone() for t in outs]

    def clear_outputs(self):
        for t in (self.out, self.outd, self.z, self.probs):
            if t is not None:
                t.fill_(float("nan"))
        for t in (self.k_part, self.v_part):
            t.fill_(0)
        for t in (self.sel, self.tok):
            t.fill_(-7)
        if self.keep is not None:
            self.keep.fill_(3)


def _same(a, b):
    assert len(a) == len(b)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.uint8 else x,
                           y.view(torch.uint8) if y.dtype != torch.uint8 else y)


def test_two_streams_at_once():
    """The verification of one input set on one stream and the draft,
    selection and logit pass of another on a second stream, enqueued with
    nothing between them, give the results of running them one after
    another."""
    banner("two streams: verify | draft + select + penalty")
    a, b = _Work(11), _Work(12)
    a.attention()
    b.draft_and_select()
    ref_a, ref_b = a.results(rest=False), b.results(attention=False)
    a.clear_outputs()
    b.clear_outputs()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    torch.cuda.synchronize()
    for _ in range(3):   # each stream's calls in order, the two streams unordered
        a.attention(stream=s1)
        b.draft_and_select(stream=s2)
    torch.cuda.synchronize()
    _same(a.results(rest=False), ref_a)
    _same(b.results(attention=False), ref_b)


def test_graph_capture_and_replay():
    """All four hot-path calls captured into one graph; each of three replays,
    with eager calls on other buffers and host synchronisation between them,
    gives the eager results again."""
    banner("graph capture: verify + draft + select + penalty")
    w, other = _Work(21), _Work(22)
    w.attention()
    w.draft_and_select()
    ref = w.results()
    other.attention()
    other.draft_and_select()
    ref_other = other.results()
    w.clear_outputs()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w.attention()
        w.draft_and_select()
    torch.cuda.synchronize()
    for r in range(3):
        w.clear_outputs()
        g.replay()
        got = w.results()
        _same(got, ref)
        # eager work on other buffers between replays
        other.clear_outputs()
        other.attention()
        other.draft_and_select()
        _same(other.results(), ref_other)
