"""The path's calls captured into one HIP graph (torch.cuda.CUDAGraph on
ROCm) and replayed: prefill (both modes), split-KV decode + merge, the
single-launch multi-latent decode, routing and the no-alloc FP8 cascade. The
library enqueues only kernels on the caller's stream (no allocation, no
memset, no host synchronisation), so every call can be captured. Each replay
runs on fresh inputs copied into the captured buffers, with eager work and a
synchronisation between replays, and must reproduce the eager calls on the
same inputs bit for bit (the kernels are deterministic)."""

import math

import pytest
import torch

import online_softmax_attention_cascaded_amd as rf
from online_softmax_attention_cascaded_amd import inputs
from gpu_util import DEV, needs_gpu, print_case

pytestmark = [pytest.mark.gpu, needs_gpu]

REPLAYS = 4


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


class Path:
    """Static device buffers of every call, one batch of inputs at a time."""

    def __init__(self):
        self.scale = 1 / math.sqrt(128)
        # prefill
        self.q = torch.empty((1, 2, 256, 128), dtype=torch.bfloat16, device=DEV)
        self.k, self.v = torch.empty_like(self.q), torch.empty_like(self.q)
        # decode, S = 4, GQA 4:1
        self.qd = torch.empty((2, 8, 128), dtype=torch.bfloat16, device=DEV)
        self.kd = torch.empty((2, 2, 3000, 128), dtype=torch.bfloat16, device=DEV)
        self.vd = torch.empty_like(self.kd)
        # multi-latent decode, one launch, S = 4
        self.mq = torch.empty((2, 16, 576), dtype=torch.bfloat16, device=DEV)
        self.mkv = torch.empty((2, 1000, 576), dtype=torch.bfloat16, device=DEV)
        # routing
        self.logits = torch.empty((100, 256), device=DEV)
        # FP8 cascade (B quantised once, outside the graph)
        self.a = torch.empty((64, 256), dtype=torch.bfloat16, device=DEV)
        _, bsrc = inputs.quant_inputs(70, 64, 128, 256)
        self.bq, self.bs = rf.absmax_quant_fp8(bsrc.to(DEV))

    def outputs(self):
        o = dict(
            o=torch.empty_like(self.q), lse=torch.empty((1, 2, 256), device=DEV),
            oc=torch.empty_like(self.q), lsec=torch.empty((1, 2, 256), device=DEV),
            pm=torch.empty((2, 8, 4), device=DEV), pl=torch.empty((2, 8, 4), device=DEV),
            pa=torch.empty((2, 8, 4, 128), device=DEV),
            od=torch.empty((2, 8, 128), dtype=torch.bfloat16, device=DEV), lsed=torch.empty((2, 8), device=DEV),
            mpm=torch.empty((2, 16, 4), device=DEV), mpl=torch.empty((2, 16, 4), device=DEV),
            mpa=torch.empty((2, 16, 4, 512), device=DEV), cnt=torch.zeros(2, dtype=torch.int32, device=DEV),
            mo=torch.empty((2, 16, 512), dtype=torch.bfloat16, device=DEV), mlse=torch.empty((2, 16), device=DEV),
            w=torch.empty((100, 8), device=DEV), idx=torch.empty((100, 8), dtype=torch.int32, device=DEV),
            sa=torch.empty(64, device=DEV), c=torch.empty((64, 128), dtype=torch.bfloat16, device=DEV))
        return o

    def load(self, seed):
        q, k, v = inputs.attention_inputs(seed, 1, 2, 2, 256, 256, 128)
        self.q.copy_(q); self.k.copy_(k); self.v.copy_(v)
        qd, kd, vd = inputs.decode_inputs(seed + 1, 2, 8, 2, 3000, 128)
        self.qd.copy_(qd); self.kd.copy_(kd); self.vd.copy_(vd)
        mq, mkv = inputs.mla_inputs(seed + 2, 2, 16, 1000)
        self.mq.copy_(mq); self.mkv.copy_(mkv)
        self.logits.copy_(inputs.routing_inputs(seed + 3, 100, 256))
        a, _ = inputs.quant_inputs(seed + 4, 64, 128, 256)
        self.a.copy_(a)

    def run(self, o):
        rf.rf_attn_fwd(self.q, self.k, self.v, o["o"], o["lse"], self.scale, False)
        rf.rf_attn_fwd(self.q, self.k, self.v, o["oc"], o["lsec"], self.scale, True)
        rf.rf_attn_decode_split(self.qd, self.kd, self.vd, o["pm"], o["pl"], o["pa"], self.scale)
        rf.rf_merge_states(o["pm"], o["pl"], o["pa"], o["od"], o["lsed"])
        rf.rf_mla_decode(self.mq, self.mkv, o["mpm"], o["mpl"], o["mpa"], o["cnt"], o["mo"], o["mlse"],
                         1 / math.sqrt(576))
        rf.rf_softmax_topk(self.logits, 8, True, o["w"], o["idx"])
        rf.rf_absmax_quant_gemm_fp8_noalloc(self.a, self.bq, self.bs, o["sa"], o["c"])


def test_graph_replays_match_eager_calls():
    path = Path()
    captured = path.outputs()
    eager = path.outputs()
    path.load(100)
    path.run(captured)             # warm-up outside the capture (loads the library, first launches)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path.run(captured)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        print_case(test="graph_replay", replay=r)
        path.load(200 + 10 * r)    # eager copies into the captured inputs
        torch.cuda.synchronize()
        for t in captured.values():
            if t.dtype != torch.int32:
                t.fill_(float("nan"))   # nothing left over from the last replay
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        path.run(eager)            # the same calls, eagerly, on the same inputs
        torch.cuda.synchronize()
        for name in captured:
            if name == "cnt":
                assert int(captured[name].abs().sum()) == 0, "counters left non-zero"
                continue
            assert _same(captured[name], eager[name]), f"replay {r}: {name} differs from the eager call"
