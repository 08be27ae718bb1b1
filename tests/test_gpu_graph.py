"""A whole forward step captured once as a HIP graph and replayed for new
routing: plan, dispatch, prefetch_weight, the grouped FFN and combine have no
host synchronisation and fixed shapes (MoonEP README, item 3: static shapes
remove per-layer host syncs), so the graph stays valid whatever the routing.
Every replay is checked bit for bit against the same step run eagerly, with
eager work and synchronisation between replays."""
import pytest
import torch

import moonep_synth as synth
from gpu_util import buffer_for, dev, dev_bf16, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["mid_r8_s1024_k4_e32", "infer_r8_s128_k8_e256_b4"])
def test_forward_step_graph_replays_equal_eager(name):
    w = synth.WORKLOADS[name]
    log(f"graph {name}")
    routings = [synth.routing(w, t) for t in (0.0, synth.SWEEPS[name][-1], "adv")]
    buf = buffer_for(w)
    plan = buf.new_plan()
    home = [torch.empty((w.E, w.H, w.Hp), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    for i in range(3):
        synth.expert_weights_device(w, i, home[i])
    pool = [torch.zeros((w.R, w.B, w.H, w.Hp), dtype=torch.bfloat16, device="cuda")
            for _ in range(3)]
    x = dev_bf16(synth.hidden(w))
    topk_in = torch.empty((w.R, w.S, w.K), dtype=torch.int32, device="cuda")
    rw_in = torch.empty((w.R, w.S, w.K), dtype=torch.float32, device="cuda")
    x_nvs = torch.empty((w.R, buf.NvS, w.H), dtype=torch.bfloat16, device="cuda")
    rw_nvs = torch.empty((w.R, buf.NvS), dtype=torch.float32, device="cuda")
    z = torch.empty((w.R, buf.NvS, w.Hp), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((w.R, w.S, w.H), dtype=torch.bfloat16, device="cuda")
    rw_sk = torch.empty((w.R, w.S, w.K), dtype=torch.float32, device="cuda")

    def step():
        buf.plan(topk_in, plan=plan)
        buf.dispatch(plan, x, rw_in, x_nvs=x_nvs, rw_nvs=rw_nvs)
        buf.prefetch_weight(plan, home, pool)
        buf.expert_ffn(plan, x_nvs, home, pool, z_ws=z, y_nvs=x_nvs)   # in place
        buf.combine(plan, x_nvs, rw_nvs, out=out, rw_sk=rw_sk)

    refs = []
    for topk, rw in routings:
        topk_in.copy_(dev(topk))
        rw_in.copy_(dev(rw))
        step()
        torch.cuda.synchronize()
        refs.append((out.clone(), rw_sk.clone()))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(2):
        for i, (topk, rw) in enumerate(routings):
            topk_in.copy_(dev(topk))
            rw_in.copy_(dev(rw))
            out.fill_(0)
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), refs[i][0].view(torch.int16)), (rep, i)
            assert torch.equal(rw_sk, refs[i][1]), (rep, i)
            # eager work between replays
            x.add_(0)
            torch.cuda.synchronize()
    del g
    buf.destroy()
