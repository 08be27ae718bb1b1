"""moonep_prefetch_weight on the GPU: every used prefetch row becomes a bit
copy of its home row (gate, up and down); unused rows are not written."""
import numpy as np
import pytest
import torch

import moonep_synth as synth
import oracle
from gpu_util import buffer_for, dev, dev_bf16, host_bf16, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,target,num_cus", [
    ("tiny_r4_s64_k2_e8", 1.0, 0), ("tiny_r4_s64_k2_e8", "adv", 0),
    ("mid_r8_s1024_k4_e32", 2.0, 0), ("mid_r8_s1024_k4_e32", 0.0, 0),
    ("mid_r8_s1024_k4_e32", 2.0, 3),                   # CU budget: workgroups loop over chunks
    ("infer_r8_s128_k8_e256_b4", 4.0, 0)])
def test_prefetch_rows_equal_home_rows(name, target, num_cus):
    w = synth.WORKLOADS[name]
    log(f"prefetch {name} target={target} num_cus={num_cus}")
    topk, _ = synth.routing(w, target)
    p = oracle.plan(topk, w.E, w.B, w.token_padding)
    buf = buffer_for(w, num_cus=num_cus)
    plan = buf.plan(dev(topk))
    if w.H * w.Hp * w.E <= 1 << 26:
        home_h = [synth.expert_weights_host(w, i) for i in range(3)]
        home = [dev_bf16(h) for h in home_h]
    else:
        home = [torch.empty((w.E, w.H, w.Hp), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
        for i in range(3):
            synth.expert_weights_device(w, i, home[i])
        home_h = None
    pool = [torch.full((w.R, w.B, w.H, w.Hp), 0x7F7F, dtype=torch.int16, device="cuda")
            .view(torch.bfloat16) for _ in range(3)]
    buf.prefetch_weight(plan, home, pool)
    torch.cuda.synchronize()
    for i in range(3):
        for d in range(w.R):
            for j in range(w.B):
                e = p.prefetch_src[d, j]
                got = host_bf16(pool[i][d, j])
                if e >= 0:
                    want = home_h[i][e] if home_h is not None else host_bf16(home[i][e])
                    assert np.array_equal(got, want), (i, d, j)
                else:
                    assert (got == 0x7F7F).all(), (i, d, j)
    buf.destroy()
