"""GPU parity of the channel-mixing layer (etp_channel_mix, matrix cores)
against the float64 oracle; bar 1e-5 per output tensor (max |gpu - oracle| /
max |oracle|)."""
import numpy as np
import pytest

import oracle
import workloads

from gpu_common import FP32_TOL, dev, np_, rel_err

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def mix_case(L, C, n, seed):
    g = workloads.rng(seed, "x")
    d = oracle.dims(L)
    inp = g.standard_normal((n, d["Dout"], C)).astype(np.float32)
    W = (g.standard_normal(sum(oracle.mix_rows(L)) * C * C) / np.sqrt(C)).astype(np.float32)
    return inp, W


@pytest.mark.parametrize("L,C,n", [(0, 8, 5), (1, 5, 7), (1, 1, 3), (2, 64, 33), (2, 128, 70), (3, 40, 11),
                                   (4, 16, 9), (2, 200, 13), (3, 256, 6)])
def test_channel_mix_small(L, C, n):
    import torch
    from equivariant_interatomic_potentials_amd import etp
    say("mix", L, C, n)
    inp, W = mix_case(L, C, n, seed=L * 1000 + C + n)
    plan = etp.etp_plan_create(L, C)
    assert etp.mix_rows(plan) == oracle.mix_rows(L)
    out = torch.full((n, (L + 1) ** 2, C), float("nan"), device="cuda")
    etp.etp_channel_mix(plan, dev(inp), dev(W), out)
    ref = oracle.channel_mix(L, inp, W)
    assert rel_err(np_(out), ref) < FP32_TOL, rel_err(np_(out), ref)


def test_channel_mix_accumulate_and_empty():
    import torch
    from equivariant_interatomic_potentials_amd import etp
    L, C, n = 2, 96, 20
    say("mix-accumulate")
    inp, W = mix_case(L, C, n, seed=5)
    plan = etp.etp_plan_create(L, C)
    base = np.random.default_rng(1).standard_normal((n, (L + 1) ** 2, C)).astype(np.float32)
    out = dev(base)
    etp.etp_channel_mix(plan, dev(inp), dev(W), out, flags=etp.ETP_FLAG_ACCUMULATE)
    ref = base + oracle.channel_mix(L, inp, W)
    assert rel_err(np_(out), ref) < FP32_TOL
    empty = torch.zeros(0, device="cuda")
    etp.etp_channel_mix(plan, empty.reshape(0, oracle.dims(L)["Dout"], C), dev(W), empty.reshape(0, 9, C))


def test_channel_mix_micro_shape():
    """The micro workload's node count and width (1024 nodes, C=128, l_max=2)."""
    import torch
    from equivariant_interatomic_potentials_amd import etp
    L, C, n = 2, 128, 1024
    say("mix-micro")
    inp, W = mix_case(L, C, n, seed=2)
    plan = etp.etp_plan_create(L, C)
    out = torch.empty((n, (L + 1) ** 2, C), device="cuda")
    etp.etp_channel_mix(plan, dev(inp), dev(W), out)
    ref = oracle.channel_mix(L, inp, W)
    assert rel_err(np_(out), ref) < FP32_TOL


@pytest.mark.parametrize("L,C,n", [(0, 8, 5), (1, 5, 7), (2, 64, 33), (2, 128, 70), (3, 40, 11), (4, 16, 9),
                                   (2, 200, 13), (3, 256, 6)])
def test_channel_mix_vjp(L, C, n):
    import torch
    from equivariant_interatomic_potentials_amd import etp
    say("mix vjp", L, C, n)
    _, W = mix_case(L, C, n, seed=L * 1000 + C + n)
    gy = workloads.rng(L + C + n, "G").standard_normal((n, (L + 1) ** 2, C)).astype(np.float32)
    plan = etp.etp_plan_create(L, C)
    gin = torch.full((n, plan.dout_rows, C), float("nan"), device="cuda")
    etp.etp_channel_mix_vjp(plan, dev(gy), dev(W), gin)
    ref = oracle.channel_mix_vjp(L, gy, W)
    assert rel_err(np_(gin), ref) < FP32_TOL, rel_err(np_(gin), ref)
    base = np.random.default_rng(0).standard_normal(ref.shape).astype(np.float32)
    acc = dev(base)
    etp.etp_channel_mix_vjp(plan, dev(gy), dev(W), acc, etp.ETP_FLAG_ACCUMULATE)
    assert rel_err(np_(acc), ref + base) < FP32_TOL
