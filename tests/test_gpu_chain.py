"""GPU parity of the chained decode pass (qw_gemv_chain): products in stages,
a later stage reading earlier stages' outputs.

Each product is checked against the oracle on the input it actually read
(the GPU's output of the earlier stage, copied back), to the GEMV bar
|y - y_ref| <= 1e-5 * sum|x * w_hat|; a stage of several products must give
exactly what qw_gemv_batched gives for the same products and inputs, and
two runs must agree bit for bit."""

import numpy as np
import pytest
import torch

import oracle
from int8_int4_dequant_amd import inputs, qw

pytestmark = pytest.mark.gpu


def _recs(bits, group, shapes, seed):
    recs, hosts = [], []
    for i, (n, k) in enumerate(shapes):
        w = inputs.weight([11, seed, i], n, k, 0.05)
        hosts.append(oracle.quantize_pack(w, bits, group))
        recs.append(qw.quantize_pack(torch.from_numpy(w).cuda(), bits, group))
    return recs, hosts


def _run_and_check(recs, hosts, wiring, stages, m, k0, seed):
    """wiring[i]: -1 = the pass input, else the product whose y is x_i."""
    x0 = torch.from_numpy(inputs.activations([11, seed, 99], m, k0)).cuda()
    ys = [torch.empty((m, h["shape"][0]), dtype=torch.float32, device="cuda") for h in hosts]
    xs = [x0 if src < 0 else ys[src] for src in wiring]
    outs = []
    for _ in range(2):
        for y in ys:
            y.fill_(float("nan"))
        qw.gemv_chain(recs, xs, ys, stages)
        torch.cuda.synchronize()
        outs.append([y.cpu().numpy().copy() for y in ys])
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    # a stage of several products against qw_gemv_batched on the same inputs
    for st in sorted(set(stages)):
        idx = [i for i, s_ in enumerate(stages) if s_ == st]
        if len(idx) < 2:
            continue
        ins = [x0.clone() if wiring[i] < 0 else torch.from_numpy(outs[0][wiring[i]]).cuda()
               for i in idx]
        outb = qw.gemv_batched([recs[i] for i in idx], ins)
        torch.cuda.synchronize()
        for i, yb in zip(idx, outb):
            assert np.array_equal(yb.cpu().numpy().view(np.uint32), outs[0][i].view(np.uint32))
    got = outs[0]
    x0h = x0.cpu().numpy()
    for i, (h, src) in enumerate(zip(hosts, wiring)):
        xin = x0h if src < 0 else got[src]
        ref = oracle.gemv_ref(h, xin)
        base = oracle.error_base(h, xin)
        assert np.all(np.abs(got[i] - ref) <= 1e-5 * base), i


@pytest.mark.parametrize("bits,group", [(4, 32), (8, 64)])
@pytest.mark.parametrize("m", [1, 3, 8])
def test_small_chain(bits, group, m):
    # stage 0: A, B read the input; stage 1: C reads A; stage 2: D reads C, E reads B
    shapes = [(96, 64), (64, 64), (80, 96), (64, 80), (40, 64)]
    wiring = [-1, -1, 0, 2, 1]
    stages = [0, 0, 1, 2, 2]
    recs, hosts = _recs(bits, group, shapes, bits * 10 + m)
    _run_and_check(recs, hosts, wiring, stages, m, 64, bits * 10 + m)


def test_stage_numbers_need_not_be_dense():
    shapes = [(64, 64), (64, 64), (64, 64)]
    recs, hosts = _recs(4, 32, shapes, 5)
    _run_and_check(recs, hosts, [-1, 0, 1], [3, 7, 100], 2, 64, 5)


def test_two_layers_of_the_7b_stack():
    """q, k, v from the input; o from v; gate and up from o; down from up;
    then the next layer from down's output (int4 g32, M = 1)."""
    d, f = 4096, 11008
    shapes, wiring, stages = [], [], []
    for layer in range(2):
        base = len(shapes)
        src = -1 if layer == 0 else base - 1
        shapes += [(d, d)] * 4 + [(f, d)] * 2 + [(d, f)]
        wiring += [src, src, src, base + 2, base + 3, base + 3, base + 5]
        stages += [4 * layer] * 3 + [4 * layer + 1] + [4 * layer + 2] * 2 + [4 * layer + 3]
    recs, hosts = _recs(4, 32, shapes, 7)
    _run_and_check(recs, hosts, wiring, stages, 1, d, 7)


def test_rejects_bad_stage_lists():
    recs, _ = _recs(4, 32, [(64, 64)] * 2, 9)
    x = torch.zeros((1, 64), device="cuda")
    ys = [torch.empty((1, 64), device="cuda") for _ in range(2)]
    arr, cnt = qw.make_gemv_descs((4, 32, 64, 64, r["payload"], r["scales"], x, y)
                                  for r, y in zip(recs, ys))
    assert qw.qw_gemv_chain(cnt, arr, [1, 0], 1) == -7
    assert qw.qw_gemv_chain(cnt, arr, [0, 1], 9) == -4


def test_zero_fill_waits_for_its_stage():
    """A product with k == 0 writes zeros to its y in its own stage: when an
    earlier stage reads that buffer as x, it still sees the values it held
    before the call (the fill is not hoisted in front of stage 0)."""
    m, n, k = 2, 64, 64
    recs, hosts = _recs(4, 32, [(n, k)], 13)
    x_host = inputs.activations([11, 13, 5], m, k)
    z = torch.from_numpy(x_host).cuda()          # read in stage 0, zeroed in stage 1
    y0 = torch.full((m, n), float("nan"), device="cuda")
    empty = dict(bits=4, group=32, shape=[k, 0],
                 payload=torch.empty(0, dtype=torch.uint8, device="cuda"),
                 scales=torch.empty(0, dtype=torch.float32, device="cuda"))
    x_empty = torch.empty((m, 0), dtype=torch.float32, device="cuda")
    qw.gemv_chain([recs[0], empty], [z, x_empty], [y0, z], [0, 1])
    torch.cuda.synchronize()
    got = y0.cpu().numpy()
    ref = oracle.gemv_ref(hosts[0], x_host)
    assert np.all(np.abs(got - ref) <= 1e-5 * oracle.error_base(hosts[0], x_host))
    assert torch.count_nonzero(z).item() == 0
