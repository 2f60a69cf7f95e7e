"""Shared helpers of the GPU parity tests: upload seeded inputs, run an entry
point through the C ABI binding, compare with the oracle."""
import numpy as np

import oracle
import synth

BITS = {"u1": 1, "u2": 2, "t5": 0}


def torch_mod():
    import torch
    return torch


def dev(a):
    torch = torch_mod()
    if a is None:
        return None
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def to_np(t):
    return t.detach().cpu().numpy()


def upload(inp):
    return dev(inp.x), dev(inp.w), dev(inp.scales), dev(inp.biases)


def run_entry(entry, inp, x=None, w=None, s=None, b=None, poison_bias=False):
    """Runs one entry point on the inputs; returns y as float64 numpy."""
    import bit_quantized_decode_qmv_amd as bq
    torch = torch_mod()
    xd, wd, sd, bd = upload(inp)
    xd = x if x is not None else xd
    wd = w if w is not None else wd
    sd = s if s is not None else sd
    bd = b if b is not None else bd
    gs = inp.group_size
    bits = BITS[inp.fmt]
    if poison_bias:
        bd = torch.full_like(sd, float("nan"))
    if entry == "qmv":
        y = bq.qmv(xd, wd, sd, bd, bits, gs)
    elif entry == "qmv_wide":
        y = bq.qmv_wide(xd, wd, sd, bd, bits, gs)
    elif entry == "qmv_sym":
        y = bq.qmv_sym(xd, wd, sd, bits, gs, biases=bd)
    elif entry == "t5_qmv":
        y = bq.t5_qmv(xd, wd, sd, gs, biases=bd)
    elif entry == "t5_qmv_wide":
        y = bq.t5_qmv_wide(xd, wd, sd, gs, biases=bd)
    elif entry == "t5_qmm":
        y = bq.t5_qmm(xd, wd, sd, gs, biases=bd)
    elif entry == "qmm":
        y = bq.qmm(xd, wd, sd, bits, gs, biases=bd)
    else:
        raise ValueError(entry)
    torch.cuda.synchronize()
    return to_np(y).astype(np.float64)


def reference(inp, rows=None, biases="stored"):
    b = inp.biases if biases == "stored" else None
    return oracle.qmv_reference(inp.fmt, inp.x, inp.w, inp.scales, b, inp.K, inp.group_size, rows)


def assert_close(y, inp, rows=None, what=""):
    y_ref, mass = reference(inp, rows)
    if rows is not None:
        y = y[:, rows]
    ok, worst = oracle.check_close(y, y_ref, mass)
    assert ok, f"{what}: worst |err|/tol = {worst:.3g}"
    return worst


def make(fmt, M, N, K, gs, variant=None, seed=0):
    return synth.make_inputs(fmt, M, N, K, gs, variant or synth.default_variant(fmt), seed)
