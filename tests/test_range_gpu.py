"""GPU parity at input magnitudes far from unit scale.

nanoGPT's train.py can train in bfloat16 on GPUs (page "nanoGPT: a real GPT
in two 300-line files", section 2 "How the code works"). Read as training
without loss scaling, which bf16's range allows, that hands the backward
upstream gradients dO of about 1e-6 and smaller. bf16 keeps fp32's exponent
range, so the kernels' fp16 matrix-core operands must not lose such values:
each operand block carries a power-of-two scale.

Each case multiplies one input by 2^k, runs forward + backward through the
C ABI and the fp64 oracle on the same (exactly scaled) inputs, and holds
error / s_out to the usual bars, where s_out is the factor the output
scales by (dO by 2^k: dQ, dK, dV by 2^k; V by 2^k: O, dQ, dK by 2^k; Q and K
by 2^k: dQ and dK by 2^k, the softmax itself changes). Scaling dO alone
must scale dK and dV bit for bit (dQ up to the order of its atomic adds).
Inputs whose magnitude varies along the sequence, beyond fp16's range
within one head, are held to max|error| / max|reference| per output.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from causal_self_attention_amd.inputs import WORKLOADS, make_inputs, workload_inputs
from tests.gpu_helpers import TOL, announce, errors, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

# (input names scaled, power of two, per-output scale exponents (multiples of k))
CASES = {
    "do": (("do",), {"o": 0, "lse": 0, "dq": 1, "dk": 1, "dv": 1}),
    "v": (("v",), {"o": 1, "lse": 0, "dq": 1, "dk": 1, "dv": 0}),
    "qk": (("q", "k"), {"o": 0, "lse": 0, "dq": 1, "dk": 1, "dv": 0}),
}


def _scaled(inp: dict, names, k: int) -> dict:
    """inp with the named inputs times 2^k, rounded to their dtype: exact for
    bf16 (fp32's exponent range); for fp16 the values that land among fp16's
    subnormals are rounded, and both sides then take the rounded input."""
    out = dict(inp)
    for n in names:
        out[n] = (inp[n].float() * 2.0 ** k).to(inp[n].dtype)
        if inp[n].dtype == torch.bfloat16:
            assert torch.equal(out[n].float(), inp[n].float() * 2.0 ** k), n
    return out


def _assert_scaled_parity(gpu, ref, dtype, k, exps, label):
    tol = TOL[dtype]
    bad = []
    for name, e in exps.items():
        s = 2.0 ** (k * e)
        d = np.abs(gpu[name].double().numpy() - ref[name]) / s
        mx, mean = float(d.max()), float(d.mean())
        if not np.isfinite(mx) or mx > tol["max"]:
            bad.append(f"{name}: max-abs/scale {mx:.3e} > {tol['max']}")
        if tol["mean"] is not None and mean > tol["mean"]:
            bad.append(f"{name}: mean-abs/scale {mean:.3e} > {tol['mean']}")
    assert not bad, f"{label}: " + "; ".join(bad)


FULL = ["gpt2_124m_bf16_b12_h12_t1024", "gpt2_774m_sharp_bf16_b8_h20_t1024"]


@pytest.mark.parametrize("case,k", [("do", -20), ("do", -24), ("do", 20), ("v", -16),
                                    ("v", 20), ("qk", -16)])
@pytest.mark.parametrize("name", FULL)
def test_scaled_inputs_full_size(name, case, k):
    w = WORKLOADS[name]
    names, exps = CASES[case]
    announce(f"range {name} {case} x 2^{k}")
    inp = _scaled(workload_inputs(w, seed=0), names, k)
    o_lo = w.qk_scale != 1.0  # the sharp workload's dQ needs delta from o + o_lo
    gpu = run_gpu(inp, o_lo=o_lo)
    ref = run_oracle(inp)
    _assert_scaled_parity(gpu, ref, w.dtype, k, exps, f"{name} {case} x 2^{k}")


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 32), ("f16", 64), ("f16", 32)])
@pytest.mark.parametrize("case,k", [("do", -10), ("v", -10), ("qk", -6), ("do", 8),
                                    ("v", 6)])
def test_scaled_inputs_small(dtype, D, case, k):
    """Every 16-bit instantiation; fp16 inputs stay inside fp16's own range."""
    names, exps = CASES[case]
    announce(f"range small dtype={dtype} D={D} {case} x 2^{k}")
    inp = _scaled(make_inputs(2, 3, 333, D, dtype, seed=40), names, k)
    for path in (False, True):
        gpu = run_gpu(inp, o_lo=path)
        _assert_scaled_parity(gpu, run_oracle(inp), dtype, k, exps,
                              f"{dtype} D={D} {case} x 2^{k} o_lo={path}")


@pytest.mark.parametrize("k", [-24, 12])
def test_do_scaling_is_exact(k):
    """Scaling dO by 2^k moves only the dO block exponent: dK and dV scale
    bit for bit, dQ to the order of its fp32 atomic adds, O and LSE do not
    change."""
    announce(f"dO scaling exactness x 2^{k}")
    inp = make_inputs(2, 5, 700, 64, "bf16", seed=41)
    a = run_gpu(inp)
    b = run_gpu(_scaled(inp, ("do",), k))
    for n in ("o", "lse"):
        assert torch.equal(a[n], b[n]), n
    for n in ("dk", "dv"):
        assert torch.equal(a[n] * 2.0 ** k, b[n]), n
    d = float((a["dq"].double() * 2.0 ** k - b["dq"].double()).abs().max())
    assert d <= 1e-6 * 2.0 ** k * float(a["dq"].abs().max())


def _relative_to_max(gpu, ref, bound, label):
    bad = []
    for name, r in ref.items():
        g = gpu[name].double().numpy()
        scale = float(np.abs(r).max())
        rel = float(np.abs(g - r).max()) / scale if scale > 0 else float(np.abs(g).max())
        if not np.isfinite(rel) or rel > bound:
            bad.append(f"{name}: max|err|/max|ref| {rel:.3e} > {bound}")
    assert not bad, f"{label}: " + "; ".join(bad)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("name", ["v", "do", "q"])
def test_magnitude_growing_along_the_sequence(name, D):
    """Row t of one input scaled by 2^(t // 64): every 64-row tile is twice
    the one before, 2^15 from first to last at T = 1000, so no single scale
    fits all of a head in fp16. The forward lowers V's exponent tile by tile
    as larger values arrive; the backward's exponents come from the maxima
    over each workgroup's rows. Bound: max|err| / max|ref| <= 2^-8 per
    output (bf16 keeps 2^-9)."""
    announce(f"growing magnitude along T: {name} D={D}")
    T = 1000
    inp = make_inputs(2, 2, T, D, "bf16", seed=42)
    f = (2.0 ** (torch.arange(T) // 64).double()).view(1, 1, T, 1)
    inp[name] = (inp[name].double() * f).to(torch.bfloat16)
    if name == "q":
        # Keep the scores near unit scale: with K at unit scale the last rows'
        # scores would reach ~3e4, where fp32 accumulation alone leaves ~0.02
        # of absolute error in a score and the softmax gradient follows it.
        inp["k"] = (inp["k"].double() * 2.0 ** -15).to(torch.bfloat16)
    for o_lo in (False, True):
        _relative_to_max(run_gpu(inp, o_lo=o_lo), run_oracle(inp), 2.0 ** -8,
                         f"{name} growing, D={D}, o_lo={o_lo}")


@pytest.mark.parametrize("D", [64, 128])
def test_magnitude_shrinking_and_zero_first_tile(D):
    """V zero on the first 64 keys and tiny (~2^-30) after them: the
    forward's first tile fixes no exponent, the first nonzero tile does."""
    announce(f"zero first tile, tiny V, D={D}")
    inp = make_inputs(1, 3, 300, D, "bf16", seed=43)
    v = inp["v"].double() * 2.0 ** -30
    v[:, :, :64, :] = 0.0
    inp["v"] = v.to(torch.bfloat16)
    gpu, ref = run_gpu(inp), run_oracle(inp)
    _relative_to_max(gpu, ref, 2.0 ** -8, f"zero first tile, D={D}")
    assert torch.equal(gpu["o"][:, :, :64], torch.zeros_like(gpu["o"][:, :, :64]))
