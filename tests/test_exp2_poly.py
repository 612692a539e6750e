"""exp2_poly (csrc/exp2_poly.h): Cody-Waite reduction plus a degree-3
minimax polynomial for 2^x, the software exponential of the FlashAttention-4
section of the cheat sheet.

CPU: the header's coefficients are the Remez fit that gen_exp2_poly.py
computes, and in exact arithmetic that polynomial stays within 7.5e-5 of 2^f
on [-1/2, 1/2] (against numpy's exp2 in fp64, independently of the fit).
GPU (through libattn_micro.so): the device function, fp32 roundings included,
stays within its stated bound 1e-4 of fp64 exp2 over [-125, 64], and within
that bound of v_exp_f32; every x below -125, -inf included, gives a
non-negative value below 2^-124 (never a NaN).
"""

import os
import re
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_io_aware_27_amd", "csrc")
BOUND = 1e-4  # kExp2PolyRelErr in exp2_poly.h


def header_coefficients():
    text = open(os.path.join(CSRC, "exp2_poly.h")).read()
    c = [float(re.search(r"kExp2C%d\s*=\s*([0-9.eE+-]+)f" % i, text).group(1)) for i in range(4)]
    b = float(re.search(r"kExp2PolyRelErr\s*=\s*([0-9.eE+-]+)f", text).group(1))
    return c, b


def test_header_holds_the_generated_fit():
    out = subprocess.check_output([sys.executable, os.path.join(CSRC, "gen_exp2_poly.py"), "3"], text=True)
    gen = [float(m) for m in re.findall(r"c\d = ([0-9.eE+-]+)f", out)]
    c, b = header_coefficients()
    assert np.float32(gen).tolist() == np.float32(c).tolist()
    assert b == BOUND


def test_polynomial_error_in_exact_arithmetic():
    c, _ = header_coefficients()
    f = np.linspace(-0.5, 0.5, 1000001)
    rel = np.abs(np.polyval(c[::-1], f) / np.exp2(f) - 1)
    assert rel.max() <= 7.5e-5, rel.max()
    # equioscillation: a minimax fit of degree 3 touches its error bound at 5 points
    assert rel.max() >= 7.4e-5


@pytest.mark.gpu
def test_device_exp2_poly_within_its_bound():
    import torch
    from exact_io_aware_27_amd import micro

    xs = np.concatenate([np.linspace(-125.0, 64.0, 2000001),
                         np.arange(-125, 65, dtype=np.float64),           # integers: f = 0
                         np.arange(-125, 64, dtype=np.float64) + 0.5,     # rounding ties of j
                         [0.0, -0.0, 1e-7, -1e-7, 16.0, -16.0]])
    x = torch.tensor(xs, dtype=torch.float32, device="cuda:0")
    poly, hw = micro.exp2(x)
    torch.cuda.synchronize()
    xf = x.double().cpu().numpy()  # the fp32 inputs the device saw
    ref = np.exp2(xf)
    p, h = poly.double().cpu().numpy(), hw.double().cpu().numpy()
    rel_poly = np.abs(p / ref - 1)
    rel_hw = np.abs(h / ref - 1)
    print("exp2_poly max rel err %.3g, v_exp_f32 max rel err %.3g" % (rel_poly.max(), rel_hw.max()))
    assert rel_poly.max() <= BOUND
    assert np.abs(p / h - 1).max() <= BOUND + rel_hw.max()
    # below the domain: tiny, non-negative, never NaN
    low = torch.cat([torch.linspace(-130.0, -125.0, 10001, dtype=torch.float32),
                     torch.tensor([-200.0, -1e30, float("-inf")])]).to("cuda:0")
    pl, _ = micro.exp2(low)
    torch.cuda.synchronize()
    assert ((pl >= 0) & (pl < 2.0 ** -124)).all()
