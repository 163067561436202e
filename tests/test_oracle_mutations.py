"""Planted mistakes: each plausible slip in the oracle's C source must fail
one of the pins (brute force, torch library routines, zero-query closed
form).  The mutants are built in a temporary directory; the oracle itself is
untouched."""
import math
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import bruteforce as bf

SRC = os.path.join(os.path.dirname(oracle.__file__), "lt_oracle.c")

MUTANTS = {
    "wrong_k_index": ("acc += qi[d] * kj[d];", "acc += qi[d] * kj[0];"),
    "dropped_scale": ("s[j] = scale * acc;", "s[j] = acc;"),
    "recent_off_by_one": ("return (j < S) || (j > i - R);", "return (j < S) || (j >= i - R);"),
    "sink_off_by_one": ("return (j < S) || (j > i - R);", "return (j <= S) || (j > i - R);"),
    "normalised_by_max": ("p[j] = exp(s[j] - L);", "p[j] = exp(s[j] - m);"),
    "lse_drops_max": ("double L = m + log(sum);", "double L = log(sum);"),
    "mean_over_w_plus_1": ("lazy_ratio[bh] = acc / (double)W;", "lazy_ratio[bh] = acc / (double)(W + 1);"),
    "gqa_map_modulo": ("long b = bh / Hq, h = bh % Hq, hk = h / G;", "long b = bh / Hq, h = bh % Hq, hk = h % Hkv;"),
    "stream_lse_full_max": ("double Ls = ms + log(ss);", "double Ls = m + log(ss);"),
    "lazy_rows_shifted": ("lz = lazy_rows + (size_t)bh * W + (i - (N - W));",
                          "lz = lazy_rows + (size_t)bh * W + ((i + 1) % W);"),
}


def _build(src_text, tmp):
    c = os.path.join(tmp, "m.c")
    so = os.path.join(tmp, "m.so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", so, c, "-lm"],
                   check=True)
    return oracle.load_library(so)


def _pins_pass(lib) -> bool:
    """A compact set of the pins; True when all hold."""
    rng = np.random.default_rng(3)
    # 1. brute force, GQA 4:2, several rows inside and outside the window
    q = rng.standard_normal((1, 4, 9, 3)) * 1.5
    k = rng.standard_normal((1, 2, 9, 3)) * 1.5
    v = rng.standard_normal((1, 2, 9, 3))
    got = oracle.prefill(q, k, v, S=2, R=3, W=4, streaming=True, lib=lib)
    want = bf.attention(q.tolist(), k.tolist(), v.tolist(), S=2, R=3, W=4)
    for key in ("out", "lse", "sout", "slse", "lazy_rows", "lazy_ratio"):
        if not np.allclose(got[key], np.array(want[key], dtype=np.float64), rtol=0, atol=1e-10):
            return False
    # 2. torch SDPA for the output
    g = torch.Generator().manual_seed(1)
    tq = torch.randn(1, 4, 40, 8, generator=g, dtype=torch.float64)
    tk = torch.randn(1, 2, 40, 8, generator=g, dtype=torch.float64)
    tv = torch.randn(1, 2, 40, 8, generator=g, dtype=torch.float64)
    r = oracle.prefill(tq.numpy(), tk.numpy(), tv.numpy(), lib=lib)
    ref = F.scaled_dot_product_attention(tq, tk.repeat_interleave(2, 1), tv.repeat_interleave(2, 1),
                                         is_causal=True)
    if not np.allclose(r["out"], ref.numpy(), atol=1e-10):
        return False
    # 3. zero-query closed form of the per-head ratio
    N, S, R, W = 50, 3, 7, 10
    z = oracle.prefill(np.zeros((1, 1, N, 2)), rng.standard_normal((1, 1, N, 2)),
                       rng.standard_normal((1, 1, N, 2)), S=S, R=R, W=W, full=False, lib=lib)
    rho = sum(min(S + R, i + 1) / (i + 1) for i in range(N - W, N)) / W
    return bool(abs(z["lazy_ratio"][0, 0] - rho) < 1e-12)


def test_unmutated_oracle_passes_pins():
    with open(SRC) as f:
        text = f.read()
    with tempfile.TemporaryDirectory() as tmp:
        assert _pins_pass(_build(text, tmp))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) >= 1, f"mutation site for {name} not found"
    with tempfile.TemporaryDirectory() as tmp:
        assert not _pins_pass(_build(text.replace(old, new), tmp)), f"mutant {name} survived"
