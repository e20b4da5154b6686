"""A seeded sweep of shapes, dtypes and backward designs against the double-precision oracle (needs
an MI355X).

The cases are drawn once, from a fixed seed, over the space the ABI supports: head_dim 32, 64, 128;
group sizes 1-8; one to four (batch, KV head) groups (few groups make the host plans split the
longest causal blocks over several workgroups, or run single dK/dV key blocks); ragged T up to 1500;
bf16 and fp16 inputs with fp32 or 16-bit outputs; the three backward designs; RoPE on or off.  Bars
and the zero-reference scale are those of test_gpu_parity.
"""
import numpy as np
import pytest
import torch

from causal_gqa_flashattention_rope_amd import binding, inputs
from tests.test_gpu_parity import BWD_FLAGS, parity

pytestmark = pytest.mark.gpu


def _cases(n=24, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D = int(rng.choice([32, 64, 128]))
        G = int(rng.choice([1, 2, 3, 4, 6, 8]))
        Hkv = int(rng.integers(1, 3))
        B = int(rng.integers(1, 3))
        T = int(rng.integers(1, 1501)) if i % 4 else int(rng.integers(1, 130))
        in_dt = [torch.bfloat16, torch.float16][int(rng.integers(0, 2))]
        out_dt = torch.float32 if rng.random() < 0.6 else in_dt
        flags = BWD_FLAGS[int(rng.integers(0, 3))]
        base = float(rng.choice([1.0e4, 5.0e5, 0.0]))
        out.append((B, T, G * Hkv, Hkv, D, in_dt, out_dt, flags, base, 7000 + i))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}T{c[1]}Hq{c[2]}Hkv{c[3]}D{c[4]}-{str(c[5])[6:]}-{str(c[6])[6:]}-f{c[7]}-b{c[8]:g}"
                                             for c in CASES])
def test_sweep_parity(case):
    B, T, Hq, Hkv, D, in_dt, out_dt, flags, base, seed = case
    q, k, v, dO = inputs.random_case(B, T, Hq, Hkv, D, seed=seed, dtype="bf16" if in_dt == torch.bfloat16 else "f16")
    parity(q, k, v, dO, base, out_dt, in_dt, flags=flags)


def test_sweep_covers_the_plans_and_designs():
    """The drawn cases include every head_dim, every backward design, 16-bit outputs, no-RoPE calls,
    single-group calls long enough for the plans to split, and T = 1-class short sequences."""
    Ds = {c[4] for c in CASES}
    flags = {c[7] for c in CASES}
    assert Ds == {32, 64, 128} and flags == set(BWD_FLAGS)
    assert any(c[6] != torch.float32 for c in CASES) and any(c[8] == 0.0 for c in CASES)
    assert any(c[0] * c[3] == 1 and c[1] > 600 for c in CASES)
    assert any(c[1] < 130 for c in CASES)
