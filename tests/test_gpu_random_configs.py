"""GPU parity over seeded random layer shapes: every entry point against the
oracle, as in test_gpu_parity's small layers, on configurations drawn from
the space the ABI accepts (expert and group counts, groups kept, k, widths,
token counts, weight types)."""

import numpy as np
import pytest
import torch

from non_gated_relu_amd import binding
from non_gated_relu_amd.synthetic import Workload
from test_gpu_parity import test_small_layer_every_entry_point as _check_layer

pytestmark = pytest.mark.gpu

DTYPES = [("f32", "f32", None), ("bf16", "bf16", None), ("bf16", "fp8", None),
          ("bf16", "fp4", "fp4"), ("bf16", "fp4", None)]


def _configs(n=30, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([16, 32, 48, 64, 128, 256]))
        groups = [g for g in (1, 2, 4, 8, 16) if E % g == 0]
        G = int(rng.choice(groups))
        tg = int(rng.integers(1, G + 1))
        k = int(rng.integers(1, min(tg * (E // G), 32) + 1))
        act, exp, sh = DTYPES[i % len(DTYPES)]
        d = int(rng.choice([64, 128, 192, 256, 512]))
        inter = int(rng.choice([64, 128, 192, 320, 448]))
        shared = int(rng.choice([0, 64, 192, 384]))
        T = int(rng.integers(1, 400))
        name = f"rand{i}-{exp}-T{T}-E{E}-G{G}-tg{tg}-k{k}-d{d}-I{inter}-Is{shared}"
        out.append(Workload(name, T, d, E, G, tg, k, inter, shared, act, exp, seed=100 + i,
                            shared_dtype=sh if shared else None))
    return out


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    binding.lib()


@pytest.mark.parametrize("wl", _configs(), ids=lambda w: w.name)
def test_random_layer_every_entry_point(wl):
    _check_layer(wl)
