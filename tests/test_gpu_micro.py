"""The microbenchmarks of libfa_micro.so (include/fa_micro.h) run on the device and give sane figures.

They are measurement tools: these tests run every mode at small sizes and check what can be checked
without assuming a clock -- the kernels finish, their outputs are finite, the clock stamps give a
plausible shader clock, MFMA rates lie between a fifth of and the clock's full rate, and the atomic
adds add exactly what they should.
"""

import pytest
import torch

from exact_tiled_attention_13_amd import micro
from parity_util import DEV

pytestmark = pytest.mark.gpu


def _sane_rate(r):
    assert 0.5 < r["clock_ghz"] < 3.0, r
    assert 0.2 < r["util_at_clock"] <= 1.05, r


@pytest.mark.parametrize("mode", [0, 1, 2, 3, 4, 5])
def test_mfma_modes(mode):
    r = micro.mfma_bf16(DEV, blocks_per_cu=2, iters=2000, reps=1, mode=mode)
    print(f"mfma mode {mode}: {r}", flush=True)
    _sane_rate(r)


@pytest.mark.parametrize("waves", [1, 2])
@pytest.mark.parametrize("nfma,nexp", [(0, 0), (4, 0), (0, 2), (4, 2)])
def test_mfma_with_valu(nfma, nexp, waves):
    r = micro.mfma_with_valu(DEV, nfma, nexp, iters=1000, reps=1, waves_per_simd=waves)
    print(f"mfma + valu {nfma} fma {nexp} exp, {waves} waves/SIMD: {r}", flush=True)
    _sane_rate(r)


def test_exp2_rate():
    r = micro.exp2_rate(DEV, blocks_per_cu=2, iters=1000, reps=1)
    print(f"v_exp_f32: {r}", flush=True)
    assert 0.5 < r["clock_ghz"] < 3.0
    assert 1.0 < r["clocks_per_wave_instr"] < 64.0


def test_atomic_add_adds_exactly():
    n, reps = 1 << 20, 3
    buf = torch.zeros(n, dtype=torch.float32, device=DEV)
    st = micro.lib().fa_micro_atomic_add(buf.data_ptr(), n, reps, torch.cuda.current_stream(DEV).cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(buf, torch.full_like(buf, float(reps)))
