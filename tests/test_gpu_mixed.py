"""The mixed continuous-batching step (pa_mixed_step): prefill chunks and
decode queries over one cache in one launch ([p1] "Chunked Prefill": chunks
are batched with decode requests in the same step).  Its prefill half runs
the 4-wave prefill workgroup body: bit for bit pa_prefill_chunk's result on an
e4m3 cache (the same body there), and within the fp16 tolerance of it on an
fp16 cache (where pa_prefill_chunk runs the 8-wave kernel).  Both halves match
the float64 oracle; decode contexts past the one-launch limit fall back to two
launches, the standalone kernels, with their results bit for bit."""

import numpy as np
import pytest
import torch

import paged_kv_cache_394_amd as pa
import workloads
from gpu_harness import Mixed, close

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dlens", [[1, 0, 37, 300, 1600],          # one block-id register per wave
                                   [5000, 3, 129],                  # two
                                   [10000, 700]])                   # four
def test_mixed_step_matches_separate_calls_and_oracle(dlens):
    wp = workloads.custom_prefill(171, [0, 37, 300], [1, 130, 200], 4, 2, 128)
    wd = workloads.custom_decode(172, dlens, 4, 2, 128)
    m = Mixed(wp, wd)
    outp, outd = m.run_mixed(wp.scale)
    sp, sd = m.run_separate(wp.scale)
    close(outp, sp.astype(np.float64))
    close(outd, sd.astype(np.float64))
    m.check_oracle(outp, outd)


def test_mixed_step_wide_decode_batch_head_dim_64():
    """80 decode sequences (beyond the 64 that are ranked by length inside a
    wave, so they keep batch order), empty and one-token contexts among them,
    beside a prefill batch with a zero-row chunk; head_dim 64, 8 heads."""
    rng = np.random.default_rng(177)
    dl = rng.integers(0, 900, size=80)
    dl[[0, 41, 79]] = [0, 1, 2048]
    wp = workloads.custom_prefill(177, [5, 300, 0, 900], [64, 0, 1, 300], 8, 8, 64)
    wd = workloads.custom_decode(178, dl, 8, 8, 64)
    m = Mixed(wp, wd)
    outp, outd = m.run_mixed(wp.scale)
    sp, sd = m.run_separate(wp.scale)
    close(outp, sp.astype(np.float64))
    close(outd, sd.astype(np.float64))
    assert np.all(outd[0] == 0)
    m.check_oracle(outp, outd)


def test_mixed_step_long_context_falls_back_to_two_launches():
    wp = workloads.custom_prefill(173, [20], [40], 2, 2, 64)
    wd = workloads.custom_decode(174, [17000, 15], 2, 2, 64)
    m = Mixed(wp, wd)
    outp, outd = m.run_mixed(wp.scale)
    sp, sd = m.run_separate(wp.scale)
    assert np.array_equal(outp, sp) and np.array_equal(outd, sd)   # the same two kernels
    m.check_oracle(outp, outd)


def test_mixed_step_with_one_part_empty():
    wp = workloads.custom_prefill(175, [10], [20], 2, 2, 128)
    wd = workloads.custom_decode(176, [50], 2, 2, 128)
    m = Mixed(wp, wd)
    pa.pa_mixed_step(m.cache, wp.scale, m.prefill, None)
    pa.pa_mixed_step(m.cache, wp.scale, None, m.decode)
    torch.cuda.synchronize()
    m.check_oracle(m.prefill["out"].cpu().numpy(), m.decode["out"].cpu().numpy())


@pytest.mark.parametrize("dlens", [[1, 0, 37, 300, 1600], [20000, 70]])
def test_mixed_step_fp8_cache(dlens):
    """An e4m3 cache: the prefill half equals pa_prefill_chunk bit for bit,
    the decode half matches pa_decode, both match the oracle over the
    dequantised cache (20000 tokens: the two-launch form)."""
    wp = workloads.custom_prefill(181, [0, 37, 300], [1, 130, 200], 4, 2, 128)
    wd = workloads.custom_decode(182, dlens, 4, 2, 128)
    m = Mixed(wp, wd, fp8=True)
    outp, outd = m.run_mixed(wp.scale)
    sp, sd = m.run_separate(wp.scale)
    assert np.array_equal(outp, sp)
    close(outd, sd.astype(np.float64))
    m.check_oracle(outp, outd)
