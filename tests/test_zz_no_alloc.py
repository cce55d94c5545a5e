"""pa_decode_noalloc, the decode entry point that allocates nothing: its split
partials live in the library's static per-GPU scratch.  Called through the C
ABI, its output must equal pa_decode's (same kernels) bit for bit and match the
float64 oracle, on two calls in a row, the second with a smaller input, and on
a batch that takes the per-sequence path; a batch whose partials exceed the
scratch is refused before anything is launched."""

import numpy as np
import pytest
import torch

import paged_kv_cache_394_amd as pa
import workloads
from gpu_harness import DecodeCase, close, oracle_decode_all

pytestmark = pytest.mark.gpu


def both(case):
    """(pa_decode with a workspace, pa_decode_noalloc) outputs of one case."""
    ref = case.decode()
    out = torch.full_like(case.out, float("nan"))
    pa.pa_decode_noalloc(case.cache, case.q, case.tables, case.lens, case.max_ctx, case.w.scale, out)
    torch.cuda.synchronize()
    return ref, out.cpu().numpy()


def check(case):
    ref, got = both(case)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    w = case.w
    close(got, oracle_decode_all(w.q, w.kv, w.batch, w.scale))
    return got


def test_two_calls_in_a_row_second_smaller():
    # narrow batch, long contexts: the split path, 18 partials for the longest
    big = workloads.custom_decode(701, [9000, 5000, 8193, 1, 0, 4097], 8, 2, 128)
    assert pa.pa_decode_workspace_bytes(6, 8, 128, 9000) > 0
    got = check(DecodeCase(big))
    assert np.all(got[4] == 0)
    # then a smaller one over the same scratch: fewer partials per sequence
    small = workloads.custom_decode(702, [1500, 513, 40], 4, 4, 64)
    check(DecodeCase(small))


def test_per_sequence_path_and_e4m3():
    rng = np.random.default_rng(703)
    w = workloads.custom_decode(703, rng.integers(1, 700, size=64), 32, 32, 128)
    check(DecodeCase(w))
    w8 = workloads.custom_decode(704, [2000, 700, 3, 1100], 4, 2, 128)
    case = DecodeCase(w8, fp8=True)
    ref, got = both(case)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_oversize_batch_is_refused_before_launch():
    w = workloads.custom_decode(705, [3, 5], 4, 4, 128)
    case = DecodeCase(w)
    out = torch.full_like(case.out, 7.0)
    need = pa.pa_decode_workspace_bytes(2, 4, 128, 1 << 22)
    assert need > pa.PA_DECODE_SCRATCH_BYTES
    with pytest.raises(pa.PaError) as e:
        pa.pa_decode_noalloc(case.cache, case.q, case.tables, case.lens, 1 << 22, w.scale, out)
    assert e.value.name == "capacity"
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)     # nothing ran
