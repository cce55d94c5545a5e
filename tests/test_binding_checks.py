"""The binding refuses tensors whose shapes do not match the call before any
pointer reaches the library, so a wrong-shaped q, out or table can never send
a kernel past the end of a buffer.  Host only: the tensors live on the CPU and
the checks fire before the device check would."""

import pytest
import torch

import paged_kv_cache_394_amd as pa

H, HKV, D, NB, BS = 4, 2, 64, 8, 16


def cache(fp8=False):
    return pa.KvCache(NB, HKV, D, block_size=BS, fp8=fp8, device="cpu")


def i32(*shape):
    return torch.zeros(shape, dtype=torch.int32)


def f16(*shape):
    return torch.zeros(shape, dtype=torch.float16)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def prefill_args(B=3, total=10):
    return dict(q=f16(total, H, D), cu_q=i32(B + 1), prior=i32(B), tables=i32(B, 4),
                out=f32(total, H, D))


def decode_args(B=3):
    return dict(q=f16(B, H, D), tables=i32(B, 4), lens=i32(B), out=f32(B, H, D))


def call_prefill(c, a):
    pa.pa_prefill_chunk(c, a["q"], a["cu_q"], a["prior"], a["tables"], 8, 0.1, a["out"])


def shape_error(fn, match):
    with pytest.raises(pa.PaError, match=match) as e:
        fn()
    assert e.value.status == pa.PA_ERR_BAD_ARG


@pytest.mark.parametrize("key,bad,match", [
    ("q", f16(10, H, 128), "head_dim"),
    ("q", f16(10, H * D), "q must be"),
    ("cu_q", i32(3), "cu_q"),
    ("prior", i32(3, 1), "prior must be"),
    ("tables", i32(2, 4), "tables must be"),
    ("tables", i32(3), "tables must be"),
    ("out", f32(9, H, D), "out"),
    ("out", f32(10, H - 1, D), "out"),
])
def test_prefill_rejects_bad_shapes(key, bad, match):
    a = prefill_args()
    a[key] = bad
    shape_error(lambda: call_prefill(cache(), a), match)


def test_prefill_shape_check_passes_good_shapes_to_the_device_check():
    # well-shaped CPU tensors get past the shape check and stop at the device check
    with pytest.raises(pa.PaError, match="CUDA tensor"):
        call_prefill(cache(), prefill_args())


@pytest.mark.parametrize("key,bad,match", [
    ("q", f16(3, H, 128), "head_dim"),
    ("tables", i32(4, 4), "tables must be"),
    ("lens", i32(2), "lens"),
    ("out", f32(3, H, D // 2), "out"),
])
def test_decode_rejects_bad_shapes(key, bad, match):
    a = decode_args()
    a[key] = bad
    shape_error(lambda: pa.pa_decode(cache(), a["q"], a["tables"], a["lens"], 64, 0.1, a["out"]), match)


def test_mixed_step_checks_both_halves_and_one_head_count():
    p, d = prefill_args(), decode_args()
    bad = dict(p, out=f32(9, H, D))
    shape_error(lambda: pa.pa_mixed_step(cache(), 0.1, bad, dict(d, max_context_len=64)), "out")
    bad = dict(d, lens=i32(5), max_context_len=64)
    shape_error(lambda: pa.pa_mixed_step(cache(), 0.1, dict(p, max_chunk=8), bad), "lens")
    # a decode batch with fewer heads than the prefill batch would get the
    # prefill's head count in the launch: refused
    fewer = dict(q=f16(3, H // 2, D), tables=i32(3, 4), lens=i32(3), out=f32(3, H // 2, D),
                 max_context_len=64)
    shape_error(lambda: pa.pa_mixed_step(cache(), 0.1, dict(p, max_chunk=8), fewer), "heads")


@pytest.mark.parametrize("fp8", [False, True])
def test_swap_blocks_checks_host_block_bytes(fp8):
    c = cache(fp8)
    dt = torch.uint8 if fp8 else torch.float16
    other = torch.float16 if fp8 else torch.uint8
    pairs = [(0, 0)]
    shape_error(lambda: pa.pa_swap_blocks(c, torch.zeros((4, HKV, BS, D), dtype=other),
                                          torch.zeros((4, HKV, BS, D), dtype=other), pairs, 0), "host blocks must be")
    shape_error(lambda: pa.pa_swap_blocks(c, torch.zeros((4, HKV, BS, D // 2), dtype=dt),
                                          torch.zeros((4, HKV, BS, D // 2), dtype=dt), pairs, 0), r"host blocks must be \[n\]")
    shape_error(lambda: pa.pa_swap_blocks(c, torch.zeros((4 * HKV * BS * D,), dtype=dt),
                                          torch.zeros((4 * HKV * BS * D,), dtype=dt), pairs, 0), r"host blocks must be \[n\]")
    t = torch.zeros((4, HKV, D, BS), dtype=dt).transpose(2, 3)
    shape_error(lambda: pa.pa_swap_blocks(c, t, t, pairs, 0), "contiguous")
