"""nvfp4_decode_attn_noalloc (decode with the library's fixed per-device
scratch instead of a workspace) against nvfp4_decode_attn: the same kernels
with the same work split, so the outputs must be identical bit for bit; two
calls in a row, the second with a smaller input, and a request beyond the
scratch refused before anything runs."""
import numpy as np
import pytest
import torch

from decode_attention_nvfp4_amd import api
from decode_attention_nvfp4_amd import workloads as W
from gpu_common import BuiltDecode, check_decode, i32, say, to_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def _both(built, q, num_splits=0):
    w = built.w
    qd = to_dev(q, w.dtype)
    lens = i32(w.lens)
    L = int(w.lens.max())
    ref = api.decode(built.cache, qd, built.pt, lens, L, num_splits=num_splits)
    got = api.decode_noalloc(built.cache, qd, built.pt, lens, L, num_splits=num_splits)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy()


def test_noalloc_matches_workspace_decode(orc):
    # first call: 4 ragged sequences, GQA 32/8, permuted pages; second call:
    # a smaller batch of shorter sequences (fewer waves, a smaller scratch
    # share), so stale partials of the first call sit in the scratch
    big = W.custom_decode(41, 4, 32, 8, [2000, 17, 900, 3333], dtype="bf16", outliers=True)
    small = W.custom_decode(42, 2, 16, 4, [40, 301], dtype="bf16")
    for name, w in (("first (B=4)", big), ("second (B=2)", small)):
        built = BuiltDecode(w, orc)
        q = w.q(0)
        say(f"noalloc decode {name}")
        ref, got = _both(built, q)
        assert np.array_equal(ref.view(np.uint32), got.view(np.uint32)), float(np.abs(ref - got).max())
        oref, mag = built.oracle_decode(orc, q, range(w.B))
        say("   ", check_decode(got, oref, mag))
    # an explicit wave count that splits every segment, on the first workload
    built = BuiltDecode(big, orc)
    say("noalloc decode, 700 waves")
    ref, got = _both(built, big.q(0), num_splits=700)
    assert np.array_equal(ref.view(np.uint32), got.view(np.uint32))


def test_noalloc_refuses_more_than_its_scratch(orc):
    w = W.custom_decode(43, 1, 16, 1, [64], dtype="bf16")
    built = BuiltDecode(w, orc)
    q = to_dev(w.q(0), w.dtype)
    need = api.decode_workspace_bytes(1, 16, 1, 64, 9000)
    assert need > api.NOALLOC_SCRATCH_BYTES
    with pytest.raises(api.Nvfp4Error) as e:
        api.decode_noalloc(built.cache, q, built.pt, i32(w.lens), 64, num_splits=9000)
    assert e.value.status == 3
    # the refused call enqueued nothing; the next call works
    ref, got = _both(built, w.q(0))
    assert np.array_equal(ref.view(np.uint32), got.view(np.uint32))
