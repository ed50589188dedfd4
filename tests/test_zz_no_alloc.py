"""vitenc_op_attention_noalloc (the attention step with its partial results in
the library's fixed device array, for callers that cannot allocate) against
vitenc_op_attention (the same kernels with a caller scratch): bit for bit, on
calls in a row whose inputs shrink, so the second reuses what the first left
in the array."""
import numpy as np
import pytest

from vision_transformer_amd import workloads as W

from gpu_util import say

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

# each needs scratch: split late query tiles plus the CLS rows (the 4097-token
# block-causal clip at 16 heads: 23 MiB; two of them: 47 MiB), then smaller
# calls, then an fp32 image whose rows are all split over runs of keys
CASES = [
    dict(dtype=W.DTYPE_BF16, B=2, H=16, N=1 + 16 * 256, hd=64, mode=1, p=1, S=256),
    dict(dtype=W.DTYPE_BF16, B=1, H=16, N=1 + 16 * 256, hd=64, mode=1, p=1, S=256),
    dict(dtype=W.DTYPE_BF16, B=1, H=2, N=1 + 4 * 300, hd=64, mode=1, p=1, S=300),
    dict(dtype=W.DTYPE_F16, B=1, H=3, N=1 + 5 * 64, hd=32, mode=1, p=1, S=64),
    dict(dtype=W.DTYPE_F32, B=1, H=3, N=257, hd=64, mode=0, p=1, S=0),
]


def _inputs(case, seed):
    from vision_transformer_amd import vitenc as V
    B, H, N, hd = case["B"], case["H"], case["N"], case["hd"]
    g = torch.Generator(device="cuda").manual_seed(seed)
    td = V.torch_dtype(case["dtype"])
    q = torch.randn((B, H, N, hd), device="cuda", generator=g).to(td)
    k = torch.randn((B, H, N, hd), device="cuda", generator=g).to(td)
    ldv = (N + 63) // 64 * 64
    vt = torch.zeros((B, H, hd, ldv), device="cuda", dtype=td)
    vt[..., :N] = torch.randn((B, H, hd, N), device="cuda", generator=g).to(td)
    return q, k, vt


def test_noalloc_matches_scratch_entry_point(gpu_lib):
    from vision_transformer_amd import vitenc as V
    for i, case in enumerate(CASES):
        say(f"noalloc attention call {i}: {case}")
        nf = gpu_lib.vitenc_attention_scratch_floats(case["dtype"], case["B"], case["N"], case["H"], case["hd"],
                                                     case["mode"], case["p"], case["S"])
        assert 0 < nf <= (16 << 20)
        q, k, vt = _inputs(case, 100 + i)
        ref = V.op_attention(case["dtype"], q, k, vt, case["mode"], case["p"], case["S"])
        got = V.op_attention_noalloc(case["dtype"], q, k, vt, case["mode"], case["p"], case["S"])
        torch.cuda.synchronize()
        assert torch.isfinite(got.float()).all()
        assert torch.equal(ref, got), (ref.float() - got.float()).abs().max().item()


def test_noalloc_refuses_calls_beyond_the_array(gpu_lib):
    from vision_transformer_amd import vitenc as V
    # prefix rows over 2^20 keys at 4 x 16 heads need 17.3 M floats of partials
    B, N, H, hd = 4, 1 + (1 << 20), 16, 64
    nf = gpu_lib.vitenc_attention_scratch_floats(W.DTYPE_BF16, B, N, H, hd, 0, 1, 0)
    assert nf > (16 << 20)
    dummy = 256  # never dereferenced: the call is refused before any device work
    st = gpu_lib.vitenc_op_attention_noalloc(W.DTYPE_BF16, dummy, dummy, dummy, B, N, H, hd, 0, 1, 0, dummy, None)
    assert st == 6, st  # VITENC_EUNSUPPORTED
    assert b"fixed array" in gpu_lib.vitenc_error_text()
