"""The allocation-free attention call against absa_sparse_attention: the
same plan and inputs must give the same output bit for bit, on two calls in
a row (the second smaller, so the static scratch holds the first call's
data), for fp32 inputs (which go through the scratch) and bf16 inputs."""
import numpy as np
import pytest
import torch

import sampled_block_sparse_amd as absa
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(B, H, N, d, seed, dtype):
    q, k, v = (torch.from_numpy(x) for x in synth.iid_qkv(B, H, N, d, seed))
    if dtype == "bf16":
        q, k, v = (x.to(torch.bfloat16) for x in (q, k, v))
    q, k, v = (x.to(DEV) for x in (q, k, v))
    plan = absa.absa_plan_create(q, k, synth.budget_blocks(15, N // 4), seed)
    return plan, q, k, v


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_noalloc_matches_allocating_call(dtype):
    # 2*3*5000*128 = 3.84M elements (within the 2^22 limit), then a smaller one
    shapes = [(2, 3, 5000, 128, 51), (1, 2, 1340, 64, 52)]
    for B, H, N, d, seed in shapes:
        print(f"[noalloc] {dtype} B={B} H={H} N={N} d={d}", flush=True)
        plan, q, k, v = _case(B, H, N, d, seed, dtype)
        want = absa.absa_sparse_attention(plan, q, k, v)
        got = torch.full_like(q, float("nan"))
        absa.absa_sparse_attention_noalloc(plan, q, k, v, got)
        torch.cuda.synchronize()
        assert torch.equal(got, want)
        plan.destroy()


def test_noalloc_rejects_fp32_beyond_its_scratch():
    B, H, N, d = 1, 1, 32768 + 4, 128         # 4,194,816 elements > 2^22
    q = torch.zeros(B, H, N, d, device=DEV)
    plan = absa.absa_plan_import(np.zeros(B * H * ((N + 127) // 128) + 1, np.int64),
                                 np.zeros(0, np.int32), np.zeros(0, np.float32), None,
                                 B, H, N, d)
    with pytest.raises(absa.AbsaError) as ei:
        absa.absa_sparse_attention_noalloc(plan, q, q, q, torch.empty_like(q))
    assert ei.value.status == absa.ABSA_ERR_UNSUPPORTED
    # bf16 inputs use no scratch: no limit
    qb = q.to(torch.bfloat16)
    out = torch.full_like(qb, 1.0)
    absa.absa_sparse_attention_noalloc(plan, qb, qb, qb, out)
    torch.cuda.synchronize()
    assert not out.any()                        # empty plan rows give zeros
