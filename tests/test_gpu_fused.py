"""The fused plan path (score pass 2 and the SIP count in one kernel, two
query blocks per workgroup, their score rows on chip) against the two-pass
path and the oracle: the plans must be identical bit for bit, since the
fused kernel computes the same fp32 scores and runs the same water-filling
and draws on them [hamidun, "Three techniques in AB-Attention", IBCS and SIP
paragraphs]."""
import numpy as np
import pytest
import torch

import oracle
import sampled_block_sparse_amd as absa
import synth
from tests.gpu_util import check_output, check_plan_exact, oracle_plan_of, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _qk(B, H, N, d, dtype, seed):
    q, k, v = (torch.from_numpy(x) for x in synth.iid_qkv(B, H, N, d, seed))
    if dtype == "bf16":
        q, k, v = (x.to(torch.bfloat16) for x in (q, k, v))
    return q, k, v


FUSED_CASES = [
    # (B, H, N, d, dtype, C, budget %, sampling)
    (1, 2, 1340, 128, "bf16", 8, 10, "poisson"),     # odd QB = 11, M = 335 (ragged tile)
    (1, 3, 5000, 64, "f32", 4, 10, "systematic"),    # d = 64, exponent groups of 8 blocks
    (2, 1, 3000, 128, "bf16", 3, 25, "poisson"),     # C = 3 (one empty cluster slot)
    (1, 2, 700, 128, "bf16", 1, 50, "systematic"),   # C = 1, groups of 32 blocks
    (1, 2, 1024, 64, "bf16", 2, 100, "poisson"),     # budget 100%: every p = 1
    (1, 2, 2000, 128, "bf16", 5, 10, "systematic"),  # C = 5
    (1, 2, 8192, 128, "bf16", 8, 10, "poisson"),     # the small layer's shape
    (1, 1, 80896, 128, "bf16", 8, 10, "poisson"),    # M = 20224, the longest fused row
    (1, 2, 1024, 128, "bf16", 8, 100, "systematic"),  # budget 100% under the fixed-size design
    (1, 1, 4, 128, "bf16", 8, 100, "poisson"),       # N = 4: one KV block, one query block
    (2, 1, 260, 64, "f32", 8, 50, "systematic"),     # QB = 3 per head: one lone row per head
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: "-".join(map(str, c)))
def test_fused_plan_is_bit_identical(case):
    B, H, N, d, dtype, C, pct, sampling = case
    print(f"[fused] {case}", flush=True)
    q, k, _ = _qk(B, H, N, d, dtype, seed=N + C)
    qd, kd = q.to(DEV), k.to(DEV)
    M = N // 4
    budget = synth.budget_blocks(pct, M)
    seed = synth.sip_seed(C)
    two = absa.absa_plan_create(qd, kd, budget, seed, n_clusters=C, sampling=sampling).export()
    one = absa.absa_plan_create(qd, kd, budget, seed, n_clusters=C, sampling=sampling,
                                fused=True).export()
    for key in two:
        assert np.array_equal(two[key], one[key]), key
    assert two["rowptr"][-1] > 0


def test_fused_plan_against_oracle():
    """The fused plan is the oracle's SIP (both designs) on the two-pass
    kernel's fp32 scores, which are within the score tolerance of the
    oracle's; the attention under it matches the oracle's HT attention."""
    q, k, v = _qk(1, 2, 3000, 128, "bf16", seed=77)
    B, H, N, d = q.shape
    M, QB = N // 4, (N + 127) // 128
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    keep = absa.absa_plan_create(qd, kd, 60, 5, keep_intermediates=True)
    s = keep.export_intermediate(absa.INTER_SCORES).reshape(B, H, QB, M)
    for sampling in ("poisson", "systematic"):
        plan = absa.absa_plan_create(qd, kd, 60, 5, sampling=sampling, fused=True)
        gp = plan.export()
        check_plan_exact(gp, oracle.plan_from_scores(s, B, H, N, d, 60, 5, sampling),
                         f"fused {sampling}")
    out = absa.absa_sparse_attention(plan, qd, kd, vd)
    torch.cuda.synchronize()
    check_output(to64(out), oracle.plan_attention(to64(q), to64(k), to64(v),
                                                  oracle_plan_of(gp, B, H, N, d)), "fused plan")


def test_fused_unsupported_requests():
    q, k, _ = _qk(1, 1, 1024, 128, "bf16", seed=3)
    qd, kd = q.to(DEV), k.to(DEV)
    with pytest.raises(absa.AbsaError, match="UNSUPPORTED"):
        absa.absa_plan_create(qd, kd, 10, 1, n_clusters=9, fused=True)
    with pytest.raises(absa.AbsaError, match="UNSUPPORTED"):
        absa.absa_plan_create(qd, kd, 10, 1, keep_intermediates=True, fused=True)
    long_q = torch.zeros(1, 1, 4 * 20225, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(absa.AbsaError, match="UNSUPPORTED"):
        absa.absa_plan_create(long_q, long_q, 10, 1, fused=True)
