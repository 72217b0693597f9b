"""GPU test at a key buffer beyond 2^31 bytes: L = 2^24 + 777 keys of d = 128
bf16 (4.3 GB), 64 queries at the end, H = 64, k = 2048 (the largest k).  The
oracle cannot score rows this long in test time, so the test checks what
holds at any size:

  * the table-free selection (here with its recovery path: at this length
    some queries' candidate buffers overflow or fall short by design) equals
    the materialise-then-top-k route bit for bit, and replay equals the
    selected scores bit for bit;
  * structure of every row (distinct in-range indices, scores non-increasing,
    equal scores in ascending position);
  * the selected scores against an fp64 recomputation of those entries;
  * the set rule against a sample: 20,000 random keys of each query's context
    are scored in fp64, and none outside the selection may exceed the
    smallest selected score by more than 1e-4 * (|v| + 1).

Inputs are seeded Gaussian draws made on the device (q, k ~ N(0, 1) / sqrt(d)
rounded to bf16, w ~ U(0, 1) / H), the distribution of the 1M workloads.
"""
import numpy as np
import pytest
import torch

from gpu_util import say

pytestmark = pytest.mark.gpu

L, N, H, D, K = (1 << 24) + 777, 64, 64, 128, 2048
SAMPLE = 20000
REL = 1e-4


def scores_fp64(q, k, w, t_idx, keys):
    """fp64 indexer scores of query rows t_idx (into q, w) against key rows
    keys [m][j] (one list of keys per query)."""
    qq = q[t_idx].double()                                                      # [m][H][D]
    kt = k[keys.reshape(-1)].double().view(keys.shape[0], keys.shape[1], D)     # [m][j][D]
    c = torch.bmm(qq, kt.transpose(1, 2).contiguous()).clamp_min(0.0)           # [m][H][j]
    return torch.bmm(w[t_idx].double().unsqueeze(1), c).squeeze(1)              # [m][j]


def test_key_buffer_beyond_2_31_bytes():
    import exact_top_token_amd as hk
    hk.load_library()
    say(f"large: L={L} n={N} H={H} d={D} k={K} (keys {L * D * 2 / 1e9:.2f} GB)")
    dev = "cuda"
    g = torch.Generator(device=dev)
    g.manual_seed(2024)
    k = (torch.randn((L, D), generator=g, device=dev) / D ** 0.5).to(torch.bfloat16)
    q = (torch.randn((N, H, D), generator=g, device=dev) / D ** 0.5).to(torch.bfloat16)
    w = torch.rand((N, H), generator=g, device=dev) / H
    q_start = L - N

    idx, sc, st = hk.select(q, k, w, K, with_stats=True)
    torch.cuda.synchronize()
    say(f"large: select done, stats {st}")
    # M is capped at 8192, so at this length the threshold is the 3rd best of
    # 8192 samples (r = ceil(3k * M / ctx) = 3) and its candidate count varies
    # widely: some queries overflow the buffer or fall short of k by design
    # and are recovered; with n = 64 there is never a full rescore.
    assert st["path"] == 0 and st["full_rescore"] == 0, st
    assert st["n_failed"] == len(st["failed"]) <= N, st
    bidx, bsc = hk.baseline_select(q, k, w, K)
    rep = hk.replay(q, k, w, idx)
    torch.cuda.synchronize()
    assert torch.equal(bidx, idx)
    assert torch.equal(bsc.view(torch.int32), sc.view(torch.int32))
    assert torch.equal(rep.view(torch.int32), sc.view(torch.int32))

    # structure
    t = torch.arange(q_start, q_start + N, device=dev)
    assert bool((idx >= 0).all()) and bool((idx <= t[:, None]).all())
    srt = torch.sort(idx, dim=1).values
    assert bool((srt[:, 1:] != srt[:, :-1]).all()), "duplicate index in a row"
    assert bool((sc[:, 1:] <= sc[:, :-1]).all()), "scores not non-increasing"
    tie = sc[:, 1:] == sc[:, :-1]
    assert bool((idx[:, 1:][tie] > idx[:, :-1][tie]).all()), "equal scores not in position order"

    # selected scores against fp64
    ref = scores_fp64(q, k, w, torch.arange(N, device=dev), idx.long())
    err = (sc.double() - ref).abs()
    assert bool((err <= REL * (ref.abs() + 1.0)).all()), float(err.max())

    # the set rule on a random sample of every context
    gs = torch.Generator(device=dev)
    gs.manual_seed(7)
    samp = (torch.rand((N, SAMPLE), generator=gs, device=dev, dtype=torch.float64)
            * (t[:, None] + 1).double()).floor().long()
    s_ref = scores_fp64(q, k, w, torch.arange(N, device=dev), samp)
    pos = torch.searchsorted(srt.long(), samp).clamp_max(K - 1)
    outside = torch.gather(srt.long(), 1, pos) != samp
    v = ref.min(dim=1).values  # the smallest selected score (fp64)
    tol = REL * (v.abs() + 1.0)
    worst = torch.where(outside, s_ref, torch.full_like(s_ref, -np.inf)).max(dim=1).values
    assert bool((worst <= v + tol).all()), float((worst - v).max())
    say("large: select == baseline == replay; structure, scores and sampled set ok")
