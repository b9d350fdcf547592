"""Speculative-sampling verification on the GPU against the oracle (aiwing.uk ch.22
sec.22.1), through the C ABI (w4a16_spec_verify).

Every decision is exact (fp64 acceptance test, integer fixed-point draw), so the
number of accepted drafts and the drawn token must match the oracle exactly.
"""
import numpy as np
import pytest

from oracle import spec
from tests.gpu_helpers import note, to_dev, to_host, torch_cuda
from workloads import verify as wv

import weight_only_int4_group_amd as w4

pytestmark = pytest.mark.gpu


def _oracle(pt, pd, dr, ua, us):
    n = np.empty(pt.shape[0], np.int32)
    t = np.empty(pt.shape[0], np.int32)
    for b in range(pt.shape[0]):
        n[b], t[b] = spec.verify(pt[b], pd[b], dr[b], ua[b], us[b])
    return n, t


def _gpu(pt, pd, dr, ua, us):
    n, t = w4.w4a16_spec_verify(to_dev(pt), to_dev(pd), to_dev(dr), to_dev(ua), to_dev(us))
    return to_host(n), to_host(t)


def _check(pt, pd, dr, ua, us, what):
    note(f"spec_verify {what} B={pt.shape[0]} K={pt.shape[1] - 1} V={pt.shape[2]}")
    n_ref, t_ref = _oracle(pt, pd, dr, ua, us)
    n, t = _gpu(pt, pd, dr, ua, us)
    bad = np.nonzero((n != n_ref) | (t != t_ref))[0]
    assert bad.size == 0, (f"{what}: {bad.size} sequences differ, first b={bad[0]}: "
                           f"gpu ({n[bad[0]]}, {t[bad[0]]}) oracle ({n_ref[bad[0]]}, {t_ref[bad[0]]})")
    return n_ref, t_ref


@pytest.mark.parametrize("B,K,V", [(64, 4, 32000), (32, 8, 128256), (48, 1, 152064),
                                   (16, 4, 1000), (40, 3, 65), (24, 2, 1)])
def test_random_batches_match_oracle(B, K, V):
    torch_cuda()
    n, _ = _check(*wv.batch(B + K, B, K, V), f"random")
    if V >= 1000:
        # a mix of outcomes: some rejections and some full acceptances
        assert (n < K).any() and (n == K).any() or K == 1


def test_no_drafts():
    torch_cuda()
    pt, pd, dr, ua, us = wv.batch(3, 20, 0, 4099)
    _check(pt, pd, dr, ua, us, "K=0")


def test_identical_draft_accepts_every_token():
    torch_cuda()
    pt, pd, dr, ua, us = wv.batch(4, 16, 4, 5000)
    pd = pt[:, :4].copy()
    dr = np.argmax(pd, axis=2).astype(np.int32)
    n, _ = _check(pt, pd, dr, ua, us, "identical")
    assert (n == 4).all()


def test_degenerate_rows_and_ids():
    torch_cuda()
    B, K, V = 32, 4, 3001
    pt, pd, dr, ua, us = wv.batch(5, B, K, V)
    pd[0, 0, dr[0, 0]] = 0.0                      # p_draft(x) = 0: accepted
    pt[1, 0, dr[1, 0]] = 0.0                      # p_target(x) = 0: rejected
    dr[2, 1] = -1                                 # ids out of range: rejected
    dr[3, 0] = V
    dr[4, 2] = 2 ** 31 - 1
    for b, i in ((2, 0), (4, 0), (4, 1)):         # (the drafts before them accepted)
        pd[b, i, dr[b, i]] = 0.0
    pd[5, 0] = pt[5, 0] * 2                       # residual has no mass: target row
    dr[5, 0] = int(np.argmax(pt[5, 0]))
    ua[5, 0] = 0.9
    pd[6, 0] = pt[6, 0] * 2                       # ... and the target row has none: -1
    pt[6, 0] = 0.0
    ua[6, 0] = 0.5
    pt[7, K] = 0.0                                # all accepted, bonus row empty: -1
    pd[7] = pt[7, :K]
    dr[7] = np.argmax(pd[7], axis=1)
    pt[8, 0, ::3] = np.nan                        # NaN and negative entries count as 0
    pd[8, 0, 1::5] = -1.0
    pt[9, 2, :100] = -np.float32(0.25)
    ua[10] = np.nan                               # NaN uniform rejects
    ua[11] = -1.0                                 # negative uniform accepts (if p_target > 0)
    us[12] = 0.0                                  # draw ends: u' = 0, just below 1, 1, NaN
    us[13] = np.nextafter(np.float32(1), np.float32(0))
    us[14] = 1.0
    us[15] = np.nan
    us[16] = -3.0
    pt[17, :, : V - 1] = 0.0                      # all mass on the last id
    pt[17, :, V - 1] = 1.0
    n, t = _check(pt, pd, dr, ua, us, "degenerate")
    assert n[0] >= 1 and n[1] == 0 and n[2] == 1 and n[3] == 0 and n[4] == 2
    assert n[5] == 0 and t[5] >= 0 and n[6] == 0 and t[6] == -1
    assert n[7] == K and t[7] == -1 and n[10] == 0 and n[11] == K and t[17] == V - 1


def test_draw_boundaries_exact():
    """Dyadic rows where the draw threshold falls exactly on a prefix sum: the token is the
    first id whose inclusive prefix sum exceeds it, on the GPU as in the oracle."""
    torch_cuda()
    V = 4096
    B = 64
    pt = np.zeros((B, 1, V), np.float32)
    pt[:, 0, :] = np.float32(1.0 / V)
    pd = np.zeros((B, 0, V), np.float32)
    dr = np.zeros((B, 0), np.int32)
    ua = np.zeros((B, 0), np.float32)
    # u' = j / 64 lands exactly on the boundary before id j * V / 64
    us = (np.arange(B, dtype=np.float32) / np.float32(B)).astype(np.float32)
    n, t = _check(pt, pd, dr, ua, us, "boundaries")
    assert (t == np.arange(B) * (V // B)).all()


def test_repeat_calls_are_identical_and_async_on_stream():
    torch = torch_cuda()
    pt, pd, dr, ua, us = (to_dev(a) for a in wv.batch(6, 32, 4, 32000))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        a = w4.w4a16_spec_verify(pt, pd, dr, ua, us)
        b = w4.w4a16_spec_verify(pt, pd, dr, ua, us)
    s.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_shared_workspace_across_calls():
    """One caller-owned workspace reused by calls of different sizes: its stale contents
    never leak into a result."""
    torch = torch_cuda()
    big = wv.batch(8, 48, 6, 20000)
    small = wv.batch(9, 5, 2, 70000)
    ws = torch.empty(max(w4.w4a16_spec_verify_workspace_size(48, 6, 20000),
                         w4.w4a16_spec_verify_workspace_size(5, 2, 70000)),
                     dtype=torch.uint8, device="cuda")
    for what, inp in (("big", big), ("small", small), ("big again", big)):
        note(f"spec_verify shared workspace {what}")
        n_ref, t_ref = _oracle(*inp)
        n, t = w4.w4a16_spec_verify(*(to_dev(a) for a in inp), workspace=ws)
        assert (to_host(n) == n_ref).all() and (to_host(t) == t_ref).all(), what


def test_unaligned_rows_take_the_scalar_path():
    """Rows whose start is not 16-byte aligned (V a multiple of 4, tensor base offset by one
    float) are read element by element; the results are the same."""
    torch = torch_cuda()
    inp = wv.batch(10, 12, 3, 32000)

    def shifted(a):
        flat = torch.empty(a.size + 1, dtype=torch.float32, device="cuda")
        t = flat[1:].view(a.shape)
        t.copy_(torch.from_numpy(a))
        assert t.data_ptr() % 16 == 4
        return t

    note("spec_verify unaligned rows")
    n_ref, t_ref = _oracle(*inp)
    pt, pd = shifted(inp[0]), shifted(inp[1])
    n, t = w4.w4a16_spec_verify(pt, pd, to_dev(inp[2]), to_dev(inp[3]), to_dev(inp[4]))
    assert (to_host(n) == n_ref).all() and (to_host(t) == t_ref).all()
