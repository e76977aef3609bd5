"""Properties of the HIP path that must hold exactly (GPU): run-to-run identity,
isolation across users, invariance to max_seqlen, to zero-length users and to
user order, exact length-one rows, plus closed-form cases within tolerance."""
import numpy as np
import pytest
import torch

import oracle
import varlen_causal_attention_amd as vlca
import workloads
from gpu_util import TOL_MAX, TOL_MEAN, assert_close, qkv64, run_fwd, say, to_gpu

pytestmark = pytest.mark.gpu


def user_rows(cu, u):
    return slice(int(cu[u]), int(cu[u + 1]))


# Users longer than this many rows (4 q-tiles) have their longest items split into
# key-range parts in the single-kernel plan; shorter users' items always run whole.
WHOLE_USER_ROWS = 256


def assert_same_or_close(a, b, w):
    """Two outputs of the same batch from launch plans that may split long items
    differently: identical bits on users that never split, the parity bound on
    the others (against each other)."""
    whole = np.zeros(w.total_tokens, dtype=bool)
    for u, L in enumerate(w.lengths):
        if L <= WHOLE_USER_ROWS:
            whole[user_rows(w.cu_seqlens, u)] = True
    whole = torch.from_numpy(whole)
    assert torch.equal(a[whole], b[whole])
    if (~whole).any():
        d = (a[~whole].double() - b[~whole].double()).abs()
        say(f"[parity] split vs whole items: max|d|={float(d.max()):.3e} mean|d|={float(d.mean()):.3e}")
        assert float(d.max()) <= TOL_MAX and float(d.mean()) <= TOL_MEAN


@pytest.mark.parametrize("idx", [2, 5])
def test_run_twice_bit_identical(gpu, idx):
    w = workloads.make_config(idx)
    say(f"[case] run twice, config {idx}")
    qkv, cu = to_gpu(w)
    a = run_fwd(w, qkv=qkv, cu=cu)
    b = run_fwd(w, qkv=qkv, cu=cu)
    assert torch.equal(a, b)


def test_isolation_other_users_bit_identical(gpu):
    w = workloads.make_config(2)
    say("[case] isolation, config 2 user 7")
    base = run_fwd(w)
    pert = workloads.make_config(2)
    r = user_rows(w.cu_seqlens, 7)
    pert.qkv_bf16[r] = (pert.qkv_bf16[r].float() * -1.5 + 0.25).to(torch.bfloat16)
    out = run_fwd(pert)
    keep = torch.ones(w.total_tokens, dtype=torch.bool)
    keep[r] = False
    assert torch.equal(base[keep], out[keep])
    assert not torch.equal(base[~keep], out[~keep])


# A larger max_seqlen may move a batch from the single-kernel plan to the
# scheduler plan; both take the same key-range split decision from the batch's
# own lengths, so the bits stay the same.
MAX_SEQLEN_CASES = [
    ("config 2 (no item split)", lambda: workloads.make_config(2), (1024, 2048, 262144)),
    ("long users, items split", lambda: workloads.make_from_lengths([1000, 700, 3, 450, 0, 320], seed=13),
     (1024, 4096, 65536, 262144)),
]


@pytest.mark.parametrize("case", range(len(MAX_SEQLEN_CASES)))
def test_max_seqlen_invariance(gpu, case):
    name, make, larger = MAX_SEQLEN_CASES[case]
    w = make()
    say(f"[case] max_seqlen {w.max_seqlen} / {larger}: {name}")
    qkv, cu = to_gpu(w)
    ref = run_fwd(w, qkv=qkv, cu=cu)
    plans = {vlca.single_kernel(w.num_users, ms, w.n_heads) for ms in (w.max_seqlen,) + larger}
    assert plans == {True, False}  # both launch plans are covered
    for ms in larger:
        assert torch.equal(ref, run_fwd(w, max_seqlen=ms, qkv=qkv, cu=cu)), ms


def test_zero_length_users_change_nothing(gpu):
    w = workloads.make_config(2)
    say("[case] zero-length users inserted")
    base = run_fwd(w)
    L = list(w.lengths)
    L2 = [0, 0] + L[:10] + [0] + L[10:30] + [0, 0, 0] + L[30:] + [0]
    w2 = workloads.Workload("padded", np.asarray(L2), workloads.cu_from_lengths(L2), w.max_seqlen, w.scale)
    w2.qkv_bf16 = w.qkv_bf16
    assert torch.equal(base, run_fwd(w2))


def _insert_zeros(lengths, n_zero, seed):
    """The same users in the same order with n_zero zero-length users at random places."""
    rng = np.random.default_rng(seed)
    out = list(lengths)
    for _ in range(n_zero):
        out.insert(int(rng.integers(0, len(out) + 1)), 0)
    return out


# A batch whose longest items split into key-range parts.  With 300 zero-length
# users inserted it has more users than the single-kernel plan takes, so it runs
# on the scheduler plan; the split decision counts only users with rows, so the
# bits must not change.
SPLIT_LENGTHS = [1000, 700, 3, 450, 0, 320]


@pytest.mark.parametrize("n_zero", [1, 100, 300, 2000])
def test_zero_length_users_change_nothing_split_batch(gpu, n_zero):
    w = workloads.make_from_lengths(SPLIT_LENGTHS, seed=13)
    L2 = _insert_zeros(SPLIT_LENGTHS, n_zero, seed=n_zero)
    w2 = workloads.Workload("padded", np.asarray(L2), workloads.cu_from_lengths(L2), w.max_seqlen, w.scale)
    w2.qkv_bf16 = w.qkv_bf16
    plans = (vlca.single_kernel(w.num_users, w.max_seqlen, 8), vlca.single_kernel(w2.num_users, w.max_seqlen, 8))
    say(f"[case] {n_zero} zero-length users inserted into {SPLIT_LENGTHS}; single kernel: {plans}")
    assert torch.equal(run_fwd(w), run_fwd(w2))


def test_zero_length_users_change_nothing_config5(gpu):
    w = workloads.make_config(5)
    L2 = _insert_zeros(w.lengths, 500, seed=5)
    w2 = workloads.Workload("padded", np.asarray(L2), workloads.cu_from_lengths(L2), w.max_seqlen, w.scale)
    w2.qkv_bf16 = w.qkv_bf16
    say("[case] 500 zero-length users inserted into config 5")
    assert torch.equal(run_fwd(w), run_fwd(w2))


PERMUTATION_CASES = [("config 3", lambda: workloads.make_config(3)),
                     ("split batch", lambda: workloads.make_from_lengths(SPLIT_LENGTHS + [900, 17, 600], seed=19))]


@pytest.mark.parametrize("case", range(len(PERMUTATION_CASES)))
def test_user_order_permutation(gpu, case):
    name, make = PERMUTATION_CASES[case]
    w = make()
    say(f"[case] user permutation, {name}")
    base = run_fwd(w)
    perm = np.random.default_rng(5).permutation(w.num_users)
    rows = np.concatenate([np.arange(w.cu_seqlens[u], w.cu_seqlens[u + 1]) for u in perm])
    L2 = w.lengths[perm]
    w2 = workloads.Workload("perm", L2, workloads.cu_from_lengths(L2), w.max_seqlen, w.scale)
    w2.qkv_bf16 = w.qkv_bf16[torch.from_numpy(rows)]
    out = run_fwd(w2)
    assert torch.equal(out, base[torch.from_numpy(rows)])


def test_length_one_rows_exact(gpu):
    w = workloads.make_from_lengths([1, 5, 1, 1, 300, 1], seed=2)
    say("[case] length-one users")
    out = run_fwd(w)
    for u, L in enumerate(w.lengths):
        if L == 1:
            r = int(w.cu_seqlens[u])
            assert torch.equal(out[r], w.qkv_bf16[r, 1024:])


def test_many_rounds_per_workgroup(gpu):
    # 70000 one-row users plus a few longer ones: about 550 items per workgroup
    # slot, past the descriptors a workgroup caches in LDS, and more users than
    # the scheduler caches in LDS.  One-row users return their own V row exactly;
    # the longer users are checked against the oracle.
    lengths = [1] * 70000
    for pos, L in ((0, 130), (35000, 257), (69999, 64)):
        lengths[pos] = L
    w = workloads.make_from_lengths(lengths, seed=9)
    say(f"[case] many rounds: {len(lengths)} users, {w.total_tokens} rows")
    out = run_fwd(w)
    cu = w.cu_seqlens
    ones = np.nonzero(np.diff(cu) == 1)[0]
    rows = torch.from_numpy(cu[ones].astype(np.int64))
    assert torch.equal(out[rows], w.qkv_bf16[rows, 1024:])
    q = w.qkv_bf16.to(torch.float64).numpy()
    for pos in (0, 35000, 69999):
        r = slice(int(cu[pos]), int(cu[pos + 1]))
        ref = oracle.varlen_causal_attention_rows(q, cu, np.arange(r.start, r.stop), w.n_heads, w.head_dim, w.scale)
        assert_close(out[r], ref, f"user {pos}")


def test_zero_query_gives_running_mean(gpu):
    w = workloads.make_from_lengths([5, 90, 200, 1], seed=3)
    w.qkv_bf16[:, :512] = 0
    say("[case] q = 0")
    out = run_fwd(w).double().numpy()
    v = qkv64(w)[:, 1024:]
    for u in range(w.num_users):
        s, e = int(w.cu_seqlens[u]), int(w.cu_seqlens[u + 1])
        want = np.cumsum(v[s:e], axis=0) / np.arange(1, e - s + 1)[:, None]
        assert np.max(np.abs(out[s:e] - want)) <= TOL_MAX


def test_constant_v(gpu):
    w = workloads.make_from_lengths([7, 150, 64], seed=4)
    c = torch.linspace(-3, 3, 512).to(torch.bfloat16)
    w.qkv_bf16[:, 1024:] = c
    say("[case] constant v")
    out = run_fwd(w)
    # weights are renormalised by the sum of the rounded weights: exact up to fp32 accumulation
    assert torch.max(torch.abs(out.float() - c.float()[None, :])) <= 2 ** -7 * 3


# Batches with at most 256 users (and few enough items per workgroup) run as one
# kernel that locates its own work; larger ones run the scheduler and the
# attention kernel over a worklist buffer.  Either plan of fwd may split the
# longest items of users of more than 4 q-tiles into key-range parts (when the
# split list fits one round of the grid), while the explicit worklist path runs
# every item whole: rows of users that never split agree bit for bit, the others
# within the parity bound.
WORKLIST_CASES = [
    ("config 2 (single kernel)", lambda: workloads.make_config(2), None),
    ("config 3 (scheduler + worklist)", lambda: workloads.make_config(3), None),
    ("256 users x 8 tiles (single kernel, at the limit)",
     lambda: workloads.make_from_lengths(list(np.random.default_rng(3).integers(1, 513, 256)), seed=3), 512),
    ("257 users x 8 tiles (just past the limit)",
     lambda: workloads.make_from_lengths(list(np.random.default_rng(4).integers(1, 513, 257)), seed=4), 512),
    ("zero-length users, 3 heads", lambda: workloads.make_from_lengths([0, 70, 0, 0, 5, 200, 0], seed=5, n_heads=3),
     None),
    ("one user of 4096 rows (64 q-tiles)", lambda: workloads.make_from_lengths([4096], seed=6), None),
    ("one user of 4096 rows, max_seqlen 262144 (scheduler plan, split)",
     lambda: workloads.make_from_lengths([4096], seed=6), 262144),
    # Scheduler plan (more than 256 users) with counters that cannot be one per head:
    # 3 heads (the grid is not a multiple of the head count) and 16 heads (more heads
    # than counters) both claim (item, head) pairs from a single counter.
    ("300 users, 3 heads (scheduler plan, one counter)",
     lambda: workloads.make_from_lengths(list(np.random.default_rng(7).integers(0, 101, 300)), seed=7, n_heads=3),
     None),
    ("300 users, 16 heads (scheduler plan, one counter)",
     lambda: workloads.make_from_lengths(list(np.random.default_rng(8).integers(0, 101, 300)), seed=8, n_heads=16),
     None),
]


@pytest.mark.parametrize("case", range(len(WORKLIST_CASES)))
def test_worklist_entry_point_matches_fwd(gpu, case):
    name, make, max_seqlen = WORKLIST_CASES[case]
    w = make()
    ms = w.max_seqlen if max_seqlen is None else max_seqlen
    say(f"[case] build_worklist + fwd_with_worklist vs fwd: {name}")
    qkv, cu = to_gpu(w)
    a = run_fwd(w, max_seqlen=ms, qkv=qkv, cu=cu)
    items, count = vlca.build_worklist(cu, ms)
    b = vlca.fwd_with_worklist(qkv, cu, ms, items, count, n_heads=w.n_heads, scale=w.scale)
    torch.cuda.synchronize()
    assert_same_or_close(a, b.cpu(), w)


def test_int64_offsets_and_preallocated_out(gpu):
    w = workloads.make_config(1)
    qkv, cu = to_gpu(w)
    a = run_fwd(w, qkv=qkv, cu=cu)
    out = torch.full((w.total_tokens, 512), 7.0, dtype=torch.bfloat16, device="cuda")
    r = vlca.fwd(qkv, cu.to(torch.int64), w.max_seqlen, scale=w.scale, out=out)
    torch.cuda.synchronize()
    assert r.data_ptr() == out.data_ptr()
    assert torch.equal(a, out.cpu())


def test_bad_shapes_raise(gpu):
    w = workloads.make_config(1)
    qkv, cu = to_gpu(w)
    with pytest.raises(ValueError):
        vlca.fwd(qkv[:, :1000], cu, 40)
    with pytest.raises(ValueError):
        vlca.fwd(qkv.float(), cu, 40)
    with pytest.raises(vlca.VlcaError):
        vlca.fwd(qkv, cu, 40, scale=-1.0)
    # A view two bytes into its storage: the kernels move 16-byte chunks, so the
    # library refuses it (VLCA_ERR_ALIGN) before any device work.
    buf = torch.empty(qkv.numel() + 8, dtype=torch.bfloat16, device="cuda")
    odd = buf[1:1 + qkv.numel()].view(qkv.shape)
    odd.copy_(qkv)
    with pytest.raises(vlca.VlcaError) as err:
        vlca.fwd(odd, cu, 40)
    assert err.value.code == -15


# Rows past cu_seqlens[-1] belong to no user: fwd must leave them as they were,
# whatever tile a user's last rows fall into.  The batches end in short users, so
# their diagonal tiles reach into the padding.
PADDED_CASES = [
    ("single kernel", [37, 3, 130, 1, 5], None),
    ("scheduler plan", [37, 3, 130, 1, 5], 65536),
    ("split items, single kernel", [700, 2, 450, 9], None),
]


@pytest.mark.parametrize("case", range(len(PADDED_CASES)))
def test_rows_past_the_last_user_untouched(gpu, case):
    name, lengths, max_seqlen = PADDED_CASES[case]
    w = workloads.make_from_lengths(lengths, seed=17)
    pad = 100
    say(f"[case] padded buffers ({name}): lengths {lengths}, {pad} rows past the end")
    qkv = torch.cat([w.qkv_bf16, torch.ones((pad, w.qkv_bf16.shape[1]), dtype=torch.bfloat16)]).cuda()
    cu = torch.from_numpy(np.asarray(w.cu_seqlens, dtype=np.int32)).cuda()
    out = torch.full((w.total_tokens + pad, 512), 7.0, dtype=torch.bfloat16, device="cuda")
    vlca.fwd(qkv, cu, w.max_seqlen if max_seqlen is None else max_seqlen, scale=w.scale, out=out)
    torch.cuda.synchronize()
    out = out.cpu()
    assert bool((out[w.total_tokens:] == 7.0).all()), "fwd wrote rows past the last user"
    ref = oracle.varlen_causal_attention(qkv64(w), w.cu_seqlens, w.n_heads, w.head_dim, w.scale)
    assert_close(out[: w.total_tokens], ref, name)
