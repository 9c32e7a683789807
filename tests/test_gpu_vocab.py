"""GPU parity of the vocabulary kernels against the oracle: greedy verification, streak
selection and drafting from fp32 logits.  Integer outputs must be bit-exact; streak scores too
(both sides use the same integer weights and the same fp64 operation order)."""
import numpy as np
import pytest
import torch

import block_diffusion_drafter_draft_amd as dbd
import synth
from oracle import accept, dnc

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _verify_gpu(logits, drafts):
    N, R, V = logits.shape
    D = drafts.shape[1]
    ws = torch.empty(dbd.verify_workspace_bytes(N, R, V), dtype=torch.uint8, device=DEV)
    n_acc = torch.full((N,), -7, dtype=torch.int32, device=DEV)
    bonus = torch.full((N,), -7, dtype=torch.int32, device=DEV)
    com = torch.full((N, D + 1), -7, dtype=torch.int32, device=DEV)
    flags = torch.full((N,), -7, dtype=torch.int32, device=DEV)
    dbd.verify_greedy(logits, drafts, n_acc, bonus, com, ws, row_flags=flags)
    torch.cuda.synchronize()
    return n_acc.cpu().numpy(), bonus.cpu().numpy(), com.cpu().numpy(), flags.cpu().numpy()


def _check_verify(logits, drafts, planted=None):
    print(f"verify_greedy shape={tuple(logits.shape)}", flush=True)
    got = _verify_gpu(logits, drafts)
    ref = accept.verify_greedy(logits.cpu().numpy(), drafts.cpu().numpy())
    for g, r in zip(got[:3], ref):
        assert np.array_equal(g, r)
    assert np.all(got[3] == 0)
    if planted is not None:
        assert np.array_equal(got[0], planted)


@pytest.mark.parametrize("name", ["tiny-fp32", "qwen3-8b", "gpt-oss-20b"])
def test_verify_greedy_workload_shapes(name):
    wl = synth.workload(name)
    V, D, N = wl.shape.vocab, wl.n_draft, wl.batch
    drafts = synth.make_drafts(N, 1, D, V, seed=3, device=DEV)[:, 0].contiguous()
    logits, a = synth.make_planted_verify_logits(drafts, wl.verify_rows, V, wl.planted_alpha,
                                                 std=wl.logit_std, seed=3, device=DEV)
    _check_verify(logits, drafts, a)


@pytest.mark.parametrize("N,D,R,V", [(3, 5, 5, 37), (4, 7, 8, 4099), (2, 64, 65, 300),
                                     (5, 1, 2, 8192), (1, 3, 4, 2)])
def test_verify_greedy_ragged_and_ties(N, D, R, V):
    g = torch.Generator(device=DEV).manual_seed(N * 1000 + V)
    # small integer logits: exact ties everywhere, so the lowest-index rule decides
    logits = torch.randint(-3, 4, (N, R, V), generator=g, device=DEV).float()
    drafts = torch.randint(0, V, (N, D), generator=g, device=DEV, dtype=torch.int32)
    # make a few prefixes match the target's argmax so acceptance lengths vary
    t = logits.argmax(-1).to(torch.int32)
    for n in range(N):
        k = (n * 3) % (D + 1)
        drafts[n, :k] = t[n, :k]
    _check_verify(logits, drafts)


def test_verify_greedy_identical_P_Q_accepts_all():
    N, D, V = 4, 15, 5000
    g = torch.Generator(device=DEV).manual_seed(5)
    q = torch.randn((N, D + 1, V), generator=g, device=DEV)
    drafts = q[:, :D].argmax(-1).to(torch.int32).contiguous()
    n_acc, bonus, com, _ = _verify_gpu(q, drafts)
    assert np.all(n_acc == D)
    assert np.array_equal(bonus, q[:, D].argmax(-1).cpu().numpy())


def test_verify_greedy_flags_non_finite():
    N, D, V = 3, 4, 1000
    logits = torch.randn((N, D + 1, V), device=DEV)
    logits[1, 2, 17] = float("nan")
    logits[2, 0, 5] = float("inf")
    drafts = torch.zeros((N, D), dtype=torch.int32, device=DEV)
    flags = _verify_gpu(logits, drafts)[3]
    assert list(flags) == [0, 1, 1]


def _select_gpu(logits, drafts):
    N, K, R, V = logits.shape
    G = drafts.shape[2]
    ws = torch.empty(dbd.select_workspace_bytes(N, K, R, V), dtype=torch.uint8, device=DEV)
    sel = torch.full((N,), -7, dtype=torch.int32, device=DEV)
    sc = torch.zeros((N, K), dtype=torch.float64, device=DEV)
    n_acc = torch.full((N,), -7, dtype=torch.int32, device=DEV)
    bonus = torch.full((N,), -7, dtype=torch.int32, device=DEV)
    com = torch.full((N, G + 1), -7, dtype=torch.int32, device=DEV)
    flags = torch.full((N,), -7, dtype=torch.int32, device=DEV)
    dbd.select_streak(logits, drafts, sel, n_acc, bonus, com, ws, scores=sc, row_flags=flags)
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in (sel, sc, n_acc, bonus, com, flags)]


def _check_select(logits, drafts):
    print(f"select_streak shape={tuple(logits.shape)}", flush=True)
    got = _select_gpu(logits, drafts)
    ref = accept.select_streak(logits.cpu().numpy(), drafts.cpu().numpy())
    assert np.array_equal(got[0], ref[0])                  # selected draft
    assert np.array_equal(got[1], ref[1])                  # fp64 streak scores, bit for bit
    for g, r in zip(got[2:5], ref[2:]):
        assert np.array_equal(g, r)
    assert np.all(got[5] == 0)
    return got


def test_select_streak_tiny():
    """[1, 4, 7, 1024] verifier logits N(0, 2) over 4 drafts of 7 tokens."""
    drafts = synth.make_drafts(1, 4, 7, 1024, seed=9, device=DEV)
    logits, _ = synth.make_planted_streak_logits(drafts, 7, 1024, 0.7, seed=9, device=DEV)
    _check_select(logits, drafts)


def test_select_streak_specdiff2_shape():
    wl = synth.workload("specdiff2-7b")
    N, K, G, V = wl.batch, wl.n_drafts, wl.n_draft, wl.shape.vocab
    drafts = synth.make_drafts(N, K, G, V, seed=2, device=DEV)
    logits, a = synth.make_planted_streak_logits(drafts, wl.verify_rows, V, wl.planted_alpha,
                                                 std=wl.logit_std, seed=2, device=DEV)
    got = _check_select(logits, drafts)
    for n in range(N):
        assert got[2][n] == a[n, got[0][n]]                # planted streak of the chosen draft


@pytest.mark.parametrize("N,K,G,R,V", [(3, 5, 4, 5, 333), (2, 1, 6, 6, 9000), (2, 8, 32, 33, 2)])
def test_select_streak_ragged(N, K, G, R, V):
    g = torch.Generator(device=DEV).manual_seed(K * 100 + V)
    logits = torch.randn((N, K, R, V), generator=g, device=DEV) * 2
    drafts = torch.randint(0, V, (N, K, G), generator=g, device=DEV, dtype=torch.int32)
    _check_select(logits, drafts)


def test_select_streak_equal_scores_pick_lowest_draft():
    V, G, K = 50, 4, 6
    row = torch.randn((G, V), device=DEV)
    logits = row.expand(1, K, G, V).contiguous()
    drafts = torch.randint(0, V, (1, 1, G), device=DEV, dtype=torch.int32).expand(1, K, G)
    got = _select_gpu(logits, drafts.contiguous())
    assert got[0][0] == 0 and np.all(got[1][0] == got[1][0][0])


def _sample_gpu(logits, K, T, seed):
    N, D, V = logits.shape
    ws = torch.empty(dbd.sample_workspace_bytes(N, D, V), dtype=torch.uint8, device=DEV)
    out = torch.full((N, K, D), -7, dtype=torch.int32, device=DEV)
    dbd.sample_from_logits(logits, K, T, seed, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("N,D,V,K,T", [(1, 7, 1024, 1, 0.0), (1, 7, 1024, 4, 1.0),
                                       (3, 5, 4097, 3, 1.5), (2, 9, 64, 8, 2.0),
                                       (16, 7, 201088, 1, 1.0), (4, 32, 152064, 8, 1.5),
                                       (32, 15, 151936, 1, 0.0)])
def test_drafting_from_fp32_logits_bit_exact(N, D, V, K, T):
    print(f"sample N={N} D={D} V={V} K={K} T={T}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(V + K)
    logits = torch.randn((N, D, V), generator=g, device=DEV) * 2
    if T <= 0:
        logits[0, 0, 10] = logits[0, 0].max() + 1      # plant a tie at two indices
        logits[0, 0, 3] = logits[0, 0, 10]
    got = _sample_gpu(logits, K, T, seed=77)
    ref = dnc.sample_drafts(logits.cpu().numpy(), K, T, 77)
    assert np.array_equal(got, ref)


def test_sampling_depends_on_seed_and_draft_index():
    logits = torch.zeros((1, 4, 1000), device=DEV)       # uniform: draws differ freely
    a = _sample_gpu(logits, 8, 1.0, 1)
    b = _sample_gpu(logits, 8, 1.0, 2)
    assert not np.array_equal(a, b)
    assert len({tuple(a[0, k]) for k in range(8)}) > 1


# ---- lossless stochastic verification ----

def _vsample_gpu(tl, dl, drafts, t_p, t_q, seed):
    N, R, V = tl.shape
    D = drafts.shape[1]
    ws = torch.empty(dbd.verify_sample_workspace_bytes(N, D, R, V), dtype=torch.uint8,
                     device=DEV)
    n_acc = torch.full((N,), -7, dtype=torch.int32, device=DEV)
    bonus = torch.full((N,), -7, dtype=torch.int32, device=DEV)
    com = torch.full((N, D + 1), -7, dtype=torch.int32, device=DEV)
    flags = torch.full((N,), -7, dtype=torch.int32, device=DEV)
    dbd.verify_sample(tl, dl, drafts, t_p, t_q, seed, n_acc, bonus, com, ws, row_flags=flags)
    torch.cuda.synchronize()
    return n_acc.cpu().numpy(), bonus.cpu().numpy(), com.cpu().numpy(), flags.cpu().numpy()


def _check_vsample(tl, dl, drafts, t_p, t_q, seed):
    print(f"verify_sample target={tuple(tl.shape)} T=({t_p}, {t_q}) seed={seed}", flush=True)
    got = _vsample_gpu(tl, dl, drafts, t_p, t_q, seed)
    ref = accept.verify_sample(tl.cpu().numpy(), dl.cpu().numpy(), drafts.cpu().numpy(), t_p,
                               t_q, seed)
    for g, r in zip(got[:3], ref):
        assert np.array_equal(g, r), (g, r)
    assert np.all(got[3] == 0)
    return got


@pytest.mark.parametrize("N,D,R,V", [(6, 5, 6, 37), (4, 7, 8, 4099), (3, 15, 16, 10000),
                                     (2, 64, 65, 300), (5, 1, 1, 8192), (2, 3, 3, 2)])
@pytest.mark.parametrize("t_p,t_q", [(1.0, 1.0), (1.0, 1.5), (0.7, 1.3)])
def test_verify_sample_bit_exact(N, D, R, V, t_p, t_q):
    """Drafts sampled from the draft logits with the library's sampler, target logits close to
    them (so acceptance lengths vary), over ragged vocabulary chunks; every output bit-exact."""
    g = torch.Generator(device=DEV).manual_seed(N * 977 + V + D)
    dl = torch.randn((N, D, V), generator=g, device=DEV) * 2.0
    tl = torch.randn((N, R, V), generator=g, device=DEV) * 2.0
    tl[:, :D] = dl + 0.6 * torch.randn((N, D, V), generator=g, device=DEV)
    drafts = torch.from_numpy(dnc.sample_drafts(dl.cpu().numpy(), 1, t_q, seed=V)[:, 0]).to(DEV)
    got = _check_vsample(tl, dl, drafts.contiguous(), t_p, t_q, seed=12345 + D)
    if N * D >= 20:
        assert len(set(got[0].tolist())) > 1           # acceptance lengths differ


def test_verify_sample_workload_shape():
    """The Qwen3-8B drafter's vocabulary and block: 15 drafted positions, 16 target rows."""
    V, D, N = 151936, 15, 4
    g = torch.Generator(device=DEV).manual_seed(5)
    dl = torch.randn((N, D, V), generator=g, device=DEV) * 3.0
    tl = torch.randn((N, D + 1, V), generator=g, device=DEV) * 3.0
    tl[:, :D] = dl + 0.3 * torch.randn((N, D, V), generator=g, device=DEV)
    drafts = torch.from_numpy(dnc.sample_drafts(dl.cpu().numpy(), 1, 1.0, seed=9)[:, 0]).to(DEV)
    _check_vsample(tl, dl, drafts.contiguous(), 1.0, 1.0, seed=77)


def test_verify_sample_identical_P_Q_accepts_all():
    N, D, V = 8, 6, 5000
    g = torch.Generator(device=DEV).manual_seed(8)
    dl = torch.randn((N, D, V), generator=g, device=DEV) * 2.0
    tl = torch.cat([dl, torch.randn((N, 1, V), generator=g, device=DEV)], 1).contiguous()
    drafts = torch.from_numpy(dnc.sample_drafts(dl.cpu().numpy(), 1, 1.0, seed=1)[:, 0]).to(DEV)
    got = _check_vsample(tl, dl, drafts.contiguous(), 1.0, 1.0, seed=3)
    assert np.all(got[0] == D) and np.all(got[1] >= 0)


def test_verify_sample_out_of_range_and_disjoint():
    """Draft tokens outside the vocabulary are rejected; Q's mass only where P is zero rejects
    at position 0 and resamples from P's support."""
    N, D, V = 4, 3, 64
    dl = torch.full((N, D, V), -1e4, device=DEV)
    dl[:, :, 40:] = 0.0
    tl = torch.full((N, D + 1, V), -1e4, device=DEV)
    tl[:, :, :8] = torch.arange(8, device=DEV, dtype=torch.float32) * 0.1
    drafts = torch.from_numpy(dnc.sample_drafts(dl.cpu().numpy(), 1, 1.0, seed=2)[:, 0]).to(DEV)
    drafts[1, 0] = V
    drafts[2, 0] = -3
    got = _check_vsample(tl, dl, drafts.contiguous(), 1.0, 1.0, seed=4)
    assert np.all(got[0] == 0) and np.all((got[1] >= 0) & (got[1] < 8))


def test_verify_sample_flags_non_finite():
    N, D, V = 3, 4, 300
    g = torch.Generator(device=DEV).manual_seed(9)
    dl = torch.randn((N, D, V), generator=g, device=DEV)
    tl = torch.randn((N, D + 1, V), generator=g, device=DEV)
    tl[1, 2, 17] = float("nan")
    dl[2, 0, 5] = float("inf")
    drafts = torch.randint(0, V, (N, D), generator=g, device=DEV, dtype=torch.int32)
    got = _vsample_gpu(tl, dl, drafts.contiguous(), 1.0, 1.0, 5)
    assert got[3].tolist() == [0, 1, 1]


def test_verify_sample_unaligned_logits():
    """Logits that start 4 bytes past a 16-byte boundary take the scalar load paths."""
    N, D, R, V = 3, 6, 7, 5003
    g = torch.Generator(device=DEV).manual_seed(12)
    tb = torch.randn(N * R * V + 1, generator=g, device=DEV) * 2.0
    db = torch.randn(N * D * V + 1, generator=g, device=DEV) * 2.0
    tl = tb[1:].view(N, R, V)
    dl = db[1:].view(N, D, V)
    tl[:, :D] = dl + 0.5
    drafts = torch.from_numpy(dnc.sample_drafts(dl.cpu().numpy(), 1, 1.0, seed=6)[:, 0]).to(DEV)
    _check_vsample(tl, dl, drafts.contiguous(), 1.0, 1.2, seed=8)


# ---- top-p nucleus drafting ----

def _top_p_gpu(logits, K, T, p, seed):
    N, D, V = logits.shape
    ws = torch.empty(dbd.sample_top_p_workspace_bytes(N, D, V), dtype=torch.uint8, device=DEV)
    out = torch.full((N, K, D), -7, dtype=torch.int32, device=DEV)
    dbd.sample_top_p(logits, K, T, p, seed, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("N,D,V,K,T,p", [(2, 5, 37, 4, 1.0, 0.9), (3, 7, 4099, 8, 1.5, 0.5),
                                         (2, 4, 10000, 3, 0.7, 0.95), (1, 3, 8192, 2, 1.0, 0.3),
                                         (2, 32, 1000, 8, 1.5, 0.99), (4, 2, 300, 1, 2.0, 0.05)])
def test_top_p_sampling_bit_exact(N, D, V, K, T, p):
    print(f"top-p N={N} D={D} V={V} K={K} T={T} p={p}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(N * 31 + V + D)
    logits = torch.randn((N, D, V), generator=g, device=DEV) * 3.0
    got = _top_p_gpu(logits, K, T, p, seed=99)
    ref = dnc.sample_drafts(logits.cpu().numpy(), K, T, 99, top_p=p)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("p", [0.2, 0.5, 0.8])
def test_top_p_boundary_inside_tie_groups(p):
    """Small integer logits: many tokens share each weight, so the nucleus boundary falls inside
    a tie group and the lowest indices of it are taken."""
    N, D, V, K = 3, 6, 5000, 6
    g = torch.Generator(device=DEV).manual_seed(int(p * 100))
    logits = torch.randint(-4, 3, (N, D, V), generator=g, device=DEV).float()
    got = _top_p_gpu(logits, K, 1.0, p, seed=5)
    ref = dnc.sample_drafts(logits.cpu().numpy(), K, 1.0, 5, top_p=p)
    assert np.array_equal(got, ref)


def test_top_p_workload_vocabulary_and_limits():
    N, D, V, K = 2, 4, 151936, 8
    g = torch.Generator(device=DEV).manual_seed(17)
    logits = torch.randn((N, D, V), generator=g, device=DEV) * 2.5
    lc = logits.cpu().numpy()
    assert np.array_equal(_top_p_gpu(logits, K, 1.5, 0.9, 4), dnc.sample_drafts(lc, K, 1.5, 4, top_p=0.9))
    # p = 1: plain sampling; tiny p: the argmax
    ws = torch.empty(dbd.sample_workspace_bytes(N, D, V), dtype=torch.uint8, device=DEV)
    plain = torch.empty((N, K, D), dtype=torch.int32, device=DEV)
    dbd.sample_from_logits(logits, K, 1.5, 4, plain, ws)
    torch.cuda.synchronize()
    assert np.array_equal(_top_p_gpu(logits, K, 1.5, 1.0, 4), plain.cpu().numpy())
    tiny = _top_p_gpu(logits, K, 1.5, 1e-7, 4)
    assert np.array_equal(tiny, np.broadcast_to(lc.argmax(-1)[:, None, :], tiny.shape))


# ---- limits of the interface ----

def test_largest_vocabulary_verify_sample_and_top_p():
    """V = 2^18 - 1, the largest vocabulary the integer weights allow (Z < 2^58): greedy and
    stochastic verification, sampling and top-p, all bit-exact."""
    V, N, D = (1 << 18) - 1, 2, 3
    g = torch.Generator(device=DEV).manual_seed(21)
    dl = torch.randn((N, D, V), generator=g, device=DEV) * 2.0
    tl = torch.cat([dl + 0.4 * torch.randn((N, D, V), generator=g, device=DEV),
                    torch.randn((N, 1, V), generator=g, device=DEV)], 1).contiguous()
    drafts = torch.from_numpy(dnc.sample_drafts(dl.cpu().numpy(), 1, 1.0, seed=2)[:, 0]).to(DEV)
    drafts = drafts.contiguous()
    _check_verify(tl, drafts)
    _check_vsample(tl, dl, drafts, 1.0, 1.0, seed=6)
    ref = dnc.sample_drafts(dl.cpu().numpy(), 4, 1.3, 11, top_p=0.8)
    assert np.array_equal(_top_p_gpu(dl, 4, 1.3, 0.8, 11), ref)


def test_sixty_four_drafts_per_position():
    N, D, V, K = 2, 5, 3000, 64
    g = torch.Generator(device=DEV).manual_seed(22)
    logits = torch.randn((N, D, V), generator=g, device=DEV) * 2.0
    ws = torch.empty(dbd.sample_workspace_bytes(N, D, V), dtype=torch.uint8, device=DEV)
    out = torch.empty((N, K, D), dtype=torch.int32, device=DEV)
    dbd.sample_from_logits(logits, K, 1.5, 123, out, ws)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(),
                          dnc.sample_drafts(logits.cpu().numpy(), K, 1.5, 123))


def _plateau_rows(V, per_chunk_counts, rest=-20.0, seed=0):
    """One row per entry: per_chunk_counts[c] tokens of chunk c (4096 wide) at logit 0, every
    other token at `rest`; the nucleus boundary then lies inside the plateau's tie group."""
    rng = np.random.default_rng(seed)
    rows = []
    for counts in per_chunk_counts:
        r = np.full(V, rest, dtype=np.float32)
        for c, k in enumerate(counts):
            lo, hi = c * 4096, min(V, (c + 1) * 4096)
            r[rng.choice(np.arange(lo, hi), size=k, replace=False)] = 0.0
        rows.append(r)
    return np.stack(rows)


def test_top_p_bin_capacities_and_row_rescan():
    """Rows at both sides of the stored-key capacities (256 per chunk, 6144 per row) in one call,
    next to ordinary rows: the LDS radix select and the rescan of the row give the oracle's draws."""
    V = 151936
    nch = (V + 4095) // 4096
    plate = _plateau_rows(V, [[256, 256] + [0] * (nch - 2),          # stored, LDS
                              [256, 257] + [0] * (nch - 2),          # chunk 1 overflows
                              [161] * nch,                           # 6118 keys: LDS
                              [162] * nch])                          # 6156 keys: rescan
    g = torch.Generator(device=DEV).manual_seed(23)
    rnd = (torch.randn((2, V), generator=g, device=DEV) * 2.0).cpu().numpy()
    logits = torch.from_numpy(np.concatenate([plate, rnd])).reshape(3, 2, V).to(DEV)
    lc = logits.cpu().numpy()
    for p in (0.3, 0.999):
        print(f"top-p capacities p={p}", flush=True)
        got = _top_p_gpu(logits, 8, 1.0, p, 31)
        assert np.array_equal(got, dnc.sample_drafts(lc, 8, 1.0, 31, top_p=p))


def test_top_p_uniform_rows():
    """All weights equal: every token lies in one bin, the boundary is an index cut."""
    N, D, V, K = 1, 3, 20000, 8
    logits = torch.zeros((N, D, V), device=DEV)
    logits[0, 1] = 5.0
    for p in (0.01, 0.5, 0.9999):
        got = _top_p_gpu(logits, K, 1.0, p, 3)
        assert np.array_equal(got, dnc.sample_drafts(logits.cpu().numpy(), K, 1.0, 3, top_p=p))
        n = int(np.ceil(p * V))
        assert got.max() < n        # the nucleus is the n lowest indices
