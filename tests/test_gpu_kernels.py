"""GPU parity of each C-ABI entry point against the CPU oracle on seeded inputs:
bit-exact FP4 codes, scores, Top-K and pool indices; attention within the
row-wise 2e-3 tolerance.  Sizes span several tiles plus ragged tails."""
import math

import numpy as np
import pytest
import torch

import oracle
from fp4_kv_cache_csa2_amd import api, inputs
from gpu_common import assert_attn_close, case, require_gpu, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    oracle.build(force=False)


# --------------------------------------------------------------------------- FP4 codec
def _codec_inputs(rows, D, tag):
    x = inputs.normal((rows, D), tag)
    # spread group magnitudes over the whole E4M3 range, incl. subnormal scales and saturation
    mag = torch.exp(inputs.uniform((rows, D // 16), tag + "/mag") * 40 - 25).float()
    x = x * mag.repeat_interleave(16, 1)
    x[0, :16] = 0.0
    x[0, 16:32] = -0.0
    x[1, :16] = torch.tensor([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0,
                              0.5])  # exact E2M1 ties at scale 1
    x[2, :16] = 1e30  # saturated scale
    return x


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_fp4_quantize_bit_exact(dtype):
    rows, D = 1037, 512
    x = _codec_inputs(rows, D, "codec").to(dtype)
    case(f"fp4_quantize rows={rows} D={D} {dtype}")
    codes = torch.empty(rows, D // 2, dtype=torch.uint8, device=DEV)
    scales = torch.empty(rows, D // 16, dtype=torch.uint8, device=DEV)
    api.csa2_fp4_quantize(x.to(DEV), codes, scales)
    y = torch.empty(rows, D, dtype=torch.float32, device=DEV)
    api.csa2_fp4_dequantize(codes, scales, y)
    torch.cuda.synchronize()
    rc, rs = oracle.fp4_encode(x.float().numpy())
    np.testing.assert_array_equal(to_np(scales), rs)
    np.testing.assert_array_equal(to_np(codes), rc)
    np.testing.assert_array_equal(to_np(y).astype(np.float64), oracle.fp4_decode(rc, rs))


def test_fp4_append_paged():
    B, D, ps = 5, 256, 64
    lengths = np.array([100, 64, 3, 200, 128])
    table, n_pages = inputs.random_page_table(lengths, ps, "app")
    codes = torch.zeros(n_pages * ps, D // 2, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(n_pages * ps, D // 16, dtype=torch.uint8, device=DEV)
    cache = api.Fp4Cache(codes, scales, D, 0, torch.from_numpy(table).to(DEV), ps)
    x = inputs.normal((B, D), "appx")
    pos = np.array([99, 0, 2, 150, 127], np.int32)
    case("fp4_append paged")
    api.csa2_fp4_append(x.to(DEV), torch.from_numpy(pos).to(DEV), cache)
    torch.cuda.synchronize()
    rc, rs = oracle.fp4_encode(x.numpy())
    for b in range(B):
        r = table[b, pos[b] // ps] * ps + pos[b] % ps
        np.testing.assert_array_equal(to_np(codes[r]), rc[b])
        np.testing.assert_array_equal(to_np(scales[r]), rs[b])
    assert int(codes.count_nonzero()) <= B * D // 2  # nothing else written


@pytest.mark.parametrize("paged,n_layers,with_k,xdtype", [(True, 4, True, torch.bfloat16),
                                                         (False, 3, True, torch.float32),
                                                         (False, 0, False, torch.bfloat16),
                                                         (True, 32, True, torch.bfloat16)])
def test_append_token(paged, n_layers, with_k, xdtype):
    B, D, D_i, T, ps = 5, 512, 128, 128, 64
    lengths = np.array([100, 64, 3, 200, 128])
    pos = np.array([99, 0, 2, 150, 127], np.int32)
    tok = pos + np.array([0, 1000, 7, 0, 129], np.int32)  # token positions (ring row = tok mod T)
    tag = f"apt{paged}{n_layers}"
    if paged:
        table, n_pages = inputs.random_page_table(lengths, ps, tag)
        n_rows, tab_d, stride = n_pages * ps, torch.from_numpy(table).to(DEV), 0
    else:
        n_rows, tab_d, stride = B * 256, None, 256
    codes = torch.zeros(n_rows, D // 2, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(n_rows, D // 16, dtype=torch.uint8, device=DEV)
    cache = api.Fp4Cache(codes, scales, D, stride, tab_d, ps if paged else 0)
    kbuf = torch.zeros(n_rows, D_i, dtype=torch.bfloat16, device=DEV)
    kview = api.IndexerK(kbuf, D_i, stride, tab_d, ps if paged else 0) if with_k else None
    x = inputs.normal((B, D), tag + "x", dtype=xdtype)
    k_new = inputs.normal((B, D_i), tag + "k", dtype=torch.bfloat16)
    swa_new = [inputs.normal((B, D), f"{tag}s{l}", dtype=torch.bfloat16).to(DEV) for l in range(n_layers)]
    swa_kv = [torch.zeros(B, T, D, dtype=torch.bfloat16, device=DEV) for _ in range(n_layers)]
    case(f"append_token paged={paged} n_layers={n_layers} k={with_k} {xdtype}")
    api.csa2_append_token(x.to(DEV), torch.from_numpy(pos).to(DEV), cache,
                          k_new.to(DEV) if with_k else None, kview, swa_new, swa_kv,
                          torch.from_numpy(tok).to(DEV))
    torch.cuda.synchronize()
    rc, rs = oracle.fp4_encode(x.float().numpy())
    rows = [(table[b, pos[b] // ps] * ps + pos[b] % ps) if paged else b * stride + pos[b] for b in range(B)]
    for b in range(B):
        np.testing.assert_array_equal(to_np(codes[rows[b]]), rc[b])
        np.testing.assert_array_equal(to_np(scales[rows[b]]), rs[b])
        if with_k:
            assert torch.equal(kbuf[rows[b]].cpu(), k_new[b])
        for l in range(n_layers):
            assert torch.equal(swa_kv[l][b, tok[b] % T].cpu(), swa_new[l][b].cpu())
    # nothing else written
    assert int(codes.count_nonzero()) <= B * D // 2
    assert int((kbuf != 0).any(dim=1).sum()) == (B if with_k else 0)
    for l in range(n_layers):
        assert int((swa_kv[l] != 0).any(dim=2).sum()) == B


# --------------------------------------------------------------------------- indexer
def _k_view(B, n_max, D_i, tag, paged, ps=64):
    K = inputs.normal((B, n_max, D_i), tag, dtype=torch.bfloat16)
    if not paged:
        return K, api.IndexerK(K.reshape(B * n_max, D_i).to(DEV), D_i, n_max)
    table, n_pages = inputs.random_page_table(np.full(B, n_max), ps, tag + "/pt")
    phys = torch.zeros(n_pages * ps, D_i, dtype=torch.bfloat16)
    for b in range(B):
        for j0 in range(0, n_max, ps):
            r = table[b, j0 // ps] * ps
            phys[r:r + min(ps, n_max - j0)] = K[b, j0:j0 + ps]
    return K, api.IndexerK(phys.to(DEV), D_i, 0, torch.from_numpy(table).to(DEV), ps)


@pytest.mark.parametrize("D_i,H_i,paged,ps", [(128, 8, False, 0), (64, 4, False, 0), (128, 8, True, 64),
                                             (128, 8, True, 16), (128, 8, True, 256)])
def test_index_full_bit_exact(D_i, H_i, paged, ps):
    """Pages of 64 entries or more hold whole 64-entry blocks (one-run loads);
    16-entry pages take the per-entry row lookup."""
    B, Q, n_max = 2, 3, 5000
    K, kview = _k_view(B, n_max, D_i, f"ifK{D_i}{paged}", paged, ps or 64)
    q = inputs.normal((B, Q, H_i, D_i), f"ifq{D_i}", dtype=torch.bfloat16)
    n_vis = np.array([[5000, 4999, 0], [1, 257, 3333]], np.int32)
    scores = torch.empty(B * Q, n_max, device=DEV)
    nb = (n_max + 7) // 8
    bmax = torch.empty(B * Q, nb, device=DEV)
    case(f"index_full D_i={D_i} paged={paged} ps={ps}")
    api.csa2_index_full(q.to(DEV), kview, torch.from_numpy(n_vis).to(DEV), n_max, scores, bmax)
    torch.cuda.synchronize()
    s, bm = to_np(scores), to_np(bmax)
    for b in range(B):
        Kb = inputs.bf16_bits(K[b])
        for qq in range(Q):
            ref = oracle.index_scores(inputs.bf16_bits(q[b, qq]), Kb, n_vis[b, qq])
            np.testing.assert_array_equal(s[b * Q + qq], ref)
            np.testing.assert_array_equal(bm[b * Q + qq], oracle.block_max(ref))


@pytest.mark.parametrize("Q,paged", [(2, False), (5, True), (8, False), (11, False), (11, True)])
def test_index_full_multi_row_bit_exact(Q, paged):
    """Several query rows per sequence share each K block (rows grouped 2/4/8,
    partial last groups, per-row visibility); scores must equal the oracle's
    row by row."""
    B, n_max, D_i, H_i = 2, 20000, 128, 8
    K, kview = _k_view(B, n_max, D_i, f"imK{Q}{paged}", paged)
    q = inputs.normal((B, Q, H_i, D_i), f"imq{Q}", dtype=torch.bfloat16)
    n_vis = inputs.small_ints((B, Q), f"imn{Q}", 0, n_max, dtype=torch.int32).numpy()
    n_vis[0, 0] = n_max
    scores = torch.empty(B * Q, n_max, device=DEV)
    nb = (n_max + 7) // 8
    bmax = torch.empty(B * Q, nb, device=DEV)
    case(f"index_full multi-row Q={Q} paged={paged}")
    api.csa2_index_full(q.to(DEV), kview, torch.from_numpy(n_vis).to(DEV), n_max, scores, bmax)
    torch.cuda.synchronize()
    s, bm = to_np(scores), to_np(bmax)
    for b in range(B):
        Kb = inputs.bf16_bits(K[b])
        for qq in range(Q):
            ref = oracle.index_scores(inputs.bf16_bits(q[b, qq]), Kb, n_vis[b, qq])
            np.testing.assert_array_equal(s[b * Q + qq], ref)
            np.testing.assert_array_equal(bm[b * Q + qq], oracle.block_max(ref))


@pytest.mark.parametrize("Q,paged", [(1, False), (1, True), (4, False)])
def test_index_full_block_max_only(Q, paged):
    """Scores left out, block maxima only (what a pool needs): the maxima must
    equal the oracle's, with several blocks per wave held back and written
    after the stream, ragged visibility and a partial last block."""
    B, n_max, D_i, H_i = 3, 300001, 128, 8
    K, kview = _k_view(B, n_max, D_i, f"bmK{Q}{paged}", paged)
    q = inputs.normal((B, Q, H_i, D_i), f"bmq{Q}", dtype=torch.bfloat16)
    n_vis = np.tile(np.array([[n_max], [n_max - 2], [12345]], np.int32), (1, Q))
    if Q > 1:
        n_vis[:, 1:] -= np.arange(1, Q, dtype=np.int32)
    nb = (n_max + 7) // 8
    bmax = torch.full((B * Q, nb), 7.0, device=DEV)
    case(f"index_full block maxima only Q={Q} paged={paged}")
    api.csa2_index_full(q.to(DEV), kview, torch.from_numpy(n_vis).to(DEV), n_max, None, bmax)
    torch.cuda.synchronize()
    bm = to_np(bmax)
    for b in range(B):
        Kb = inputs.bf16_bits(K[b])
        for qq in range(Q):
            ref = oracle.index_scores(inputs.bf16_bits(q[b, qq]), Kb, n_vis[b, qq])
            np.testing.assert_array_equal(bm[b * Q + qq], oracle.block_max(ref))


@pytest.mark.parametrize("paged", [False, True])
def test_index_reindex_bit_exact(paged):
    B, n_max, D_i, H_i, P = 2, 40000, 128, 8, 700
    K, kview = _k_view(B, n_max, D_i, f"riK{paged}", paged)
    q = inputs.normal((B, 1, H_i, D_i), "riq", dtype=torch.bfloat16)
    n_vis = np.array([[40000], [39990]], np.int32)
    pool = np.full((B, P), -1, np.int32)
    rng = np.random.default_rng(0)
    pool[0, :600] = np.sort(rng.choice(5000, 600, replace=False))
    pool[1, :P] = np.sort(rng.choice(5000, P, replace=False))
    pool[1, -1] = 4999  # block 4999 holds entries 39992.. -> partly invisible
    ps = torch.empty(B, 8 * P, device=DEV)
    case(f"index_reindex paged={paged}")
    api.csa2_index_reindex(q.to(DEV), kview, torch.from_numpy(n_vis).to(DEV), torch.from_numpy(pool).to(DEV), ps)
    torch.cuda.synchronize()
    got = to_np(ps)
    for b in range(B):
        ref = oracle.reindex_scores(inputs.bf16_bits(q[b, 0]), inputs.bf16_bits(K[b]), n_vis[b, 0], pool[b])
        np.testing.assert_array_equal(got[b], ref)


# --------------------------------------------------------------------------- Top-K
def _topk_case(rows, n, k, kind, tag):
    if kind == "normal":
        s = inputs.normal((rows, n), tag).numpy() * 30
    elif kind == "ties":
        s = inputs.small_ints((rows, n), tag, -40, 40, dtype=torch.float32).numpy()
    elif kind == "coarse":  # a few equal keys per value: short runs of ties at the threshold
        s = np.round(inputs.normal((rows, n), tag).numpy() * 120) / 4
    elif kind == "empty":  # no valid entry in any row: every output is -1
        return np.full((rows, n), -np.inf, np.float32)
    else:  # "flat": one value everywhere -> the threshold bin overflows any candidate buffer
        s = np.full((rows, n), 1.5, np.float32)
        s[:, ::5] = 2.5
    s[:, ::11] = -np.inf
    if rows > 1:
        s[1, 100:] = -np.inf  # a row with few valid entries
    return s


@pytest.mark.parametrize("rows,n,k,kind", [
    (3, 1, 512, "normal"), (4, 700, 512, "ties"), (2, 16384, 512, "normal"), (5, 16384, 2048, "ties"),
    (3, 16385, 512, "normal"), (4, 100000, 512, "ties"), (4, 100000, 1, "normal"), (2, 300000, 2048, "normal"),
    (2, 70000, 512, "flat"), (1, 1 << 20, 512, "normal"),
    # one-workgroup path: threshold bin resolved by ranking, by the radix fallback
    # (long ties, k > 1024), k at the bound's limit, single key, short rows
    (3, 16384, 512, "coarse"), (2, 16384, 512, "ties"), (2, 16384, 512, "flat"), (4, 16384, 1024, "normal"),
    (4, 16384, 1025, "coarse"), (2, 16384, 1, "normal"), (3, 5000, 512, "coarse"), (2, 600, 512, "normal"),
    # short rows with 4 and 8 keys per thread (up to 4096 and 8192 positions)
    (3, 4096, 512, "normal"), (3, 4096, 512, "flat"), (2, 4096, 2048, "normal"), (2, 4097, 512, "ties"),
    (2, 8192, 512, "ties"), (2, 8192, 1024, "coarse"),
    # rows without a single valid entry, on both paths
    (3, 16384, 512, "empty"), (2, 100000, 512, "empty"),
    # one workgroup with 32 keys per thread (16384 < n <= 32768), and the first
    # length past it
    (3, 32768, 512, "normal"), (2, 20000, 512, "ties"), (2, 32768, 2048, "coarse"), (2, 32768, 512, "flat"),
    (2, 16392, 1, "normal"), (4, 30001, 1024, "coarse"), (2, 32768, 512, "empty"), (2, 32769, 512, "normal")])
def test_topk_bit_exact(rows, n, k, kind):
    s = _topk_case(rows, n, k, kind, f"tk{rows}_{n}_{k}_{kind}")
    out = torch.empty(rows, k, dtype=torch.int32, device=DEV)
    nbytes = api.csa2_topk_workspace_size(rows, n, k)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV)
    case(f"topk rows={rows} n={n} k={k} {kind}")
    api.csa2_topk(torch.from_numpy(s).to(DEV), k, out, ws=ws)
    torch.cuda.synchronize()
    got = to_np(out)
    for r in range(rows):
        np.testing.assert_array_equal(got[r], oracle.topk(s[r], k), err_msg=f"row {r}")


@pytest.mark.parametrize("P", [2048, 4096])
def test_topk_with_pool_map(P):
    rows, k = 3, 512
    n = 8 * P
    s = inputs.normal((rows, n), "tkpool").numpy()
    pool = np.full((rows, P), -1, np.int32)
    rng = np.random.default_rng(1)
    for r in range(rows):
        nb = [P, 1500, 10][r]
        pool[r, :nb] = np.sort(rng.choice(200000, nb, replace=False))
        s[r, 8 * nb:] = -np.inf
    out = torch.empty(rows, k, dtype=torch.int32, device=DEV)
    case(f"topk pool map P={P}")
    api.csa2_topk(torch.from_numpy(s).to(DEV), k, out, pool_blocks=torch.from_numpy(pool).to(DEV))
    torch.cuda.synchronize()
    for r in range(rows):
        np.testing.assert_array_equal(to_np(out)[r], oracle.topk(s[r], k, pool[r]))


def test_topk_deterministic_and_workspace_reuse():
    rows, n, k = 4, 200000, 512
    s = torch.from_numpy(_topk_case(rows, n, k, "ties", "det")).to(DEV)
    ws = torch.empty(api.csa2_topk_workspace_size(rows, n, k), dtype=torch.uint8, device=DEV)
    outs = []
    case("topk determinism")
    for _ in range(3):
        o = torch.empty(rows, k, dtype=torch.int32, device=DEV)
        api.csa2_topk(s, k, o, ws=ws)
        outs.append(o)
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


# --------------------------------------------------------------------------- attention
def _attn_inputs(B, Q, H, D, n, K, T, qdtype, tag):
    lat = inputs.normal((B, n, D), tag + "/lat")
    codes = torch.empty(B * n, D // 2, dtype=torch.uint8, device=DEV)
    scales = torch.empty(B * n, D // 16, dtype=torch.uint8, device=DEV)
    api.csa2_fp4_quantize(lat.reshape(B * n, D).to(DEV), codes, scales)
    cache = api.Fp4Cache(codes, scales, D, n)
    q = inputs.normal((B, Q, H, D), tag + "/q", dtype=qdtype)
    idx = inputs.small_ints((B, Q, K), tag + "/idx", -1, n - 1, dtype=torch.int32)
    swa = inputs.normal((B, T, D), tag + "/swa", dtype=torch.bfloat16)
    # query token positions: early ones (short windows) and wrapped rings
    qpos = inputs.small_ints((B, Q), tag + "/qpos", 0, 5000, dtype=torch.int32)
    qpos.view(-1)[0] = 3
    rc, rs = oracle.fp4_encode(lat.reshape(B * n, D).numpy())
    return cache, q, idx, swa, qpos, rc.reshape(B, n, -1), rs.reshape(B, n, -1)


@pytest.mark.parametrize("B,Q,H,D,K,qdtype,window", [
    (2, 1, 64, 512, 512, torch.bfloat16, 128), (1, 1, 16, 128, 512, torch.float32, 128),
    (3, 2, 32, 256, 100, torch.bfloat16, 128), (600, 1, 16, 128, 48, torch.bfloat16, 128),
    # long lists at one or two rows: 16 splits, and 32 splits merged in two
    # batches of at most 24
    (2, 1, 32, 256, 1024, torch.float32, 128), (1, 1, 64, 512, 2048, torch.bfloat16, 128),
    # 5 sparse + 4 window chunks in 3 splits of 3: every split of the
    # producer/consumer kernel pads its odd range, with a sparse, a window and
    # a past-the-end chunk's kind
    (100, 1, 64, 512, 80, torch.bfloat16, 64),
    # many rows at D = 512, H = 64 (rows sampled): bf16 queries take the
    # producer/consumer kernel (chunks in pairs; 13 sparse chunks and a
    # one-chunk window exercise its padding chunk), fp32 queries the
    # one-workgroup kernel
    (520, 1, 64, 512, 512, torch.bfloat16, 128), (520, 1, 64, 512, 200, torch.bfloat16, 8),
    (300, 2, 64, 512, 200, torch.float32, 128),
    # a few more rows than four head groups x ten key splits fit in one round
    # over the CUs: fewer key splits keep the head split (12 rows: 5 splits of
    # 8 chunks; 7 rows: 9 splits of 5 chunks, each padded to an even count)
    (12, 1, 64, 512, 512, torch.bfloat16, 128), (7, 1, 64, 512, 512, torch.bfloat16, 128)])
def test_sparse_then_swa_merge(B, Q, H, D, K, qdtype, window):
    n, T = (3000 if B < 100 else 520), 200
    cache, q, idx, swa, qpos, rc, rs = _attn_inputs(B, Q, H, D, n, K, T, qdtype, f"at{B}{H}{D}{K}")
    sc = 1 / math.sqrt(D)
    o = torch.empty(B, Q, H, D, device=DEV)
    lse = torch.empty(B, Q, H, device=DEV)
    ws = torch.empty(max(api.csa2_attn_workspace_size(B, Q, H, D), 16), dtype=torch.uint8, device=DEV)
    case(f"sparse_attn B={B} Q={Q} H={H} D={D} K={K}")
    api.csa2_sparse_attn_fp4(q.to(DEV), cache, idx.to(DEV), sc, o, lse, ws=ws)
    torch.cuda.synchronize()
    o1, l1 = to_np(o), to_np(lse)
    case(f"swa_attn merge window={window}")
    api.csa2_swa_attn(q.to(DEV), swa.to(DEV), qpos.to(DEV), window, sc, 1, o, lse, ws=ws)
    torch.cuda.synchronize()
    o2, l2 = to_np(o), to_np(lse)
    qn = q.double().numpy()
    sw = swa.double().numpy()
    worst = 0.0
    rows = [(b, qq) for b in range(B) for qq in range(Q)]
    if len(rows) > 64:  # first, last and a seeded sample
        pick = np.random.default_rng(B * Q).choice(len(rows), 14, replace=False)
        rows = [rows[0], rows[-1]] + [rows[i] for i in pick]
    for b, qq in rows:
        ra, la = oracle.attention(qn[b, qq], rc[b], rs[b], idx[b, qq].numpy(), None, 0, 0, sc)
        worst = max(worst, assert_attn_close(o1[b, qq], l1[b, qq], ra, la, "sparse"))
        ru, lu = oracle.attention(qn[b, qq], rc[b], rs[b], idx[b, qq].numpy(), sw[b], int(qpos[b, qq]), window, sc)
        worst = max(worst, assert_attn_close(o2[b, qq], l2[b, qq], ru, lu, "merged"))
    print(f"worst row-relative error {worst:.2e}")


def test_swa_only_short_window_and_empty_sparse():
    B, Q, H, D, T = 2, 1, 64, 512, 128
    cache, q, idx, swa, qpos, rc, rs = _attn_inputs(B, Q, H, D, 100, 16, T, torch.bfloat16, "swo")
    qpos = torch.tensor([[0], [5]], dtype=torch.int32)  # first tokens: windows of 1 and 6 rows
    idx[:] = -1  # no selected entries at all
    sc = 0.05
    o = torch.empty(B, Q, H, D, device=DEV)
    lse = torch.empty(B, Q, H, device=DEV)
    ws = torch.empty(api.csa2_attn_workspace_size(B, Q, H, D), dtype=torch.uint8, device=DEV)
    case("sparse with empty selection")
    api.csa2_sparse_attn_fp4(q.to(DEV), cache, idx.to(DEV), sc, o, lse, ws=ws)
    torch.cuda.synchronize()
    assert torch.all(torch.isneginf(lse)) and torch.all(o == 0)
    case("swa merge after empty sparse")
    api.csa2_swa_attn(q.to(DEV), swa.to(DEV), qpos.to(DEV), 128, sc, 1, o, lse, ws=ws)
    torch.cuda.synchronize()
    for b in range(B):
        ref, lr = oracle.attention(q[b, 0].double().numpy(), None, None, None, swa[b].double().numpy(),
                                   int(qpos[b, 0]), 128, sc)
        assert_attn_close(to_np(o)[b, 0], to_np(lse)[b, 0], ref, lr, "swa-only")


@pytest.mark.parametrize("B,K,window", [(300, 512, 128), (290, 200, 24)])
def test_many_rows_paged_cache(B, K, window):
    """More query rows than compute units at D = 512, H = 64 (persistent
    workgroups, each walking several rows) over a paged FP4 cache, so that every
    key row goes through the page table; the second case's 13 sparse chunks
    give an odd count (padding chunk).  Sampled rows against the oracle, the
    window merged into the sparse output."""
    H, D, n, T, ps = 64, 512, 640, 200, 64
    tag = f"mrp{B}{K}"
    lat = inputs.normal((B, n, D), tag + "/lat")
    c_log = torch.empty(B * n, D // 2, dtype=torch.uint8, device=DEV)
    s_log = torch.empty(B * n, D // 16, dtype=torch.uint8, device=DEV)
    api.csa2_fp4_quantize(lat.reshape(B * n, D).to(DEV), c_log, s_log)
    table, n_pages = inputs.random_page_table(np.full(B, n), ps, tag + "/pages")
    phys = (table.astype(np.int64)[:, :, None] * ps + np.arange(ps)[None, None, :]).reshape(-1)
    codes = torch.zeros(n_pages * ps, D // 2, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(n_pages * ps, D // 16, dtype=torch.uint8, device=DEV)
    pr = torch.from_numpy(phys).to(DEV)
    codes[pr] = c_log
    scales[pr] = s_log
    cache = api.Fp4Cache(codes, scales, D, 0, torch.from_numpy(table).to(DEV), ps)
    q = inputs.normal((B, 1, H, D), tag + "/q", dtype=torch.bfloat16)
    idx = inputs.small_ints((B, 1, K), tag + "/idx", -1, n - 1, dtype=torch.int32)
    swa = inputs.normal((B, T, D), tag + "/swa", dtype=torch.bfloat16)
    qpos = inputs.small_ints((B, 1), tag + "/qpos", 0, 5000, dtype=torch.int32)
    qpos.view(-1)[1] = 5
    rc, rs = oracle.fp4_encode(lat.reshape(B * n, D).numpy())
    rc, rs = rc.reshape(B, n, -1), rs.reshape(B, n, -1)
    sc = 1 / math.sqrt(D)
    o = torch.empty(B, 1, H, D, device=DEV)
    lse = torch.empty(B, 1, H, device=DEV)
    ws = torch.empty(max(api.csa2_attn_workspace_size(B, 1, H, D), 16), dtype=torch.uint8, device=DEV)
    case(f"many rows paged B={B} K={K} window={window}")
    api.csa2_sparse_attn_fp4(q.to(DEV), cache, idx.to(DEV), sc, o, lse, ws=ws)
    api.csa2_swa_attn(q.to(DEV), swa.to(DEV), qpos.to(DEV), window, sc, 1, o, lse, ws=ws)
    torch.cuda.synchronize()
    og, lg = to_np(o), to_np(lse)
    qn, sw = q.double().numpy(), swa.double().numpy()
    pick = [0, 1, B - 1] + list(np.random.default_rng(B + K).choice(B, 13, replace=False))
    worst = 0.0
    for b in pick:
        ru, lu = oracle.attention(qn[b, 0], rc[b], rs[b], idx[b, 0].numpy(), sw[b], int(qpos[b, 0]), window, sc)
        worst = max(worst, assert_attn_close(og[b, 0], lg[b, 0], ru, lu, f"row {b}"))
    print(f"worst row-relative error {worst:.2e}")


@pytest.mark.parametrize("qdtype,qlog_lo,qlog_hi,sc", [
    (torch.bfloat16, -6.0, 1.5, None), (torch.float32, -6.0, 1.5, None),
    (torch.bfloat16, 3.0, 6.0, 1e-6), (torch.float32, 3.0, 6.0, 1e-6)])
def test_sparse_attn_extreme_magnitudes(qdtype, qlog_lo, qlog_hi, sc):
    """Entry rows spanning 10^-2.5 .. 10^1 (many E4M3 scales subnormal) and query
    heads spanning 10^qlog_lo .. 10^qlog_hi (scaled up or down by a power of two
    before the fp16 products; a tiny logit scale keeps the large ones' logits
    moderate): the fp16 datapath must stay within the tolerance."""
    B, Q, H, D, n, K = 2, 1, 64, 512, 2000, 512
    rmag = torch.pow(10.0, inputs.uniform((B * n, 1), "xm/rmag").double() * 3.5 - 2.5)
    lat = (inputs.normal((B * n, D), "xm/lat").double() * rmag).float()
    codes = torch.empty(B * n, D // 2, dtype=torch.uint8, device=DEV)
    scales = torch.empty(B * n, D // 16, dtype=torch.uint8, device=DEV)
    api.csa2_fp4_quantize(lat.to(DEV), codes, scales)
    rc, rs = oracle.fp4_encode(lat.numpy())
    assert np.any((rs > 0) & (rs < 8)), "no subnormal E4M3 scale in the sample"
    cache = api.Fp4Cache(codes, scales, D, n)
    qmag = torch.pow(10.0, inputs.uniform((B, Q, H, 1), "xm/qmag").double() * (qlog_hi - qlog_lo) + qlog_lo)
    q = (inputs.normal((B, Q, H, D), "xm/q").double() * qmag).to(qdtype)
    idx = inputs.small_ints((B, Q, K), "xm/idx", -1, n - 1, dtype=torch.int32)
    sc = 1 / math.sqrt(D) if sc is None else sc
    o = torch.empty(B, Q, H, D, device=DEV)
    lse = torch.empty(B, Q, H, device=DEV)
    ws = torch.empty(max(api.csa2_attn_workspace_size(B, Q, H, D), 16), dtype=torch.uint8, device=DEV)
    case(f"sparse_attn extreme magnitudes q={qdtype}")
    api.csa2_sparse_attn_fp4(q.to(DEV), cache, idx.to(DEV), sc, o, lse, ws=ws)
    torch.cuda.synchronize()
    rc, rs = rc.reshape(B, n, -1), rs.reshape(B, n, -1)
    worst = 0.0
    for b in range(B):
        ra, la = oracle.attention(q[b, 0].double().numpy(), rc[b], rs[b], idx[b, 0].numpy(), None, 0, 0, sc)
        worst = max(worst, assert_attn_close(to_np(o)[b, 0], to_np(lse)[b, 0], ra, la, "extreme"))
    print(f"worst row-relative error {worst:.2e}")


# --------------------------------------------------------------------------- Top-K: overflowing threshold bin
@pytest.mark.parametrize("k,n_above,n_ties,span", [
    (512, 300, 10000, 70000),   # > 8192 candidates in the row, 300 positions above the bin
    (2048, 300, 10000, 70000),  # k = 2048: the above-bin positions plus k would overrun a 2048-slot list
    (2048, 1900, 9000, 70000),  # only 148 picked inside the bin
    (512, 200, 5000, 16384),    # > 4096 candidates inside one 16384-position chunk (local overflow only)
    (1024, 0, 9000, 70000)])    # no position above the bin
def test_topk_overflowing_bin_with_positions_above(k, n_above, n_ties, span):
    """The threshold bin holds more candidates than the candidate lists keep,
    so the selection falls back to the whole row, while other positions lie
    above the bin and are already selected: the fallback may pick only inside
    the bin."""
    rows, n = 2, 70000
    rng = np.random.default_rng(k + n_above + span)
    s = (rng.standard_normal((rows, n)) - 6.0).astype(np.float32)   # below the tie value's bin
    s[:, ::13] = -np.inf
    for r in range(rows):
        tie_pos = rng.choice(span, n_ties, replace=False)
        s[r, tie_pos] = 1.5
        rest = np.setdiff1d(np.arange(n), tie_pos)
        above = rng.choice(rest, n_above, replace=False)
        s[r, above] = (10.0 + rng.random(n_above)).astype(np.float32)
    out = torch.empty(rows, k, dtype=torch.int32, device=DEV)
    ws = torch.empty(api.csa2_topk_workspace_size(rows, n, k), dtype=torch.uint8, device=DEV)
    case(f"topk overflow k={k} above={n_above} ties={n_ties} span={span}")
    api.csa2_topk(torch.from_numpy(s).to(DEV), k, out, ws=ws)
    torch.cuda.synchronize()
    got = to_np(out)
    for r in range(rows):
        np.testing.assert_array_equal(got[r], oracle.topk(s[r], k), err_msg=f"row {r}")


# --------------------------------------------------------------------------- canary guards
GUARD = 4096  # bytes before and after an output


def _guarded(shape, dtype):
    """(whole buffer, view): the view sits between two guard regions filled with 0xA5 bytes."""
    nbytes = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
    whole = torch.full((GUARD + nbytes + GUARD,), 0xA5, dtype=torch.uint8, device=DEV)
    view = whole[GUARD:GUARD + nbytes].view(dtype).view(shape)
    return whole, view


def _guards_intact(whole, what):
    g = to_np(whole)
    assert (g[:GUARD] == 0xA5).all() and (g[-GUARD:] == 0xA5).all(), f"{what}: write outside the output"


@pytest.mark.parametrize("rows,n,k", [(3, 5000, 512), (4, 16384, 2048), (2, 100000, 512), (2, 100000, 2048)])
def test_topk_writes_only_its_output(rows, n, k):
    s = _topk_case(rows, n, k, "coarse", f"guard{n}{k}")
    whole, out = _guarded((rows, k), torch.int32)
    ws = torch.empty(max(api.csa2_topk_workspace_size(rows, n, k), 16), dtype=torch.uint8, device=DEV)
    case(f"topk guards rows={rows} n={n} k={k}")
    api.csa2_topk(torch.from_numpy(s).to(DEV), k, out, ws=ws)
    torch.cuda.synchronize()
    _guards_intact(whole, "topk out")
    for r in range(rows):
        np.testing.assert_array_equal(to_np(out)[r], oracle.topk(s[r], k), err_msg=f"row {r}")


@pytest.mark.parametrize("B,H,D,K", [(4, 64, 512, 512), (300, 64, 512, 512), (3, 16, 128, 100)])
def test_attention_writes_only_its_outputs(B, H, D, K):
    n, T, Q = 3000, 200, 1
    cache, q, idx, swa, qpos, rc, rs = _attn_inputs(B, Q, H, D, n, K, T, torch.bfloat16, f"gd{B}{H}")
    wo, o = _guarded((B, Q, H, D), torch.float32)
    wl, lse = _guarded((B, Q, H), torch.float32)
    ws = torch.empty(max(api.csa2_attn_workspace_size(B, Q, H, D), 16), dtype=torch.uint8, device=DEV)
    sc = 1 / math.sqrt(D)
    case(f"attention guards B={B} H={H} D={D}")
    api.csa2_sparse_attn_fp4(q.to(DEV), cache, idx.to(DEV), sc, o, lse, ws=ws)
    api.csa2_swa_attn(q.to(DEV), swa.to(DEV), qpos.to(DEV), 128, sc, 1, o, lse, ws=ws)
    torch.cuda.synchronize()
    _guards_intact(wo, "o")
    _guards_intact(wl, "lse")
    for b in (0, B - 1):
        ru, lu = oracle.attention(q[b, 0].double().numpy(), rc[b], rs[b], idx[b, 0].numpy(), swa[b].double().numpy(),
                                  int(qpos[b, 0]), 128, sc)
        assert_attn_close(to_np(o)[b, 0], to_np(lse)[b, 0], ru, lu, "guarded")


# --------------------------------------------------------------------------- FP4 decode inside attention
def _all_codes_cache(n, D):
    """n entries whose code bytes run through all 256 values and whose scale
    bytes run through every finite non-negative E4M3 code 0x00..0x7E."""
    e = np.arange(n)[:, None]
    codes = ((e * (D // 2) + np.arange(D // 2)[None]) % 256).astype(np.uint8)
    scales = ((e * (D // 16) + np.arange(D // 16)[None]) % 127).astype(np.uint8)
    return codes, scales


@pytest.mark.parametrize("D,H,qdtype,rows", [
    (128, 16, torch.float32, 2), (128, 16, torch.bfloat16, 300), (256, 32, torch.bfloat16, 3),
    (256, 64, torch.float32, 400), (512, 64, torch.float32, 4),
    (512, 64, torch.bfloat16, 4),     # producer/consumer kernel, keys split over workgroups
    (512, 64, torch.bfloat16, 12),    # the same with fewer key splits (five) so that heads split too
    (512, 64, torch.bfloat16, 300)])  # producer/consumer kernel, whole list per workgroup
def test_attention_fp4_decode_bit_exact(D, H, qdtype, rows):
    """A query row that selects exactly one entry (window empty) has softmax
    weight exactly 1 on it, so its output is that entry's decoded value: the
    decode attention performs in registers must equal the oracle's FP4 decode
    bit for bit (signed zeros compare equal: the output sums from +0)."""
    K = 512
    n = 64  # entries 0 .. ceil(127 / (D/16)) - 1 already hold every code and scale byte
    codes, scales = _all_codes_cache(n, D)
    need = max(-(-127 // (D // 16)), -(-256 // (D // 2)))
    ref = oracle.fp4_decode(codes, scales)
    # every query row is its own sequence: one copy of the n entries per sequence
    # (entry j of sequence b is physical row b * n + j)
    codes_d = torch.from_numpy(np.tile(codes, (rows, 1))).to(DEV)
    scales_d = torch.from_numpy(np.tile(scales, (rows, 1))).to(DEV)
    cache = api.Fp4Cache(codes_d, scales_d, D, n)
    assert rows * cache.seq_stride <= codes_d.shape[0] and rows * cache.seq_stride <= scales_d.shape[0]
    sc = 1 / math.sqrt(D)
    checked = set()
    for g0 in range(0, n, rows):
        ent = (np.arange(rows) + g0) % n
        idx = np.full((rows, 1, K), -1, np.int32)
        idx[np.arange(rows), 0, (ent * 37) % K] = ent      # the one selected entry at varying list positions
        q = inputs.normal((rows, 1, H, D), f"fpx{D}{g0}", dtype=qdtype)
        o = torch.empty(rows, 1, H, D, device=DEV)
        lse = torch.empty(rows, 1, H, device=DEV)
        ws = torch.empty(max(api.csa2_attn_workspace_size(rows, 1, H, D), 16), dtype=torch.uint8, device=DEV)
        case(f"fp4 decode through attention D={D} H={H} {qdtype} rows={rows} group {g0}")
        api.csa2_sparse_attn_fp4(q.to(DEV), cache, torch.from_numpy(idx).to(DEV), sc, o, lse, ws=ws)
        torch.cuda.synchronize()
        got = to_np(o).astype(np.float64)
        for r in range(rows):
            np.testing.assert_array_equal(got[r, 0], np.broadcast_to(ref[ent[r]], (H, D)),
                                          err_msg=f"entry {ent[r]}")
            checked.add(int(ent[r]))
        if len(checked) >= need:
            break
    cb = np.unique(codes[sorted(checked)])
    sb = np.unique(scales[sorted(checked)])
    assert len(cb) == 256 and len(sb) == 127, (len(cb), len(sb))
