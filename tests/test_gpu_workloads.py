"""End-to-end GPU parity of the layer-mode dispatcher on the five workloads
(at full size, in the launch configuration the benchmark uses), against the
CPU oracle: Top-K / pool indices bit-exact on every checked row, FP4 codes
bit-exact on every entry the oracle attends, attention within 2e-3.  The
layer outputs, selections and pool sit between guard regions that must stay
untouched.  The oracle runs on a thread pool (its C calls release the GIL)."""
import concurrent.futures
import os

import numpy as np
import pytest
import torch

import oracle
from fp4_kv_cache_csa2_amd import api, inputs, workload
from gpu_common import assert_attn_close, case, require_gpu, to_np

pytestmark = pytest.mark.gpu
GUARD = 4096
WORKERS = min(16, os.cpu_count() or 1)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    oracle.build(force=False)


def _host_seq(inst, b):
    lo, hi = int(inst.offsets[b]), int(inst.offsets[b + 1])
    return inputs.bf16_bits(inst.k_logical[lo:hi])


def _guarded(shape, dtype, dev):
    nbytes = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
    whole = torch.full((GUARD + nbytes + GUARD,), 0xA5, dtype=torch.uint8, device=dev)
    return whole, whole[GUARD:GUARD + nbytes].view(dtype).view(shape)


def guard_runner(run):
    """Move the runner's outputs, selection and pool into guarded buffers."""
    w, dev = run.inst.w, run.inst.latent.device
    wholes = []
    for l in range(w.layers):
        a, run.o[l] = _guarded(tuple(run.o[l].shape), torch.float32, dev)
        b, run.lse[l] = _guarded(tuple(run.lse[l].shape), torch.float32, dev)
        wholes += [a, b]
    a, run.state.idx = _guarded(tuple(run.state.idx.shape), torch.int32, dev)
    b, run.state.pool = _guarded(tuple(run.state.pool.shape), torch.int32, dev)
    wholes += [a, b]
    run.state.c.idx = run.state.idx.data_ptr()
    run.state.c.pool = run.state.pool.data_ptr()
    return wholes


def check_guards(wholes):
    for i, g in enumerate(wholes):
        g = to_np(g)
        assert (g[:GUARD] == 0xA5).all() and (g[-GUARD:] == 0xA5).all(), f"guard {i}: write outside an output"


def _oracle_row(inst, r):
    """Oracle selections of query row r (and the visible count it derives from
    the row's token position)."""
    w = inst.w
    b, q = divmod(r, w.Q)
    nv = oracle.visible_entries(int(inst.q_pos_host[b, q]), w.ratio)
    K_b = _host_seq(inst, b)
    qi = [None if L["q_idx"] is None else inputs.bf16_bits(L["q_idx"][b, q]) for L in inst.layers]
    sel, pool = oracle.select_stack(w.pattern, K_b, nv, qi, w.K, w.P)
    return dict(r=r, nv=nv, sel=sel, pool=pool)


def check_instance(inst, rows_idx, rows_attn, heads=None, run=None):
    """Run the pattern on the GPU once and compare the given rows."""
    w = inst.w
    run = workload.StackRunner(inst) if run is None else run
    wholes = guard_runner(run)
    case(f"{w.name}: B={w.B} Q={w.Q} N={inst.n_max} pattern={w.pattern}")
    run.step(keep_indices=True)
    torch.cuda.synchronize()
    check_guards(wholes)
    gidx = [to_np(t) for t in run.idx]
    gpool = to_np(run.pool)
    go = [to_np(t) for t in run.o]
    gl = [to_np(t) for t in run.lse]
    sc = inst.sm_scale
    rows_attn = set(rows_attn)
    need_rows = sorted(set(rows_idx) | rows_attn)
    hs = slice(None) if heads is None else heads
    swa_h = [L["swa"].double().cpu().numpy() for L in inst.layers]
    q_h = [L["q"][:, :, hs].double().cpu().numpy() for L in inst.layers]

    def one(r):
        b, q = divmod(r, w.Q)
        res = _oracle_row(inst, r)
        assert res["nv"] == int(inst.n_vis_host[b, q]), f"row {r}: visible entries differ"
        for l in range(w.layers):
            np.testing.assert_array_equal(gidx[l][r], res["sel"][l], err_msg=f"{w.name} row {r} layer {l} idx")
        if res["pool"] is not None:
            np.testing.assert_array_equal(gpool[r], res["pool"], err_msg=f"{w.name} row {r} pool")
        return res

    with concurrent.futures.ThreadPoolExecutor(WORKERS) as ex:
        results = {res["r"]: res for res in ex.map(one, need_rows)}
    # FP4 codes of exactly the entries the checked rows attend, checked against the cache
    enc = {}
    for r in sorted(rows_attn):
        b, q = divmod(r, w.Q)
        sel = results[r]["sel"]
        ids = np.unique(np.concatenate([s[s >= 0] for s in sel]))
        lat = inst.latent[torch.from_numpy(inst.offsets[b] + ids).to(inst.latent.device)]
        rc, rs = oracle.fp4_encode(to_np(lat))
        phys = torch.from_numpy(inst.phys_rows(b, ids)).to(inst.latent.device)
        np.testing.assert_array_equal(to_np(inst.cache.codes[phys]), rc, err_msg="FP4 codes")
        np.testing.assert_array_equal(to_np(inst.cache.scales[phys]), rs, err_msg="FP4 scales")
        enc[r] = (ids, rc, rs)

    def attn(args):
        r, l = args
        b, q = divmod(r, w.Q)
        ids, rc, rs = enc[r]
        sel = results[r]["sel"][l]
        idx_c = np.where(sel >= 0, np.searchsorted(ids, sel), -1).astype(np.int32)
        o, lse = oracle.attention(q_h[l][b, q], rc, rs, idx_c, swa_h[l][b], int(inst.q_pos_host[b, q]), w.window, sc)
        return assert_attn_close(go[l][b, q, hs], gl[l][b, q, hs], o, lse, f"{w.name} r{r} L{l}")

    jobs = [(r, l) for r in sorted(rows_attn) for l in range(w.layers)]
    with concurrent.futures.ThreadPoolExecutor(WORKERS) as ex:
        worst = max(ex.map(attn, jobs), default=0.0)
    print(f"{w.name}: {len(need_rows)} rows' indices, {len(rows_attn)} rows' attention; "
          f"worst attention row-relative error {worst:.2e}")
    return run


def test_small_stack_all_modes():
    w = inputs.Workload("small_stack", B=3, Q=1, N=40000, D=256, H=32, H_i=8, D_i=128, pattern="FUURUU", P=300)
    inst = workload.make_instance(w)
    check_instance(inst, range(3), range(3))


def test_short_context_pool_is_whole_context():
    # N <= 2048 * 8: the pool covers everything, Reindex behaves like Full.
    w = inputs.Workload("short_pool", B=2, Q=1, N=9000, D=128, H=16, H_i=4, D_i=64, pattern="FRUR")
    inst = workload.make_instance(w)
    check_instance(inst, range(2), range(2))


@pytest.mark.parametrize("distinct", [8, 96])
def test_tied_scores_pool_and_topk(distinct):
    """Indexer-K rows drawn from a few distinct vectors: scores and block
    maxima tie in large groups, so the pool and every Top-K are decided by the
    lower-position rule.  A pool-building Full layer takes its Top-K from its
    pool (K <= P), which must still equal the Top-K over every entry; the
    pool-less Full layer and the P < K layer take theirs from all scores."""
    import dataclasses
    base = inputs.Workload("tied", B=2, Q=1, N=30000, D=128, H=16, H_i=4, D_i=64, pattern="FRU", P=2048)
    for w in (base, dataclasses.replace(base, name="tied_small_pool", P=300),
              dataclasses.replace(base, name="tied_no_pool", pattern="FUU")):
        inst = workload.make_instance(w)
        g = torch.Generator(device="cpu").manual_seed(11 + distinct)
        rows = torch.randn(distinct, w.D_i, generator=g).to(torch.bfloat16)
        pick = torch.randint(0, distinct, (inst.k_logical.shape[0],), generator=g)
        # the contiguous view shares the logical K tensor
        assert inst.kview.k.data_ptr() == inst.k_logical.data_ptr()
        inst.k_logical.copy_(rows[pick].to(inst.k_logical.device))
        check_instance(inst, range(2), range(2))


def _set_positions(inst, q_pos):
    """Give every query row its own token position (and so its visible count)."""
    q_pos = np.asarray(q_pos, np.int32).reshape(inst.w.B, inst.w.Q)
    inst.q_pos_host = q_pos
    inst.q_pos = torch.from_numpy(q_pos).to(inst.q_pos.device)
    inst.n_vis_host = ((q_pos + 1) // inst.w.ratio).astype(np.int32)
    inst.n_vis = torch.from_numpy(inst.n_vis_host).to(inst.q_pos.device)


def _screen_instance(name, N, Q=80, B=2, seed=0):
    w = inputs.Workload(name, B=B, Q=Q, N=N, D=128, H=16, H_i=8, D_i=128, pattern="FU", window=64)
    inst = workload.make_instance(w, seed=seed)
    assert inst.kview.k.data_ptr() == inst.k_logical.data_ptr()
    return inst


def test_screened_selection_many_rows():
    """Many query rows (the matrix-core screen with exact rescoring): every
    row's Top-K equals the oracle's, with row tiles and entry tiles both cut
    short (80 rows of 2 sequences, 5000 entries) and visible counts from 0 to
    all, including rows with fewer than K entries or blocks."""
    inst = _screen_instance("screen_rows", N=5000)
    rng = np.random.default_rng(5)
    q_pos = rng.integers(0, 5000, size=(2, 80))
    q_pos[0, :6] = [0, 1, 100, 511, 512, 4999]
    q_pos[1, :4] = [4999, 4998, 8190 // 2, 7000 // 2]
    _set_positions(inst, q_pos)
    check_instance(inst, range(160), [0, 5, 81], heads=slice(0, 16, 4))


@pytest.mark.parametrize("kind", ["ties", "near_ties_all_candidates", "near_ties_overflow"])
def test_screened_selection_adversarial(kind):
    """Scores that the screen cannot separate: exact ties (K rows from four
    vectors), and near-ties (one vector plus single-ulp changes) whose scores
    all fall inside the screen's error band -- every entry is a candidate
    (exact ranking among them), or more than the candidate buffer holds (the
    full exact fallback)."""
    N = 3000 if kind == "near_ties_all_candidates" else 6000
    inst = _screen_instance("screen_" + kind, N=N, Q=64, B=1, seed=3)
    n = inst.k_logical.shape[0]
    g = torch.Generator(device="cpu").manual_seed(17)
    if kind == "ties":
        base = torch.randn(4, 128, generator=g).to(torch.bfloat16)
        k = base[torch.randint(0, 4, (n,), generator=g)]
    else:
        base = torch.randn(128, generator=g).to(torch.bfloat16)
        bits = base.view(torch.int16).repeat(n, 1)
        # one ulp up or down on three random channels of every row
        ch = torch.randint(0, 128, (n, 3), generator=g)
        step = torch.randint(0, 2, (n, 3), generator=g).to(torch.int16) * 2 - 1
        bits.scatter_add_(1, ch, step)
        k = bits.view(torch.bfloat16)
    inst.k_logical.copy_(k.to(inst.k_logical.device))
    rng = np.random.default_rng(9)
    _set_positions(inst, rng.integers(N // 2, N, size=(1, 64)))
    check_instance(inst, range(64), [0, 63], heads=slice(0, 16, 8))


def test_full_decode_n4k():
    inst = workload.make_instance(inputs.WORKLOADS["full_decode_n4k"])
    check_instance(inst, [0], [0])


def test_decoder_group_b8_n64k():
    inst = workload.make_instance(inputs.WORKLOADS["decoder_group_b8_n64k"])
    check_instance(inst, range(8), range(8))


def test_hier_decode_b4_n1m():
    inst = workload.make_instance(inputs.WORKLOADS["hier_decode_b4_n1m"])
    run = check_instance(inst, range(4), range(4))
    # determinism: a second step reproduces every index and output bit for bit
    first = [t.clone() for t in run.o] + [t.clone() for t in run.idx]
    case("hier_decode_b4_n1m: second step")
    run.step(keep_indices=True)
    torch.cuda.synchronize()
    for a, b in zip(first, list(run.o) + list(run.idx)):
        assert torch.equal(a, b)


def test_ragged_paged_b64():
    inst = workload.make_instance(inputs.WORKLOADS["ragged_paged_b64"])
    assert inst.page_table_host is not None and inst.lengths.min() >= 4096
    rows = sorted(set(range(0, 64, 4)) | {int(np.argmax(inst.lengths)), int(np.argmin(inst.lengths))})
    assert len(rows) >= 16
    check_instance(inst, range(64), rows)


def test_encoder_prefill_q2k_n32k():
    inst = workload.make_instance(inputs.WORKLOADS["encoder_prefill_q2k_n32k"])
    # indices of every query row; attention of every head of 32 rows, among
    # them all eight rows of the first and of the last persistent workgroup
    # (rows w, w + 256, ...: each row's set-up overlaps the previous row's end)
    rows = sorted({w + 256 * i for w in (0, 255) for i in range(8)} | {1, 2, 100, 700, 1300, 1500, 1800, 1999, 2046,
                                                                       2030, 77, 333, 901, 1777, 1100, 1650})
    assert len(rows) == 32
    check_instance(inst, range(2048), rows)


def _fp4_path_rerun(inst, run):
    """Every Reuse layer again with the staged copy switched off (the FP4 path:
    each selected entry dequantised by the attention itself): outputs must be
    bit for bit the staged ones."""
    w = inst.w
    staged_o = [t.clone() for t in run.o]
    staged_l = [t.clone() for t in run.lse]
    n = 0
    for l, mode in enumerate(w.pattern):
        if mode != "U":
            continue
        L = inst.layers[l]
        run.state.c.has_stage = 0
        case(f"{w.name}: layer {l} without the staged copy")
        api.csa2_layer_forward("U", q=L["q"], q_idx=None, swa_kv=L["swa"], q_pos=inst.q_pos, window=w.window,
                               sm_scale=inst.sm_scale, o=run.o[l], lse=run.lse[l], cache=inst.cache,
                               kview=inst.kview, n_vis=inst.n_vis, n_max=inst.n_max, K=w.K, P=0, build_pool=False,
                               ws=run.ws, state=run.state)
        torch.cuda.synchronize()
        bad = staged_o[l].view(torch.int32) != run.o[l].view(torch.int32)
        if bool(bad.any()):
            rows_bad = bad.reshape(bad.shape[0] * bad.shape[1], -1).any(dim=1).nonzero().flatten().tolist()
            d = (staged_o[l] - run.o[l]).abs().max().item()
            raise AssertionError(f"layer {l} o: {int(bad.sum())} elements differ in {len(rows_bad)} rows "
                                 f"(first {rows_bad[:12]}), max |diff| {d:.3e}")
        assert torch.equal(staged_l[l].view(torch.int32), run.lse[l].view(torch.int32)), f"layer {l} lse"
        n += 1
    assert n >= 1


@pytest.mark.parametrize("B,Q,N,K,window,paged", [
    (2, 300, 8192, 200, 128, True),   # paged cache; 13 + 8 = 21 chunks (a padding chunk); 2 or 3 rows per workgroup
    (1, 256, 4096, 512, 0, False),    # no window; one row per workgroup
])
def test_staged_prefill_attention(B, Q, N, K, window, paged):
    """Many query rows per sequence: the Full layer stages an fp16 copy of the
    shared cache and the group's layers attend from it.  Indices and sampled
    attention rows against the oracle, then the Reuse layers rerun on the FP4
    path must reproduce the staged outputs bit for bit."""
    import dataclasses
    w = dataclasses.replace(inputs.WORKLOADS["encoder_prefill_q2k_n32k"], name=f"staged_b{B}_q{Q}", B=B, Q=Q, N=N,
                            K=K, window=window, pattern="FUU", ragged=paged)
    inst = workload.make_instance(w, lengths=np.full(B, N, np.int32))
    rows = B * Q
    run = check_instance(inst, [0, rows // 2, rows - 1], [0, 1, 255, rows - 1])
    assert run.state.c.has_stage == 1 and run.state.c.stage_n == N
    _fp4_path_rerun(inst, run)


def test_fp4_ring_slots_change_kind():
    """Persistent FP4 attention whose ring slots change kind inside a row (13
    FP4 chunks, then window chunks, so a chunk pair holds one of each) and back
    at each row's start: every producer copies into its own quarter of a slot,
    so none overwrites another's unread copies.  Four instances, each checked
    bit for bit against the staged path (a shared slot layout made a row or two
    of most instances wrong)."""
    import dataclasses
    w = dataclasses.replace(inputs.WORKLOADS["encoder_prefill_q2k_n32k"], name="ring_kinds", B=2, Q=300, N=8192,
                            K=208, window=128, pattern="FUU", ragged=True)
    for seed in range(4):
        inst = workload.make_instance(w, seed=seed, lengths=np.full(2, 8192, np.int32))
        run = workload.StackRunner(inst)
        case(f"ring_kinds seed {seed}")
        run.step()
        torch.cuda.synchronize()
        assert run.state.c.has_stage == 1
        _fp4_path_rerun(inst, run)


def test_staged_prefill_bit_identical_at_full_size():
    """The 2048-row prefill chunk (eight rows per persistent workgroup): staged
    and FP4-path outputs of every Reuse layer bit for bit equal."""
    inst = workload.make_instance(inputs.WORKLOADS["encoder_prefill_q2k_n32k"])
    run = workload.StackRunner(inst)
    case("encoder_prefill_q2k_n32k: staged step")
    run.step()
    torch.cuda.synchronize()
    assert run.state.c.has_stage == 1
    _fp4_path_rerun(inst, run)


def test_multi_decode_b4_q4_n1m():
    # 4 causal query tokens per sequence: the scan shares K blocks among a
    # sequence's rows, the pool and Top-K histograms come from their own pass
    inst = workload.make_instance(inputs.WORKLOADS["multi_decode_b4_q4_n1m"])
    assert list(inst.n_vis_host[0]) == [inst.n_max - 3, inst.n_max - 2, inst.n_max - 1, inst.n_max]
    run = check_instance(inst, range(16), [0, 7, 13], heads=slice(0, 64, 8))
    # a second step on the same workspace (its Top-K counters left cleared by the
    # first, not zeroed again) reproduces every index and output
    first = [t.clone() for t in run.o] + [t.clone() for t in run.idx]
    case("multi_decode_b4_q4_n1m: second step")
    run.step(keep_indices=True)
    torch.cuda.synchronize()
    for a, b in zip(first, list(run.o) + list(run.idx)):
        assert torch.equal(a, b)


def test_workspace_shared_across_context_lengths():
    """One workspace and group state serve calls whose n_max changes (a growing
    context) and whose row count changes: the selection counters sit at the
    start of the workspace, where no other size moves them, and a different
    workspace or row count makes the next call clear them again."""
    import dataclasses
    base = inputs.Workload("grow_a", B=2, Q=1, N=100000, D=256, H=32, H_i=8, D_i=128, pattern="FRU", P=2048)
    insts = [workload.make_instance(base),
             workload.make_instance(dataclasses.replace(base, name="grow_b", N=70000), seed=1),
             workload.make_instance(dataclasses.replace(base, name="grow_c", B=3, N=90000), seed=2)]
    nbytes = max(api.csa2_layer_workspace_size(i.w.B, 1, i.w.H, i.w.D, i.n_max, i.w.K, i.w.P) for i in insts)
    dev = insts[0].latent.device
    ws = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(2)]
    state = api.GroupState(3, base.K, base.P, dev)
    for step, (k, wsi) in enumerate([(0, 0), (1, 0), (0, 0), (2, 0), (1, 0), (0, 1), (1, 0)]):
        inst = insts[k]
        run = workload.StackRunner(inst)
        run.ws = ws[wsi]
        rows = inst.rows
        # the same state (its flags and workspace record) with buffers of this row count
        state.idx = torch.empty(rows, base.K, dtype=torch.int32, device=dev)
        state.pool = torch.empty(rows, base.P, dtype=torch.int32, device=dev)
        run.state = state
        case(f"shared workspace step {step}: {inst.w.name} N={inst.n_max} rows={rows} ws={wsi}")
        check_instance(inst, range(rows), [0], heads=slice(0, 32, 4), run=run)
        assert state.c.ws_clean == 1 and state.c.clean_rows == rows
