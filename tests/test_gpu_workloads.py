"""End-to-end GPU parity of the layer-mode dispatcher on the five workloads
(at full size, in the launch configuration the benchmark uses), against the
CPU oracle: Top-K / pool indices bit-exact on every checked row, FP4 codes
bit-exact on every entry the oracle attends, attention within 2e-3."""
import numpy as np
import pytest
import torch

import oracle
from fp4_kv_cache_csa2_amd import inputs, workload
from gpu_common import assert_attn_close, case, require_gpu, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    oracle.build(force=False)


def _host_seq(inst, b):
    lo, hi = int(inst.offsets[b]), int(inst.offsets[b + 1])
    return inputs.bf16_bits(inst.k_logical[lo:hi])


def check_instance(inst, rows_idx, rows_attn, heads=None):
    """Run the pattern on the GPU once and compare the given rows."""
    w = inst.w
    run = workload.StackRunner(inst)
    case(f"{w.name}: B={w.B} Q={w.Q} N={inst.n_max} pattern={w.pattern}")
    run.step(keep_indices=True)
    torch.cuda.synchronize()
    gidx = [to_np(t) for t in run.idx]
    gpool = to_np(run.pool)
    go = [to_np(t) for t in run.o]
    gl = [to_np(t) for t in run.lse]
    sc = inst.sm_scale
    worst = 0.0
    need_rows = sorted(set(rows_idx) | set(rows_attn))
    for r in need_rows:
        b, q = divmod(r, w.Q)
        K_b = _host_seq(inst, b)
        qi = [None if L["q_idx"] is None else inputs.bf16_bits(L["q_idx"][b, q]) for L in inst.layers]
        sel, pool = oracle.select_stack(w.pattern, K_b, int(inst.n_vis_host[b, q]), qi, w.K, w.P)
        for l in range(w.layers):
            np.testing.assert_array_equal(gidx[l][r], sel[l], err_msg=f"{w.name} row {r} layer {l} idx")
        if pool is not None:
            np.testing.assert_array_equal(gpool[r], pool, err_msg=f"{w.name} row {r} pool")
        if r not in rows_attn:
            continue
        # oracle FP4 codes of exactly the entries attended, checked against the cache
        ids = np.unique(np.concatenate([s[s >= 0] for s in sel]))
        lat = inst.latent[torch.from_numpy(inst.offsets[b] + ids).to(inst.latent.device)]
        rc, rs = oracle.fp4_encode(to_np(lat))
        phys = torch.from_numpy(inst.phys_rows(b, ids)).to(inst.latent.device)
        np.testing.assert_array_equal(to_np(inst.cache.codes[phys]), rc, err_msg="FP4 codes")
        np.testing.assert_array_equal(to_np(inst.cache.scales[phys]), rs, err_msg="FP4 scales")
        hs = slice(None) if heads is None else heads
        for l, L in enumerate(inst.layers):
            idx_c = np.where(sel[l] >= 0, np.searchsorted(ids, sel[l]), -1).astype(np.int32)
            qn = L["q"][b, q, hs].double().cpu().numpy()
            swa = L["swa"][b].double().cpu().numpy()
            o, lse = oracle.attention(qn, rc, rs, idx_c, swa, int(inst.q_slot_host[b, q]), w.window, sc)
            worst = max(worst, assert_attn_close(go[l][b, q, hs], gl[l][b, q, hs], o, lse, f"{w.name} r{r} L{l}"))
    print(f"{w.name}: worst attention row-relative error {worst:.2e}")
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


def test_full_decode_n4k():
    inst = workload.make_instance(inputs.WORKLOADS["full_decode_n4k"])
    check_instance(inst, [0], [0])


def test_decoder_group_b8_n64k():
    inst = workload.make_instance(inputs.WORKLOADS["decoder_group_b8_n64k"])
    check_instance(inst, range(8), [0, 5, 7])


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
    check_instance(inst, range(64), [0, 17, int(np.argmax(inst.lengths)), int(np.argmin(inst.lengths))],
                   heads=slice(0, 64, 4))


def test_encoder_prefill_q2k_n32k():
    inst = workload.make_instance(inputs.WORKLOADS["encoder_prefill_q2k_n32k"])
    rows = [0, 1, 2, 100, 1023, 1024, 2046, 2047]
    check_instance(inst, rows, rows[::2], heads=slice(0, 64, 8))


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
