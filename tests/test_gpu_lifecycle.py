"""GPU tests of the paged-cache lifecycle calls (gva_copy_blocks, gva_fork,
gva_rollback): block contents and tables bit for bit, and decodes after
fork + copy-on-write + divergent appends, and after rollback + new appends,
against the CPU oracle on each sequence's own token history."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests import gpu_setup as S

pytestmark = pytest.mark.gpu

gva = pytest.importorskip("compact_kv_cache_amd")
from compact_kv_cache_amd.cache import GvaCache  # noqa: E402

BASE = 10000.0


@pytest.fixture(autouse=True)
def _gpu():
    S.need_gpu()
    yield
    torch.cuda.synchronize()


def _i32(x):
    return torch.tensor(np.asarray(x, dtype=np.int32), device="cuda")


def test_copy_blocks_bitwise_and_remap():
    torch.manual_seed(3)
    table = np.full((2, 4), -1, dtype=np.int32)
    table[0, :3] = [5, 2, 7]
    cache = GvaCache(2, 16, 4, 64, 64, 24, dtype="bf16", block_table=torch.tensor(table), num_blocks=12)
    cache.v_cache.copy_(torch.randn_like(cache.v_cache, dtype=torch.float32).bfloat16())
    cache.kr_cache.copy_(torch.randn_like(cache.kr_cache, dtype=torch.float32).bfloat16())
    v0, k0 = cache.v_cache.clone(), cache.kr_cache.clone()
    shape = cache.shape(256)
    print("[case] copy_blocks", flush=True)
    gva.gva_copy_blocks(shape, _i32([2, 7]), _i32([9, 11]), cache.v_cache, cache.kr_cache)
    torch.cuda.synchronize()
    for s, d in ((2, 9), (7, 11)):
        assert torch.equal(cache.v_cache[d], v0[s]) and torch.equal(cache.kr_cache[d], k0[s])
    untouched = [i for i in range(12) if i not in (9, 11)]
    assert torch.equal(cache.v_cache[untouched], v0[untouched])
    assert torch.equal(cache.kr_cache[untouched], k0[untouched])
    # copy-on-write form: copy block 5 to 10 and point sequence 1, slot 0 at it
    gva.gva_copy_blocks(shape, _i32([5]), _i32([10]), cache.v_cache, cache.kr_cache, cache.block_table,
                        remap_seqs=_i32([1]), remap_slots=_i32([0]))
    torch.cuda.synchronize()
    assert torch.equal(cache.v_cache[10], v0[5])
    assert cache.block_table.cpu().tolist() == [[5, 2, 7, -1], [10, -1, -1, -1]]
    # out-of-range pairs are skipped
    gva.gva_copy_blocks(shape, _i32([99]), _i32([0]), cache.v_cache, cache.kr_cache)
    torch.cuda.synchronize()
    assert torch.equal(cache.v_cache[0], v0[0])


def test_fork_copy_on_write_then_diverge():
    """Beam-style: sequence 0 holds a 150-token prefix; sequences 1 and 2 are
    forked from it (sharing its blocks), the partly filled last block is
    copied for each fork before it appends, then all three append different
    tokens and decode; each decode equals the oracle on its own history."""
    wl = W.Workload("fork", 9, B=3, H=16, G=4, d_n=64, d_v=64, d_r=16, S=0, dtype="bf16")
    prefix, extra = 150, 5
    inp = W.make_gva_inputs(wl, lens=np.full(3, prefix), extra=extra, seed=100)
    # sequence b's history: the prefix of sequence 0, then its own new tokens
    hist_v = [np.concatenate([inp.V[0][:, :prefix], inp.V[b][:, prefix:]], axis=1) for b in range(3)]
    hist_k = [np.concatenate([inp.kr[0][:prefix], inp.kr[b][prefix:]], axis=0) for b in range(3)]
    table = np.full((3, 4), -1, dtype=np.int32)
    table[0, :3] = [4, 0, 6]
    free = [1, 2, 3, 5, 7, 8, 9]
    cache = GvaCache(3, 16, 4, 64, 64, 16, dtype="bf16", block_table=torch.tensor(table), num_blocks=10)
    cache.append_one(0, S.dev(inp.V[0][:, :prefix], "bf16"), S.dev(inp.kr[0][:prefix], "bf16"), BASE)
    shape = cache.shape(256)
    print("[case] fork + copy-on-write", flush=True)
    gva.gva_fork(shape, _i32([0, 0]), _i32([1, 2]), cache.seq_lens, cache.block_table)
    torch.cuda.synchronize()
    assert cache.seq_lens.cpu().tolist() == [prefix] * 3
    assert cache.block_table.cpu().tolist() == [[4, 0, 6, -1]] * 3
    # the shared last block (slot 2, tokens 128..191, 22 filled) is copied for each fork
    cow = [free.pop(0), free.pop(0)]
    gva.gva_copy_blocks(shape, _i32([6, 6]), _i32(cow), cache.v_cache, cache.kr_cache, cache.block_table,
                        remap_seqs=_i32([1, 2]), remap_slots=_i32([2, 2]))
    for b in range(3):
        cache.append_one(b, S.dev(inp.V[b][:, prefix:], "bf16"), S.dev(inp.kr[b][prefix:], "bf16"), BASE)
    torch.cuda.synchronize()
    assert cache.block_table.cpu().tolist() == [[4, 0, 6, -1], [4, 0, cow[0], -1], [4, 0, cow[1], -1]]
    n = prefix + extra
    q_rot = torch.empty(3, 16, 16, dtype=torch.bfloat16, device="cuda")
    gva.gva_rope_query(shape, S.dev(inp.q_rope, "bf16"), q_rot, cache.seq_lens, BASE)
    out = torch.empty(3, 16, 64, dtype=torch.bfloat16, device="cuda")
    cache.decode(S.dev(inp.q_nope, "bf16"), q_rot, S.dev(inp.M, "bf16"), wl.scale, out, 256)
    torch.cuda.synchronize()
    ref = O.gva_decode_step(hist_v, hist_k, inp.q_nope, inp.q_rope, inp.M, np.full(3, n), wl.scale, BASE, "bf16")
    S.assert_close(S.host(out), ref, "bf16", "fork + copy-on-write + divergent appends")
    # the forks' appends did not touch sequence 0's block
    ref0 = O.append_positional_keys(hist_k[0][128:n], 128, BASE, "bf16")
    assert np.array_equal(S.host(cache.kr_cache[6])[:n - 128], ref0)


@pytest.mark.parametrize("paged", [False, True])
def test_rollback_then_new_tokens(paged):
    """Append 4 draft tokens, verify them as 4 queries, accept 1 (roll back 3),
    append the corrected token with a fused step: the result equals the oracle
    on the accepted history, and the step equals a cache that never saw the
    rejected drafts."""
    wl = W.Workload("rollback", 9, B=2, H=16, G=4, d_n=64, d_v=64, d_r=16, S=0, dtype="bf16")
    lens = np.array([500, 64])
    inp = W.make_gva_inputs(wl, lens=lens, extra=5, seed=110)
    rng = np.random.default_rng(111)
    drafts_v = W.round_storage(rng.standard_normal((2, 4, 4, 64)), "bf16")   # [B, G, 4, d_v]
    drafts_k = W.round_storage(rng.standard_normal((2, 4, 16)), "bf16")
    cap = 600

    def make():
        if paged:
            table, nblk = W.paged_pool(np.full(2, cap), 64, 112)
            c = GvaCache(2, 16, 4, 64, 64, 16, dtype="bf16", block_table=torch.tensor(table), num_blocks=nblk)
        else:
            c = GvaCache(2, 16, 4, 64, 64, 16, dtype="bf16", capacity=cap)
        for b, n in enumerate(lens):
            c.append_one(b, S.dev(inp.V[b][:, :n], "bf16"), S.dev(inp.kr[b][:n], "bf16"), BASE)
        return c

    ca, cb = make(), make()
    print(f"[case] rollback paged={paged}", flush=True)
    # speculative round on ca: 4 drafts (the first equal to the true next token)
    drafts_v[:, :, 0] = np.stack([inp.V[b][:, n] for b, n in enumerate(lens)])
    drafts_k[:, 0] = np.stack([inp.kr[b][n] for b, n in enumerate(lens)])
    ca.append(S.dev(drafts_v, "bf16"), S.dev(drafts_k, "bf16"), BASE)
    shape = ca.shape(cap)
    qn4 = W.round_storage(rng.standard_normal((2, 4, 16, 64)), "bf16")
    qr4 = W.round_storage(rng.standard_normal((2, 4, 16, 16)), "bf16")
    q_rot = torch.empty(2, 4, 16, 16, dtype=torch.bfloat16, device="cuda")
    gva.gva_rope_query_multi(shape, 4, S.dev(qr4, "bf16"), q_rot, ca.seq_lens, BASE)
    out4 = torch.empty(2, 4, 16, 64, dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(gva.gva_decode_multi_workspace_bytes(shape, 4) // 4 + 1, device="cuda")
    gva.gva_decode_multi(shape, 4, S.dev(qn4, "bf16"), q_rot, S.dev(inp.M, "bf16"), ca.v_cache, ca.kr_cache,
                         ca.seq_lens, ca.block_table, wl.scale, out4, ws)
    torch.cuda.synchronize()
    hv = [np.concatenate([inp.V[b][:, :n], drafts_v[b]], axis=1) for b, n in enumerate(lens)]
    hk = [np.concatenate([inp.kr[b][:n], drafts_k[b]], axis=0) for b, n in enumerate(lens)]
    ref4 = O.gva_decode_multi_step(hv, hk, qn4, qr4, inp.M, lens + 4, wl.scale, BASE, "bf16")
    for j in range(4):
        S.assert_close(S.host(out4)[:, j], ref4[:, j], "bf16", f"speculative verify query {j}")
    # accept one draft, roll back three
    gva.gva_rollback(shape, ca.seq_lens, _i32([3, 3]))
    torch.cuda.synchronize()
    assert ca.seq_lens.cpu().tolist() == (lens + 1).tolist()
    # the reference cache appends only the accepted token
    cb.append(S.dev(drafts_v[:, :, :1], "bf16"), S.dev(drafts_k[:, :1], "bf16"), BASE)
    # then both take the next true token with a fused step
    v1 = S.dev(np.stack([inp.V[b][:, n + 1] for b, n in enumerate(lens)]), "bf16")
    k1 = S.dev(np.stack([inp.kr[b][n + 1] for b, n in enumerate(lens)]), "bf16")
    outs = []
    for c in (ca, cb):
        o = torch.empty(2, 16, 64, dtype=torch.bfloat16, device="cuda")
        c.step(v1, k1, S.dev(inp.q_nope, "bf16"), S.dev(inp.q_rope, "bf16"), S.dev(inp.M, "bf16"), wl.scale, o,
               cap)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    ref = O.gva_decode_step(inp.V, inp.kr, inp.q_nope, inp.q_rope, inp.M, lens + 2, wl.scale, BASE, "bf16")
    S.assert_close(S.host(outs[0]), ref, "bf16", f"after rollback paged={paged}")


def test_rollback_clamps_and_ignores_negative():
    shape = gva.make_shape(3, 16, 4, 64, 64, 16, capacity=64, max_seq_len=64, dtype="bf16")
    lens = _i32([5, 10, 0])
    gva.gva_rollback(shape, lens, _i32([7, -2, 1]))
    torch.cuda.synchronize()
    assert lens.cpu().tolist() == [0, 10, 0]


@pytest.mark.parametrize("paged", [False, True])
def test_snapshot_restore_resumes_bit_for_bit(paged):
    """Checkpoint and resume of the cache state ([gqa] 与位置编码和 KV Cache 的关系:
    an engine commits or rolls back cache state): copy the caches, lengths and
    block table to the host, clobber the device copies, restore them, and
    continue with fused decode steps. Every output, length and cache row
    equals that of a cache that was never interrupted."""
    wl = W.Workload("snap", 9, B=3, H=16, G=4, d_n=64, d_v=64, d_r=16, S=0, dtype="bf16")
    lens = np.array([700, 65, 1300])
    steps = 4
    inp = W.make_gva_inputs(wl, lens=lens, extra=steps, seed=91)
    cap = int(lens.max()) + steps
    caches = []
    for _ in range(2):
        if paged:
            table, nblk = W.paged_pool(lens + steps, 64, 92)
            c = GvaCache(wl.B, wl.H, wl.G, 64, 64, wl.d_r, dtype="bf16",
                         block_table=torch.tensor(table), num_blocks=nblk)
        else:
            c = GvaCache(wl.B, wl.H, wl.G, 64, 64, wl.d_r, dtype="bf16", capacity=cap)
        for b, n in enumerate(lens):
            c.append_one(b, S.dev(inp.V[b][:, :n], "bf16"), S.dev(inp.kr[b][:n], "bf16"), BASE)
        caches.append(c)
    ref_c, c = caches
    qn, qr, Md = (S.dev(x, "bf16") for x in (inp.q_nope, inp.q_rope, inp.M))
    outs = [torch.empty(wl.B, wl.H, 64, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    ws = [x.step_workspace(cap) for x in caches]

    def step(which, i):
        x = caches[which]
        v1 = S.dev(np.stack([inp.V[b][:, n + i] for b, n in enumerate(lens)]), "bf16")
        k1 = S.dev(np.stack([inp.kr[b][n + i] for b, n in enumerate(lens)]), "bf16")
        x.step(v1, k1, qn, qr, Md, wl.scale, outs[which], int(lens.max()) + i + 1, workspace=ws[which])

    print(f"[case] snapshot/restore paged={paged}", flush=True)
    for i in range(2):
        step(0, i)
        step(1, i)
    torch.cuda.synchronize()
    state = c.snapshot()
    # clobber everything the snapshot holds
    c.v_cache.fill_(7.0)
    if c.kr_cache is not None:
        c.kr_cache.fill_(-3.0)
    c.seq_lens.fill_(5)
    if c.block_table is not None:
        c.block_table.fill_(0)
    torch.cuda.synchronize()
    c.restore(state)
    for i in range(2, steps):
        step(0, i)
        step(1, i)
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1])
        assert torch.equal(ref_c.seq_lens, c.seq_lens)
    assert torch.equal(ref_c.v_cache, c.v_cache)
    assert torch.equal(ref_c.kr_cache, c.kr_cache)
    ref = O.gva_decode_step(inp.V, inp.kr, inp.q_nope, inp.q_rope, inp.M, lens + steps, wl.scale, BASE, "bf16")
    S.assert_close(S.host(outs[1]), ref, "bf16", "resumed step")
    # a snapshot of another layout is refused
    with pytest.raises(ValueError):
        c.restore({k: v[:1] for k, v in state.items()})
