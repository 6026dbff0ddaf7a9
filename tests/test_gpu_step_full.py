"""GPU tests of the fused decode step (gva_decode_step) at full workload sizes
and under the automatic split into thirds: every step is compared bit for bit
with gva_append + gva_rope_query + gva_decode on an identical cache (output,
lengths and both caches) and element by element with the oracle's step.

The decode loop these follow is the GQA tutorial page's (section KV Cache
为什么会不断变大): append the new token's state, then its query reads every
cached token including itself."""
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


def _two_caches(wl, inp, lens, steps, paged, seed):
    """Two identical caches holding the first lens[b] tokens of every sequence
    (appended through gva_append from the pre-RoPE keys), with room for
    `steps` more tokens per sequence."""
    caches = []
    if paged:
        table, nblk = W.paged_pool(np.asarray(lens) + steps, 64, seed)
    for _ in range(2):
        if paged:
            c = GvaCache(wl.B, wl.H, wl.G, 64, 64, wl.d_r, dtype=wl.dtype,
                         block_table=torch.tensor(table), num_blocks=nblk)
        else:
            c = GvaCache(wl.B, wl.H, wl.G, 64, 64, wl.d_r, dtype=wl.dtype,
                         capacity=int(np.max(lens)) + steps)
        for b, n in enumerate(lens):
            if n > 0:
                c.append_one(b, S.dev(inp.V[b][:, :n], wl.dtype), S.dev(inp.kr[b][:n], wl.dtype), BASE)
        caches.append(c)
    torch.cuda.synchronize()
    return caches


def _run_steps(wl, inp, lens, steps, caches, split, expect_thirds=False):
    ca, cb = caches
    qn, qr, Md = (S.dev(x, wl.dtype) for x in (inp.q_nope, inp.q_rope, inp.M))
    td = W.torch_dtype(wl.dtype)
    out_a = torch.full((wl.B, wl.H, 64), float("nan"), dtype=td, device="cuda")
    out_b = torch.full_like(out_a, float("nan"))
    q_rot = torch.empty_like(qr)
    top = int(np.max(lens)) + steps
    ws_a = ca.workspace(top, split)
    ws_b = cb.step_workspace(top, split)
    for i in range(steps):
        max_len = int(np.max(lens)) + i + 1
        sh = cb.shape(max_len, split)
        used = gva.gva_decode_split_tokens(sh)
        if expect_thirds:
            assert 3 * used >= max_len > 2 * used, "the automatic split cuts the longest sequence into thirds"
        print(f"[case] {wl.name} step {i} max_len={max_len} split={used}", flush=True)
        v1 = S.dev(np.stack([inp.V[b][:, n + i] for b, n in enumerate(lens)]), wl.dtype)  # [B, G, d_v]
        k1 = S.dev(np.stack([inp.kr[b][n + i] for b, n in enumerate(lens)]), wl.dtype)    # [B, d_r]
        ca.append(v1.unsqueeze(2).contiguous(), k1.unsqueeze(1).contiguous(), BASE)
        gva.gva_rope_query(ca.shape(max_len, split), qr, q_rot, ca.seq_lens, BASE)
        ca.decode(qn, q_rot, Md, wl.scale, out_a, max_len, split, workspace=ws_a)
        cb.step(v1, k1, qn, qr, Md, wl.scale, out_b, max_len, split, workspace=ws_b)
        torch.cuda.synchronize()
        assert torch.equal(ca.seq_lens, cb.seq_lens)
        assert cb.seq_lens.cpu().numpy().tolist() == (np.asarray(lens) + i + 1).tolist()
        assert torch.equal(out_a, out_b), (out_a.float() - out_b.float()).abs().max()
        ref = O.gva_decode_step(inp.V, inp.kr, inp.q_nope, inp.q_rope, inp.M, np.asarray(lens) + i + 1,
                                wl.scale, BASE, wl.dtype)
        S.assert_close(S.host(out_b), ref, wl.dtype, f"{wl.name} fused step {i}")
    assert torch.equal(ca.v_cache, cb.v_cache)
    assert torch.equal(ca.kr_cache, cb.kr_cache)


def test_step_ragged_paged_full_auto_thirds():
    """The ragged paged workload (B=64, lengths uniform in [1024, 32768],
    shuffled 64-token pages) with the automatic split, which cuts it into
    thirds; one new token per sequence per step, two steps."""
    wl = W.WORKLOADS["ragged_paged"]
    steps = 2
    inp = W.make_gva_inputs(wl, extra=steps)
    lens = inp.lens
    assert (lens == W.ragged_lens(wl)).all()
    caches = _two_caches(wl, inp, lens, steps, paged=True, seed=wl.seed)
    _run_steps(wl, inp, lens, steps, caches, split=0, expect_thirds=True)


def test_step_auto_thirds_with_empty_and_ties():
    """A batch that fills the compute units by itself (B*G = 256), mostly short
    sequences, four of about 30.8K tokens (480 tiles and more, with a tie in
    length) and one empty sequence that receives its first tokens."""
    wl = W.Workload("thirds_step", 9, B=64, H=16, G=4, d_n=64, d_v=64, d_r=16, S=0, dtype="bf16")
    rng = np.random.default_rng(71)
    lens = rng.integers(1, 3000, size=wl.B)
    lens[[5, 17, 40, 63]] = [30800, 31000, 30721, 30800]
    lens[3] = 0
    steps = 2
    inp = W.make_gva_inputs(wl, lens=lens, extra=steps, seed=72)
    caches = _two_caches(wl, inp, lens, steps, paged=True, seed=73)
    _run_steps(wl, inp, lens, steps, caches, split=0, expect_thirds=True)


def test_step_long_split_full():
    """The long workload (B=4, 131072 tokens per sequence after the step,
    4096-token partitions): prefill 131071 tokens, then one fused step."""
    wl = W.WORKLOADS["long_split"]
    steps = 1
    lens = np.full(wl.B, wl.S - steps)
    inp = W.make_gva_inputs(wl, lens=lens, extra=steps)
    caches = _two_caches(wl, inp, lens, steps, paged=False, seed=0)
    _run_steps(wl, inp, lens, steps, caches, split=wl.split_tokens)
