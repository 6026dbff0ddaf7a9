"""Randomized GPU parity sweep: decode, fused-step, several-query, prefill and
GQA-reference cases drawn once from a fixed seed over the shapes the library
accepts (G in {1, 2, 4, 8}, H/G in {1, 2, 4}, d_r in {0, 8, 16, 24, 32}, bf16
and fp32, contiguous and paged, automatic and explicit partitions) and length
mixes that include empty sequences, single tokens and tile boundaries. Each
case is checked against the CPU oracle at the decode tolerances; the
fused-step cases are also checked bit for bit against the three separate
calls on an identical cache. A case's id names its draw."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests import gpu_setup as S
from tests.test_gpu_multi import _run as _multi_run
from tests.test_gpu_parity import _decode_post_rope, _gqa_run
from tests.test_gpu_prefill import _cache as _prefill_cache
from tests.test_gpu_prefill import _prefill, _queries, _rotate
from tests.test_gpu_step import BASE, _new_token, _pair_of_caches

pytestmark = pytest.mark.gpu

gva = pytest.importorskip("compact_kv_cache_amd")

_EDGE_LENS = (0, 1, 2, 63, 64, 65, 127, 128, 129, 511, 512, 513)


def _draw_lens(rng, B, hi):
    lens = rng.integers(1, hi, size=B, endpoint=True)
    for b in range(B):                       # about a third of the rows take an edge length
        if rng.random() < 0.35:
            lens[b] = min(int(rng.choice(_EDGE_LENS)), hi)
    return lens


def _decode_cases(n=32, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        G = int(rng.choice([1, 2, 4, 8]))
        hpg = int(rng.choice([1, 2, 4]))
        d_r = int(rng.choice([0, 8, 16, 24, 32]))
        dtype = "f32" if rng.random() < 0.25 else "bf16"
        paged = bool(rng.random() < 0.5)
        split = int(rng.choice([0, 0, 64, 128, 320, 1024]))
        B = int(rng.integers(1, 5, endpoint=True))
        lens = _draw_lens(rng, B, int(rng.choice([200, 700, 1500])))
        if lens.max() == 0:
            lens[0] = 1
        cases.append(dict(i=i, G=G, hpg=hpg, d_r=d_r, dtype=dtype, paged=paged, split=split, lens=lens))
    return cases


def _step_cases(n=12, seed=20261204):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        cases.append(dict(i=i, G=int(rng.choice([1, 2, 4, 8])), hpg=int(rng.choice([1, 2, 4])),
                          d_r=int(rng.choice([0, 8, 16, 24, 32])),
                          dtype="f32" if rng.random() < 0.25 else "bf16", paged=bool(rng.random() < 0.5),
                          split=int(rng.choice([0, 64, 192, 512])),
                          lens=_draw_lens(rng, int(rng.integers(1, 4, endpoint=True)), 900)))
    return cases


def _other_cases(kind, n, seed, d_rs):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        c = dict(i=i, G=int(rng.choice([1, 2, 4, 8])), hpg=int(rng.choice([1, 2, 4])), d_r=int(rng.choice(d_rs)),
                 dtype="bf16", paged=bool(rng.random() < 0.5), split=int(rng.choice([0, 64, 256])),
                 lens=np.maximum(_draw_lens(rng, int(rng.integers(1, 3, endpoint=True)), 700), 1))
        if kind == "multi":
            c["nq"] = int(rng.choice([2, 4]))
        elif kind == "prefill":
            c["split"] = 0
            c["nq"] = int(rng.choice([0, 1, 4, 37, 100]))    # 0: the whole prompt
        cases.append(c)
    return cases


def _id(c):
    nq = f"-q{c['nq']}" if "nq" in c else ""
    return (f"{c['i']}-G{c['G']}h{c['hpg']}r{c['d_r']}-{c['dtype']}-{'paged' if c['paged'] else 'contig'}"
            f"-s{c['split']}{nq}-n{'_'.join(str(int(x)) for x in c['lens'])}")


@pytest.fixture(autouse=True)
def _gpu():
    S.need_gpu()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("c", _decode_cases(), ids=_id)
def test_decode_sweep(c):
    wl = W.Workload("sweep", 9 + c["i"], B=len(c["lens"]), H=c["G"] * c["hpg"], G=c["G"], d_n=64, d_v=64,
                    d_r=c["d_r"], S=0, dtype=c["dtype"])
    out, ref = _decode_post_rope(wl, c["lens"], paged=c["paged"], split=c["split"], seed=100 + c["i"])
    for b, n in enumerate(c["lens"]):
        if n == 0:       # an empty sequence attends to nothing: exact zeros
            assert np.array_equal(out[b], np.zeros_like(out[b]))
    S.assert_close(out, ref, c["dtype"], f"sweep {_id(c)}")


@pytest.mark.parametrize("c", _step_cases(), ids=_id)
def test_step_sweep(c):
    dtype = c["dtype"]
    lens = c["lens"]
    wl = W.Workload("sweep_step", 9 + c["i"], B=len(lens), H=c["G"] * c["hpg"], G=c["G"], d_n=64, d_v=64,
                    d_r=c["d_r"], S=0, dtype=dtype)
    cap = int(lens.max()) + 8
    split = c["split"]
    inp, (ca, cb) = _pair_of_caches(wl, lens, cap, c["paged"], seed=200 + c["i"])
    qn, qr, Md = (S.dev(x, dtype) for x in (inp.q_nope, inp.q_rope, inp.M))
    if c["d_r"] == 0:
        qr = None
    out_a = torch.empty(wl.B, wl.H, 64, dtype=W.torch_dtype(dtype), device="cuda")
    out_b = torch.empty_like(out_a)
    q_rot = None if qr is None else torch.empty_like(qr)
    ws_b = cb.step_workspace(cap, split)
    for i in range(2):
        max_len = int(lens.max()) + i + 1
        print(f"[case] step sweep {_id(c)} i={i}", flush=True)
        v1, k1 = _new_token(inp, lens, i, dtype)
        k_app = None if c["d_r"] == 0 else k1.unsqueeze(1).contiguous()
        ca.append(v1.unsqueeze(2).contiguous(), k_app, BASE)
        if qr is not None:
            gva.gva_rope_query(ca.shape(max_len, split), qr, q_rot, ca.seq_lens, BASE)
        ca.decode(qn, q_rot, Md, wl.scale, out_a, max_len, split)
        cb.step(v1, None if c["d_r"] == 0 else k1, qn, qr, Md, wl.scale, out_b, max_len, split, workspace=ws_b)
        torch.cuda.synchronize()
        assert torch.equal(ca.seq_lens, cb.seq_lens)
        assert torch.equal(out_a, out_b), (out_a.float() - out_b.float()).abs().max()
        ref = O.gva_decode_step(inp.V, inp.kr, inp.q_nope, inp.q_rope, inp.M, lens + i + 1, wl.scale, BASE,
                                dtype)
        S.assert_close(S.host(out_b), ref, dtype, f"step sweep {_id(c)} i={i}")
    assert torch.equal(ca.v_cache, cb.v_cache)
    if c["d_r"] > 0:
        assert torch.equal(ca.kr_cache, cb.kr_cache)


@pytest.mark.parametrize("c", _other_cases("multi", 10, 20261205, [8, 16, 24, 32]), ids=_id)
def test_multi_sweep(c):
    lens = c["lens"]
    wl = W.Workload("sweep_multi", 9 + c["i"], B=len(lens), H=c["G"] * c["hpg"], G=c["G"], d_n=64, d_v=64,
                    d_r=c["d_r"], S=0, dtype="bf16")
    print(f"[case] multi sweep {_id(c)}", flush=True)
    got, ref, _ = _multi_run(wl, lens, c["nq"], paged=c["paged"], split=c["split"], seed=300 + c["i"])
    S.assert_close(got, ref, "bf16", f"multi sweep {_id(c)}")


@pytest.mark.parametrize("c", _other_cases("prefill", 10, 20261206, [0, 8, 16, 24, 32]), ids=_id)
def test_prefill_sweep(c):
    lens = c["lens"]
    wl = W.Workload("sweep_prefill", 9 + c["i"], B=len(lens), H=c["G"] * c["hpg"], G=c["G"], d_n=64, d_v=64,
                    d_r=c["d_r"], S=0, dtype="bf16")
    nq = c["nq"] or int(lens.max())
    inp = W.make_gva_inputs(wl, lens=lens, seed=400 + c["i"])
    print(f"[case] prefill sweep {_id(c)}", flush=True)
    cache = _prefill_cache(wl, inp, lens, c["paged"], seed=401 + c["i"])
    shape = cache.shape(int(lens.max()))
    qn, qr = _queries(wl, nq, seed=402 + c["i"])
    got = _prefill(cache, shape, nq, S.dev(qn, "bf16"), _rotate(cache, shape, nq, qr), S.dev(inp.M, "bf16"),
                   wl.scale)
    ref = O.gva_prefill_step(inp.V, inp.kr, qn, qr, inp.M, lens, wl.scale, BASE, "bf16")
    assert not np.isnan(got).any()
    S.assert_close(got, ref, "bf16", f"prefill sweep {_id(c)}")
    for b, n in enumerate(lens):      # queries before a sequence's first token read nothing
        assert np.all(got[b, :max(nq - n, 0)] == 0)


@pytest.mark.parametrize("c", _other_cases("gqa", 8, 20261207, [0]), ids=_id)
def test_gqa_sweep(c):
    lens = c["lens"]
    wl = W.Workload("sweep_gqa", 9 + c["i"], B=len(lens), H=c["G"] * c["hpg"], G=c["G"], d_n=64, d_v=64,
                    d_r=0, S=0, dtype="bf16")
    out, ref = _gqa_run(wl, lens, paged=c["paged"], split=c["split"], seed=500 + c["i"])
    S.assert_close(out, ref, "bf16", f"gqa sweep {_id(c)}")
