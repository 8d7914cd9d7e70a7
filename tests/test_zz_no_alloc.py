"""er_op_attention_noalloc (the attention op for callers that cannot allocate:
its split partials live in the library's fixed device scratch) against
er_op_attention on the same inputs: identical outputs, bit for bit (same
kernels, same split, same merge order), on two calls in a row, the second
smaller than the first, so the second reads scratch the first left behind;
and a call whose partials exceed the scratch is refused before any launch.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from speculative_decoding_rl_amd import ops as o
    return o


def _case(hq, hkv, hd, items, bf16, L=2, layer=1, seed=0):
    rng = np.random.Generator(np.random.PCG64(seed))
    nblk = [(c + q + 15) // 16 for c, q in items]
    total = sum(nblk) + 3
    perm = rng.permutation(total)
    bt = np.zeros((len(items), max(nblk)), dtype=np.int32)
    k = 0
    for i, nb in enumerate(nblk):
        bt[i, :nb] = perm[k:k + nb]
        k += nb
    tdt = torch.bfloat16 if bf16 else torch.float32
    pool = torch.from_numpy(rng.standard_normal((total, L, 2, hkv, 16, hd)).astype(np.float32)).to(tdt).cuda()
    Mq = sum(q for _, q in items)
    q = torch.from_numpy(rng.standard_normal((Mq, hq, hd)).astype(np.float32)).to(tdt).cuda()
    row0 = np.cumsum([0] + [q for _, q in items[:-1]]).astype(np.int32)
    i32 = lambda a: torch.from_numpy(np.asarray(a, dtype=np.int32)).cuda()
    args = dict(n_layers=L, layer=layer, hq=hq, hkv=hkv, hd=hd, block_table=i32(bt),
                bt_row=i32(np.arange(len(items))), q_row0=i32(row0), q_pos0=i32([c for c, _ in items]),
                q_count=i32([q for _, q in items]), max_q_count=max(q for _, q in items),
                max_ctx=max(c + q for c, q in items))
    return q, pool, Mq, tdt, args


def _run(fn, q, pool, Mq, tdt, hq, hd, args):
    out = torch.full((Mq, hq * hd), float("nan"), dtype=tdt, device="cuda")
    fn(q, out, pool, args["n_layers"], args["layer"], args["hq"], args["hkv"], args["hd"], args["block_table"],
       args["bt_row"], args["q_row0"], args["q_pos0"], args["q_count"], args["max_q_count"], args["max_ctx"])
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


@pytest.mark.parametrize("bf16", [True, False])
def test_noalloc_matches_attention_on_two_calls(ops, bf16):
    # first call: many split units (long contexts, verify rows); second: fewer, shorter
    cases = [dict(hq=28, hkv=4, hd=128, items=[(0, 1), (300, 5), (2000, 4), (4100, 1), (37, 3)], seed=1),
             dict(hq=28, hkv=4, hd=128, items=[(600, 2), (15, 1)], seed=2)]
    if not bf16:
        cases = [dict(hq=4, hkv=2, hd=64, items=[(3000, 4), (5, 3), (700, 1)], seed=3),
                 dict(hq=4, hkv=2, hd=64, items=[(900, 2)], seed=4)]
    for c in cases:
        q, pool, Mq, tdt, args = _case(c["hq"], c["hkv"], c["hd"], c["items"], bf16, seed=c["seed"])
        got = _run(ops.attention_noalloc, q, pool, Mq, tdt, c["hq"], c["hd"], args)
        ref = _run(ops.attention, q, pool, Mq, tdt, c["hq"], c["hd"], args)
        assert np.isfinite(ref).all()
        assert np.array_equal(got, ref), np.max(np.abs(got - ref))


def test_noalloc_refuses_partials_beyond_the_scratch(ops):
    from speculative_decoding_rl_amd import _lib
    # 72 items of 9 verify rows each (63 rows per KV head) with a 4096-key bound: 144 units x 4 heads
    # x 63 rows x 130 floats = 4.72 M floats of partials, over the 4 M-float (16 MiB) scratch
    items = [(8, 9)] * 72
    q, pool, Mq, tdt, args = _case(28, 4, 128, items, True, seed=5)
    args["max_ctx"] = 4096
    out = torch.zeros(Mq, 28 * 128, dtype=tdt, device="cuda")
    with pytest.raises(_lib.ErError) as ei:
        ops.attention_noalloc(q, out, pool, args["n_layers"], args["layer"], 28, 4, 128, args["block_table"],
                              args["bt_row"], args["q_row0"], args["q_pos0"], args["q_count"], 9, 4096)
    assert ei.value.code == _lib.ER_ENOMEM
    torch.cuda.synchronize()
    assert float(out.float().abs().sum()) == 0.0     # nothing was launched
