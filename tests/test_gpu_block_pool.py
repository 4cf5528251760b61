"""End to end through the host block pool: requests get their blocks from
the pool (three share a cached prefix), only their uncached tokens are
written through the pool's slot mapping, and decode attention over the pool's
block tables matches the oracle on the same cache contents."""
import numpy as np
import pytest

import oracle
from paged_kv_cache_50_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_50_amd import pagedkv
    pagedkv.lib()
    yield
    torch.cuda.synchronize()


def _kv_rows(tokens, first_pos, hkv, d, salt):
    """bf16 K or V rows as a fixed function of (token id, position): the same
    prefix gives the same rows in every request, as a model would."""
    rows = []
    for i, t in enumerate(tokens):
        rng = np.random.default_rng([salt, int(t), first_pos + i])
        rows.append(rng.standard_normal((hkv, d), dtype=np.float32))
    return W.f32_to_bf16_bits(np.stack(rows)) if rows else np.zeros((0, hkv, d), np.uint16)


def test_decode_over_pool_tables_with_prefix_cache():
    torch = G.torch()
    from paged_kv_cache_50_amd import pagedkv
    hq, hkv, d, bs, nb = 16, 4, 128, 16, 96
    rng = np.random.default_rng(5)
    shared = list(rng.integers(0, 1000, 40))
    prompts = [shared + list(rng.integers(0, 1000, n)) for n in (7, 30, 61)]
    prompts += [list(rng.integers(0, 1000, n)) for n in (1, 100, 333)]
    pool = pagedkv.BlockPool(nb, bs, prefix_caching=True)
    kc = np.full((nb, bs, hkv, d), W.BF16_QNAN, dtype=np.uint16)
    vc = kc.copy()
    dk, dv = G.np_to_dev(kc, "bf16"), G.np_to_dev(vc, "bf16")
    cached = []
    for r, toks in enumerate(prompts):
        c = pool.allocate(r, len(toks), toks)
        assert c >= 0
        cached.append(c)
        new = toks[c:]
        slots = pool.slot_mapping(r, c, len(new))
        key = _kv_rows(new, c, hkv, d, 1)
        val = _kv_rows(new, c, hkv, d, 2)
        oracle.kv_cache_write(kc, vc, key, val, slots, bs)
        if len(new):
            pagedkv.kv_cache_write(dk, dv, G.np_to_dev(key, "bf16"), G.np_to_dev(val, "bf16"),
                                   torch.from_numpy(slots).cuda())
        pool.cache_full_blocks(r, toks, len(toks))
    # requests 1 and 2 reuse the two full blocks of the shared 40-token prefix
    assert cached[:3] == [0, 32, 32]
    t0 = pool.block_table([0], 4)[0]
    for r in (1, 2):
        assert list(pool.block_table([r], 8)[0][:2]) == list(t0[:2])
    reqs = list(range(len(prompts)))
    lens = np.array([len(p) for p in prompts], dtype=np.int32)
    mb = int(max(pool.num_blocks_of(r) for r in reqs))
    bt = pool.block_table(reqs, mb)
    q = W.f32_to_bf16_bits(rng.standard_normal((len(reqs), hq, d)).astype(np.float32))
    torch.cuda.synchronize()
    assert np.array_equal(G.dev_to_bits(dk), kc) and np.array_equal(G.dev_to_bits(dv), vc)
    dq = G.np_to_dev(q, "bf16")
    out = torch.empty_like(dq)
    for ps in (0, -1, 64):
        pagedkv.paged_attention_decode(out, dq, dk, dv, torch.from_numpy(bt).cuda(),
                                       torch.from_numpy(lens).cuda(), 1 / np.sqrt(d),
                                       int(lens.max()), partition_size=ps)
        ref, _ = oracle.paged_attention(q, kc, vc, bt, lens, 1 / np.sqrt(d), bs, "bf16")
        G.assert_close(G.dev_to_f64(out), ref, "bf16", f"pool decode ps={ps}")
    pool.close()
