"""Pins of the shared seeded input generator (CPU)."""
import numpy as np
import pytest
from scipy import stats

from vcsynth import configs, rng, tensors
from vcsynth.normal_table import normal_table


def test_splitmix64_published_vectors():
    # SplitMix64 started from state 0 (Steele, Lea, Flood 2014; the reference seeding generator of
    # the xoshiro family) emits e220a8397b1dcdaf, 6e789e6aa1b965f4, 06c45d188009454f.
    with np.errstate(over="ignore"):
        got = [int(rng.mix64(np.uint64(k) * rng.GAMMA)) for k in (1, 2, 3)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_counter_form_equals_sequential_generator():
    seed, stream = 0x5EED0002, 3
    key = int(rng.stream_key(seed, stream))
    state = key
    seq = []
    for _ in range(50):
        state = (state + int(rng.GAMMA)) & 0xFFFFFFFFFFFFFFFF
        seq.append(int(rng.mix64(np.uint64(state))))
    assert [int(v) for v in rng.u64(seed, stream, np.arange(50))] == seq


def test_streams_and_seeds_differ():
    a = rng.u32(1, 2, np.arange(1000))
    b = rng.u32(1, 3, np.arange(1000))
    c = rng.u32(2, 2, np.arange(1000))
    assert (a != b).mean() > 0.99 and (a != c).mean() > 0.99


@pytest.mark.parametrize("sigma", [1.0, 1 / np.sqrt(512), 1 / 64.0])
def test_normal_table_is_rounded_inverse_cdf(sigma):
    t = normal_table(sigma)
    assert np.all(np.diff(t.thresholds.astype(np.int64)) > 0)
    vals = rng.bf16_bits_to_f64(t.values_bits)
    assert np.all(np.diff(vals) > 0)
    # spot-check buckets against the definition RNE_bf16(sigma * Phi^-1((u + .5) / 2^32))
    u = rng.u32(7, 1, np.arange(20000))
    x = sigma * stats.norm.ppf((u.astype(np.float64) + 0.5) / 2.0 ** 32)
    want = np.asarray(x, dtype=np.float32)
    want_bits = (want.view(np.uint32) + 0x7FFF + ((want.view(np.uint32) >> 16) & 1)) >> 16
    got = rng.normal_bf16_bits(7, 1, np.arange(20000), t)
    # x rounded twice (f64 -> f32 -> bf16) can differ from a single rounding only on exact
    # bf16 half-way points, which have probability 0 here
    assert np.array_equal(got.astype(np.uint32), want_bits.astype(np.uint32))


@pytest.mark.parametrize("sigma", [1.0, 1 / 64.0])
def test_bucketed_lookup_equals_the_threshold_search(sigma):
    """The per-bucket shortcut gives #{thresholds <= u} exactly: random u, every threshold and
    its neighbours, bucket edges, and the ends of the range."""
    t = normal_table(sigma)
    th = t.thresholds.astype(np.int64)
    edges = np.arange(0, 1 << 32, 1 << 12, dtype=np.int64)
    u = np.concatenate([rng.u32(3, 4, np.arange(200000)).astype(np.int64), th - 1, th, th + 1,
                        edges, edges - 1, [0, (1 << 32) - 1]])
    u = np.clip(u, 0, (1 << 32) - 1).astype(np.uint32)
    assert np.array_equal(rng.bucket_of(t, u), np.searchsorted(t.thresholds, u, side="right"))
    assert rng.normal_bf16_bits(3, 4, 5, t).shape == ()  # scalar index, scalar result


def test_normal_moments_and_ks():
    t = normal_table(1.0)
    x = rng.bf16_bits_to_f64(rng.normal_bf16_bits(11, 2, np.arange(400000), t))
    assert abs(x.mean()) < 5 / np.sqrt(400000)
    assert abs(x.var() - 1) < 0.01
    # bf16 rounding moves values by <= 2^-9 relative; KS distance stays tiny
    assert stats.kstest(x, "norm").statistic < 0.005


def test_ragged_batch_draws():
    c = configs.get("C5")
    assert c.B == 64 and c.L == 1
    kinds = [r.kind for r in c.reqs]
    assert kinds.count(configs.KIND_DRAFT) == 32
    for r in c.reqs:
        assert 4096 <= r.ctx_len <= 131072
        if r.kind == configs.KIND_VERIFY:
            assert 8 <= r.x <= 40 and r.comp == configs.COMP_DROP
        else:
            assert 0 <= r.step <= 39 and r.x == r.step + 1
            assert r.comp in (configs.COMP_DROP, configs.COMP_KIVI2)
    assert {r.comp for r in c.reqs if r.kind == configs.KIND_DRAFT} == {
        configs.COMP_DROP, configs.COMP_KIVI2}


def test_config_byte_sizes():
    # full bf16 KV per config: 2 * n * L * Hkv * d * 2 bytes per request
    assert configs.get("C2").full_kv_bytes() == 34359738368
    assert configs.get("C3").full_kv_bytes() == 52428800000
    assert configs.get("C4").full_kv_bytes() == 68719476736
    assert configs.get("C1").full_kv_bytes() == 524288


def test_tensor_slices_are_layout_independent():
    c = configs.get("C1")
    full = tensors.kctx_bits(c, 0, 0, 1, 64)
    part = tensors.kctx_bits(c, 0, 0, 1, 16, p0=32)
    assert np.array_equal(full[32:48], part)


def test_page_tables_are_permutations():
    tab, total = configs.page_tables(123, [100, 33, 16], salt=0)
    used = tab[tab >= 0]
    assert total == 7 + 3 + 1
    assert sorted(used.tolist()) == list(range(total))
    assert tab.shape == (3, 7) and tab[1, 3] == -1 and tab[2, 1] == -1
