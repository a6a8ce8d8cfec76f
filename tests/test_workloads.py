"""Seeded generators and workload shapes (CPU only)."""
import json
import os

import numpy as np

import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_generators_are_deterministic_and_seed_separated():
    a = wl.activation_bf16(2, 8, 5120, outliers=True)
    b = wl.activation_bf16(2, 8, 5120, outliers=True)
    assert wl.sha256(a) == wl.sha256(b)
    assert wl.sha256(a) != wl.sha256(wl.activation_bf16(2, 4, 5120, outliers=True))
    w1 = wl.weight_f32(1, 384, 256)
    assert np.array_equal(w1, wl.weight_f32(1, 384, 256))
    assert not np.array_equal(w1, wl.weight_f32(1, 384, 256, tensor=wl.T_DOWN_W))


def test_outlier_count_and_distributions():
    M, K = 8, 5120
    plain = wl.activation_bf16(2, M, K, outliers=False)
    witho = wl.activation_bf16(2, M, K, outliers=True)
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    changed = np.flatnonzero(plain != witho)
    assert changed.size == round(0.01 * M * K)
    ratio = f(witho).reshape(-1)[changed] / f(plain).reshape(-1)[changed]
    assert np.all(np.abs(ratio - 20) < 0.2)
    w = wl.weight_f32(1, 384, 256)
    assert abs(w.std() - 0.02) < 0.001 and abs(w.mean()) < 0.001
    g = f(wl.gamma_bf16(3, 5120))
    assert abs(g.mean() - 1) < 0.01 and abs(g.std() - 0.1) < 0.01
    codes = wl.random_codes(1, 64, 256)
    assert not np.isin(codes, [0x7F, 0xFF]).any() and len(np.unique(codes)) == 254


def test_pages_tower_shapes_reproduce_printed_bytes():
    """The per-layer projection shapes reproduce the bytes/step the paired trace
    prints, and the printed per-shape rates follow from bytes / time."""
    g = json.load(open(os.path.join(GOLDEN, "tower_bytes.json")))
    gdn = [(10240, 5120), (6144, 5120), (5120, 6144)]            # in_proj_qkv, in_proj_z, out_proj
    attn = [(12288, 5120), (1024, 5120), (1024, 5120), (5120, 6144)]  # q, k, v, o
    total = 48 * sum(n * k for n, k in gdn) + 16 * sum(n * k for n, k in attn)
    assert total == g["bytes_per_step"]
    assert round(total / 2 ** 30, 4) == g["gib_per_step"]
    assert 48 + 48 + 48 + 16 + 16 + 32 == g["launches"]["total"]
    for r in g["rates"]:
        n = int(r["shape"].split("N=")[1].split()[0])
        k = int(r["shape"].split("K=")[1].split()[0])
        gib_s = r["launches"] * n * k / (r["ms_per_step"] * 1e-3) / 2 ** 30
        assert abs(gib_s - r["gib_per_s"]) < 0.05
    # merged qkvz = in_proj_qkv + in_proj_z
    assert 10240 + 6144 == 16384


def test_workload_table():
    assert wl.DECODE_MLP.projections[0].shards == (17408, 17408)
    assert sum(wl.PREFILL.projections[0].shards) == wl.PREFILL.projections[0].N
    layer_bytes = sum(p.N * p.K for p in wl.DECODE_STEP_LAYER)
    assert layer_bytes * wl.DECODE_STEP_LAYERS == 23_152_558_080
    # the pages' tower as merged launches: its projections read exactly the
    # printed bytes/step, plus the MLP pair's ~0.996 GiB; 136 launches
    g = json.load(open(os.path.join(GOLDEN, "tower_bytes.json")))
    tower = sum(n * sum(p.N * p.K for p in ps) for n, ps in wl.DECODE_STEP_4B)
    mlp = 4 * (34816 * 5120 + 5120 * 17408)
    assert tower - mlp == g["bytes_per_step"]
    assert round(mlp / 2 ** 30, 3) == 0.996
    assert tower == 8_283_750_400
    assert sum(n * len(ps) for n, ps in wl.DECODE_STEP_4B) == 136
    assert 48 * 2 + 16 * 2 == g["vllm_merged_launches"]["total"]
