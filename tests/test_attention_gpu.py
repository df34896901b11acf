"""Parity of the attention consumer (through the C ABI) with the CPU oracle (GPU).

O = softmax(scale Q K^T) V per (batch, head) slice.  Every producer variant
and stage count runs the same arithmetic in the same order (only the way key
and value blocks reach LDS differs), so their outputs must be bit-identical;
each must match the oracle within the normalised tolerance of tests/parity.py
(the probabilities are rounded to the input type before the second product).
Shapes span several query and key blocks with ragged tails; closed forms
check the mask of keys past Sk, one-key rows and a selection by huge logits.
"""
from __future__ import annotations

import numpy as np
import pytest

import software_pipelined_tiling_amd as spt
from software_pipelined_tiling_amd import inputs as I
from tests import parity

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

VARIANTS = [("sync", 1), ("reg", 1), ("reg", 2), ("direct", 2), ("direct", 3), ("auto", 0)]


@pytest.fixture(scope="module", autouse=True)
def gpu(built_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    spt.lib()


def dev(x: np.ndarray, dtype: str):
    t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16).copy())
    return t.view(torch.float16 if dtype == "f16" else torch.bfloat16).cuda()


def run(Q, K, V, dtype, scale, variant="auto", stages=0):
    BH, Sq, D = Q.shape
    Sk = K.shape[1]
    print(f"[gpu] attention {dtype} BH={BH} Sq={Sq} Sk={Sk} D={D} {variant}/{stages}", flush=True)
    dQ, dK, dV = dev(Q, dtype), dev(K, dtype), dev(V, dtype)
    O = torch.full((BH, Sq, D), float("nan"), dtype=torch.float32, device="cuda")
    rc = spt.spt_attention(BH, Sq, Sk, D, dQ.data_ptr(), dK.data_ptr(), dV.data_ptr(), O.data_ptr(), scale,
                           spt.DTYPE_CODES[dtype], torch.cuda.current_stream().cuda_stream,
                           spt.VARIANT_CODES[variant], stages)
    assert rc == 0, f"{spt.spt_status_string(rc)}: {spt.spt_last_error()}"
    torch.cuda.synchronize()
    return O.cpu().numpy()


def qkv(dtype, BH, Sq, Sk, D, seed, dist="normal"):
    w = I.AttentionWorkload("t", seed, BH, Sq, Sk, D, dtype, dist)
    return I.make_qkv(w)


SHAPES = [(1, 1, 1, 64), (2, 100, 33, 64), (1, 256, 64, 128), (3, 300, 200, 128), (2, 513, 65, 64),
          (1, 70, 1000, 128), (2, 257, 129, 128)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("BH,Sq,Sk,D", SHAPES)
def test_every_variant_matches_oracle_and_each_other(oracle_mod, dtype, BH, Sq, Sk, D):
    Q, K, V = qkv(dtype, BH, Sq, Sk, D, 60 + D)
    scale = 1.0 / np.sqrt(D)
    ref = oracle_mod.attention(Q, K, V, dtype, scale)
    outs = []
    for v, s in VARIANTS:
        O = run(Q, K, V, dtype, scale, v, s)
        parity.check_attention(O, ref, V, dtype)
        outs.append(O)
    for O in outs[1:]:
        assert np.array_equal(O.view(np.uint32), outs[0].view(np.uint32)), "variants differ"


@pytest.mark.parametrize("D", [64, 128])
def test_scales_and_distributions(oracle_mod, D):
    """Scale 0 (equal weights), a large scale (peaked rows), uniform inputs."""
    for scale, dist in [(0.0, "normal"), (2.0, "normal"), (0.3, "uniform")]:
        Q, K, V = qkv("f16", 2, 130, 150, D, 70, dist)
        O = run(Q, K, V, "f16", scale)
        parity.check_attention(O, oracle_mod.attention(Q, K, V, "f16", scale), V, "f16")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("variant,stages", [("direct", 2), ("reg", 2), ("sync", 1)])
def test_one_key_gives_its_value_row(D, variant, stages):
    """Sk = 1: every weight is exactly 1, so O is V's only row, exactly."""
    Q, K, V = qkv("f16", 3, 40, 1, D, 71)
    O = run(Q, K, V, "f16", 0.125, variant, stages)
    want = parity.values(V, "f16")  # (3, 1, D)
    assert np.array_equal(O, np.broadcast_to(want, O.shape).astype(np.float32))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
def test_equal_value_rows_give_that_value_exactly(dtype, D):
    """Every value row 0.5: the row sums come from the same rounded probabilities as
    O += P V (an MFMA against ones), each product with 0.5 is exact and so is every
    partial sum's halving, so O = l / 2 / l = 0.5 exactly, for every producer, a ragged
    last block and any logits."""
    Q, K, V = qkv(dtype, 2, 70, 333, D, 74)
    half = I.f64_to_f16_bits(np.full((1,), 0.5))[0] if dtype == "f16" else I.f32_to_bf16_bits(np.full((1,), 0.5, np.float32))[0]
    V = np.full_like(V, half)
    for variant, stages in VARIANTS:
        O = run(Q, K, V, dtype, 0.3, variant, stages)
        assert np.array_equal(O, np.full(O.shape, 0.5, np.float32)), (variant, stages)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Sk", [64, 100, 1000])
def test_selection_by_huge_logits(D, Sk):
    """Query i one-hot at column i mod D times 8, key j one-hot at column pi(j) mod D
    times 8, scale 64: row i scores 4096 on its selected keys and 0 elsewhere, so O
    averages exactly the selected value rows (whatever block they fall in)."""
    Sq = 50
    rng = np.random.default_rng(72)
    q = np.zeros((1, Sq, D))
    q[0, np.arange(Sq), np.arange(Sq) % D] = 8.0
    perm = rng.permutation(Sk)
    k = np.zeros((1, Sk, D))
    k[0, np.arange(Sk), perm % D] = 8.0
    V = I.draw("intgrid", -4, 4, (1, Sk, D), rng, "f16")
    Q, K = I.f64_to_f16_bits(q), I.f64_to_f16_bits(k)
    O = run(Q, K, V, "f16", 64.0)
    v = parity.values(V, "f16")[0]
    for i in range(Sq):
        sel = np.flatnonzero(perm % D == i % D)
        want = v[sel].mean(axis=0) if sel.size else v.mean(axis=0)
        assert np.allclose(O[0, i], want, rtol=0, atol=2e-3 * max(1.0, np.abs(v).max())), i


def test_keys_past_sk_are_masked(oracle_mod):
    """A ragged last block whose missing keys would dominate if they were read as
    zeros: every real logit is very negative, so a zero logit would take all the
    weight."""
    D, Sq, Sk = 64, 20, 70
    q = -np.ones((1, Sq, D))
    k = np.ones((1, Sk, D))
    Q, K = I.f64_to_f16_bits(q), I.f64_to_f16_bits(k)
    V = I.draw("uniform", -1, 1, (1, Sk, D), np.random.default_rng(73), "f16")
    for variant, stages in VARIANTS:
        O = run(Q, K, V, "f16", 1.0, variant, stages)
        parity.check_attention(O, oracle_mod.attention(Q, K, V, "f16", 1.0), V, "f16")


def test_empty_and_invalid():
    z = torch.zeros(1024, dtype=torch.float16, device="cuda")
    o = torch.zeros(1024, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    p = z.data_ptr()
    assert spt.spt_attention(0, 5, 5, 64, p, p, p, o.data_ptr(), 1.0, spt.F16, s, 0, 0) == 0
    assert spt.spt_attention(1, 0, 5, 64, p, p, p, o.data_ptr(), 1.0, spt.F16, s, 0, 0) == 0
    assert spt.spt_attention(1, 2, 0, 64, p, p, p, o.data_ptr(), 1.0, spt.F16, s, 0, 0) == spt.SPT_ERR_INVALID
    assert spt.spt_attention(1, 2, 2, 96, p, p, p, o.data_ptr(), 1.0, spt.F16, s, 0, 0) == spt.SPT_ERR_UNSUPPORTED
    assert spt.spt_attention(1, 2, 2, 64, p, p, p, p, 1.0, spt.F16, s, 0, 0) == spt.SPT_ERR_INVALID  # O overlaps


def test_torch_wrapper(oracle_mod):
    Q, K, V = qkv("bf16", 2, 77, 90, 128, 74)
    O = spt.attention(dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16"))
    torch.cuda.synchronize()
    parity.check_attention(O.cpu().numpy(), oracle_mod.attention(Q, K, V, "bf16", 1 / np.sqrt(128)), V, "bf16")


@pytest.mark.parametrize("variant,stages", [("auto", 0), ("direct", 2), ("direct", 3), ("reg", 1), ("reg", 2),
                                            ("sync", 1)])
def test_full_size_workload(oracle_mod, variant, stages):
    """The benchmark's workload (32 slices x 4096 x 4096 x 128, fp16) in every
    configuration bench.py times, against the oracle over all of O."""
    w = I.W_ATTN_4096
    if not hasattr(test_full_size_workload, "ref"):
        Q, K, V = I.make_qkv(w)
        print("[gpu] oracle attention full size", flush=True)
        test_full_size_workload.ref = (Q, K, V, oracle_mod.attention(Q, K, V, "f16", 1 / np.sqrt(w.D)))
    Q, K, V, ref = test_full_size_workload.ref
    O = run(Q, K, V, "f16", 1 / np.sqrt(w.D), variant, stages)
    parity.check_attention(O, ref, V, "f16")


def test_full_size_bf16_d64_sampled_rows(oracle_mod):
    """bf16 at head dimension 64: 64 slices x 4096 queries x 4096 keys (the benchmark
    workload's FLOP, 64 key blocks per slice) under every producer, bit-identical to each
    other over all of O, and against the oracle on 48 query rows of every slice spread
    over all 16 query blocks (attention is row-wise: those rows of O are the attention
    of those rows of Q alone)."""
    w = I.AttentionWorkload("bf16 attention 64 x 4096 x 4096 x 64", 75, 64, 4096, 4096, 64, "bf16")
    Q, K, V = I.make_qkv(w)
    scale = 1 / np.sqrt(w.D)
    rows = np.unique(np.concatenate([np.arange(0, w.Sq, 256) + o for o in (0, 127, 255)]))
    print("[gpu] oracle attention bf16 d64, sampled rows", flush=True)
    ref = oracle_mod.attention(np.ascontiguousarray(Q[:, rows]), K, V, "bf16", scale)
    first = None
    for variant, stages in VARIANTS:
        O = run(Q, K, V, "bf16", scale, variant, stages)
        parity.check_attention(np.ascontiguousarray(O[:, rows]), ref, V, "bf16")
        if first is None:
            first = O
        else:
            assert np.array_equal(O.view(np.uint32), first.view(np.uint32)), (variant, stages)

