"""Layer-level GPU parity against the oracle (gfx950 only)."""

import numpy as np
import pytest

import synth
from oracle import moe, weights
from tests import parity
from tests.frag_layout import from_fragment_order
from tests.gpu_harness import gpu_layer, gpu_weights, run_traced, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check_weight_codes(cfg, gw, W, row_major=False):
    """The GPU-encoded MX weights equal the oracle's codes, in fragment order
    (read back through the layout's numpy statement) or row-major."""
    from oracle import mx
    if W.precision == "bf16":   # bfloat16 dense weights: the oracle's own rounding of the same fp32
        for name in ("w_down", "w_up", "w_gate_s", "w_up_s", "w_down_s"):
            ref = getattr(W, name)
            got = gw[name + "_bf16"].cpu().numpy().view(np.uint16)
            if isinstance(ref, list):
                for i, r in enumerate(ref):
                    assert np.array_equal(got[i], r.bits), (name, i)
            else:
                assert np.array_equal(got, ref.bits), name
    for name in ("w_down", "w_up"):
        if getattr(W, name) is None or W.precision == "bf16":   # no MX latent projections
            assert gw[name] is None, name
            continue
        c, s = gw[name]
        c, s = c.cpu().numpy(), s.cpu().numpy()
        if not row_major:
            c, s = from_fragment_order(c, s)
        ref = getattr(W, name)
        assert np.array_equal(s, ref.scales), name
        assert np.array_equal(c, mx.pack_e2m1(ref.codes)), name
    for name in ("w_gate_e", "w_up_e", "w_down_e", "w_gate_s", "w_up_s", "w_down_s"):
        lst = getattr(W, name)
        if not lst or not isinstance(lst[0], moe.MXTensor):
            continue
        c, s = gw[name]
        c, s = c.cpu().numpy(), s.cpu().numpy()
        if not row_major:
            c, s = from_fragment_order(c, s)
        for i, ref in enumerate(lst):
            assert np.array_equal(s[i], ref.scales), (name, i)
            assert np.array_equal(c[i], mx.pack_e2m1(ref.codes)), (name, i)


def _layer_case(cfg, x=None, selection_bias=None, check_codes=True):
    say(f"layer parity {cfg.name} T={cfg.T} d={cfg.d_model} L={cfg.d_latent} E={cfg.n_routed} k={cfg.top_k}")
    W = weights.layer(cfg, selection_bias=selection_bias)
    lay, gw = gpu_layer(cfg, selection_bias=selection_bias)
    if check_codes:
        _check_weight_codes(cfg, gw, W)
    if x is None:
        x = synth.gen_hidden(cfg)
    y, tr = run_traced(lay, x)
    o = moe.forward(x, W, cfg.top_k)
    rep = parity.check_layer(cfg, W, o, y, tr, x=x, say=say)
    lay.close()
    return rep, y, tr, o


def test_tiny_layer_parity():
    _layer_case(synth.config("tiny"))


def test_tiny_ragged_tokens():
    for T in (1, 5, 63, 65, 130):
        _layer_case(synth.config("tiny", T=T), check_codes=(T == 1))


def test_tiny_selection_bias_and_top1():
    cfg = synth.config("tiny", T=48)
    _layer_case(cfg, selection_bias=synth.gen_selection_bias(cfg, 0.05), check_codes=False)
    import dataclasses
    _layer_case(dataclasses.replace(cfg, top_k=1), check_codes=False)


def test_zero_input_gives_zero_output():
    cfg = synth.config("tiny", T=16)
    lay, _ = gpu_layer(cfg)
    y, tr = run_traced(lay, np.zeros((16, cfg.d_model), np.float32))
    assert np.all(y == 0)
    assert np.all(tr["ids"] == np.arange(cfg.top_k)[None, :])
    lay.close()


def test_determinism_two_forwards_bitwise_equal():
    cfg = synth.config("tiny")
    lay, _ = gpu_layer(cfg)
    x = synth.gen_hidden(cfg)
    y1, t1 = run_traced(lay, x)
    y2, t2 = run_traced(lay, x)
    assert np.array_equal(y1, y2)
    for k in ("ids", "pair_of_row", "zq_codes", "hq_codes", "yq_codes"):
        assert np.array_equal(t1[k], t2[k]), k
    lay.close()


def test_mid_layer_parity():
    _layer_case(synth.config("mid"))


def test_mid_concentrated_routing():
    """A selection bias of +10 on experts 0..k-2: every token picks those seven
    (2048 rows each: 16 full 128-row M-tiles per expert in the prefill GEMMs),
    and its last slot goes to one of the other 121 experts by score (about 17
    rows each, a single part-filled tile); the M-tile-to-expert table, the
    permutation and the ragged tails all against the oracle."""
    cfg = synth.config("mid", T=2048)
    b = np.zeros(cfg.n_routed, np.float32)
    b[: cfg.top_k - 1] = 10.0
    rep, y, tr, o = _layer_case(cfg, selection_bias=b, check_codes=False)
    ids = tr["ids"]
    assert np.all(np.sort(ids, axis=1)[:, : cfg.top_k - 1] == np.arange(cfg.top_k - 1)[None, :])


def test_tiny_many_experts_lds_topk():
    """More than 1024 routed experts: top-k keeps its keys in LDS instead of
    registers (the K3 router has 896)."""
    import dataclasses
    cfg = dataclasses.replace(synth.config("tiny", T=40), n_routed=1280, top_k=6)
    _layer_case(cfg, check_codes=False)


def test_tiny_many_tokens_split_bf16_router():
    """Enough (token, expert) tiles for the router to run as three-piece bf16
    products (2048 tokens x 1024 experts = 128 tiles of 128 x 128)."""
    import dataclasses
    cfg = dataclasses.replace(synth.config("tiny", T=2048), n_routed=1024, top_k=8)
    _layer_case(cfg, check_codes=False)


# --------------------------------------------------------------------------- no latent, softmax gates


def test_k2_tiny_layer_parity():
    """Non-latent layer: the router reads x, the experts read xq, the combined
    routed output is y's routed part; gates are the softmax of the winners'
    logits."""
    rep, y, tr, o = _layer_case(synth.config("k2_tiny"))
    assert "yq_codes" not in tr


def test_k2_tiny_ragged_tokens():
    for T in (1, 7, 130):
        _layer_case(synth.config("k2_tiny", T=T), check_codes=False)


def test_k2_tiny_selection_bias_and_top1():
    """The selection bias shifts the logit keys only; with top-1 every gate is
    exactly one."""
    import dataclasses
    cfg = synth.config("k2_tiny", T=48)
    _layer_case(cfg, selection_bias=synth.gen_selection_bias(cfg, 0.5), check_codes=False)
    _, _, tr, _ = _layer_case(dataclasses.replace(cfg, top_k=1), check_codes=False)
    assert np.all(tr["gates"] == 1.0)


def test_k2_tiny_no_shared_expert():
    """Without a shared expert and without a latent, y is the combine's output
    alone (no output GEMM runs)."""
    import dataclasses
    cfg = dataclasses.replace(synth.config("k2_tiny", T=40), n_shared=0)
    _, y, tr, _ = _layer_case(cfg, check_codes=False)
    assert np.array_equal(y, tr["y_lat"])


def test_k2_many_tokens_split_bf16_router():
    """The three-piece bf16 router on x itself (2048 tokens x 1024 experts)."""
    import dataclasses
    cfg = dataclasses.replace(synth.config("k2_tiny", T=2048), n_routed=1024, top_k=8)
    _layer_case(cfg, check_codes=False)


# --------------------------------------------------------------------------- higher-precision map


def test_bf16_map_tiny_layer_parity():
    """bfloat16 latent projections and shared experts (split-K weight
    streaming at 64 tokens), MXFP4 routed experts."""
    rep, y, tr, o = _layer_case(synth.config("tiny_bf16"))
    assert "xq_codes" not in tr and "yb" in tr


def test_bf16_map_ragged_tokens_both_kernels():
    """1 and 17 tokens (16- and 64-row split-K tiles), 256 (the last few-row
    size), 257 and 300 (the 512-thread LDS kernel, ragged M-tiles)."""
    for T in (1, 17, 256, 257, 300):
        _layer_case(synth.config("tiny_bf16", T=T), check_codes=(T == 257))


def test_bf16_map_mid_layer_two_shared_experts():
    """4096 tokens, 2 shared experts: the output GEMM runs three K segments
    [L | Fs | Fs] on the LDS kernel; the shared gate/up two dense groups."""
    import dataclasses
    cfg = dataclasses.replace(synth.config("mid"), name="mid_bf16", precision="bf16")
    _layer_case(cfg, check_codes=False)


def test_bf16_map_mid_decode_two_shared_experts():
    """The same layer at 48 tokens: every bf16 GEMM on the split-K path, the
    output one cutting its K slices across three segments."""
    import dataclasses
    cfg = dataclasses.replace(synth.config("mid", T=48), name="mid_bf16", precision="bf16")
    _layer_case(cfg, check_codes=False)


def test_repeated_decode_forwards_bitwise_equal():
    """Eight forwards of the same 48-token batch (bf16 map, two shared
    experts: the K-split path reuses one partial-sum buffer for several
    GEMMs) give bitwise equal outputs and latents."""
    import dataclasses
    cfg = dataclasses.replace(synth.config("mid", T=48), name="mid_bf16", precision="bf16")
    lay, _ = gpu_layer(cfg)
    x = synth.gen_hidden(cfg)
    y0, t0 = run_traced(lay, x)
    for _ in range(7):
        y, t = run_traced(lay, x)
        assert np.array_equal(y, y0)
        assert np.array_equal(t["z"], t0["z"])
    lay.close()


def test_no_shared_expert_latent_layers():
    """n_shared = 0 on the latent layer: the output GEMM is the up-projection
    alone (MX map and higher-precision map, few and many tokens)."""
    import dataclasses
    for name in ("tiny", "tiny_bf16"):
        for T in (40, 300):
            cfg = dataclasses.replace(synth.config(name, T=T), n_shared=0)
            _layer_case(cfg, check_codes=False)


# --------------------------------------------------------------------------- weight layouts


def _y(lay, x):
    xt = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    y = lay.forward(xt)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("name,T", [("tiny", 64), ("mid", 48), ("mid", 600), ("tiny_bf16", 300), ("k2_tiny", 64)])
def test_row_major_weights_give_the_fragment_order_result(name, T):
    """MX weights handed over row-major [out][in] (weight_layout = ROW_MAJOR,
    the codes as a checkpoint stores them) give bit for bit the forward on the
    same codes in fragment order: the kernels stage identical operands and
    only their global addresses differ.  48 tokens run the weight-streaming
    and K-split kernels, 600 the LDS-staged ones and the bf16 image of
    W_down."""
    from latent_routing_mxfp4_amd import _lib
    cfg = synth.config(name, T=T)
    say(f"row-major weights {name} T={T}")
    W = weights.layer(cfg)
    lay_f, _ = gpu_layer(cfg)
    lay_r, gw_r = gpu_layer(cfg, weight_layout=_lib.MOE_WEIGHTS_ROW_MAJOR)
    _check_weight_codes(cfg, gw_r, W, row_major=True)
    x = synth.gen_hidden(cfg)
    yf, yr = _y(lay_f, x), _y(lay_r, x)
    lay_f.close()
    lay_r.close()
    assert np.array_equal(yf.view(np.uint32), yr.view(np.uint32))


def test_checkpoint_row_major_weights_packed_to_fragment_order():
    """Row-major MXFP4 weights (as stored) converted by moe_mx_pack_weights and
    run in fragment order: the oracle's result, and bit for bit the row-major
    forward on the unpacked codes."""
    from latent_routing_mxfp4_amd import _lib
    from latent_routing_mxfp4_amd import layer as LY
    cfg = synth.config("tiny")
    say(f"packed checkpoint weights {cfg.name} T={cfg.T}")
    W = weights.layer(cfg)
    lay_r, gw_r = gpu_layer(cfg, weight_layout=_lib.MOE_WEIGHTS_ROW_MAJOR)
    packed = dict(gw_r)
    for name in LY.DENSE + LY.ROUTED + LY.SHARED:
        if gw_r.get(name) is not None:
            packed[name] = LY.mx_pack_weights(*gw_r[name])
    _check_weight_codes(cfg, packed, W)
    lay_p = LY.LatentMoE(LY.LayerShape.of(cfg), packed, cfg.T)
    x = synth.gen_hidden(cfg)
    y, tr = run_traced(lay_p, x)
    o = moe.forward(x, W, cfg.top_k)
    parity.check_layer(cfg, W, o, y, tr, x=x, say=say)
    assert np.array_equal(y.view(np.uint32), _y(lay_r, x).view(np.uint32))
    lay_p.close()
    lay_r.close()
