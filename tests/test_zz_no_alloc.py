"""mlp_forward_noalloc (the library's own per-GPU scratch as workspace)
against mlp_forward with a caller workspace: the same kernels run, so the
outputs must be bit-identical. Each case makes two calls in a row, the
second with a smaller input, so the second runs on the scratch as the first
left it."""
import numpy as np
import pytest
import torch

import nvfp4_synth as synth
import oracle
from gpu_helpers import calibrate_activation_scales, dev, gemm_close, mlp_weights, packed_weights, scalar, to_dev, \
    to_host

pytestmark = pytest.mark.gpu

nv = None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global nv
    import nvfp4_quantized_dense_amd as _nv
    nv = _nv
    nv.lib()
    assert torch.cuda.is_available()
    nv.set_path(nv.PATH_AUTO)
    yield


def _calls(mode, x, w, sc, p_gu, p_d, I):
    """(with a fresh caller workspace, on the scratch) for one input."""
    if mode == 0:
        args = (0, to_dev(x), p_gu, scalar(sc["a_gu"]), p_d, scalar(sc["a_d"]), I)
        kw = dict(g1_inv=scalar(sc["g1_inv"]), g2_inv=scalar(sc["g2_inv"]))
    else:
        args = (1, to_dev(x), p_gu, scalar(w["g_gu"]), p_d, scalar(w["g_d"]), I)
        kw = {}
    ref = nv.mlp_forward(*args, **kw)
    out = torch.full_like(ref, float("nan"))
    nv.mlp_forward_noalloc(*args, out=out, **kw)
    torch.cuda.synchronize()
    return to_host(ref), to_host(out)


# (mode, H, I, first M, second M): decode-size shapes on the single-launch
# decode and the streaming kernels; 64, 256 and 300 tokens with the down
# projection K-split on the mid-size kernels (8, 2 and 3 ways; 128-token
# tiles at 300), its partial tiles in the scratch.
CASES = [
    (0, 5120, 17408, 16, 1),
    (0, 7168, 18432, 64, 1),
    (0, 7168, 18432, 256, 3),
    (0, 7168, 18432, 300, 17),
    (1, 5120, 17408, 768, 48),
    (1, 5120, 17408, 64, 16),
    (1, 5120, 17408, 16, 1),
    (0, 512, 4352, 200, 1),
]


@pytest.mark.parametrize("mode,H,I,m1,m2", CASES)
def test_noalloc_matches_mlp_forward(mode, H, I, m1, m2):
    print(f"noalloc case mode={mode} H={H} I={I} M={m1} then {m2}", flush=True)
    w = mlp_weights(H, I, 0)
    p_gu, p_d = packed_weights(H, I, 0)
    x1 = synth.activations(31 + m1, m1, H)
    x2 = synth.activations(37 + m2, m2, H)
    sc = calibrate_activation_scales(x1[:64], w) if mode == 0 else None
    for x in (x1, x2):
        ref, out = _calls(mode, x, w, sc, p_gu, p_d, I)
        assert np.array_equal(ref, out), f"noalloc differs from mlp_forward at M={x.shape[0]}"
    # the smaller call also against the oracle
    if mode == 0:
        r = oracle.mlp_w4a4(x2, w["c_gu"], w["s_gu"], sc["a_gu"], w["c_d"], w["s_d"], sc["a_d"], sc["g1_inv"],
                            sc["g2_inv"])
    else:
        r = oracle.mlp_w4a16(x2, w["c_gu"], w["s_gu"], w["g_gu"], w["c_d"], w["s_d"], w["g_d"])
    gemm_close(out, r["out"], f"noalloc mode={mode} M={m2}")


def test_noalloc_bf16_out_and_limit():
    H, I = 7168, 18432
    w = mlp_weights(H, I, 0)
    p_gu, p_d = packed_weights(H, I, 0)
    x = synth.activations(5, 1, H)
    sc = calibrate_activation_scales(x, w)
    args = (0, to_dev(x), p_gu, scalar(sc["a_gu"]), p_d, scalar(sc["a_d"]), I)
    kw = dict(g1_inv=scalar(sc["g1_inv"]), g2_inv=scalar(sc["g2_inv"]), out_dtype=torch.bfloat16)
    ref = to_host(nv.mlp_forward(*args, **kw))
    out = to_host(nv.mlp_forward_noalloc(*args, **kw))
    assert np.array_equal(ref, out)
    # past the scratch: rejected on the host, nothing launched
    xb = torch.zeros((8192, H), dtype=torch.bfloat16, device=dev())
    with pytest.raises(nv.Nvfp4Error, match="scratch"):
        nv.mlp_forward_noalloc(0, xb, *args[2:], **kw)
