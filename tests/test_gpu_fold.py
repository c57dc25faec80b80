"""A convolution followed by batch normalisation, run as one libconv call with
the normalisation folded into the weights and bias on the host (the detector
of "PP-OCR on Vulkan compute shaders" folds its BN layers this way), against
the fp64 oracle's convolution followed by the normalisation."""
import numpy as np
import pytest

import oracle
import workloads as W
from convcheck import assert_gates, metrics, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_conv_bn_folded(dtype):
    import direct_implicit_gemm_amd as L
    r = np.random.default_rng(93)
    layer = W.Layer("bn", dtype, 2, 16, 1, 20, 72, 40, 1, 3, 3, (0, 1, 1), (1, 1, 1), "relu",
                    2, "N01", "N01", "U0.05")
    x, w, b = W.make_inputs(layer, 94)
    gamma, beta = r.uniform(0.5, 1.5, 40), r.uniform(-0.2, 0.2, 40)
    mean, var, eps = r.uniform(-0.3, 0.3, 40), r.uniform(0.5, 2.0, 40), 1e-5
    wf, bf = L.fold_batchnorm(w.f64(), b.f64(), gamma, beta, mean, var, eps)
    wq, bq = W.Tensor.quantise(wf.astype(np.float64), dtype), W.Tensor.quantise(
        bf.astype(np.float64), dtype)
    print(f"[gpu] conv+BN folded {dtype} x={layer.x_shape}", flush=True)
    y = to_f64(L.conv_nd(x.torch("cuda"), wq.torch("cuda"), bq.torch("cuda"), 1, 1, "relu"))
    # reference: the unfolded convolution, then the normalisation, then ReLU, in fp64
    conv, s = oracle.conv(x.f64(), w.f64(), b.f64(), 1, 1)
    scale = gamma / np.sqrt(var + eps)
    ref = np.maximum((conv - mean[:, None, None]) * scale[:, None, None] + beta[:, None, None],
                     0.0)
    # error scale: the folded products |x * w_f| and |b_f|, i.e. S scaled per channel
    s_f = s * scale[:, None, None] + np.abs(bf)[:, None, None]
    m = metrics(y, ref, s_f, dtype)
    print(f"[gpu]   {m}", flush=True)
    if dtype == "f32":
        assert_gates(m, dtype, "conv+bn")
    else:
        # the folded weights are rounded to the storage dtype once more than
        # the reference's: allow that rounding in the relative bound
        assert m["g1_raw"] <= 2 ** -7, m
        assert m["nrmse_unrounded"] <= 1e-2, m
