"""Train/rollout mismatch of the forward, measured with the multiplicative
probability error of the nmedialink NeMo-RL FP8 page (section
"FP8面临的关键挑战：数值分歧"; oracle/mismatch.py).

A rollout scores its tokens with a small decode batch; the trainer re-scores
the same tokens inside a training batch.  Here the rollout batch is 64 rows
(M = 64, the weight-streaming forward) and the training batch the 8192 rows
that contain them (the tiled forward).  The layer is a Llama-3.1-8B linear
that writes the 4096-wide hidden state (O or down projection); its BF16
output is projected to synthetic logits by a fixed BF16 output projection
(vocabulary 32768, N(0, 0.02^2) weights) in float64 on the host -- the
output projection stays BF16 on the pages -- and each row's token is the
one the rollout samples from its own logits (seeded Gumbel-max).

The batch-invariant forward makes the rollout's Y the training Y bit for
bit, so the metric is exactly 1; the default split-K forward sums its K
ranges in another FP32 order and the metric shows how far that moves the
token probabilities (printed, and bounded well inside the page's accepted
1.03-1.05 band)."""
import numpy as np
import pytest
import torch

from oracle import mismatch as MM
from fp8_blockwise_quantized_amd import inputs
from tests.gpu_helpers import dev_bf16, host

pytestmark = pytest.mark.gpu

LAYERS = {"o": (4096, 4096), "down": (4096, 14336)}
VOCAB = 32768
M_TRAIN, M_ROLL = 8192, 64


def _logits(y_bf16_rows, head):
    return host(y_bf16_rows).astype(np.float64) @ head.T


def _sampled_ids(logits, seed):
    g = np.random.default_rng(seed).gumbel(size=logits.shape)
    return np.argmax(logits + g, axis=1)


@pytest.mark.parametrize("name", list(LAYERS))
def test_token_mult_prob_error_rollout_vs_training(gpu_lib, name):
    J = gpu_lib
    N, K = LAYERS[name]
    x = inputs.activations_with_outliers(M_TRAIN, K, seed=21)
    w = inputs.normal_bf16((N, K), 0.02, seed=21, tensor_id=inputs.ID_W)
    head = inputs.normal_bf16((VOCAB, N), 0.02, seed=22, tensor_id=inputs.ID_W).astype(np.float64)
    xq, xs = J.jet_quant_act_1x128(dev_bf16(x))
    wq, ws, _ = J.jet_quant_weight_128x128(dev_bf16(w), transposed=False)
    y_train = J.jet_fp8_linear_fwd(xq, xs, wq, ws)                              # tiled, M = 8192
    r0 = 1000
    rows = slice(r0, r0 + M_ROLL)
    xq_r, xs_r = xq[rows].contiguous(), xs[:, rows].contiguous()
    y_split = J.jet_fp8_linear_fwd(xq_r, xs_r, wq, ws)                          # split-K, M = 64
    y_inv = J.jet_fp8_linear_fwd_batch_invariant(xq_r, xs_r, wq, ws)           # one K range, M = 64
    torch.cuda.synchronize()
    lt = _logits(y_train[rows], head)
    out = {}
    for kind, y in (("batch_invariant", y_inv), ("split_k", y_split)):
        lr = _logits(y, head)
        ids = _sampled_ids(lr, 23)
        out[kind] = MM.token_mult_prob_error(MM.token_logprobs(lt, ids), MM.token_logprobs(lr, ids))
    print(f"token-mult-prob-error {name}: batch-invariant {out['batch_invariant']!r}, "
          f"split-K {out['split_k']!r}", flush=True)
    assert out["batch_invariant"] == 1.0
    assert 1.0 <= out["split_k"] < 1.01
