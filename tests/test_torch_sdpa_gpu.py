"""Cross-check against a third-party implementation: torch's
scaled_dot_product_attention, evaluated on the CPU in float64 on the same
bf16 inputs.  Informative only (the oracle is the reference); torch's causal
mask is aligned top-left, so causal cases use T_q = T_kv, where both
alignments agree.  GQA is given to torch as MHA with each kv head repeated
for its group of consecutive q heads."""
import math

import numpy as np
import pytest

import gpu_util as G
from transformer_scaled_dot_flash_amd import attn as abi
from transformer_scaled_dot_flash_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    abi.load_library()


@pytest.mark.parametrize("B,H_q,H_kv,T_q,T_kv,D,causal", [
    (1, 4, 4, 128, 128, 64, True),
    (2, 8, 2, 300, 300, 128, True),
    (1, 6, 3, 77, 200, 64, False),
    (1, 8, 1, 513, 513, 128, False),
])
def test_matches_torch_sdpa(B, H_q, H_kv, T_q, T_kv, D, causal):
    torch = G.torch_mod()
    seed = 950 + T_q + D
    q = inputs.normal(seed, (B, H_q, T_q, D), "bf16")
    k = inputs.normal(seed + 1, (B, H_kv, T_kv, D), "bf16")
    v = inputs.normal(seed + 2, (B, H_kv, T_kv, D), "bf16")
    scale = float(np.float32(1.0 / math.sqrt(D)))
    got = G.prefill(q, k, v, causal, scale, "bf16")
    G_ = H_q // H_kv
    Q = torch.from_numpy(inputs.as_f64(q, "bf16"))
    K = torch.from_numpy(inputs.as_f64(k, "bf16")).repeat_interleave(G_, dim=1)
    V = torch.from_numpy(inputs.as_f64(v, "bf16")).repeat_interleave(G_, dim=1)
    want = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=causal, scale=scale).numpy()
    assert G.max_err(got, want) <= G.TOL["bf16"]
