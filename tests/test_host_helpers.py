"""Host-side helpers of the GPU tests, checked on the CPU."""
import numpy as np

from grouped_query_kv_amd.inputs import prefill_inputs
from gpu_util import f64, oracle_by_kv_head, scale_of
from oracle import cross_attention_ref, prefill_causal_ref, prefill_chunk_ref


def test_oracle_by_kv_head_equals_the_whole_batch_call():
    """The threaded per-(sequence, KV head) evaluation used for the full-size
    prefill checks returns exactly what one oracle call over the batch does."""
    inp = prefill_inputs(2, 12, 3, 37, 64, "bf16", seed=5)
    q, k, v = f64(inp["q"]), inp["k"].float().numpy(), inp["v"].float().numpy()
    s = scale_of(64)
    whole = prefill_causal_ref(q, k, v, s)
    assert np.array_equal(oracle_by_kv_head(lambda a, b, c: prefill_causal_ref(a, b, c, s), q, k, v, workers=3),
                          whole)
    lens = np.array([37, 30])
    qc = q[:, :, :9]
    whole = prefill_chunk_ref(qc, k, v, lens, s)
    got = oracle_by_kv_head(lambda a, b, c, l: prefill_chunk_ref(a, b, c, l, s), qc, k, v, lens, workers=2)
    assert np.array_equal(got, whole)
    whole = cross_attention_ref(qc, k, v, lens, s)
    got = oracle_by_kv_head(lambda a, b, c, l: cross_attention_ref(a, b, c, l, s), qc, k, v, lens)
    assert np.array_equal(got, whole)
