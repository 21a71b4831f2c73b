"""GPU parity of the dense 1-bit key layout (the 1.5-bit point: half of the
pairs at one bit, none salient; PN-Mix abstract, down to 1.5 bits), through
the C ABI against the oracle: every byte of the 768-byte plane-order k_lo
records and of k_meta after prefill and after appends, and decode within
2e-3 at split counts 1 (the fp32 record too), 3 and 16, on both MFMA column
modes (G <= 8 and G = 16), both io dtypes and with two value precisions."""
import numpy as np
import pytest
import torch

import kvq_synth
import oracle
from decode_attention_select_amd import kvq
from tests._gpu_case import SM_SCALE, Case, check_output, check_single_split, compare_cache, dev

pytestmark = pytest.mark.gpu

ATOL = 2e-3

DENSE = [
    kvq_synth.Workload("dense-g1-fp16", 2, 2, 2, 32 * 9 + 32 + 11, n_qry=8, n_app=70,
                       io_dtype="fp16", outliers="pct2x10", n_pairs_hi=0, n_pairs_lo1=32,
                       residual=32, seed=71),
    kvq_synth.Workload("dense-g4", 1, 16, 4, 32 * 17 + 128 + 3, n_qry=8, n_app=70,
                       io_dtype="bf16", outliers="pairs4x8", n_pairs_hi=0, n_pairs_lo1=32,
                       residual=128, seed=72),
    kvq_synth.Workload("dense-g16", 1, 16, 1, 32 * 6 + 64 + 30, n_qry=4, n_app=70,
                       io_dtype="bf16", n_pairs_hi=0, n_pairs_lo1=32, residual=64, seed=73),
    kvq_synth.Workload("dense-vmix", 2, 8, 2, 32 * 8 + 64 + 1, n_qry=8, n_app=70,
                       io_dtype="bf16", outliers="pct2x10", n_pairs_hi=0, n_pairs_lo1=32,
                       residual=64, seed=74, n_vblk_hi=1, bits_vhi=3),
]


def _ids(w):
    return w.name


@pytest.mark.parametrize("w", DENSE, ids=_ids)
def test_dense1_prefill_decode_appends(w):
    print("case", w.name, flush=True)
    assert oracle.dense1(w.n_pairs_hi, w.n_pairs_lo1)
    case = Case(w, T=w.tokens, max_tokens=w.max_tokens)
    assert case.cache.sizes[0] == w.batch * w.n_kv_heads * case.NG * 768
    pairs = case.oracle_select()[1]
    q = case.d["q_dec"][:, :, 0]
    qz = case.oracle_quant(pairs=pairs)
    compare_cache(case, qz, qz.nq // 32)
    ref = oracle.attention(qz, q, SM_SCALE)
    _, part = case.decode(q, 1, partials=True)
    check_single_split(part, ref, ATOL)
    for S in (3, 16):
        check_output(case.decode(q, S), ref, w.io_dtype, ATOL)
    kn = dev(np.ascontiguousarray(case.d["k"][:, :, w.tokens:]))
    vn = dev(np.ascontiguousarray(case.d["v"][:, :, w.tokens:]))
    for i in range(w.n_app):
        kvq.kvq_append(case.layout, kn[:, :, i].contiguous(), vn[:, :, i].contiguous(),
                       case.cache.struct)
    torch.cuda.synchronize()
    assert kvq.kvq_check(case.cache.struct) == 0
    case.T = w.tokens + w.n_app
    qz = case.oracle_quant(pairs=pairs)
    compare_cache(case, qz, qz.nq // 32)
    got = case.decode(q, 5)
    check_output(got, oracle.attention(qz, q, SM_SCALE), w.io_dtype, ATOL)
    out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.int16, device="cuda")
    kvq.kvq_decode_attn_noalloc(case.layout, dev(q), case.cache.struct, SM_SCALE, 5, out)
    torch.cuda.synchronize()
    assert np.array_equal(kvq_synth.bits_to_f64(out.cpu().numpy().view(np.uint16), w.io_dtype),
                          got)
    assert case.pruned_unsupported()
