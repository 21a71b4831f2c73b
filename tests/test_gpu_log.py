"""KVQ_LOG: with the variable set, every launch prints its call, shape and
launch geometry on stderr (host side); unset, the library prints nothing."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = """
import numpy as np, torch, kvq_synth
from decode_attention_select_amd import kvq
from tests._gpu_case import Case, SM_SCALE, dev
w = kvq_synth.workload("tiny")
case = Case(w)
q = dev(case.d["q_dec"][:, :, 0])
ws = torch.zeros(kvq.kvq_workspace_bytes(case.layout, 3), dtype=torch.uint8, device="cuda")
out = torch.empty((1, 1, 128), dtype=torch.int16, device="cuda")
kvq.kvq_decode_attn(case.layout, q, case.cache.struct, SM_SCALE, 3, ws, out)
torch.cuda.synchronize()
print("done")
"""


@pytest.mark.timeout(300)
@pytest.mark.parametrize("value", ["1", None])
def test_launch_log(value):
    env = dict(os.environ)
    env.pop("KVQ_LOG", None)
    if value is not None:
        env["KVQ_LOG"] = value
    r = subprocess.run([sys.executable, "-c", SCRIPT], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=280)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip().endswith("done")
    lines = [l for l in r.stderr.splitlines() if l.startswith("kvq: ")]
    if value is None:
        assert lines == []
    else:
        calls = [l.split()[1] for l in lines]
        assert calls == ["kvq_select_pairs", "kvq_quant_keys", "kvq_quant_values",
                         "kvq_decode_attn"], lines
        assert "splits=3" in lines[-1] and "Hq=1 Hkv=1" in lines[-1]
