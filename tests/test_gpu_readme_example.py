"""The README's usage example, run as it stands: its code block is taken
from README.md and executed, and the decode output it leaves is checked
against the oracle on the same cache contents."""
import os
import re

import numpy as np
import pytest

from tests import gpu_util as G

pytestmark = pytest.mark.gpu

README = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "README.md")


def _example_code() -> str:
    text = open(README).read()
    section = text[text.index("## Using it"):]
    m = re.search(r"```python\n(.*?)```", section, re.S)
    assert m, "no python block under 'Using it'"
    return m.group(1)


def test_readme_example_runs_and_matches_oracle():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import oracle
    ns = {}
    exec(compile(_example_code(), "README.md", "exec"), ns)
    torch.cuda.synchronize()
    kc, vc = G.dev_to_bits(ns["k_cache"]), G.dev_to_bits(ns["v_cache"])
    bt = ns["block_tables"].cpu().numpy()
    lens = ns["seq_lens"].cpu().numpy()
    ref, _ = oracle.paged_attention(G.dev_to_bits(ns["q"]), kc, vc, bt, lens,
                                    1 / np.sqrt(ns["head_size"]), ns["block_size"], "bf16")
    G.assert_close(G.dev_to_f64(ns["out"]), ref, "bf16", "README example")
