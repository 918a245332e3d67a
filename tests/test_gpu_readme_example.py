"""The Python example in README.md runs as written."""

import os
import re

import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_example_runs():
    if not torch.cuda.is_available():
        pytest.fail("the GPU tests need a visible MI355X")
    text = open(os.path.join(ROOT, "README.md")).read()
    code = re.search(r"```python\n(.*?)```", text, re.S).group(1)
    env = {}
    exec(compile(code, "README.md", "exec"), env)
    torch.cuda.synchronize()
    buf = env["buf"]
    assert buf.combined.shape == (buf.tokens, buf.hidden)
    assert int((buf.dst_row >= 0).sum()) == buf.tokens * buf.top_k
