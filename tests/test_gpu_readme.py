"""The Python example in README.md runs as written (GPU)."""
import os
import re

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.gpu
def test_readme_python_example_runs():
    path = os.path.join(HERE, "..", "README.md")
    if not os.path.exists(path):
        pytest.skip("README.md is not in this copy of the tree")
    with open(path) as f:
        text = f.read()
    blocks = re.findall(r"```python\n(.*?)```", text, re.S)
    assert len(blocks) == 1, "README holds one Python example"
    print("[gpu] README example", flush=True)
    exec(compile(blocks[0], "README.md example", "exec"), {})
