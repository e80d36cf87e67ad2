"""The usage example in README.md runs as written (on one GPU)."""
import os
import re

import pytest

pytestmark = pytest.mark.gpu


def test_readme_example_runs():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    text = open(os.path.join(root, "README.md")).read()
    code = re.search(r"```python\n(.*?)```", text, re.S).group(1)
    env = {}
    exec(compile(code, "README.md", "exec"), env)
    torch.cuda.synchronize()
    assert tuple(env["y"].shape) == (32768, 11008) and env["y"].dtype == torch.bfloat16
    assert tuple(env["dx"].shape) == (32768, 4096) and env["dx"].dtype == torch.float32
    assert tuple(env["y_mx"].shape) == (32768, 11008)
    assert torch.isfinite(env["y"].float()).all() and torch.isfinite(env["dx"]).all()
    # the forward product is close to the unquantized one (FP4: a few percent)
    x, w = env["x"].float(), env["w"].float()
    ref = x[:64] @ w.t()
    err = (env["y"][:64].float() - ref).norm() / ref.norm()
    assert err < 0.2, float(err)
