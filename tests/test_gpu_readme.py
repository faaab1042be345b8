"""The usage example in README.md runs as written.  Its gradients are zero, so
each of its ten steps is the decay alone (u = 0, clip coefficient 1):
p = p0 * (1 - lr*wd)^10 within the fp32 bar."""
import os
import re

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_example_runs():
    import torch
    text = open(os.path.join(ROOT, "README.md")).read()
    code = re.search(r"```python\n(.*?)```", text, re.S).group(1)
    torch.manual_seed(0)
    env = {}
    exec(compile(code, "README.md", "exec"), env)
    torch.cuda.synchronize()
    torch.manual_seed(0)
    p0 = [torch.randn(4096, 4096, device="cuda"), torch.randn(4096, device="cuda")]
    d = (1.0 - 3e-4 * 0.1) ** 10
    # ten fp32 products (half an ulp each) and the rounded decay factor taken to
    # the tenth power (ten times its half-ulp error): under 20 * 2^-24 relative
    bound = 24 * 2.0 ** -24
    for p, q in zip(env["params"], p0):
        want = q.double() * d
        assert float(((p.double() - want).abs() / want.abs().clamp_min(1e-30)).max()) <= bound
    assert float(env["coef"].cpu()[0]) == 1.0
