"""Helpers shared by the test modules (host side only)."""
import numpy as np

ULP1 = 2.0 ** -24   # unit roundoff of binary32


def f64(x):
    return np.asarray(x, dtype=np.float64)


def run_oracle(opt, fmt, n, steps, hp_kw, grad_fn=None, p=None, qs=None, qu=None,
               tensor_index=0, seed=0, decay_after=False, scale_fn=None):
    """Run the oracle for `steps` steps on one tensor of n elements from zero
    state.  grad_fn(t) -> gradient (float32 or BF16 words).  Returns (p, state)."""
    import oracle
    import synth
    if p is None:
        p = synth.params(n, tensor_index)
    st = oracle.state_zeros(fmt, n, opt, qs, qu)
    for t in range(1, steps + 1):
        g = grad_fn(t) if grad_fn is not None else synth.grads(n, t, tensor_index)
        hp = oracle.make_hp(step=t, seed=seed, tensor_index=tensor_index,
                            decay_after=decay_after, **hp_kw)
        scale = scale_fn(hp, p, g, st) if scale_fn is not None else 1.0
        oracle.step(opt, fmt, hp, p, g, qs=qs, qu=qu, scale=scale, **st)
    return p, st
