"""The allocation-free decode step (specdec_decode_step_noalloc, for callers that cannot
allocate) against the workspace entry point (specdec_decode_step), through the C ABI:
two calls in a row, the second with fewer rows, on the tiny decoder and on the
1.5B shape at a 2048-token cache.  Both run the same kernels, so logits, argmax,
log-sum-exp and the appended K/V are compared bit for bit."""
import numpy as np
import pytest
import torch

from gpu_helpers import say, to_np

pytestmark = pytest.mark.gpu


def _pair(b, shape, model, prompt, max_len):
    out = []
    for _ in range(2):
        cache, ws = b.Cache(shape, max_len), b.Workspace(shape, max_len)
        b.prefill(model, cache, torch.from_numpy(prompt).cuda(), ws)
        out.append((cache, ws))
    return out


def _run_both(b, shape, model, caches, toks, err):
    (ca, wa), (cb, _) = caches
    V, M = shape.vocab, len(toks)
    t = torch.from_numpy(np.asarray(toks, np.int32)).cuda()
    la, lb = (torch.empty((M, V), dtype=torch.float32, device="cuda") for _ in range(2))
    aa, ab = (torch.empty(M, dtype=torch.int32, device="cuda") for _ in range(2))
    sa, sb = (torch.empty(M, dtype=torch.float32, device="cuda") for _ in range(2))
    b.decode_step(model, ca, t, wa, logits=la, argmax=aa, lse=sa)
    b.decode_step_noalloc(model, cb, t, err, logits=lb, argmax=ab, lse=sb)
    torch.cuda.synchronize()
    assert torch.equal(la.view(torch.int32), lb.view(torch.int32))
    assert torch.equal(aa, ab) and torch.equal(sa.view(torch.int32), sb.view(torch.int32))
    assert ca.length() == cb.length()
    n = ca.length()
    ka, va = ca.kv()
    kb, vb = cb.kv()
    assert torch.equal(ka[:, :, :n], kb[:, :, :n]) and torch.equal(va[:, :, :n], vb[:, :, :n])
    assert int(err.item()) == 0 and wa.error_bits() == 0


@pytest.mark.parametrize("which", ["tiny", "1.5b"])
def test_no_alloc_step_equals_workspace_step(which):
    from block_verify_amd import lib as b
    from block_verify_amd.shapes import QWEN_1_5B, SEED_TARGET, TINY
    from block_verify_amd.synth import make_prompt, make_weights
    shape, P = (TINY, 128) if which == "tiny" else (QWEN_1_5B, 2048)
    say(f"no-alloc step: {which}, {P}-token cache")
    model = b.Model(shape, make_weights(shape, SEED_TARGET))
    prompt = make_prompt(shape.vocab, P)
    b.static_init()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    caches = _pair(b, shape, model, prompt, P + 64)
    rng = np.random.default_rng(7)
    for rows in (5, 1):          # two calls in a row, the second smaller
        _run_both(b, shape, model, caches, rng.integers(0, shape.vocab, rows), err)
    say(f"no-alloc step: {which} equal bit for bit for 5 then 1 rows")


def test_no_alloc_step_refuses_oversized_plans_and_a_missing_error_word():
    from block_verify_amd import lib as b
    from block_verify_amd.shapes import TINY, SEED_TARGET
    from block_verify_amd.synth import make_weights
    model = b.Model(TINY, make_weights(TINY, SEED_TARGET))
    b.static_init()
    big = b.Cache(TINY, 65536)      # its workspace plan passes the 128 MiB scratch
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    t = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(b.SpecdecError, match=r"\[-2\]"):
        b.decode_step_noalloc(model, big, t, err)
    small = b.Cache(TINY, 256)
    rc = b.lib().specdec_decode_step_noalloc(model.handle, small.handle, t.data_ptr(), 1, None, None, None, None,
                                             torch.cuda.current_stream().cuda_stream)
    assert rc == b.EINVAL
    assert small.length() == 0 and int(err.item()) == 0
