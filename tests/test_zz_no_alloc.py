"""simsd_accept_prefix_noalloc (no workspace argument: its scratch is the
library's fixed device array) against simsd_accept_prefix (the caller's
workspace), both through the C ABI, on the same inputs.

The outputs are integers (accepted prefix length, replacement token, status
flags) and must be equal bit for bit.  Calls run back to back on one stream,
larger first and then smaller, so the second finds the first one's contents
in the shared array; the draw and no-draw forms and faulted sequences are
covered.
"""
import pytest
import torch

import diffusion_lm_speculative_amd as sd
from diffusion_lm_speculative_amd import synth
from tests.gpu_helpers import dev

pytestmark = pytest.mark.gpu


def _both(inp, gamma, seed, offset, with_next=True):
    p, q, x, tau = (inp[k].to(dev()) for k in ("p", "q", "draft_tok", "tau"))
    NB, B, V = p.shape
    print(f"noalloc NB={NB} B={B} V={V} gamma={gamma} with_next={with_next}", flush=True)
    ref = sd.accept_prefix(p, q, x, tau, gamma, seed, offset, with_next=with_next)
    got = sd.accept_prefix_noalloc(p, q, x, tau, gamma, seed, offset, with_next=with_next)
    torch.cuda.synchronize()
    for a, b, name in zip(got, ref, ("n_accepted", "next_token", "status")):
        if b is None:
            assert a is None
            continue
        assert torch.equal(a, b), (name, a.cpu().tolist(), b.cpu().tolist())
    return got


def test_noalloc_matches_workspace_entry_point_on_two_calls_in_a_row():
    # batch 32, B = gamma = 8, V = 151936 (the headline step's acceptance), then a smaller call
    big = synth.make_accept_inputs(32, 8, 151936, seed=9001, device=dev())
    n1, nx1, _ = _both(big, 8, 1234, 0)
    small = synth.make_accept_inputs(7, 4, 5000, seed=9002, device=dev())
    n2, nx2, _ = _both(small, 4, 77, 3)
    assert (n1 < 8).any() and (nx1 >= 0).any()  # some sequences drew a replacement
    assert (nx2 >= -1).all()


def test_noalloc_other_forms():
    inp = synth.make_accept_inputs(64, 16, 151936, seed=9003, device=dev())
    _both(inp, 16, 5, 1)                   # batch 64, B = gamma = 16
    _both(inp, 5, 5, 2)                    # gamma < B
    _both(inp, 16, 5, 3, with_next=False)  # walk only: the array is not touched
    bad = synth.make_accept_inputs(4, 3, 20, seed=9)
    bad["tau"] = torch.tensor([[1, 2, 3], [-1, 2, 3], [1, 1, 3], [3, 2, 1]], dtype=torch.int32)
    bad["draft_tok"] = bad["draft_tok"].clone()
    bad["draft_tok"][3, 2] = 20
    n, _, st = _both(bad, 3, 1, 0)         # faulted sequences: n = next = -1 with their flags
    assert n.cpu().tolist()[1:] == [-1, -1, -1] and st.cpu().tolist()[1:] != [0, 0, 0]
    empty = synth.make_accept_inputs(3, 1, 100, seed=11)
    _both({k: (v[:, :0].contiguous() if v.dim() > 1 else v) for k, v in empty.items()}, 0, 1, 0)  # B == 0
