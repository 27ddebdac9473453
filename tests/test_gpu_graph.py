"""The whole drafter forward captured into a HIP graph: every replay, with
eager work and synchronisation between replays, must equal the eager result
bit for bit (tokens, layer output, written KV rows)."""
import numpy as np
import pytest
import torch

from drafter_pe_build_amd.step import DraftStep, GraphStep
from helpers import bits, say
from synth import inputs as si

pytestmark = pytest.mark.gpu


def _case(name):
    if name == "tiny":
        return si.decode_config(0)
    dims = si.DrafterDims(hidden=128, n_q_heads=8, n_kv_heads=2, head_dim=64, ffn=256, vocab=1000, dtype="bf16")
    W = si.drafter_weights(dims, 31)
    c = si.decode_case(dims, 31, R=2, K=7, W=[3, 0], kv_len=[300, 1200], n_rej=[1, 0])
    return dims, W, c


@pytest.mark.parametrize("name", ["tiny", "small_bf16_split_kv"])
def test_graph_replay_equals_eager(name):
    say("graph %s" % name)
    dims, W, c = _case(name)
    st = DraftStep(dims, W, c)
    st.run()
    torch.cuda.synchronize()
    tok, xo, kc = st.tokens.clone(), st.x_out.clone(), st.k_cache.clone()
    gs = GraphStep(st)
    for i in range(3):
        st.x_out.zero_()
        st.tokens.fill_(-7)
        gs.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.tokens, tok), i
        assert np.array_equal(bits(st.x_out), bits(xo)), i
        assert np.array_equal(bits(st.k_cache), bits(kc)), i
        st.run()                       # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(st.tokens, tok)
