"""cdb_init_static, the context whose workspace is the library's static
device scratch (for callers that cannot allocate device memory), against
cdb_init with a caller workspace (needs an MI355X).

Two contexts in a row on the static scratch, the second with a smaller
input (fewer slots and requests, so a smaller carved workspace over the
first one's leftovers): each decodes the same requests as a cdb_init
context and must give the same tokens, exit depths and exit states bit for
bit (the same kernels run on the same inputs).  (That maxima whose
workspace exceeds the static scratch are rejected is a host-side check,
tested on the CPU in test_abi.py.)
"""
import sys

import numpy as np
import pytest

import cdb_synth as S

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mods():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from continuous_depth_batching_amd import _lib, engine
    return engine, _lib


def _decode(engine, static, d, w, prompts, W, n_out):
    dm = engine.DeviceModel(d, w)
    max_len = max(len(p) for p in prompts) + n_out
    e = engine.Engine(dm, n_slots=W, max_rows=engine.pow2(W), num_blocks=len(prompts) * (max_len // 16 + 2),
                      max_seqs=len(prompts), max_blocks_per_seq=max_len // 16 + 2, max_out=n_out,
                      max_prefill_tokens=256, static_workspace=static)
    assert (e.workspace is None) == static
    sch = engine.Scheduler(e, prompts, n_out, mode="refill", W=W, K=1, M=256, capture_states=True).run()
    res = sch.results()
    states = {k: v.copy() for k, v in sch.exit_states.items()}
    e.close()
    return res, states


@pytest.mark.parametrize("W,lens,n_out", [(4, [16, 9, 23, 12, 30, 5, 16, 7], 10), (2, [11, 4, 19], 6)])
def test_static_scratch_matches_caller_workspace(mods, W, lens, n_out):
    engine, L = mods
    d = S.CONFIGS["c0"]
    _say(f"[case] cdb_init_static vs cdb_init: c0 fp32, W={W}, prompts {lens}, {n_out} outputs")
    w = S.make_weights(d, seed=0)
    prompts = S.make_prompts(d.vocab, lens, seed=1)
    ref, ref_states = _decode(engine, False, d, w, prompts, W, n_out)
    got, got_states = _decode(engine, True, d, w, prompts, W, n_out)
    assert got == ref
    assert sorted(got_states) == sorted(ref_states)
    for k in ref_states:
        assert np.array_equal(got_states[k], ref_states[k]), k
    _say(f"  identical tokens, exits and {len(ref_states)} exit states")
