"""Out-of-range descriptor values written by a caller into device memory are
reported at the next cdb_sync as CDB_EINVAL (needs an MI355X).

The kernels clamp every index they read from device memory into its buffer,
so these cases make no access out of bounds and every kernel exits
normally; what is tested is that the clamp is reported rather than silent.
Each case then checks that the error word was cleared: the next sync after
valid work returns CDB_OK.
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


def _engine(engine, B=4, L=20):
    d = S.CONFIGS["c0"]
    w = S.make_weights(d, seed=0)
    dm = engine.DeviceModel(d, w)
    mbps = (L + 32) // 16 + 1
    e = engine.Engine(dm, n_slots=B, max_rows=B, num_blocks=B * mbps, max_seqs=B, max_blocks_per_seq=mbps,
                      max_out=4, max_prefill_tokens=16, kv_fill=0.0)
    e.btab.copy_(torch.arange(B * mbps, dtype=torch.int32, device="cuda"))
    e.emap.fill_(d.r_max)
    e.state.copy_(torch.randn((B, d.hidden), device="cuda"))
    return d, e


def _desc(e, d, B, L, **over):
    cap = e.max_rows
    cols = dict(slot=np.arange(B), seq=np.arange(B), pos=np.full(B, L), depth=np.ones(B), exit_at=np.full(B, d.r_max))
    for k, (row, v) in over.items():
        cols[k] = cols[k].copy()
        cols[k][row] = v
    desc = np.zeros(5 * cap + 1, dtype=np.int32)
    desc[0] = B
    for i, k in enumerate(("slot", "seq", "pos", "depth", "exit_at")):
        desc[1 + i * cap:1 + i * cap + B] = cols[k]
    e.desc_t.copy_(torch.from_numpy(desc))


@pytest.mark.parametrize("field,value,word", [("depth", 9, "depth"), ("depth", 0, "depth"), ("slot", 7, "slot"),
                                              ("seq", -3, "sequence"), ("pos", 10 ** 6, "position")])
def test_core_step_reports_clamped_descriptor(mods, field, value, word):
    engine, L = mods
    d, e = _engine(engine)
    _say(f"[case] core step with {field} = {value} in row 2 (r_max {d.r_max}, 4 rows)")
    _desc(e, d, 4, 20, **{field: (2, value)})
    e.core_step(4)
    with pytest.raises(L.CDBError) as ei:
        e.sync()
    assert ei.value.code == L.CDB_EINVAL and word in str(ei.value), str(ei.value)
    _desc(e, d, 4, 20)
    e.core_step(4)
    e.sync()                                     # cleared, and valid work reports nothing
    e.close()


def test_gate_reports_row_count_above_launch_rows(mods):
    engine, L = mods
    d, e = _engine(engine)
    _say("[case] gate/compaction with n_valid 6 > rows_pad 4")
    _desc(e, d, 4, 20)
    e.desc_t[0] = 6
    e.q_t.zero_()
    e.gate_compact(4, True)
    with pytest.raises(L.CDBError) as ei:
        e.sync()
    assert ei.value.code == L.CDB_EINVAL and "row count" in str(ei.value)
    assert int(e.desc_t[0].item()) <= 4         # the rows past the launch were dropped, not read
    e.close()


def test_boundary_reports_exit_queue_beyond_rows_pad(mods):
    engine, L = mods
    d, e = _engine(engine)
    _say("[case] boundary with 4 queued exits and rows_pad 2")
    _desc(e, d, 4, 20, depth=(0, d.r_max))
    e.desc_t[0] = 0
    cap = e.max_rows
    q = np.zeros(4 * cap + 1, dtype=np.int32)
    q[0] = 4
    q[1:1 + 4] = np.arange(4)
    q[1 + cap:1 + cap + 4] = np.arange(4)
    q[1 + 2 * cap:1 + 2 * cap + 4] = 20
    q[1 + 3 * cap:1 + 3 * cap + 4] = 3
    e.q_t.copy_(torch.from_numpy(q))
    e.n_gen.fill_(1)
    e.n_out.fill_(4)
    e.boundary(2)
    with pytest.raises(L.CDBError) as ei:
        e.sync()
    assert ei.value.code == L.CDB_EINVAL and "row count" in str(ei.value)
    e.close()
