"""Round dump and replay: one round's inputs and outputs written to an .npz,
then the same round run again from the file on fresh buffers.  Every output
must come back bit for bit (the kernels use no floating-point atomics, so a
round is deterministic); this is also the run-twice check of the round."""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("name,T,round_id", [("mid_bf16", 1.0, 3), ("mid_bf16", 0.0, 0), ("tiny", 1.0, 1)])
def test_round_dump_replay_bit_exact(tmp_path, name, T, round_id):
    import bench
    path = str(tmp_path / f"{name}.npz")
    meta = bench.dump_round(path, name, T, round_id=round_id)
    assert meta["status"] & ~0x8 == 0, hex(meta["status"])
    r = bench.replay_round(path)
    print(r)
    assert r["outputs"] >= 10
    assert r["match"], r["mismatched"]
