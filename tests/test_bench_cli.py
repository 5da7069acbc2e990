"""bench.py's command line on the CPU: refusals happen before any GPU work."""

import pytest

import bench


def test_more_than_one_gpu_is_refused(capsys, monkeypatch):
    monkeypatch.setenv("WORLD_SIZE", "1")
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_a_multi_rank_launch_is_refused(capsys, monkeypatch):
    monkeypatch.setenv("WORLD_SIZE", "8")
    assert bench.main([]) == 2
    assert "--gpus 1" in capsys.readouterr().err


@pytest.mark.parametrize("p", ["1.0", "-0.1", "1.5"])
def test_dropout_probability_out_of_range_is_an_error(p):
    with pytest.raises(SystemExit) as e:
        bench.main(["--dropout", p])
    assert e.value.code == 2


def test_unknown_workload_is_an_error():
    with pytest.raises(SystemExit) as e:
        bench.main(["--workload", "no_such_workload"])
    assert e.value.code == 2
