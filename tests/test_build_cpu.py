"""Host logic of the build: parallel jobs whose output outgrows a pipe buffer
finish, and a failing job is reported."""
import sys

import pytest

from exact_attention_backward_fa_amd import build


def test_jobs_with_large_output_finish(tmp_path, monkeypatch):
    monkeypatch.setattr(build, "BUILD_DIR", str(tmp_path))
    big = [sys.executable, "-c", "import sys; sys.stdout.write('x' * 300000)"]
    build._run_jobs([(f"job{i}", big) for i in range(3)], verbose=False)
    assert (tmp_path / "logs" / "job0.log").stat().st_size == 300000


def test_failing_job_raises(tmp_path, monkeypatch):
    monkeypatch.setattr(build, "BUILD_DIR", str(tmp_path))
    with pytest.raises(RuntimeError, match="bad"):
        build._run_jobs([("bad", [sys.executable, "-c", "raise SystemExit(3)"])], verbose=False)
