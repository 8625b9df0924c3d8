"""The rocprofv3 summaries under profiles/ each state the command that made them, and that
command runs committed files only (nothing under the working folder _work/)."""
import glob
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_every_profile_names_its_command_and_runs_committed_files():
    files = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md")))
    assert files, "no profile summaries"
    for f in files:
        text = open(f).read()
        assert "rocprofv3" in text and "Command" in text, f"{f}: no command"
        assert "_work" not in text, f"{f}: refers to the working folder"
        assert os.path.getsize(f) < 16 * 1024, f"{f}: a summary should stay short"
