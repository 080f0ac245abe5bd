"""The committed rocprofv3 summaries (profiles/): short text files, each naming
the command that produced it, and every command runs committed files only (the
benchmark under the profiler, from the repository root) with its raw output
kept out of the repository."""

import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")


def _files():
    return sorted(f for f in os.listdir(PROFILES) if not f.startswith("."))


def test_profiles_are_short_text_summaries():
    files = _files()
    assert files
    for f in files:
        assert f.endswith((".txt", ".md")), f
        assert os.path.getsize(os.path.join(PROFILES, f)) < 64 * 1024, f


def test_every_profile_names_a_command_on_committed_files():
    with open(os.path.join(ROOT, ".gitignore")) as fh:
        ignored = {l.strip() for l in fh if l.strip() and not l.startswith("#")}
    for f in _files():
        with open(os.path.join(PROFILES, f)) as fh:
            text = fh.read()
        cmds = re.findall(r"(?:rocprofv3[^\n]*|python3 bench\.py[^\n]*)", text)
        assert cmds, f
        for c in cmds:
            assert "_work" not in c, (f, c)
            # raw profiler output goes to a folder that git ignores, never into the tree
            for d in re.findall(r"-d (\S+)", c):
                assert d.split("/")[0] + "/" in ignored, (f, c)
            for script in re.findall(r"python3 (\S+\.py)", c):
                assert os.path.exists(os.path.join(ROOT, script)), (f, script)
