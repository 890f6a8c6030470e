"""The committed measurement summaries under profiles/ name the command that made each figure, and
every such command runs committed files only: bench.py (with options it defines) or the issue-rate
probe, under rocprofv3 with either a kernel trace or counters, never both."""
import json
import os
import re
import shlex

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")


def _bench_options():
    src = open(os.path.join(ROOT, "bench.py")).read()
    return set(re.findall(r'add_argument\("(--[a-z0-9-]+)"', src))


def _commands():
    out = []
    for name in sorted(os.listdir(PROFILES)):
        path = os.path.join(PROFILES, name)
        if name.endswith(".txt"):
            cmds = [l[len("command: "):].strip() for l in open(path) if l.startswith("command: ")]
        elif name.endswith(".json"):
            cmds = json.load(open(path))["commands"]
        else:
            cmds = []
        out.append((name, cmds))
    return out


def test_profiles_are_text_summaries():
    names = os.listdir(PROFILES)
    assert names
    for name in names:
        assert name.endswith((".txt", ".json", ".md")), f"{name}: profiles/ holds short text summaries only"
        assert os.path.getsize(os.path.join(PROFILES, name)) < 64 * 1024, f"{name} is not a short summary"


@pytest.mark.parametrize("name,cmds", _commands(), ids=lambda v: v if isinstance(v, str) else "")
def test_profile_commands_run_committed_files(name, cmds):
    assert cmds, f"{name} names no command"
    opts = _bench_options()
    for cmd in cmds:
        assert "_work" not in cmd, f"{name}: {cmd}"
        for part in cmd.split("&&"):
            tok = shlex.split(part.replace("<these commands as JSON>", "JSON"))
            if tok[0] == "rocprofv3":
                pre = tok[:tok.index("--")]
                assert ("--kernel-trace" in pre) != ("--pmc" in pre), f"{name}: trace or counters, not both: {cmd}"
                assert not any(t in pre for t in ("-s", "--sys-trace", "-r", "--runtime-trace")), cmd
                tok = tok[tok.index("--") + 1:]
            if tok[0] == "python3" and tok[1] == "-m":
                assert tok[2] == "selective_state_space_41_amd.build", cmd
                continue
            if tok[0] == "python3":
                assert tok[1] == "bench.py", cmd
                used = {t for t in tok[2:] if t.startswith("--")}
                assert used <= opts, f"{name}: options bench.py does not define: {sorted(used - opts)}"
                continue
            assert tok[0] == "./selective_state_space_41_amd/vmscan_probe", cmd
            assert os.path.exists(os.path.join(ROOT, "selective_state_space_41_amd", "csrc", "probe.hip"))


def test_traffic_record_is_tied_to_a_source_digest():
    for name in os.listdir(PROFILES):
        if name.startswith("traffic_") and name.endswith(".json"):
            rec = json.load(open(os.path.join(PROFILES, name)))
            assert re.fullmatch(r"[0-9a-f]{16}", rec["source_sha256_16"]), name
            assert rec["traffic_bytes_per_launch"] > 0
