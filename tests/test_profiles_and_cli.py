"""The committed profile summaries against the sources they were measured on, and the bench's
command line (no GPU needed).

Each summary under profiles/ names the source files of the kernels it measured, with the
sha256[:16] of their bytes concatenated in the order listed; a summary whose hash no longer
matches describes a kernel that has since changed.  The commands a summary records must run
files of this repository that are under version control.
"""
import hashlib
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "kv_cache_attention_02_amd", "csrc")
ATTN_FILES = ["attn_bf16.hip", "attn_tiles.h", "fastdiv.h", "wmk_internal.h"]

ONE_FILE = re.compile(r"^([\w.]+) sha256\[:16\]: ([0-9a-f]{16})\s*$")
FILE_LIST = re.compile(r"sources sha256\[:16\] \(([^)]*)\): ([0-9a-f]{16})")
COUNTER_KEY = re.compile(r"^kernel_source_sha256_16: ([0-9a-f]{16})\s*$")


def _hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _summaries():
    return sorted(os.path.join(PROFILES, f) for f in os.listdir(PROFILES) if f.endswith((".txt", ".md")))


def _recorded_hashes(path):
    out = []
    for line in open(path, encoding="utf-8"):
        m = ONE_FILE.match(line)
        if m:
            out.append(([m.group(1)], m.group(2)))
            continue
        m = FILE_LIST.search(line)
        if m:
            out.append(([f.strip() for f in m.group(1).split(",")], m.group(2)))
            continue
        m = COUNTER_KEY.match(line)
        if m:
            out.append((ATTN_FILES, m.group(1)))
    return out


def test_every_summary_records_the_hash_of_its_kernel_sources():
    paths = _summaries()
    assert paths, "no profile summaries"
    for path in paths:
        assert _recorded_hashes(path), f"{os.path.basename(path)} records no source hash"


def test_recorded_hashes_match_the_current_sources():
    stale = []
    for path in _summaries():
        for files, recorded in _recorded_hashes(path):
            now = _hash(files)
            if now != recorded:
                stale.append(f"{os.path.basename(path)}: {', '.join(files)} recorded {recorded}, now {now}")
    assert not stale, "profiles measured on other sources:\n" + "\n".join(stale)


def test_recorded_commands_run_tracked_files_only():
    tracked = set(subprocess.run(["git", "ls-files"], cwd=ROOT, capture_output=True, text=True,
                                 check=True).stdout.split())
    if not tracked:                       # an exported tree without git metadata
        tracked = None
    ran = 0
    for path in _summaries():
        text = open(path, encoding="utf-8").read()
        assert "_work" not in text, f"{os.path.basename(path)} names a scratch file"
        for rel in re.findall(r"\$R/([\w./-]+)", text):
            if rel.startswith("gpurun_out/"):
                continue                  # the profiler's output folder
            assert os.path.isfile(os.path.join(ROOT, rel)), f"{os.path.basename(path)} runs missing {rel}"
            if tracked is not None:
                assert rel in tracked, f"{os.path.basename(path)} runs untracked {rel}"
            ran += 1
    assert ran > 0


def test_bench_runs_on_one_gpu_only():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_bench_help_lists_its_modes():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--append-only", "--step-profile", "--rates-only"):
        assert flag in r.stdout
