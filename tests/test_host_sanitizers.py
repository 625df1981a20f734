"""The host part of the library (label parsing, trie construction, decision-word
cut) built alone with AddressSanitizer and UndefinedBehaviorSanitizer and run on
the configs' label sets, random and malformed label sets and short output
capacities (tests/host_sanitized_run.py, in a child process that preloads the ASan
runtime).  These functions parse caller-supplied label CSR, so out-of-bounds reads
or writes and undefined arithmetic there are what this guards against."""
import os
import subprocess
import sys

from trie_constrained_scoring_amd.build import build_host_sanitized

HERE = os.path.dirname(os.path.abspath(__file__))


def test_host_library_under_asan_and_ubsan():
    so = build_host_sanitized()
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, os.path.join(HERE, "host_sanitized_run.py"), so],
                       capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0 and "SANITIZED_OK" in r.stdout, (r.returncode, r.stdout[-2000:],
                                                                r.stderr[-4000:])
