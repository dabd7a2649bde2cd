"""Host-side checks of the benchmark's inputs (no GPU): the traffic record it
reports, and that the files a GPU run loads are not left off the upload."""
import fnmatch
import hashlib
import importlib.util
import re
from pathlib import Path

ROOT = Path(__file__).resolve().parents[1]


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", ROOT / "bench.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_traffic_records_match_the_kernel_sources():
    """bench.py reports a counted HBM traffic figure only while the kernel
    sources hash to the value recorded with the counters."""
    bench = _bench()
    for key, (name, files) in bench.TRAFFIC_PROFILES.items():
        path = ROOT / "profiles" / name
        if not path.exists():
            assert bench.measured_traffic(key) is None
            continue
        text = path.read_text()
        want = re.search(r"kernel_sources_sha256_16: ([0-9a-f]+)", text).group(1)
        h = hashlib.sha256()
        for f in files:
            h.update((ROOT / "bit_trellis_quantized_amd" / "csrc" / f).read_bytes())
        if h.hexdigest()[:16] == want:
            got = int(re.search(r"traffic_bytes_per_launch: (\d+)", text).group(1))
            assert bench.measured_traffic(key) == got
        else:
            assert bench.measured_traffic(key) is None


def _ignored(rel: str, patterns) -> bool:
    """tar-style exclusion as the upload applies it: './x' anchors at the
    root, a bare pattern matches the name or the path at any depth."""
    parts = rel.split("/")
    for p in patterns:
        if p.startswith("./"):
            anchored = p[2:]
            if any(fnmatch.fnmatch("/".join(parts[:i]), anchored) for i in range(1, len(parts) + 1)):
                return True
        else:
            if any(fnmatch.fnmatch(x, p) for x in parts) or fnmatch.fnmatch(rel, p):
                return True
    return False


def test_gpu_runs_ship_what_bench_and_tests_load():
    ign = ROOT / ".gpurunignore"
    patterns = [ln.strip() for ln in ign.read_text().splitlines() if ln.strip()] if ign.exists() else []
    bench = _bench()
    needed = ["profiles/" + name for name, _ in bench.TRAFFIC_PROFILES.values()
              if (ROOT / "profiles" / name).exists()]
    needed += ["bench.py", "__graft_entry__.py", "bit_trellis_quantized_amd/escha.py",
              "bit_trellis_quantized_amd/synth.py", "bit_trellis_quantized_amd/libescha.so"]
    needed += [p.relative_to(ROOT).as_posix() for p in (ROOT / "tests").rglob("*") if p.is_file()
               and "__pycache__" not in p.parts]
    needed += [p.relative_to(ROOT).as_posix() for p in (ROOT / "oracle").rglob("*") if p.is_file()
               and "__pycache__" not in p.parts]
    left_off = [n for n in needed if _ignored(n, patterns)]
    assert not left_off, left_off
