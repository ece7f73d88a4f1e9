"""Host-side checks of bench.py that need no GPU: every global name a function
uses is defined (a missing helper would otherwise surface only when the
benchmark reaches it on the device), the --gpus guard, and the traffic record
parser on a stored counter file."""

import builtins
import json
import os
import subprocess
import symtable
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _module_definitions(table):
    return {s.get_name() for s in table.get_symbols()
            if s.is_assigned() or s.is_imported() or s.is_namespace()}


def _global_uses(table, out):
    for child in table.get_children():
        for s in child.get_symbols():
            if s.is_referenced() and (s.is_global() and not s.is_declared_global()):
                out.add((child.get_name(), s.get_name()))
        _global_uses(child, out)
    return out


def test_every_global_name_is_defined():
    src = open(BENCH).read()
    top = symtable.symtable(src, BENCH, "exec")
    defined = _module_definitions(top) | set(dir(builtins))
    missing = sorted((fn, name) for fn, name in _global_uses(top, set()) if name not in defined)
    assert not missing, f"bench.py uses undefined globals: {missing}"


def test_functions_the_default_run_calls_exist():
    import ast
    tree = ast.parse(open(BENCH).read())
    defs = {n.name for n in tree.body if isinstance(n, ast.FunctionDef)}
    for name in ("ablation_leg", "small_batch_leg", "chunked_leg", "decode_leg", "gdn_leg",
                 "gdn_cpu_baseline", "cpu_baseline", "traffic_record", "write_traffic",
                 "tile_sweep_leg", "stream_ceiling", "mfma_ceiling", "time_workload"):
        assert name in defs, name


def test_several_gpus_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_record_reads_the_stored_summary():
    sys.path.insert(0, ROOT)
    import bench
    rec = bench.traffic_record()  # HBM bytes per launch of the dominant kernel
    if rec is not None:  # null when the kernels changed after the counters were taken
        json.dumps(rec)
        assert rec > 0
