"""bench.py's host-side contract (CPU): it measures one GPU and refuses
--gpus N > 1 (or a multi-rank launch) with a message and exit status 2,
before touching a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, env=e, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_a_multi_rank_launch_is_refused():
    r = _run([], env={"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_launch_form_labels_follow_the_dispatch_rules():
    """step_kernels names the launches kin_sparse_decode_step makes (bf16, no
    scores output): one kernel when the pairs cover the chip (at most 8192
    blocks and 2048 kept), the split select + attend alone when few pairs
    keep every block, score tiles + select/attend for few pairs otherwise,
    and four launches past 2048 kept blocks; the tiny fp32 layer is one
    fp32 kernel."""
    sys.path.insert(0, ROOT)
    import bench
    from block_top_sparse_amd import workloads

    cu = 256
    form = {w.name: bench.step_kernels(w, cu) for w in workloads.sweep()}
    assert bench.step_kernels(workloads.QWEN3_8B, cu) == "one"
    assert bench.step_kernels(workloads.TINY, cu) == "one-f32"                # 640 KiB per pair
    assert form["sweep-b32-ctx32768-blk16-budget1024"] == "one"        # 256 pairs
    assert form["sweep-b8-ctx32768-blk16-budget8192"] == "two"         # 64 pairs, 512 of 2048
    assert form["sweep-b8-ctx8192-blk16-allblocks"] == "one-split"     # 64 pairs, all 512 kept
    assert form["sweep-b32-ctx131072-blk16-allblocks"] == "four"       # 8192 kept blocks
    for w in workloads.sweep():
        f = form[w.name]
        if w.topk > 2048:
            assert f == "four", w.name
        elif w.pairs >= cu and w.nb <= 8192:
            assert f == "one", w.name
        else:
            assert f in ("two", "one-split"), w.name
            assert (f == "one-split") == (w.topk >= w.nb), w.name
