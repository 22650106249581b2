"""bench.py's contract that needs no GPU: it measures one GPU's share only."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_visible_pairs_matches_brute_force_count():
    sys.path.insert(0, ROOT)
    import bench
    import oracle
    from long_sequence_causal_cp_amd import binding as cb
    for N, r, L in ((2, 0, 64), (4, 3, 64), (8, 0, 64)):
        q_tab = cb.CpChunks.make(list(oracle.local_positions(2 * N * L, N, r)[::L]), L)
        kv = [cb.CpChunks.make(list(oracle.local_positions(2 * N * L, N, (r - j) % N)[::L]), L) for j in range(N)]
        qpos = oracle.local_positions(2 * N * L, N, r)
        brute = sum(int((oracle.local_positions(2 * N * L, N, (r - j) % N)[None, :] <= qpos[:, None]).sum())
                    for j in range(N))
        assert bench.visible_pairs(q_tab, kv) == brute == 2 * N * L * L + L
