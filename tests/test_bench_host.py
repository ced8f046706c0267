"""bench.py's host logic, without a GPU: the byte and FLOP accounting behind
`kv_gbps` and `roofline.achieved`, the key and hash that tie counter records
to a run and to the kernel code, and the one-GPU guard."""

import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_of_the_batch64_launch():
    # 64 streams x 2 KV heads x 4096 keys x 128 dims x 2 bytes, for K and for V,
    # plus one query and one output row of 16 x 128 bf16 per stream
    wl = synth.WORKLOADS["qwen3b_batch64"]
    kv = 64 * 2 * 4096 * 128 * 2 * 2
    q_and_out = 2 * 64 * 16 * 128 * 2
    assert bench.algorithmic_bytes(wl, [4096] * 64) == kv + q_and_out == 268_959_744
    # a partly filled stream moves only its live keys
    live = [4096] * 63 + [100]
    assert bench.algorithmic_bytes(wl, live) == kv + q_and_out - 2 * 2 * 3996 * 128 * 2


def test_append_bytes_read_and_write_each_new_key_and_value():
    wl = synth.WORKLOADS["qwen3b_chunk8"]
    per_token = wl.n_kv_heads * wl.head_dim * 2 * 2          # K and V, bf16
    assert bench.append_bytes(wl) == 2 * wl.n_streams * wl.chunk * per_token


def test_attention_flops_count_the_causal_keys_of_a_chunk():
    # C = 8 queries over a window of n live keys: query j sees n - 8 + 1 + j keys
    wl = synth.WORKLOADS["qwen3b_chunk8"]
    n = 37
    keys = sum(n - 8 + 1 + j for j in range(8))
    assert keys == 8 * n - 28
    assert bench.attention_flops(wl, [n]) == 4 * wl.head_dim * wl.n_q_heads * keys
    one = synth.WORKLOADS["qwen3b_batch64"]
    assert bench.attention_flops(one, [4096]) == 4 * 128 * 16 * 4096


def test_profile_key_names_workload_prefix_and_cache_mode():
    class A:
        workload = "qwen3b_batch64"
        prefix = 0
        cache_mode = "rotate_on_read"
    a = A()
    assert bench.profile_key(a) == "qwen3b_batch64"
    a.prefix = 256
    assert bench.profile_key(a) == "qwen3b_batch64+prefix256"
    a.prefix = 0
    a.cache_mode = "rebase_on_evict"
    assert bench.profile_key(a) == "qwen3b_batch64+rebase_on_evict"


def test_kernel_hash_follows_the_code_not_its_comments(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    src.write_text("__global__ void k(int* p) {\n    p[0] = 1;   // one\n}\n")
    h0 = bench.kernel_hash()
    src.write_text("// header\n__global__ void k(int* p) {\n  /* a\n block */ p[0] = 1;  // another\n\n}\n")
    assert bench.kernel_hash() == h0
    src.write_text("__global__ void k(int* p) {\n    p[0] = 2;   // one\n}\n")
    assert bench.kernel_hash() != h0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
