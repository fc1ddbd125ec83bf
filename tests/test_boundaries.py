"""Boundaries the product keeps (CPU only): the library package never imports the oracle, no
product source reads the reference pages, the benchmark refuses more than one GPU with a
message, and its measured-traffic figure is tied to the kernels' code."""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mla_latent_cache_absorb_amd")


def test_package_does_not_import_the_oracle():
    code = ("import sys; sys.path.insert(0, %r); import mla_latent_cache_absorb_amd.binding, "
            "mla_latent_cache_absorb_amd.workloads, mla_latent_cache_absorb_amd.build; "
            "print('oracle' in sys.modules)" % ROOT)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True).stdout
    assert out.strip() == "False"


def test_product_sources_name_no_oracle_and_no_pages():
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if not f.endswith((".py", ".hip", ".h")):
                continue
            text = open(os.path.join(dirpath, f)).read()
            assert not re.search(r"^\s*(import|from)\s+oracle\b", text, flags=re.M), f
            assert "/root/reference" not in text, f
    for f in ("bench.py", "__graft_entry__.py"):
        assert "/root/reference" not in open(os.path.join(ROOT, f)).read(), f


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_counter_digest_follows_code_not_comments():
    # bench.py reports measured HBM traffic only while the kernels' code matches the code the
    # counters were taken on: comments and layout must not change the digest, code must
    sys.path.insert(0, ROOT)
    import bench

    src = "int f(int x) {  // doubles x\n  /* no-op */ return 2 * x;\n}\n"
    assert bench.code_text(src) == bench.code_text("int f(int x)\n{\n return 2 * x; // twice\n}")
    assert bench.code_text(src) != bench.code_text(src.replace("2 * x", "3 * x"))
    assert bench.code_text("a /* b */ c // d\ne") == "a c e"
    digest = bench.kernel_source_digest()
    assert re.fullmatch(r"[0-9a-f]{16}", digest)
    assert bench.kernel_source_digest() == digest
