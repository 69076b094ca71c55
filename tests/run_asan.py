"""Run the host-side CPU tests (block pool, argument validation) against a host
AddressSanitizer build of the library.

    python -m kv_cache_flashattention_attn_amd.build --asan   # writes libattn_asan.so
    python tests/run_asan.py

The sanitizer runtime is preloaded into a child Python process (the interpreter
itself is not instrumented, so leak checking is off); any invalid access in the
library's host code aborts the run.  Not collected by pytest: it starts a process
of its own.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def main() -> int:
    from kv_cache_flashattention_attn_amd import build
    if not os.path.exists(build.ASAN_LIB_PATH):
        print(f"{build.ASAN_LIB_PATH} is missing: python -m kv_cache_flashattention_attn_amd.build --asan")
        return 2
    clang = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang++")
    rt = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", PYTHONPATH=ROOT)
    code = ("import sys, pytest\n"
            "import kv_cache_flashattention_attn_amd as K\n"
            f"K.lib_path = {build.ASAN_LIB_PATH!r}\n"
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', 'tests/test_block_pool.py', "
            "'tests/test_library_cpu.py']))\n")
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env).returncode


if __name__ == "__main__":
    sys.exit(main())
