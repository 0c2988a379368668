"""Host-sanitizer build of the library: every source compiled as for
liblizard.so, with AddressSanitizer and UndefinedBehaviorSanitizer on the host
side only (the gfx950 device code is built as usual), into _build_san/.

The C ABI's argument checks (lizard_abi.cpp, static_scratch.hip) are the host
code a caller reaches with arbitrary arguments; tests/test_host_sanitizers.py
runs the host-side ABI tests against this build with the sanitizer runtime
preloaded.  Not part of the product build.
"""
import concurrent.futures
import glob
import os
import subprocess

from . import build as _b

OUT = os.path.join(_b.HERE, "_build_san")
LIB = os.path.join(OUT, "liblizard_san.so")
# sanitizers for the host compilation only: each flag right after -Xarch_host
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def runtime():
    """Path of the shared AddressSanitizer runtime of the ROCm clang, or None."""
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _compile(src, obj):
    cmd = [_b.hipcc(), *_b.HIPCC_FLAGS, *SAN, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{r.stderr}")
    return obj


def build(jobs=None):
    os.makedirs(OUT, exist_ok=True)
    sources = sorted(f for f in os.listdir(_b.CSRC) if f.endswith((".hip", ".cpp")))
    objs = [os.path.join(OUT, os.path.splitext(f)[0] + ".o") for f in sources]
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs or min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(_compile, [os.path.join(_b.CSRC, f) for f in sources], objs))
    cmd = [_b.hipcc(), f"--offload-arch={_b.ARCH}", "-shared", "-fPIC", *SAN, *objs, "-o", LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return LIB


if __name__ == "__main__":
    print(build())
