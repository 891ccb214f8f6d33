"""Host-sanitizer build of liblcmoe.so, for CPU-only checks of the C ABI.

The host code (argument validation, workspace layout, launch sequencing) is
built with AddressSanitizer and UndefinedBehaviorSanitizer; the gfx950 device
code is built as usual (the sanitizer options go to the host pass only). The
result is _build/sanitize/liblcmoe.so; nothing else uses it. Run the host
test suites against it with the binding's LCMOE_LIBRARY override and the
sanitizer runtime preloaded (python itself is not instrumented):

    python -m mixture_experts_layer_biased_amd.build_sanitized
    LD_PRELOAD=$(hipcc -print-file-name=libclang_rt.asan-x86_64.so) \\
    ASAN_OPTIONS=detect_leaks=0 UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 \\
    LCMOE_LIBRARY=_build/sanitize/liblcmoe.so \\
    python -m pytest tests/test_abi.py tests/test_binding_checks.py -p no:cacheprovider
"""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

from mixture_experts_layer_biased_amd.build import ARCH, CSRC, FLAGS, ROOT, SOURCES, _hipcc, _run

OUT_DIR = os.path.join(ROOT, "_build", "sanitize")
LIB = os.path.join(OUT_DIR, "liblcmoe.so")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def build():
    hipcc = _hipcc()
    os.makedirs(OUT_DIR, exist_ok=True)
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(OUT_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([hipcc, *FLAGS, "-O1", "-g", *HOST_SAN, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        list(ex.map(_run, cmds))
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *HOST_SAN, "-shared-libsan", *objs,
          "-o", LIB])
    return LIB


if __name__ == "__main__":
    print(build())
    sys.exit(0)
