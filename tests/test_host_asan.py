"""The library's host code under AddressSanitizer (CPU only, no GPU needed).

The host side of every entry point (argument validation, workspace layout arithmetic, the
error strings) is built with -fsanitize=address into _build/asan/ (the device code is
built as usual) and driven from a C program that calls every entry point include/kvm.h
declares with arguments that validation must reject: all-NULL arguments, an all-zero
descriptor with non-NULL pointers, and undersized workspaces.  Validation runs before any
HIP call, so nothing reaches a device; any out-of-bounds host access or use after free
makes ASan abort the program."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"


def _prototypes():
    src = open(os.path.join(ROOT, "include", "kvm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    out = []
    for m in re.finditer(r"\n([a-z_0-9]+)\s+(kvm_[a-z0-9_]+)\s*\(([^;]*)\)\s*;", src):
        ret, name, params = m.group(1), m.group(2), " ".join(m.group(3).split())
        ps = [] if params == "void" else [p.strip() for p in params.split(",")]
        out.append((ret, name, ps))
    return out


def _arg(p, variant, first):
    if "*" in p:
        if variant == "null":
            return "NULL"
        if first and "desc" in p:
            t = p.rsplit("*", 1)[0].strip()
            return f"({t}*)zero_desc"
        return "(void*)FAKE"
    return "0"


def _harness():
    lines = ["#include <stdio.h>", "#include <stdint.h>", "#include <string.h>", '#include "kvm.h"',
             "#define FAKE 0x7f0000000000ull", "static unsigned char zero_desc[4096];",
             "static int bad = 0;",
             "#define EXPECT_FAIL(call) do { int s = (int)(call); if (s == 0) { printf(\"accepted: %s\\n\", #call); bad++; } } while (0)",
             "int main(void) {", "  memset(zero_desc, 0, sizeof zero_desc);"]
    n = 0
    for ret, name, ps in _prototypes():
        if name in ("kvm_check_device",):
            continue     # a HIP call: needs a device
        for variant in ("null", "zero"):
            args = ", ".join(_arg(p, variant, i == 0) for i, p in enumerate(ps))
            call = f"{name}({args})"
            if ret == "kvm_status":
                lines.append(f"  EXPECT_FAIL({call});")
            elif ret == "size_t":
                lines.append(f"  if ({call} != 0 && {len(ps)} > 0) {{ printf(\"size for a bad desc: %s\\n\", \"{name}\"); bad++; }}")
            elif ret == "int32_t":
                lines.append(f"  if ({call} != -1) {{ printf(\"count for a bad desc: %s\\n\", \"{name}\"); bad++; }}")
            else:
                lines.append(f"  (void){call};")
            n += 1
            if not ps:
                break
    # undersized workspaces (the messages format sizes with %zu)
    lines += [
        "  { kvm_decode_desc d = {1, 32, 8, 128, 64, 0, KVM_BF16, KVM_READ_NONE, 0.088f, 1e-6f};",
        "    size_t need = kvm_decode_workspace_size(&d);",
        "    int s = (int)kvm_decode_attn_mem(&d, (void*)FAKE, NULL, NULL, NULL, (void*)FAKE, (void*)FAKE, (void*)FAKE,",
        "        NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, (void*)FAKE, NULL, (void*)FAKE, need - 1, NULL);",
        "    if (s != KVM_ERR_WORKSPACE) { printf(\"decode ws: %d\\n\", s); bad++; }",
        "    if (!strstr(kvm_last_error(), \"workspace\")) { printf(\"message: %s\\n\", kvm_last_error()); bad++; } }",
        "  { kvm_topk_desc t = {2, 40000, 100, 0, 1};",
        "    size_t need = kvm_topk_workspace_size(&t);",
        "    int s = (int)kvm_topk_select(&t, (void*)FAKE, (void*)FAKE, (void*)FAKE, (void*)FAKE, need - 1, NULL);",
        "    if (s != KVM_ERR_WORKSPACE) { printf(\"topk ws: %d\\n\", s); bad++; } }",
        "  for (int s = -1; s < 12; ++s) if (!kvm_status_string((kvm_status)s)) bad++;",
        "  printf(\"abi %d calls %d bad %d\\n\", kvm_abi_version(), " + str(n) + ", bad);",
        "  return bad != 0;",
        "}"]
    return "\n".join(lines) + "\n"


@pytest.fixture(scope="module")
def asan_lib():
    import importlib.util
    spec = importlib.util.spec_from_file_location("_kvm_build_asan", os.path.join(ROOT, "learned_kv_cache_mqa_amd",
                                                                                  "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.build(asan=True)


@pytest.mark.skipif(not os.path.exists(CLANG), reason="needs the ROCm clang for the host AddressSanitizer build")
def test_entry_points_reject_bad_arguments_under_asan(asan_lib, tmp_path):
    src = tmp_path / "asan_harness.c"
    src.write_text(_harness())
    exe = tmp_path / "asan_harness"
    libdir = os.path.dirname(asan_lib)
    subprocess.run([CLANG, "-std=c99", "-g", "-fsanitize=address", "-I", os.path.join(ROOT, "include"), str(src),
                    "-L", libdir, "-lkvmem", f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=99")
    p = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert "AddressSanitizer" not in p.stderr, p.stderr[-4000:]
    assert p.returncode == 0, p.stdout + p.stderr[-2000:]
    assert "bad 0" in p.stdout
