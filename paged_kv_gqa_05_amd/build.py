"""Builds libpkv.so (every HIP/C++ source under csrc/) for gfx950 with hipcc.

Run ``python paged_kv_gqa_05_amd/build.py`` (or __graft_entry__.build()); it is a
plain script so that it never imports the package (which needs the library).  It
always recompiles.  Objects go to csrc/_obj/, the library next to this file.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(CSRC, "_obj")
LIB = os.path.join(HERE, "libpkv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-result", "-munsafe-fp-atomics",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src):
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    return src, obj, r.returncode, errs


def build(verbose=True):
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    bad = [r for r in results if r[2] != 0]
    for src, _, rc, errs in results:
        if errs.strip() and verbose:
            print(f"[{os.path.basename(src)}]\n{errs}", file=sys.stderr)
    if bad:
        raise RuntimeError("hipcc failed for: " + ", ".join(os.path.basename(b[0]) for b in bad))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp,
           *[r[1] for r in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


# Host-side sanitizer build (AddressSanitizer + UndefinedBehaviorSanitizer on
# the host code only; the CPU tests that load it run no kernel): the
# host runtime's argument checks, allocator and validation run under it in the
# CPU tests.  Each -fsanitize= follows -Xarch_host.
SAN_OBJ = os.path.join(CSRC, "_obj_hostsan")
SAN_LIB = os.path.join(HERE, "libpkv_hostsan.so")
SAN_FLAGS = ["-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _compile_san(src):
    obj = os.path.join(SAN_OBJ, os.path.basename(src) + ".o")
    cmd = [HIPCC, "--offload-arch=gfx950", *SAN_FLAGS, "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    return src, obj, r.returncode, r.stdout + r.stderr


def build_host_sanitized():
    os.makedirs(SAN_OBJ, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile_san, srcs))
    bad = [r for r in results if r[2] != 0]
    if bad:
        raise RuntimeError("hipcc (host sanitizer build) failed:\n" + "\n".join(b[3] for b in bad))
    tmp = SAN_LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-shared-libasan", "-o", tmp, *[r[1] for r in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


# Measurement variants: the library with some sources compiled with extra
# defines, linked with the other objects of build().  attn_qk_valu computes
# the f16 attention scores with v_dot2 on the VALU instead of the 16x16x32
# MFMA (libpkv_attn_qk_valu.so; select it with PKV_LIB_PATH), to time that
# choice against the MFMA form.  attn_stamps records wall-clock stamps per
# attention workgroup or work-list item (start, context known, partition
# computed, end; read back with pkv_debug_attn_stamps), for timelines.
VARIANTS = {"attn_qk_valu": (("attn.hip", "persist.hip"), ["-DPKV_ATTN_QK_VALU"]),
            "attn_stamps": (("attn.hip",), ["-DPKV_ATTN_STAMPS"])}


def build_variant(name):
    files, defines = VARIANTS[name]
    vobj = os.path.join(CSRC, "_obj_" + name)
    os.makedirs(vobj, exist_ok=True)
    objs = []
    for src in sources():
        base = os.path.basename(src)
        if base in files:
            obj = os.path.join(vobj, base + ".o")
            cmd = [HIPCC, *FLAGS, *defines, "-x", "hip", "-c", src, "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed for {base} ({name}):\n" + r.stdout + r.stderr)
        else:
            obj = os.path.join(OBJ, base + ".o")
            if not os.path.exists(obj):
                raise RuntimeError(f"{obj} missing: run build() first")
        objs.append(obj)
    lib = os.path.join(HERE, f"libpkv_{name}.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib + ".tmp", *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--host-sanitized":
        print(build_host_sanitized())
    elif len(sys.argv) > 2 and sys.argv[1] == "--variant":
        print(build_variant(sys.argv[2]))
    else:
        print(build())
