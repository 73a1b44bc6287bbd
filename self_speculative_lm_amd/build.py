"""Build libtrimode.so in-tree with hipcc for gfx950.

    python -m self_speculative_lm_amd.build
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["k_gemm.hip", "k_attn.hip", "k_misc.hip", "runtime.hip"]
OUT = os.path.join(HERE, "libtrimode.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed float32 VALU forms are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# Per-source additions.  The attention kernel rescales and reads its MFMA
# results with VALU code every tile; in the VGPR form they need no moves
# between accumulation and vector registers.
EXTRA_FLAGS = {
    "k_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    return "hipcc"


def compile_flags(src: str) -> list:
    """Flags for one source file (without -c / -o)."""
    return [*HIPCC_FLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []),
            "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(HERE, "csrc")]


# Host-code sanitizers (AddressSanitizer + UndefinedBehaviorSanitizer) for a
# checking build of the runtime: each -fsanitize applies to the host pass only
# (device code is built as usual).  The library then needs the sanitizer
# runtime preloaded (sanitizer_runtime()).
SANITIZE_FLAGS = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer"]


def sanitizer_runtime() -> str:
    """Path of the shared AddressSanitizer runtime of the HIP toolchain."""
    out = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        rt = subprocess.run(["/opt/rocm/llvm/bin/clang", "-print-resource-dir"], capture_output=True, text=True)
        path = os.path.join(rt.stdout.strip(), "lib", "linux", "libclang_rt.asan-x86_64.so")
    return path


def build(verbose: bool = False, sanitize: bool = False, out: str = OUT) -> str:
    """Compile every source to an object (in parallel), then link the library.
    sanitize: the host-sanitizer checking build (objects and library at `out`'s
    directory, never the in-tree library)."""
    objdir = os.path.join(os.path.dirname(out) if sanitize else HERE, "_build_san" if sanitize else "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    for s in SOURCES:
        src = os.path.join(HERE, "csrc", s)
        obj = os.path.join(objdir, s + ".o")
        flags = compile_flags(src)
        if sanitize:
            flags = [f for f in flags if f != "-O3"] + SANITIZE_FLAGS
        cmd = [hipcc(), *flags, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((obj, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for obj, cmd, p in procs:
        log, _ = p.communicate()
        if p.returncode != 0:
            failed.append((cmd, log))
    if failed:
        for cmd, log in failed:
            sys.stderr.write(" ".join(cmd) + "\n" + log)
        raise RuntimeError(f"hipcc failed for {len(failed)} source(s)")
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-fPIC", "-shared", *[o for o, _, _ in procs], "-o", tmp]
    if sanitize:
        cmd += ["-fsanitize=address,undefined", "-shared-libsan"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"link failed with exit code {r.returncode}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
