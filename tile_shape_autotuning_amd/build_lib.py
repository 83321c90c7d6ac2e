"""Build libtilegemm.so for gfx950.

Steps:
  1. compile the host selection rules with g++ into a small program that
     prints the kernel instantiation set (every configuration of the space
     that passes the shape-independent rules; split-K is a run-time value);
  2. generate instantiation units (a few kernels each) under _build/;
  3. compile them with hipcc in parallel, recording each kernel's register,
     scratch and LDS use from the compiler's resource remarks;
  4. generate the kernel registry (with those resource figures) and link
     everything into tile_shape_autotuning_amd/_lib/libtilegemm.so.

Usage: python -m tile_shape_autotuning_amd.build_lib [--incremental] [-j N]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import os
import re
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(REPO, "_build", "tilegemm")
GEN = os.path.join(BUILD, "gen")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libtilegemm.so")
RES_JSON = os.path.join(LIBDIR, "kernel_resources.json")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
ARCH = "gfx950"
HIP_FLAGS = ["-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument", "-I", CSRC]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall", "-I", CSRC]
KERNELS_PER_UNIT = 6

HEADERS = [os.path.join(CSRC, f) for f in ("select.hpp", "registry.hpp", "runtime.hpp")] + \
    [os.path.join(CSRC, "kernels", f) for f in os.listdir(os.path.join(CSRC, "kernels")) if f.endswith(".hpp")] + \
    [os.path.join(REPO, "include", "tilegemm.h")]


def kernel_source_digest() -> str:
    """SHA-256 over what decides a GEMM call's memory traffic: the GEMM
    kernel sources, the launch path (grid, block order, instantiation chosen)
    and the split-K second pass, and the device compile flags, without
    file-system paths.  Measurements taken with one digest describe every
    build of the same sources (the toolchain is the same image everywhere)."""
    import hashlib
    files = sorted(os.path.join(CSRC, "kernels", f) for f in os.listdir(os.path.join(CSRC, "kernels"))
                   if f.endswith(".hpp"))
    files += [os.path.join(CSRC, f) for f in ("api.cpp", "splitk_reduce.hip", "pad.hip", "workspace.cpp")]
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.relpath(f, CSRC).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    h.update(" ".join(x for x in HIP_FLAGS if x != CSRC).encode())
    return h.hexdigest()


def _run(cmd, verbose=False, capture=False):
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r.stderr if capture else None


def _stale(obj, deps):
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(d) > t for d in deps)


def instantiation_set(verbose=False):
    exe = os.path.join(BUILD, "tg_space")
    srcs = [os.path.join(CSRC, "select.cpp"), os.path.join(CSRC, "space_main.cpp")]
    _run(["g++", *HOST_FLAGS, "-o", exe, *srcs], verbose)
    out = subprocess.run([exe], stdout=subprocess.PIPE, text=True, check=True).stdout
    return [tuple(int(x) for x in line.split()) for line in out.splitlines() if line.strip()]


def _kernel_expr(e, stream_b=False):
    in_bf16, kind, bm, bn, bk, wgm, wgn, st, kg = e
    if kind == 1:
        return f"launch_skinny<{bm // 16}, {wgm}, {st}>"
    if kind == 3:
        return f"launch_streamk<{bm}, {bn}, {bk}, {wgm}, {wgn}, {st}>"
    if kind in (0, 4):
        f32 = "false" if in_bf16 else "true"
        return (f"launch_tiled_dma<{bm}, {bn}, {bk}, {wgm}, {wgn}, {st}, {'true' if stream_b else 'false'}, {f32}, "
                f"{kg if kind == 4 else 1}>")
    # the unaligned kind: the element-load kernel
    bf = "true" if in_bf16 else "false"
    return f"launch_tiled<{bf}, {bm}, {bn}, {bk}, {wgm}, {wgn}, {st}>"


STREAM_B_MAX_BM = 64     # tallest tile with a B-streaming twin (M <= BM: the decode regime)


def _has_stream_b(e):
    """bf16 DMA tiles short enough to cover M in one tile row (M <= BM <= 64)
    also get the instantiation that streams B with the non-temporal policy."""
    in_bf16, kind, bm = e[0], e[1], e[2]
    return in_bf16 == 1 and kind == 0 and bm <= STREAM_B_MAX_BM


def generate_units(entries):
    os.makedirs(GEN, exist_ok=True)
    units = []
    for u in range(0, len(entries), KERNELS_PER_UNIT):
        part = entries[u:u + KERNELS_PER_UNIT]
        idx = u // KERNELS_PER_UNIT
        lines = ["// generated by build_lib.py: kernel instantiations", '#include "kernels/instantiate.hpp"',
                 '#include "registry.hpp"', "#if !defined(__HIP_DEVICE_COMPILE__)", "namespace tg {",
                 f"extern const KernelEntry kPart{idx}[] = {{"]
        for e in part:
            lines.insert(3, f"template hipError_t tg::{_kernel_expr(e)}(const tg::GemmParams&, int, hipStream_t);")
            if _has_stream_b(e):
                lines.insert(3, f"template hipError_t tg::{_kernel_expr(e, True)}(const tg::GemmParams&, int, "
                                f"hipStream_t);")
        for e in part:
            in_bf16, kind, bm, bn, bk, wgm, wgn, st, kg = e
            sb = f"&{_kernel_expr(e, True)}" if _has_stream_b(e) else "nullptr"
            threads = 64 * wgm * (1 if kind == 1 else wgn) * (kg if kind == 4 else 1)
            lines.append(f"    {{{in_bf16}, {{{kind}, {bm}, {bn}, {bk}, {wgm}, {wgn}, {st}, {kg}}}, "
                         f"&{_kernel_expr(e)}, {threads}, {{0, 0, 0, 0, 0}}, {sb}}},")
        lines += ["};", f"extern const int kPart{idx}Count = {len(part)};", "}  // namespace tg", "#endif", ""]
        path = os.path.join(GEN, f"inst_{idx:03d}.hip")
        text = "\n".join(lines)
        if not os.path.exists(path) or open(path).read() != text:
            with open(path, "w") as f:
                f.write(text)
        units.append(path)
    return units


_TILED_RE = re.compile(r"gemm_tiled_kernelILb(\d)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)EE")
_SKINNY_RE = re.compile(r"gemm_skinny_kernelILi(\d+)ELi(\d+)ELi(\d+)E")
_DMA_RE = re.compile(r"gemm_tiled_dma_kernelILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELb(\d)ELb(\d)ELi(\d+)E")
_SK_RE = re.compile(r"gemm_streamk_kernelILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)EE")


def parse_resources(text):
    """Kernel resource remarks -> {(in_bf16, kind, bm, bn, bk, wgm, wgn, st, k_groups): {...}}."""
    res = {}
    cur = None
    for line in text.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            t = _TILED_RE.search(name)
            s = _SKINNY_RE.search(name)
            dm = _DMA_RE.search(name)
            sk = _SK_RE.search(name)
            if sk:
                bm, bn, bk, wgm, wgn, st = (int(x) for x in sk.groups())
                cur = (1, 3, bm, bn, bk, wgm, wgn, st, 0)
            elif dm:
                bm, bn, bk, wgm, wgn, st, stream_b, f32, wk = (int(x) for x in dm.groups())
                # the registry records the plain instantiation's figures; the
                # B-streaming twin differs only in a cache-policy bit.  K
                # groups > 1: the sliced-K kind
                kind = 4 if wk > 1 else 0
                cur = (1 - f32, kind, bm, bn, bk, wgm, wgn, st, wk if kind == 4 else 0) if not stream_b else None
            elif t:
                bf, bm, bn, bk, wgm, wgn, st = (int(x) for x in t.groups())
                cur = (bf, 2, bm, bn, bk, wgm, wgn, st, 0)
            elif s:
                mt, w, u = (int(x) for x in s.groups())
                cur = (1, 1, 16 * mt, 128, 32, w, 1, u, 0)
            else:
                cur = None
            if cur is not None:
                res[cur] = {}
            continue
        if cur is None:
            continue
        for key, pat in (("vgpr", r"\bVGPRs: (\d+)"), ("agpr", r"AGPRs: (\d+)"),
                         ("scratch", r"ScratchSize \[bytes/lane\]: (\d+)"),
                         ("occupancy", r"Occupancy \[waves/SIMD\]: (\d+)"),
                         ("lds", r"LDS Size \[bytes/block\]: (\d+)")):
            m = re.search(pat, line)
            if m:
                res[cur][key] = int(m.group(1))
    return res


def generate_registry(entries, resources):
    lines = ["// generated by build_lib.py: kernel registry", "#include <algorithm>", "#include <vector>",
             '#include "registry.hpp"', '#include "select.hpp"', "namespace tg {"]
    nunits = (len(entries) + KERNELS_PER_UNIT - 1) // KERNELS_PER_UNIT
    for i in range(nunits):
        lines.append(f"extern const KernelEntry kPart{i}[]; extern const int kPart{i}Count;")
    lines.append("struct ResRow { int key[9]; KernelResources r; };")
    lines.append("static const ResRow kRes[] = {")
    for e in entries:
        r = resources.get(tuple(e), {})
        lines.append(f"    {{{{{', '.join(str(x) for x in e)}}}, {{{r.get('vgpr', -1)}, {r.get('agpr', -1)}, "
                     f"{r.get('scratch', -1)}, {r.get('lds', -1)}, {r.get('occupancy', -1)}}}}},")
    lines.append("};")
    lines.append("static std::vector<KernelEntry> build() {")
    lines.append("    std::vector<KernelEntry> v;")
    for i in range(nunits):
        lines.append(f"    v.insert(v.end(), kPart{i}, kPart{i} + kPart{i}Count);")
    lines += [
        "    for (KernelEntry& k : v)",
        "        for (const ResRow& r : kRes)",
        "            if (r.key[0] == k.in_bf16 && r.key[1] == k.cfg.kind && r.key[2] == k.cfg.bm && r.key[3] == k.cfg.bn &&",
        "                r.key[4] == k.cfg.bk && r.key[5] == k.cfg.wgm && r.key[6] == k.cfg.wgn && r.key[7] == k.cfg.stages &&",
        "                r.key[8] == k.cfg.split_k)",
        "                k.res = r.r;",
        "    std::sort(v.begin(), v.end(), [](const KernelEntry& a, const KernelEntry& b) {",
        "        return a.in_bf16 != b.in_bf16 ? a.in_bf16 < b.in_bf16 : cfg_less(a.cfg, b.cfg); });",
        "    return v;",
        "}",
        "static const std::vector<KernelEntry>& table() { static const std::vector<KernelEntry> t = build(); return t; }",
        "const KernelEntry* registry_begin() { return table().data(); }",
        "const KernelEntry* registry_end() { return table().data() + table().size(); }",
        "const KernelEntry* find_kernel(int dtype, const tg_cfg& c) {",
        "    KernelEntry key{};",
        "    key.in_bf16 = dtype == TG_F32 ? 0 : 1;",
        "    key.cfg = c;",
        "    key.cfg.split_k = c.kind == TG_KIND_SLICEDK ? c.split_k : 0;   // compiled in only for sliced-K",
        "    const auto& t = table();",
        "    auto it = std::lower_bound(t.begin(), t.end(), key, [](const KernelEntry& a, const KernelEntry& b) {",
        "        return a.in_bf16 != b.in_bf16 ? a.in_bf16 < b.in_bf16 : cfg_less(a.cfg, b.cfg); });",
        "    if (it == t.end() || it->in_bf16 != key.in_bf16 || !cfg_equal(it->cfg, key.cfg)) return nullptr;",
        "    return &*it;",
        "}",
        "bool compiled_alloc(int dtype, const tg_cfg& c, Alloc* out) {",
        "    const KernelEntry* k = find_kernel(dtype, c);",
        "    if (!k) return false;",
        "    *out = Alloc{k->res.vgpr, k->res.agpr, k->res.lds, k->res.scratch};",
        "    return true;",
        "}",
        "}  // namespace tg", ""]
    path = os.path.join(GEN, "registry_gen.cpp")
    with open(path, "w") as f:
        f.write("\n".join(lines))
    return path


C_EXAMPLE_SRC = os.path.join(REPO, "tests", "c_abi", "gemm_from_c.c")
C_EXAMPLE = os.path.join(LIBDIR, "gemm_from_c")
ROCM = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))


def build_c_example(verbose=False):
    """The C program of tests/c_abi, compiled as C99 by the host compiler
    against include/tilegemm.h and linked with the library (found beside the
    executable at run time)."""
    _run(["gcc", "-std=c99", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(ROCM, "include"), "-I", os.path.join(REPO, "include"), C_EXAMPLE_SRC,
          "-o", C_EXAMPLE, "-L", LIBDIR, "-ltilegemm", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
          "-Wl,-rpath,$ORIGIN", "-Wl,-rpath," + os.path.join(ROCM, "lib")], verbose)
    return C_EXAMPLE


def build(force: bool = True, jobs: int | None = None, verbose: bool = False) -> str:
    t0 = time.time()
    os.makedirs(GEN, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    entries = instantiation_set(verbose)
    units = generate_units(entries)
    jobs = jobs or min(16, os.cpu_count() or 8)

    def compile_unit(src):
        obj = src[:-4] + ".o"
        resf = src[:-4] + ".res"
        if force or _stale(obj, [src] + HEADERS) or not os.path.exists(resf):
            err = _run([HIPCC, *HIP_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj],
                       verbose, capture=True)
            with open(resf, "w") as f:
                f.write(err)
        return obj

    host_objs = []

    def compile_host(src, hip):
        obj = os.path.join(BUILD, os.path.basename(src).rsplit(".", 1)[0] + ".o")
        if force or _stale(obj, [src] + HEADERS):
            if hip:
                _run([HIPCC, *HIP_FLAGS, "-c", src, "-o", obj], verbose)
            else:
                _run(["g++", *HOST_FLAGS, "-c", src, "-o", obj], verbose)
        return obj

    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(compile_unit, u) for u in units]
        hfuts = [ex.submit(compile_host, os.path.join(CSRC, "select.cpp"), False),
                 ex.submit(compile_host, os.path.join(CSRC, "api.cpp"), True),
                 ex.submit(compile_host, os.path.join(CSRC, "workspace.cpp"), True),
                 ex.submit(compile_host, os.path.join(CSRC, "tune.cpp"), True),
                 ex.submit(compile_host, os.path.join(CSRC, "tune_kernels.hip"), True),
                 ex.submit(compile_host, os.path.join(CSRC, "splitk_reduce.hip"), True),
                 ex.submit(compile_host, os.path.join(CSRC, "pad.hip"), True),
                 ex.submit(compile_host, os.path.join(CSRC, "rmsnorm.hip"), True),
                 ex.submit(compile_host, os.path.join(CSRC, "noalloc.hip"), True)]
        unit_objs = [f.result() for f in futs]
        host_objs = [f.result() for f in hfuts]

    resources = {}
    for u in units:
        with open(u[:-4] + ".res") as f:
            resources.update(parse_resources(f.read()))
    reg = generate_registry(entries, resources)
    reg_obj = os.path.join(BUILD, "registry_gen.o")
    _run([HIPCC, *HIP_FLAGS, "-c", reg, "-o", reg_obj], verbose)

    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *unit_objs, *host_objs, reg_obj], verbose)
    os.replace(tmp, LIB)
    build_c_example(verbose)
    table = [{"in_bf16": e[0], "kind": e[1], "bm": e[2], "bn": e[3], "bk": e[4], "wgm": e[5], "wgn": e[6],
              "stages": e[7], "k_groups": e[8], **resources.get(tuple(e), {})} for e in entries]
    with open(RES_JSON, "w") as f:
        json.dump(table, f, indent=0)
    if verbose:
        print(f"built {LIB}: {len(entries)} kernels in {time.time() - t0:.1f}s", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--incremental", action="store_true")
    ap.add_argument("-j", type=int, default=None)
    ap.add_argument("-v", action="store_true")
    a = ap.parse_args()
    print(build(force=not a.incremental, jobs=a.j, verbose=a.v))
