"""Build libhkg.so (gfx950) in-tree from csrc/ with hipcc.

Every kernel file is compiled with the compiler's kernel-resource-usage
report; the build parses it, refuses any kernel with scratch use or VGPR
spills, and compiles the figures into the library (hkg_plan_t reports them).
"""
import concurrent.futures
import json
import os
import re
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libhkg.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

KERNEL_SOURCES = ["hkg_tile.hip", "hkg_tile_mx.hip", "hkg_skinny.hip", "hkg_generic.hip", "hkg_noalloc.hip"]
HOST_SOURCES = ["hkg_resources.cpp", "hkg_abi.cpp"]

# -packed-fp32-ops: no v_pk_*_f32 from the compiler (kept off on this target).
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function",
          "-I" + INCLUDE, "-I" + CSRC, "-I" + BUILD]



def tile_configs(mx=False, grouped=False, mx4=False):
    """(BM, BN, BK, STAGES, WM, WN, SCHED) per tile variant (bf16; MXFP8 with mx=True;
    MXFP4 with mx4=True; grouped with grouped=True), from hkg_tile_configs.h."""
    text = open(os.path.join(CSRC, "hkg_tile_configs.h")).read()
    start = text.index("#define HKG_MX_TILE_CONFIGS(X)" if mx else "#define HKG_MX4_TILE_CONFIGS(X)" if mx4 else
                       "#define HKG_GROUPED_CONFIGS(X)" if grouped else "#define HKG_TILE_CONFIGS(X)")
    body = text[start:]
    end = body.find("#define", 10)
    body = body if end < 0 else body[:end]
    return [tuple(int(v) for v in m) for m in re.findall(
        r"X\((\d+),\s*(\d+),\s*(\d+),\s*(\d+),\s*(\d+),\s*(\d+),\s*(\d+)\)", body)]


TILE_VARIANTS = tile_configs()
MX_TILE_VARIANTS = tile_configs(mx=True)
MX4_TILE_VARIANTS = tile_configs(mx4=True)
GROUPED_VARIANTS = tile_configs(grouped=True)
def skinny_configs(mx=False, mx4=False):
    """(MB, NB, WK, U, CP, AL) per skinny variant (MXFP8 with mx=True, MXFP4 with mx4=True), from
    hkg_skinny_configs.h."""
    text = open(os.path.join(CSRC, "hkg_skinny_configs.h")).read()
    body = text[text.index("#define HKG_MX_SKINNY_CONFIGS(X)" if mx else "#define HKG_MX4_SKINNY_CONFIGS(X)" if mx4
                           else "#define HKG_SKINNY_CONFIGS(X)"):]
    end = body.find("#define", 10)
    body = body if end < 0 else body[:end]
    fields = r"X\(" + r",\s*".join([r"(\d+)"] * 6) + r"\)"
    return [tuple(int(v) for v in m) for m in re.findall(fields, body)]


SKINNY_VARIANTS = skinny_configs()
MX_SKINNY_VARIANTS = skinny_configs(mx=True)
MX4_SKINNY_VARIANTS = skinny_configs(mx4=True)


class BuildError(RuntimeError):
    pass


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    if p.returncode != 0:
        raise BuildError("command failed (%d): %s\n%s%s" % (p.returncode, " ".join(cmd), p.stdout, p.stderr))
    return p.stderr


def _parse_resources(text):
    """kernel mangled name -> dict of the resource-usage remark fields."""
    out = {}
    cur = None
    for ln in text.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", ln)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z][A-Za-z /\[\]]*?)(?: \[[A-Za-z/]+\])?: (\S+) \[-Rpass", ln)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    return out


def _compile(src, want_remarks):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    if want_remarks:
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    err = _run(cmd)
    return obj, (_parse_resources(err) if want_remarks else {})


def _entry(name, r):
    def g(key):
        v = r.get(key)
        try:
            return int(v)
        except (TypeError, ValueError):
            return -1
    return dict(name=name, vgprs=g("VGPRs"), agprs=g("AGPRs"), sgprs=g("TotalSGPRs"),
                scratch=g("ScratchSize"), lds=g("LDS Size"),
                vgpr_spill=g("VGPRs Spill"), sgpr_spill=g("SGPRs Spill"),
                occupancy=g("Occupancy"))


def _table(resources):
    tile = [None] * len(TILE_VARIANTS)
    mx_tile = [None] * len(MX_TILE_VARIANTS)
    mx4_tile = [None] * len(MX4_TILE_VARIANTS)
    grouped = [None] * len(GROUPED_VARIANTS)
    skinny = [None] * len(SKINNY_VARIANTS)
    mx_skinny = [None] * len(MX_SKINNY_VARIANTS)
    mx4_skinny = [None] * len(MX4_SKINNY_VARIANTS)
    generic = None
    for mangled, r in resources.items():
        # The table holds the plain instantiations (no fused epilogue); the
        # gate below checks every kernel, epilogue instantiations included.
        m = re.search(r"tile_kernelILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)"
                      r"ELb([01])ELb([01])ELb([01])E", mangled)
        if m:
            key = tuple(int(g) for g in m.groups()[:7])
            plain, mx, grp = m.group(8) == "0", m.group(9) == "1", m.group(10) == "1"
            if plain and grp and key in GROUPED_VARIANTS:
                grouped[GROUPED_VARIANTS.index(key)] = _entry("grouped_%dx%dx%d_s%d_w%dx%d_p%d" % key, r)
            elif plain and not mx and not grp and key in TILE_VARIANTS:
                tile[TILE_VARIANTS.index(key)] = _entry("tile_%dx%dx%d_s%d_w%dx%d_p%d" % key, r)
            elif plain and mx and key in MX_TILE_VARIANTS:
                mx_tile[MX_TILE_VARIANTS.index(key)] = _entry("mxtile_%dx%dx%d_s%d_w%dx%d_p%d" % key, r)
            elif plain and mx and key in MX4_TILE_VARIANTS:
                mx4_tile[MX4_TILE_VARIANTS.index(key)] = _entry("mx4tile_%dx%dx%d_s%d_w%dx%d_p%d" % key, r)
            continue
        m = re.search(r"skinny_kernelILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELb([01])ELb([01])ELb([01])E"
                      r"Lb([01])ELb([01])E", mangled)
        if m:
            key = tuple(int(g) for g in m.groups()[:5])
            al, plain, mx = int(m.group(6)), m.group(7) == "0", m.group(8) == "1"
            nat, f4 = m.group(9) == "1", m.group(10) == "1"
            if plain and f4 and key + (al,) in MX4_SKINNY_VARIANTS:
                mx4_skinny[MX4_SKINNY_VARIANTS.index(key + (al,))] = _entry(
                    "mx4skinny_m%d_n%d_w%d_u%d_c%d" % ((16 * key[0], 16 * key[1]) + key[2:]) + ("_lds" if al else ""),
                    r)
                continue
            if f4 or (mx and nat):
                continue
            label = (16 * key[0], 16 * key[1]) + key[2:]
            if plain and not mx and key + (al,) in SKINNY_VARIANTS:
                skinny[SKINNY_VARIANTS.index(key + (al,))] = _entry(
                    "skinny_m%d_n%d_w%d_u%d_c%d" % label + ("_lds" if al else ""), r)
            elif plain and mx and key + (al,) in MX_SKINNY_VARIANTS:
                mx_skinny[MX_SKINNY_VARIANTS.index(key + (al,))] = _entry(
                    "mxskinny_m%d_n%d_w%d_u%d_c%d" % label + ("_lds" if al else ""), r)
            continue
        if "generic_kernel" in mangled:
            generic = _entry("generic", r)
        elif "zero_kernel" in mangled:
            pass
    missing = [i for i, e in enumerate(tile) if e is None] + \
              [100 + i for i, e in enumerate(skinny) if e is None] + \
              [200 + i for i, e in enumerate(mx_tile) if e is None] + \
              [300 + i for i, e in enumerate(grouped) if e is None] + \
              [400 + i for i, e in enumerate(mx_skinny) if e is None] + \
              [500 + i for i, e in enumerate(mx4_tile) if e is None] + \
              [600 + i for i, e in enumerate(mx4_skinny) if e is None] + ([-1] if generic is None else [])
    if missing:
        raise BuildError("resource report missing kernels: %s" % missing)
    return tile, mx_tile, grouped, skinny, mx_skinny, mx4_tile, mx4_skinny, generic


def _gate(entries):
    # Refused: any scratch use, any VGPR spill (memory traffic that the
    # hand-placed vmcnt waits do not account for).  SGPR spills with no
    # scratch live in VGPR lanes (v_writelane / v_readlane, no memory access)
    # and are allowed.
    bad = [e for e in entries if e["scratch"] != 0 or e["vgpr_spill"] > 0]
    if bad:
        raise BuildError("kernels use scratch / spill registers (refused): %s" % bad)


def _write_inc(tile, mx_tile, grouped, skinny, mx_skinny, mx4_tile, mx4_skinny, generic):
    def row(e):
        return '{"%s", %d, %d, %d, %d, %d}' % (e["name"], e["vgprs"], e["agprs"], e["sgprs"], e["scratch"], e["lds"])
    text = "// generated by tile_level_dense_amd/build.py -- do not edit\n"
    text += "const KernelResources kTileResources[] = {\n    " + ",\n    ".join(row(e) for e in tile) + "};\n"
    text += "const KernelResources kMxTileResources[] = {\n    " + ",\n    ".join(row(e) for e in mx_tile) + "};\n"
    text += "const KernelResources kGroupedResources[] = {\n    " + ",\n    ".join(row(e) for e in grouped) + "};\n"
    text += "const KernelResources kSkinnyResources[] = {\n    " + ",\n    ".join(row(e) for e in skinny) + "};\n"
    text += "const KernelResources kMxSkinnyResources[] = {\n    " + ",\n    ".join(row(e) for e in mx_skinny) + "};\n"
    text += "const KernelResources kMx4TileResources[] = {\n    " + ",\n    ".join(row(e) for e in mx4_tile) + "};\n"
    text += "const KernelResources kMx4SkinnyResources[] = {\n    " + ",\n    ".join(row(e) for e in mx4_skinny) + "};\n"
    text += "const KernelResources kGenericResources = " + row(generic) + ";\n"
    path = os.path.join(BUILD, "hkg_resources.inc")
    with open(path, "w") as f:
        f.write(text)
    with open(os.path.join(BUILD, "kernel_resources.json"), "w") as f:
        json.dump(dict(tile=tile, mx_tile=mx_tile, grouped=grouped, skinny=skinny, mx_skinny=mx_skinny,
                       mx4_tile=mx4_tile, mx4_skinny=mx4_skinny, generic=generic), f, indent=1)


def build(verbose=False):
    """Compile every kernel for gfx950, gate resources, link libhkg.so."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        futs = [ex.submit(_compile, s, True) for s in KERNEL_SOURCES]
        results = [f.result() for f in futs]
    objs = [o for o, _ in results]
    res = {}
    for _, r in results:
        res.update(r)
    tile, mx_tile, grouped, skinny, mx_skinny, mx4_tile, mx4_skinny, generic = _table(res)
    _gate([_entry(name, r) for name, r in res.items()])
    _write_inc(tile, mx_tile, grouped, skinny, mx_skinny, mx4_tile, mx4_skinny, generic)
    with concurrent.futures.ThreadPoolExecutor(max_workers=2) as ex:
        objs += [f.result()[0] for f in [ex.submit(_compile, s, False) for s in HOST_SOURCES]]
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs)
    os.replace(tmp, LIB)
    if verbose:
        for e in tile + mx_tile + grouped + skinny + mx_skinny + mx4_tile + mx4_skinny + [generic]:
            print("%-18s vgpr %3d agpr %3d sgpr %3d scratch %d lds %6d occ %d" % (
                e["name"], e["vgprs"], e["agprs"], e["sgprs"], e["scratch"], e["lds"], e["occupancy"]))
    return LIB


if __name__ == "__main__":
    build(verbose=True)
