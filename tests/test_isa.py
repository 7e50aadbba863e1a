"""The instructions in the library as built: its gfx950 code objects are
taken out of libgemmf16.so and disassembled (this build's own AMD GPU code),
and each kernel's instruction set is checked on the CPU.

- Every dense-contraction kernel keeps its matrix instructions: the
  256x256 LDS-DMA kernels (final, partial, grouped and packed-B forms) the
  fp16 or bfloat16 32x32x16 MFMA of their format, the register-path tiles and
  the decode kernels an MFMA of their format, and the FP8 kernels the
  32x32x64 f8f6f4 MFMA.  An
  optimisation that silently lost the matrix core would fail here (the C500
  log keeps a change only if the matrix instruction is still in the
  generated code: its final-kernel summary and its record template).
- No kernel converts with the round-toward-zero packed instruction, and the
  kernels that write binary16 convert with v_cvt_f16_f32 (round to nearest
  even under the default mode), the output rounding the pages fix.
"""
import collections
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "dense_tiled_gemm_fp16_amd", "libgemmf16.so")
LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"


def _tools():
    need = [shutil.which("objcopy"), shutil.which("c++filt"),
            os.path.join(LLVM, "clang-offload-bundler"), os.path.join(LLVM, "llvm-objdump")]
    return all(t and os.path.exists(t) for t in need)


@pytest.fixture(scope="module")
def kernels():
    """{demangled kernel name: Counter of mnemonics} over every gfx950 code
    object in the library."""
    if not os.path.exists(LIB):
        pytest.fail("libgemmf16.so is not built")
    if not _tools():
        pytest.skip("objcopy / c++filt / ROCm llvm tools not available")
    out = collections.defaultdict(collections.Counter)
    with tempfile.TemporaryDirectory() as tmp:
        fat = os.path.join(tmp, "fatbin")
        # (-O binary writes the section to its own file; objcopy given only an
        # input file would rewrite the library in place.)
        subprocess.run(["objcopy", "-O", "binary", "--only-section=.hip_fatbin", LIB, fat],
                       check=True, capture_output=True)
        data = open(fat, "rb").read()
        starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)] + [len(data)]
        assert len(starts) > 1, "no offload bundle in the library"
        for n, (a, b) in enumerate(zip(starts, starts[1:])):
            part, co = os.path.join(tmp, f"b{n}"), os.path.join(tmp, f"co{n}")
            open(part, "wb").write(data[a:b])
            subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o",
                            f"--input={part}", f"--targets={TARGET}", f"--output={co}"],
                           check=True, capture_output=True)
            dis = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", co], check=True,
                                 capture_output=True, text=True).stdout
            dis = subprocess.run(["c++filt"], input=dis, check=True, capture_output=True,
                                 text=True).stdout
            name = None
            for line in dis.splitlines():
                m = re.match(r"^[0-9a-f]+ <(.*)>:$", line)
                if m:
                    name = m.group(1)
                    continue
                m = re.match(r"^\s+([a-z_][a-z0-9_]*)\b", line)
                if name and m:
                    out[name][m.group(1)] += 1
    return out


def _of(kernels, prefix):
    found = {k: v for k, v in kernels.items() if k.startswith("void gemmf16::" + prefix + "<")}
    assert found, f"no {prefix} in the library"
    return found


def _targs(name):
    """Top-level template arguments of a demangled kernel name."""
    body = name[name.index("<") + 1:name.rindex(">(")]
    args, depth, cur = [], 0, ""
    for ch in body:
        if ch == "," and depth == 0:
            args.append(cur.strip())
            cur = ""
            continue
        depth += (ch == "<") - (ch == ">")
        cur += ch
    return args + [cur.strip()]


def test_dma_tiles_keep_their_mfma(kernels):
    for name, ops in _of(kernels, "gemm_dma_a128_kernel").items():
        dt = int(_targs(name)[4])           # <Cfg<.., ..>, kmajor, partial, grouped, format, packed>
        want = {0: "v_mfma_f32_32x32x16_f16", 1: "v_mfma_f32_32x32x16_bf16"}[dt]
        assert ops[want] >= 16, (name, want, ops[want])
    for name, ops in _of(kernels, "gemm_dma_kernel").items():
        args = _targs(name)                 # <Cfg<..>, kmajor, partial, format, FP8 formats>
        dt, f8 = int(args[3]), int(args[4])
        want = ("v_mfma_f32_32x32x64_f8f6f4" if f8 >= 0 else
                {0: "v_mfma_f32_32x32x16_f16", 1: "v_mfma_f32_32x32x16_bf16"}[dt])
        assert ops[want] >= 4 if f8 >= 0 else ops[want] >= 16, (name, want, ops[want])


def test_register_tiles_keep_their_mfma(kernels):
    for name, ops in _of(kernels, "gemm_tile_kernel").items():
        bf16 = _targs(name)[-1] == "1"
        mf = [k for k in ops if k.startswith("v_mfma_f32_")]
        assert mf and all(k.endswith("_bf16" if bf16 else "_f16") for k in mf), (name, mf)


def test_decode_kernels_keep_their_mfma(kernels):
    found = _of(kernels, "decode_kernel")
    assert len(found) == 24                 # 16, 32, 64 rows of A with N-contiguous B, 16 with
                                            # K-contiguous B; fp16, bfloat16 and the four FP8
                                            # format pairs
    for name, ops in found.items():
        want = {"0": "v_mfma_f32_16x16x32_f16", "1": "v_mfma_f32_16x16x32_bf16"}[_targs(name)[1]]
        assert ops[want] >= 8, (name, want)
        if int(_targs(name)[3]) >= 0:       # FP8 bytes widened by the packed convert
            conv = ops["v_cvt_scalef32_pk_f16_fp8"] + ops["v_cvt_scalef32_pk_f16_bf8"]
            assert conv >= 8, (name, conv)


def test_f8_kernels_keep_their_mfma(kernels):
    found = _of(kernels, "gemm_f8_kernel")
    assert len(found) >= 32                 # 4 format pairs x 8 forms
    for name, ops in found.items():
        assert ops["v_mfma_f32_32x32x64_f8f6f4"] >= 16, name


def test_output_rounding_instructions(kernels):
    for name, ops in kernels.items():
        assert not [k for k in ops if k.startswith("v_cvt_pkrtz")], name
    writers = ["gemm_dma_a128_kernel", "gemm_tile_kernel", "gemm_f8_kernel", "decode_kernel",
               "splitk_reduce_quad", "splitk_reduce_elem", "sk_fixup"]
    for w in writers:
        for name, ops in _of(kernels, w).items():
            args = _targs(name)
            if w == "gemm_dma_a128_kernel" and args[4] == "1":
                continue                    # bfloat16 output
            if w == "decode_kernel" and args[1] == "1":
                continue
            if w in ("splitk_reduce_quad", "splitk_reduce_elem") and args[-1] == "1":
                continue
            if w == "sk_fixup" and args[0] == "1":
                continue
            if w == "gemm_tile_kernel" and args[-1] == "1":
                continue
            partial = (w in ("gemm_dma_a128_kernel", "gemm_tile_kernel", "gemm_f8_kernel")
                       and args[2 if w != "gemm_tile_kernel" else 3] == "true")
            if partial:
                continue                    # fp32 partials, no conversion
            assert ops["v_cvt_f16_f32_e32"] + ops["v_cvt_f16_f32_e64"] > 0, name
