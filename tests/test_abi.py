"""CPU checks of the C ABI: the library loads without a GPU, exports every
entry point include/sharq.h declares, and rejects invalid arguments with the
documented status code before making any HIP call (so nothing here touches a
device).  Also records the sparse-MFMA decision as a compile probe."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sharq.h")
LIB = os.path.join(ROOT, "sparsity_prep_amd", "libsharq.so")

OK, NULL, SHAPE, NM, DTYPE, ALIGN, WORKSPACE, UNSUPPORTED = 0, 1, 2, 3, 4, 5, 6, 7
BF16, F16, F32 = 1, 0, 2
MX, NV, SP = 0, 1, 2


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} not built (python -m sparsity_prep_amd.build)")
    import sparsity_prep_amd
    return sparsity_prep_amd.lib()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"SHARQ_API[^;(]*?\b(sharq_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_symbols()
    for n in ("sharq_prepare", "sharq_prepare_swiglu", "sharq_linear", "sharq_quantize_weight",
              "sharq_linear_swiglu", "sharq_quantize_weight_gate_up"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for name in declared_symbols():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (\w+)", out))
    assert set(declared_symbols()) == {s for s in exported if s.startswith("sharq_")}


def test_version_and_strings(L):
    assert L.sharq_abi_version() == 7
    for code in range(9):
        assert L.sharq_status_string(code)
    assert L.sharq_status_string(99) == b"unknown status"


def test_last_hip_error_untouched_by_validation(L, monkeypatch):
    """Calls rejected before any HIP call leave the last HIP error at its
    previous value (no HIP call has run in this process), check mode or not."""
    assert L.sharq_last_hip_error() == 0
    for debug in ("0", "1"):
        monkeypatch.setenv("SHARQ_DEBUG", debug)
        assert prep(L, x=None) == NULL
        assert lin(L, bc=None) == NULL
        assert L.sharq_last_hip_error() == 0


FAKE = ctypes.c_void_p(0x10000)       # never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p(0x10002)


def prep(L, x=FAKE, dt=BF16, T=4, K=256, ldx=None, norm=1, gamma=FAKE, beta=None, n=2, m=4,
         fmt=MX, mask=FAKE, bc=FAKE, bs=FAKE, rc=FAKE, rs=FAKE, G=None, ws=None, wsb=0):
    return L.sharq_prepare(x, dt, T, K, K if ldx is None else ldx, norm, gamma, beta, 1e-5, n, m,
                           fmt, mask, bc, bs, rc, rs, G, ws, wsb, None)


def test_prepare_validation(L):
    assert prep(L, fmt=3) == UNSUPPORTED
    assert prep(L, dt=F32) == DTYPE
    assert prep(L, norm=7) == UNSUPPORTED
    assert prep(L, K=100) == SHAPE                # not a multiple of 32
    assert prep(L, K=256, ldx=128) == SHAPE
    assert prep(L, T=-1) == SHAPE
    assert prep(L, T=2**31) == SHAPE               # rows beyond the one-workgroup-per-row grid
    assert prep(L, n=5, m=4) == NM
    assert prep(L, n=-1, m=4) == NM
    assert prep(L, n=2, m=3) == NM
    assert prep(L, n=2, m=32) == NM
    assert prep(L, K=40, fmt=NV, G=FAKE) == SHAPE  # not a multiple of 16
    assert prep(L, x=None) == NULL
    assert prep(L, gamma=None) == NULL
    assert prep(L, norm=0, gamma=None, x=MISALIGNED) == ALIGN
    assert prep(L, ldx=256 + 4) == ALIGN
    assert prep(L, fmt=NV) == NULL                 # NVFP4 needs the tensor-scale output
    assert prep(L, fmt=NV, G=FAKE) == WORKSPACE
    assert prep(L, fmt=NV, G=FAKE, ws=FAKE, wsb=1) == WORKSPACE
    assert prep(L, T=0, x=None) == OK              # empty tensor is a no-op, no HIP call


def test_prepare_sp24_validation(L):
    # the compressed backbone exists for the 2:4 mask only
    assert prep(L, fmt=SP, G=FAKE, n=1, m=4) == NM
    assert prep(L, fmt=SP, G=FAKE, n=4, m=8) == NM
    # whole K tiles and 32-bit code offsets (T*K/2 < 2^32)
    assert prep(L, fmt=SP, G=FAKE, K=160) == SHAPE
    assert prep(L, fmt=SP, G=FAKE, T=2**24, K=512) == SHAPE
    assert prep(L, fmt=SP, G=FAKE, T=2**24 - 1, K=512) == WORKSPACE  # just under: shape accepted
    assert prep(L, fmt=SP) == NULL                 # NVFP4 tensor scale
    assert prep(L, fmt=SP, G=FAKE) == WORKSPACE
    assert swiglu(L, fmt=SP, G=FAKE, n=1) == NM
    assert swiglu(L, fmt=SP, G=FAKE, K=160) == SHAPE
    assert swiglu(L, fmt=SP) == NULL
    assert swiglu(L, fmt=SP, G=FAKE) == WORKSPACE
    assert lin(L, fmt=SP) == NULL                  # both tensor scales
    assert lin(L, fmt=SP, xg=FAKE, wg=FAKE, y=MISALIGNED) == ALIGN
    assert L.sharq_prepare_workspace_size(100, 256, SP) == L.sharq_prepare_workspace_size(100, 256, NV)
    assert L.sharq_linear_workspace_size(64, 14336, 4096, 1, SP) == 0


def swiglu(L, gu=FAKE, T=4, K=256, ld=None, n=2, m=4, fmt=MX, bc=FAKE, G=None, ws=None, wsb=0):
    return L.sharq_prepare_swiglu(gu, T, K, 2 * K if ld is None else ld, n, m, fmt, FAKE, bc, FAKE, FAKE,
                                  FAKE, G, ws, wsb, None)


def test_prepare_swiglu_validation(L):
    L.sharq_prepare_swiglu.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int32, ctypes.c_int32, ctypes.c_int32] + \
                                      [ctypes.c_void_p] * 7 + [ctypes.c_size_t, ctypes.c_void_p]
    assert swiglu(L, fmt=4) == UNSUPPORTED
    assert swiglu(L, ld=300) == SHAPE              # ld < 2K
    assert swiglu(L, K=100) == SHAPE
    assert swiglu(L, T=-1) == SHAPE
    assert swiglu(L, T=2**31) == SHAPE
    assert swiglu(L, n=5) == NM
    assert swiglu(L, gu=None) == NULL
    assert swiglu(L, bc=None) == NULL
    assert swiglu(L, gu=MISALIGNED) == ALIGN
    assert swiglu(L, ld=2 * 256 + 2) == ALIGN      # rows not 16-byte aligned
    assert swiglu(L, fmt=NV) == NULL
    assert swiglu(L, fmt=NV, G=FAKE) == WORKSPACE
    assert swiglu(L, T=0, gu=None) == OK


def test_quantize_weight_validation(L):
    def q(w=FAKE, dt=BF16, E=1, nout=16, K=256, ldw=None, fmt=MX, codes=FAKE, G=None, ws=None, wsb=0):
        return L.sharq_quantize_weight(w, dt, E, nout, K, K if ldw is None else ldw, fmt, codes, FAKE, G,
                                       ws, wsb, None)
    assert q(fmt=9) == UNSUPPORTED
    assert q(dt=F32) == DTYPE
    assert q(E=0) == SHAPE
    assert q(K=40) == SHAPE
    assert q(ldw=128) == SHAPE                    # row stride shorter than a row
    assert q(w=None) == NULL
    assert q(fmt=NV) == NULL
    assert q(fmt=NV, G=FAKE) == WORKSPACE
    assert q(w=MISALIGNED) == ALIGN
    assert q(ldw=256 + 4) == ALIGN                # rows not 16-byte aligned
    assert q(w=None, nout=0) == OK
    assert q(fmt=NV, G=FAKE, ws=MISALIGNED, wsb=1 << 20) == ALIGN


def test_quantize_weight_gate_up_validation(L):
    def q(nout=128, K=256, fmt=MX, codes=FAKE, w=FAKE):
        return L.sharq_quantize_weight_gate_up(w, BF16, 1, nout, K, K, fmt, codes, FAKE, None, None, 0, None)
    assert q(nout=96) == SHAPE                    # gate/up pairs of 32-row groups: nout % 64
    assert q(fmt=9) == UNSUPPORTED
    assert q(w=None) == NULL
    assert q(codes=MISALIGNED) == ALIGN
    assert q(nout=0, w=None) == OK


def lsw(L, T=4, K=256, E=1, nout=512, offs=None, ridx=None, rows=None, n=2, m=4, mask=FAKE, obc=FAKE, obs=FAKE,
        orc=FAKE, ors=FAKE, y=None, ldy=0, bc=FAKE):
    return L.sharq_linear_swiglu(bc, FAKE, FAKE, FAKE, T, K, FAKE, FAKE, E, nout, offs, ridx,
                                 T if rows is None else rows, n, m, mask, obc, obs, orc, ors, y, ldy, None)


def test_linear_swiglu_validation(L):
    assert lsw(L, K=160) == SHAPE                 # K not a multiple of 128
    assert lsw(L, nout=320) == SHAPE              # hidden width nout/2 not whole 128-element tiles
    assert lsw(L, rows=7) == SHAPE                # dense rows must equal T without a gather
    assert lsw(L, n=5) == NM
    assert lsw(L, m=3) == NM
    assert lsw(L, m=8) == UNSUPPORTED             # mask groups wider than a lane's four
    assert lsw(L, E=4) == NULL                    # grouped needs offsets
    assert lsw(L, y=FAKE, ldy=100) == SHAPE       # product output narrower than nout
    assert lsw(L, bc=None) == NULL
    assert lsw(L, obs=None) == NULL
    assert lsw(L, mask=None, obc=MISALIGNED) == ALIGN
    assert lsw(L, mask=MISALIGNED) == ALIGN
    assert lsw(L, y=MISALIGNED, ldy=512) == ALIGN
    assert lsw(L, T=0, rows=0, bc=None) == OK
    assert lsw(L, nout=0, bc=None) == OK
    assert lsw(L, T=1 << 24, K=256) == SHAPE      # T*K/2 at the 2 GiB operand limit


def lin(L, T=4, K=256, fmt=MX, E=1, nout=64, offs=None, ridx=None, rows=None, y=FAKE, ydt=F32, ldy=None,
        bc=FAKE, xg=None, wg=None, ws=None, wsb=0):
    return L.sharq_linear(bc, FAKE, FAKE, FAKE, xg, T, K, fmt, FAKE, FAKE, wg, E, nout, offs, ridx,
                          T if rows is None else rows, y, ydt, nout if ldy is None else ldy, ws, wsb, None)


def test_linear_validation(L):
    assert lin(L, fmt=5) == UNSUPPORTED
    assert lin(L, ydt=7) == DTYPE                 # output must be F32, BF16 or F16
    assert lin(L, K=160) == SHAPE                 # not a multiple of 128
    assert lin(L, ldy=10) == SHAPE
    assert lin(L, rows=7) == SHAPE                # dense rows must equal T without a gather
    assert lin(L, E=4) == NULL                    # grouped needs offsets
    assert lin(L, bc=None) == NULL
    assert lin(L, fmt=NV) == NULL                 # NVFP4 needs both tensor scales
    assert lin(L, y=MISALIGNED) == ALIGN          # 2 bytes past a boundary: not float-aligned
    assert lin(L, y=ctypes.c_void_p(0x10001), ydt=BF16) == ALIGN
    assert lin(L, rows=0, T=0) == OK
    assert lin(L, T=64, K=14336, nout=4096) == WORKSPACE   # a K-split product needs its workspace
    need = L.sharq_linear_workspace_size(64, 14336, 4096, 1, MX)
    assert lin(L, T=64, K=14336, nout=4096, ws=ctypes.c_void_p(0x10004), wsb=need) == ALIGN
    assert lin(L, T=0, rows=3, ridx=FAKE) == SHAPE


def test_workspace_sizes(L):
    assert L.sharq_prepare_workspace_size(100, 256, MX) == 0
    assert L.sharq_prepare_workspace_size(100, 256, NV) >= 100 * 12
    assert L.sharq_quantize_weight_workspace_size(2, 64, 256, NV) >= 128 * 4
    assert L.sharq_linear_workspace_size(64, 256, 64, 1, MX) == 0
    # decode batch with a long K: partial products of a K split (S * rows * nout floats)
    need = L.sharq_linear_workspace_size(64, 14336, 4096, 1, MX)
    assert need > 0 and need % (64 * 4096 * 4) == 0 and need // (64 * 4096 * 4) in (2, 4, 8)
    assert L.sharq_linear_workspace_size(16, 14336, 4096, 1, MX) == 0     # 16 rows and fewer: no split
    assert L.sharq_linear_workspace_size(64, 14336, 4096, 1, NV) == 0
    assert L.sharq_linear_workspace_size(65, 14336, 4096, 1, MX) == 0
    assert L.sharq_linear_workspace_size(64, 14336, 4096, 8, MX) == 0     # grouped products


HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _compiles(tmp_path, body):
    src = tmp_path / "probe.hip"
    src.write_text("#include <hip/hip_runtime.h>\n"
                   "typedef int v4i __attribute__((ext_vector_type(4)));\n"
                   "typedef int v8i __attribute__((ext_vector_type(8)));\n"
                   "typedef float v4f __attribute__((ext_vector_type(4)));\n" + body)
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "--offload-device-only", "-c", str(src),
                        "-o", str(tmp_path / "p.o")], capture_output=True, text=True)
    return r.returncode == 0


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_gfx950_has_block_scaled_fp4_mfma_but_no_sparse_fp4(tmp_path):
    """The backbone runs dense on its zero-filled form because gfx950's sparse
    matrix instructions take fp8/bf8/f16/bf16 operands only and no block
    scale; the block-scaled FP4 instruction is dense."""
    assert _compiles(tmp_path, "__global__ void k(v8i*a,v8i*b,v4f*c){int i=threadIdx.x;"
                     "c[i]=__builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[i],b[i],c[i],4,4,0,127,0,127);}")
    assert _compiles(tmp_path, "__global__ void k(v4i*a,v8i*b,v4f*c,int*x){int i=threadIdx.x;"
                     "c[i]=__builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(a[i],b[i],c[i],x[i],0,0);}")
    for name in ("smfmac_f32_16x16x128_fp4_fp4", "smfmac_f32_16x16x256_fp4_fp4",
                 "smfmac_scale_f32_16x16x128_f8f6f4", "smfmac_f32_16x16x128_f8f6f4"):
        assert not _compiles(tmp_path, "__global__ void k(v4i*a,v8i*b,v4f*c,int*x){int i=threadIdx.x;"
                             f"c[i]=__builtin_amdgcn_{name}(a[i],b[i],c[i],x[i],0,0);}}"), name


LLVM_MC = "/opt/rocm/llvm/bin/llvm-mc"


def _assembles(tmp_path, line):
    src = tmp_path / "probe.s"
    src.write_text(line + "\n")
    r = subprocess.run([LLVM_MC, "-arch=amdgcn", "-mcpu=gfx950", str(src), "-o", os.devnull],
                       capture_output=True, text=True)
    return r.returncode == 0


@pytest.mark.skipif(not os.path.exists(LLVM_MC), reason="llvm-mc not available")
def test_gfx950_assembler_sparse_matrix_instructions(tmp_path):
    """The gfx950 assembler's sparse matrix instructions: f16, bf16, fp8 and
    int8 operands with an index register and no scale operands; no FP4
    (f8f6f4) or block-scaled sparse form exists, while the dense
    block-scaled FP4 instruction does."""
    ops = "v[0:15], v[16:19], v[20:27], v28"
    for mnemonic in ("v_smfmac_f32_32x32x32_f16", "v_smfmac_f32_32x32x32_bf16",
                     "v_smfmac_f32_32x32x64_fp8_fp8", "v_smfmac_i32_32x32x64_i8"):
        assert _assembles(tmp_path, f"{mnemonic} {ops}"), mnemonic
    assert _assembles(tmp_path, "v_mfma_scale_f32_32x32x64_f8f6f4 v[0:15], v[16:23], v[24:31], v[0:15], v32, v33")
    for line in ("v_smfmac_f32_32x32x128_fp4_fp4 " + ops, "v_smfmac_f32_32x32x64_f8f6f4 " + ops,
                 "v_smfmac_scale_f32_32x32x64_f8f6f4 " + ops + ", v29, v30",
                 "v_smfmac_f32_16x16x128_fp4 v[0:3], v[16:19], v[20:27], v28"):
        assert not _assembles(tmp_path, line), line


def test_prepare_noalloc_validation(L):
    def na(T=4, K=256, fmt=MX, x=FAKE, G=None, norm=1):
        return L.sharq_prepare_noalloc(x, BF16, T, K, K, norm, FAKE, None, 1e-5, 2, 4, fmt, FAKE, FAKE, FAKE,
                                       FAKE, FAKE, G, None)
    assert na(fmt=3) == UNSUPPORTED
    assert na(K=100) == SHAPE
    assert na(x=None) == NULL
    assert na(fmt=NV) == NULL
    assert na(x=MISALIGNED) == ALIGN
    # NVFP4 rows beyond the built-in scratch are refused before any HIP call
    assert na(T=65536 + 1, fmt=NV, G=FAKE) == WORKSPACE
    assert na(T=0, x=None) == OK
