"""Checks on the gfx950 ISA the library's sources compile to (hipcc runs on the
CPU; nothing is launched).  They guard assumptions the kernels make about code
generation that no numerical test would catch reliably."""
import importlib.util
import os
import re

import pytest

# the build script itself, not the package (whose import loads the built library)
_spec = importlib.util.spec_from_file_location(
    "_sq_hip_build", os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                                  "int8_quantization_amd", "build.py"))
B = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(B)


def kernels(asm):
    """{kernel symbol: list of its instruction lines}, in order."""
    out, name = {}, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            name = m.group(1)
            out[name] = []
            continue
        if name is not None:
            if line.strip().startswith("s_endpgm"):
                out[name].append(line)
                name = None
            else:
                out[name].append(line)
    return out


@pytest.fixture(scope="module")
def gemm_asm():
    return B.device_asm("gemm.hip")


@pytest.fixture(scope="module")
def stream_asm():
    return B.device_asm("quant_stream.hip")


def _check_m0(ks):
    for name, lines in ks.items():
        inside, n_dma = False, 0
        for l in lines:
            t = l.strip()
            if t.startswith(";;#ASMSTART"):
                inside = True
                prev = None
                continue
            if t.startswith(";;#ASMEND"):
                inside = False
                continue
            if not t or t.startswith(";") or t.startswith("."):
                continue
            ops = t.split(None, 1)
            writes_m0 = len(ops) > 1 and ops[1].split(",")[0].strip() == "m0"
            is_lds_dma = " lds" in t and t.startswith("buffer_load")
            if not inside:
                assert not writes_m0, f"{name}: compiler writes M0: {t}"
                assert not is_lds_dma, f"{name}: LDS DMA outside the asm helper: {t}"
            elif is_lds_dma:
                n_dma += 1
        assert n_dma > 0, name


def test_gemm_m0_only_written_by_the_dma_asm(gemm_asm):
    """The tile kernel's operand DMA is issued from inline asm that loads M0
    itself; nothing the compiler emits may depend on M0 surviving it, so M0 must
    be written (and buffer ... lds issued) only inside those asm blocks."""
    ks = {k: v for k, v in kernels(gemm_asm).items() if "gemm_i8_kernel" in k}
    assert len(ks) >= 6
    _check_m0(ks)


def test_stream_quantizer_m0_only_written_by_the_dma_asm(stream_asm):
    """The same for the streaming quantizer's row DMA."""
    ks = {k: v for k, v in kernels(stream_asm).items() if "quant_stream_kernel" in k}
    assert len(ks) >= 10
    _check_m0(ks)


def test_stream_quantizer_stores_every_step_unconditionally(stream_asm):
    """Its vmcnt waits count CH code stores and L DMA loads per wave per step, so no
    branch may skip them: between the last branch target before the step's code
    stores and the DMA that follows them there is no conditional branch, and the
    kernel uses no scratch (spill loads and stores would be extra vector-memory
    instructions in the loop)."""
    for name, lines in kernels(stream_asm).items():
        if "quant_stream_kernel" not in name:
            continue
        ch = int(re.search(r"quant_stream_kernelILi\d+ELi(\d)E", name).group(1))
        body = [l.strip() for l in lines if l.strip() and not l.strip().startswith(";")]
        stores = [i for i, l in enumerate(body) if l.startswith("buffer_store_dword ")]
        assert len(stores) == ch, (name, len(stores))
        dma = [i for i, l in enumerate(body) if l.startswith("buffer_load_dwordx4") and " lds" in l]
        after = [i for i in dma if i > stores[-1]]
        assert after, name
        block_start = max(i for i, l in enumerate(body[:stores[0]]) if l.endswith(":") or l.startswith("s_cbranch"))
        region = body[block_start + 1:after[0]]
        assert not any(l.startswith("s_cbranch") for l in region), name
        assert not any(l.endswith(":") for l in region), name
        assert "scratch_" not in "\n".join(body), name


def test_gemm_kernels_do_not_spill(gemm_asm):
    """Scratch use in the tile kernels means register spills in the MFMA loop."""
    meta = re.findall(r"\.name:\s+(_Z\w+gemm_i8_kernel\w*)\s*\n(?:.*\n)*?\s+\.private_segment_fixed_size:\s+(\d+)",
                      gemm_asm)
    sizes = dict(meta)
    assert len(sizes) >= 6
    for name, size in sizes.items():
        assert int(size) == 0, f"{name} uses {size} bytes of scratch"


@pytest.mark.parametrize("src", B.SOURCES)
def test_no_packed_fp32_instructions(src):
    """The library is built with packed fp32 disabled; no v_pk_{add,mul,fma}_f32 may appear."""
    asm = B.device_asm(src)
    bad = re.findall(r"^\s*v_pk_(?:add|mul|fma)_f32\b.*$", asm, re.M)
    assert not bad, bad[:3]
