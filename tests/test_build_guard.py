"""The build's register guard (CPU only: kernels are compiled, never run).

A kernel that spills registers or uses scratch memory must fail the build:
the library's MFMA kernels keep accumulators tied to inline-asm MFMAs, and a
spilled accumulator would silently give wrong results.  Each toy kernel here
is compiled for gfx950 with the library's own flags and checked by the same
function the build uses."""
import os
import shutil

import pytest

from tiled_dense_gemm_tile_amd import build as B

pytestmark = pytest.mark.skipif(shutil.which(B.HIPCC) is None and not os.path.exists(B.HIPCC),
                                reason="hipcc not available")

SPILLS = r"""
#include <hip/hip_runtime.h>
// 1024 threads per block leave at most 128 VGPRs; 192 live values do not fit
__global__ void __launch_bounds__(1024) too_many_live(const float *x, float *y, int n) {
    float v[192];
#pragma unroll
    for (int i = 0; i < 192; ++i) v[i] = x[threadIdx.x + i * n];
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < 192; ++i) s = s * v[(i + r) % 192] + v[191 - i];
    y[threadIdx.x] = s;
}
"""

SCRATCH = r"""
#include <hip/hip_runtime.h>
// a private array indexed at run time lives in scratch memory
__global__ void indexed_array(const int *idx, float *y) {
    float a[64];
    for (int i = 0; i < 64; ++i) a[i] = (float)(i * threadIdx.x);
    y[threadIdx.x] = a[idx[threadIdx.x] & 63];
}
"""

FITS = r"""
#include <hip/hip_runtime.h>
__global__ void fits(const float *x, float *y) { y[threadIdx.x] = 2.0f * x[threadIdx.x]; }
"""


def _compile(tmp_path, name, text):
    src = tmp_path / (name + ".hip")
    src.write_text(text)
    return B.compile_unit(str(src), str(tmp_path / (name + ".o")))


@pytest.mark.parametrize("name,text", [("spills", SPILLS), ("scratch", SCRATCH)])
def test_guard_rejects(tmp_path, name, text):
    with pytest.raises(B.ResourceError):
        _compile(tmp_path, name, text)


def test_guard_accepts_and_reports(tmp_path):
    ks = _compile(tmp_path, "fits", FITS)
    assert len(ks) == 1 and ks[0]["ScratchSize"] == 0 and ks[0]["VGPRs"] > 0


def test_remark_parser():
    text = ("x.hip:3:1: remark: Function Name: _Z1kv [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:3:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:3:1: remark:     AGPRs: 256 [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:3:1: remark:     ScratchSize [bytes/lane]: 144 [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:3:1: remark:     VGPRs Spill: 35 [-Rpass-analysis=kernel-resource-usage]\n")
    ks = B.resource_usage(text)
    assert ks == [{"name": "_Z1kv", "VGPRs": 256, "AGPRs": 256, "ScratchSize": 144, "VGPRs Spill": 35}]
    assert B.offenders(ks) == ks
