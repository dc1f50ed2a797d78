"""The measurement kernels of include/msa_peaks.h run through the C ABI on a
small buffer and a short MFMA loop (they return no result to compare: the
benchmark times them)."""
import pytest
import torch

import block_sparse_attention_04_amd as msa

pytestmark = pytest.mark.gpu


def test_peaks_kernels_run():
    buf = torch.ones(1 << 20, dtype=torch.int32, device="cuda")
    sink = torch.zeros(256, dtype=torch.float32, device="cuda")
    msa.msa_peaks_stream_read(buf, sink)
    msa.msa_peaks_stream_read(buf[:16], sink)        # 64 bytes: fewer words than threads
    msa.msa_peaks_mfma(sink, 4, 10)
    for unroll in (1, 2, 4, 8, 16):
        for width in (4, 8, 16):
            for nt in (0, 1):
                msa.msa_peaks_stream_read_variant(buf, sink, unroll, width, nt, 2)
    msa.msa_peaks_stream_read_variant(buf[:16], sink, 16, 16, 1, 64)   # fewer words than threads
    torch.cuda.synchronize()
    with pytest.raises(msa.MsaError):
        msa.msa_peaks_stream_read(buf[:3], sink)     # 12 bytes: not a multiple of 16
    with pytest.raises(msa.MsaError):
        msa.msa_peaks_stream_read_variant(buf, sink, 3, 16, 0, 2)      # unroll not in the set
