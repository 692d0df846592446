"""Host-side checks of the measurement tooling (no GPU): the rocprofv3 summary's
kernel classes, and bench.py's single-GPU contract."""
import os
import subprocess
import sys

from dependent_position_encoding_fwd_amd import profsum

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_profsum_classifies_decode_variants():
    c = profsum.classify
    assert c("void path::decode_chunk_kernel<path::bf16_t, 64, false, path::ContigRows>(path::ContigRows, int)") \
        == "decode_chunk"
    assert c("void path::decode_chunk_kernel<path::bf16_t, 64, true, path::ContigRows>(path::ContigRows)") \
        == "decode_chunk_fox"
    assert c("void path::decode_merge_kernel<path::bf16_t, 64, false, path::PagedRows>(path::PagedRows)") \
        == "decode_merge_paged"
    assert c("void path::decode_chunk_kernel<path::bf16_t, 64, true, path::PagedRows>(path::PagedRows)") \
        == "decode_chunk_paged_fox"
    assert c("_ZN4path13scan64_kernelILb0EEEvliiifPKDF16_S2_S2_PKfS4_S4_S4_S4_S4_PtPf") == "scan"
    assert c("_ZN4path19prepare_mfma_kernelILi64EEEvlifPKtS2_S2_S2_PKfPDF16_S5_PfS6_S6_S6_S5_") == "prepare"
    assert c("void path::bwd_pair_kernel<path::bf16_t, 64, false>(long)") is None
    assert profsum.short("_ZN4path14project_kernelILi64EEEvlllliiPKtS2_S2_PKffPtPf") == "project_kernel (projection)"


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
