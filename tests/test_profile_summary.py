"""Host-side checks of the rocprofv3 summary helper used for roofline.traffic."""
import os

import profile_summary as ps


def test_short_name_strips_arguments_keeps_templates():
    assert ps.short_name("void qmm::mmvq_q4k_kernel<1, 4, false>(unsigned char const*, int)") == \
        "qmm::mmvq_q4k_kernel<1, 4, false>"
    assert ps.short_name("at::cuda::(anonymous namespace)::spin_kernel(long)") == \
        "at::cuda::{anonymous}::spin_kernel"
    assert ps.short_name("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def test_sources_hash_only_for_library_kernels():
    assert ps.sources_sha256("qmm::mmvq_q4k_kernel<1, 4, false>") is not None
    assert ps.sources_sha256("qmm::mmq_q4k_kernel<4, 2, false>") != ps.sources_sha256("qmm::mmvq_q4k_kernel<1, 4, false>")
    assert ps.sources_sha256("__amd_rocclr_copyBuffer") is None
    assert ps.sources_sha256("qmm::mmq_k4_q8k_kernel<4, 2, 1, false, false>") != ps.sources_sha256("qmm::mmq_q4k_kernel<4, 2, 1, false>")
    assert ps.sources_sha256("qmm::mmq_q6k_q8k_kernel<4, 2, false, true>") == \
        ps.sources_sha256("qmm::mmq_k4_q8k_kernel<4, 2, 1, false, false>")
    fused = ps.sources_sha256("qmm::{anonymous}::silu_mul_kernel<1>")
    assert fused is not None and fused == ps.sources_sha256("qmm::{anonymous}::rmsnorm_kernel<4, true, 1>")
    assert ps.short_name("void qmm::(anonymous namespace)::silu_mul_kernel<true>(HIP_vector_type<float, 4u> const*)") \
        == "qmm::{anonymous}::silu_mul_kernel<true>"


def _summary(tmp_path, lines):
    p = tmp_path / "s.md"
    p.write_text("# x\n```\n" + "\n".join(lines) + "\n```\n")
    return str(p)


def test_read_traffic_current_stale_and_ambiguous(tmp_path):
    k = "qmm::mmq_q4k_kernel<4, 2, false>"
    sha = ps.sources_sha256(k)
    p = _summary(tmp_path, [
        f"traffic: kernel=qmm::mmq_q4k_kernel<4,2,false> grid=393216 bytes_per_launch=1000 sources_sha256={sha}",
        f"traffic: kernel=qmm::mmq_q4k_kernel<4,2,false> grid=131072 bytes_per_launch=2000 sources_sha256={'0' * 64}",
    ])
    assert ps.read_traffic(p, k, 393216) == 1000
    assert ps.read_traffic(p, k, 131072) is None          # counters taken from other sources
    assert ps.read_traffic(p, k, None) is None             # two grids: ambiguous
    assert ps.read_traffic(p, k, 4096) is None             # not profiled
    assert ps.read_traffic(os.path.join(str(tmp_path), "missing.md"), k, None) is None
