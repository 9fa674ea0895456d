"""Host logic of the rocprofv3 summarizer: kernel classification, the
schedule window and the source-hash guard on stored traffic figures."""
from bit_quantized_video_amd import profsum as P


def test_classify_kernel_names():
    cases = {
        "hdq::k_stats_partial(unsigned short const*)": "select_stats",
        "void hdq::k_stats_partial<0>(unsigned short const*)": "select_stats",
        "void hdq::k_stats_partial<2>(unsigned short const*)": "select_stats",
        "void hdq::k_stats_partial<1>(unsigned short const*)": "delta_sums",
        "hdq::k_stats_final(double const*)": "select_final",
        "void hdq::k_quant_int_rows<128, 3, false>(int)": "quant_int8",
        "void hdq::k_quant_int_rows<256, 6, true>(int)": None,  # INT4 weight preparation
        "void hdq::k_quant_int_rows<256, 6, true, false>(int)": None,
        "void hdq::k_quant_int_rows<128, 3, false, false>(int)": "quant_int8",
        "void hdq::k_quant_int_rows<128, 3, false, true>(int)": "select_quant_int8",
        "void hdq::k_quant_nvfp4<3>(int)": "quant_nvfp4_mx",
        "void hdq::k_quant_nvfp4<4>(int)": "quant_nvfp4_p2",
        "void hdq::k_quant_nvfp4<2>(int)": "quant_nvfp4",
        # with the Hadamard block as a template argument
        "void hdq::k_quant_int_rows<192, 2, false, true, 128>(int)": "select_quant_int8",
        "void hdq::k_quant_int_rows<128, 3, false, false, 128>(int)": "quant_int8",
        "void hdq::k_quant_int_rows<128, 3, false, false, 128, true>(int)": "quant_int8",
        "void hdq::k_quant_int_rows<64, 6, false, true, 128, true>(int)": "select_quant_int8",
        "void hdq::k_quant_int_rows<256, 6, false, true, 128, false>(int)": "select_quant_int8",
        "void hdq::k_quant_int_rows<128, 3, true, false, 0>(int)": None,
        "void hdq::k_quant_int_rows<128, 3, true, false, 0, false>(int)": None,
        "void hdq::k_quant_nvfp4<3, 128>(int)": "quant_nvfp4_mx",
        "void hdq::k_quant_nvfp4<4, 0>(int)": "quant_nvfp4_p2",
        "void hdq::k_quant_nvfp4<2, 128>(int)": "quant_nvfp4",
        "void hdq::k_gemm_i8i4_pipe<2, 4, 4, 2, 1>(int)": "gemm_int8",
        "void hdq::k_gemm_i8i4_pipe<2, 4, 4, 2, 0>(int)": None,  # f32 output: quality check
        "void hdq::k_gemm_fp4mx_pipe<1, false>(int)": "gemm_nvfp4_mx",
        "void hdq::k_gemm_fp4mx_pipe<1, true>(int)": "gemm_nvfp4_p2",
        "void hdq::k_gemm_bf16_pipe<1, 1>(int)": "gemm_nvfp4",
        "void hdq::k_gemm_bf16_pipe<0, 1>(int)": "gemm_bf16",
        "__amd_rocclr_copyBuffer": None,
    }
    for name, kind in cases.items():
        assert P.classify(name) == kind, name


def test_schedule_window_starts_after_weight_prep():
    rows = [(0, "void hdq::k_quant_int_rows<128, 3, true>"), (1, "hdq::k_stats_partial"),
            (2, "void hdq::k_quant_int_rows<128, 3, true, false>"), (3, "hdq::k_stats_partial"),
            (4, "void hdq::k_gemm_i8i4_pipe<2, 4, 4, 2, 1>"), (5, "void hdq::k_gemm_i8i4_pipe<2, 4, 4, 2, 0>")]
    assert [r[0] for r in P.schedule_window(rows)] == [3, 4]
    rows[2] = (2, "void hdq::k_quant_int_rows<128, 3, true, false, 0>")
    assert [r[0] for r in P.schedule_window(rows)] == [3, 4]
    rows[2] = (2, "void hdq::k_quant_int_rows<128, 3, true, false, 0, false>")  # the full-row argument
    assert [r[0] for r in P.schedule_window(rows)] == [3, 4]


def test_stored_traffic_guarded_by_source_hash(tmp_path):
    f = tmp_path / "t.txt"
    f.write_text(f"header\ntraffic gemm_int8 123 {P.sources_hash('gemm_int8')}\n"
                 f"traffic quant_int8 456 0000000000000000\n")
    assert P.current_traffic(str(f), "gemm_int8") == 123.0
    assert P.current_traffic(str(f), "quant_int8") is None  # sources changed
    assert P.current_traffic(str(f), "gemm_bf16") is None  # never measured
    assert P.current_traffic(str(tmp_path / "missing.txt"), "gemm_int8") is None


def test_one_launch_gemms_take_their_calls_decisions():
    P.DECISIONS = [1, 0, 2, 1]
    try:
        c = P.Classifier()
        mx = "void hdq::k_gemm_dispatch<1, 3>(int const*)"
        plain = "void hdq::k_gemm_dispatch<1, 2>(int const*)"
        decoded = "void hdq::k_gemm_dispatch<1, 16>(int const*)"   # plain NVFP4 from decoded operands
        got = [c(mx) for _ in range(5)] + [c(plain) for _ in range(3)] + [c(decoded) for _ in range(2)]
        assert got == ["gemm_int8", "gemm_nvfp4_mx", "gemm_bf16", "gemm_int8", "gemm_int8",
                       "gemm_int8", "gemm_nvfp4", "gemm_bf16", "gemm_int8", "gemm_nvfp4"]
        assert P.classify("hdq::k_dq_decode_w(unsigned char const*)") == "decode_nvfp4"
        for name, kind in (("void hdq::k_quant_nvfp4<3, 128, false>(unsigned short const*)", "quant_nvfp4_mx"),
                           ("void hdq::k_quant_nvfp4<2, 128, true>(unsigned short const*)", "quant_nvfp4"),
                           ("void hdq::k_quant_nvfp4<4, 0, false>(unsigned short const*)", "quant_nvfp4_p2"),
                           ("void hdq::k_quant_nvfp4_w32<3>(unsigned short const*)", "quant_nvfp4_mx"),
                           ("void hdq::k_quant_nvfp4_w32<2>(unsigned short const*)", "quant_nvfp4"),
                           ("void hdq::k_quant_nvfp4_w32<4>(unsigned short const*)", "quant_nvfp4_p2")):
            assert P.classify(name) == kind, name
        assert c("void hdq::k_gemm_dispatch<0, 3>(int const*)") is None  # f32 output: not the schedule
    finally:
        P.DECISIONS = None
    assert P.Classifier()("void hdq::k_gemm_dispatch<1, 3>(int const*)") == "gemm_dispatch"
