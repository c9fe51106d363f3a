"""Host checks of the profile summariser: the kernel names rocprofv3 reports
map to the short names under which bench.py looks up the committed traffic
and counter records (a wrong mapping would silently drop them from the bench
line or merge two kernels' timings)."""
from __future__ import annotations

import pytest

import profile_summary as P

NAMES = [
    ("void w8a8::pipe::gemm_i8_pipelined<(w8a8::Epilogue)0, true>(signed char const*, long)",
     "gemm_postscale"),
    ("void w8a8::pipe::gemm_i8_pipelined<(w8a8::Epilogue)1, true>(signed char const*, long)",
     "gemm_i32"),
    ("void w8a8::pipe::gemm_i8_pipelined<(w8a8::Epilogue)5, false>(signed char const*, long)",
     "gemm_postscale_bias_gelu"),
    ("_ZN4w8a84pipe17gemm_i8_pipelinedILNS_8EpilogueE3ELb1EEEvPKalS4_lPKfS6_PKtPvliiiiii",
     "gemm_postscale_bias"),
    ("void w8a8::pipe::t160::gemm_i8_t160_postscale<(w8a8::Epilogue)0>(signed char const*)",
     "gemm_postscale_t160"),
    ("void w8a8::pipe::t160::gemm_i8_t160_blockwise(signed char const*, long)",
     "gemm_blockwise_t160"),
    ("void w8a8::pipe::bw::gemm_i8_blockwise<3>(signed char const*, long)", "gemm_blockwise"),
    ("void w8a8::splitk::postscale_kernel<false, false>(int const*, int, int, int)",
     "splitk_postscale"),
    ("void w8a8::rmsnorm_quant_kernel<8, true>(unsigned short const*)", "rmsnorm_quant"),
    ("void w8a8::layernorm_quant_f32_kernel<8, true, false, true, 8>(unsigned short const*)",
     "layernorm_quant"),
    ("void w8a8::quant_rows_kernel<27, false, true>(unsigned short const*, long)", "quant_rows"),
    ("void w8a8::quant_rows_kernel<10, true, true>(unsigned short const*, long)",
     "quant_rows_1x128"),
    ("void w8a8::quant_rows_split_kernel<3, false, true>(unsigned short const*, long)",
     "quant_rows_split"),
    ("void w8a8::quant_rows_split_kernel<2, true, true>(unsigned short const*, long)",
     "quant_rows_1x128_split"),
    ("void w8a8::quant_rows_long_kernel<false>(unsigned short const*, long)", "quant_rows_long"),
    ("void w8a8::quant_block128_kernel(unsigned short const*, long)", "quant_block128"),
    ("__amd_rocclr_copyBuffer", "hip_copy_buffer"),
    ("void (anonymous namespace)::mainloop<true>(signed char const*, int, int*)",
     "probe_mainloop"),
    ("void (anonymous namespace)::mainloop<false>(signed char const*, int, int*)",
     "probe_mainloop_norefill"),
]


@pytest.mark.parametrize("full,short", NAMES)
def test_short_names(full, short):
    assert P.short_name(full) == short


def test_short_names_are_distinct():
    # every kernel of the library keeps a name of its own
    shorts = [s for _, s in NAMES]
    assert len(set(shorts)) == len(shorts)
