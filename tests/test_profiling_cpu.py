"""The rocprofv3 summary helpers: kernel-symbol naming and the staleness
check of committed traffic figures (host only)."""
import json

from token_transformer_layer_amd import profiling


def test_gemm_symbols_map_to_trace_names():
    m = "_ZN3tpk19gemm_bf16_dl_kernelINS_5DlCfgILi128ELi128ELi2ELi2ELi2ELi64EEELb0ELb0ENS_11EpiStoreF32IDF16bEEEEvNS_8GemmArgsET2_i"
    assert profiling.trace_name(m) == "gemm_bf16_128_tn_store_f32"
    d = "void tpk::gemm_bf16_pp_kernel<tpk::DlCfg<256, 256, 2, 2, 4, 32, 1>, true, true, tpk::EpiQkv<__bf16> >(tpk::GemmArgs)"
    assert profiling.trace_name(d) == "gemm_bf16_256_nt_qkv"
    p = "_ZN3tpk19gemm_bf16_pp_kernelINS_5DlCfgILi256ELi128ELi2ELi2ELi3ELi32ELi2EEELb0ELb0ENS_11EpiStoreF32IDF16bEEEEvNS_8GemmArgsET2_i"
    assert profiling.trace_name(p) == "gemm_bf16_256x128_tn_store_f32"
    p = "_ZN3tpk19gemm_bf16_pp_kernelINS_5DlCfgILi128ELi128ELi2ELi2ELi2ELi64ELi1EEELb1ELb0ENS_11EpiStoreF32IDF16bEEEEvNS_8GemmArgsET2_i"
    assert profiling.trace_name(p) == "gemm_bf16_p128_nn_store_f32"
    p = "_ZN3tpk19gemm_bf16_pp_kernelINS_5DlCfgILi256ELi192ELi4ELi2ELi2ELi64ELi1EEELb1ELb1ENS_11EpiBiasGeluIDF16bEEEEvNS_8GemmArgsET2_i"
    assert profiling.trace_name(p) == "gemm_bf16_256x192w8_nt_bias_gelu"
    d = "void tpk::gemm_bf16_pp_kernel<tpk::DlCfg<256, 256, 2, 4, 2, 64, 1>, false, false, tpk::EpiStoreF32<__bf16> >(tpk::GemmArgs)"
    assert profiling.trace_name(d) == "gemm_bf16_256w8_tn_store_f32"
    # a short slice's input-gradient product computed transposed (split partial sums)
    p = "_ZN3tpk19gemm_bf16_pp_kernelINS_5DlCfgILi256ELi128ELi4ELi2ELi3ELi64ELi1EEELb0ELb1ENS_8EpiSplitELb1EEEvNS_8GemmArgsET2_i"
    assert profiling.trace_name(p) == "gemm_bf16_sk256x128_mk_split"
    assert profiling.trace_name("_ZN3tpk12_GLOBAL__N_113ln_bwd_kernelIDF16bEEviiiPKf") == "ln_bwd_kernel<bf16>"
    # split reductions are told apart by their epilogue
    r = "_ZN3tpk22splitk_reduce_t_kernelINS_6EpiQkvIDF16bEEEEvPKfiiiiT_"
    assert profiling.trace_name(r) == "splitk_reduce_t_kernel<qkv>"
    r = "_ZN3tpk20splitk_reduce_kernelINS_11EpiStoreF32IDF16bEEEEvPKfiiiT_"
    assert profiling.trace_name(r) == "splitk_reduce_kernel<store_f32>"


def test_traffic_is_dropped_when_sources_change(tmp_path):
    k, w = "gemm_bf16_128_tn_store_f32", "wl"
    rec = dict(kernel=k, workload=w, bytes_per_launch=123, source_sha256=profiling.source_hash(k))
    (tmp_path / ("traffic_%s_%s.json" % (k, w))).write_text(json.dumps(rec))
    assert profiling.load_traffic(str(tmp_path), k, w) == 123
    rec["source_sha256"] = "0" * 64
    (tmp_path / ("traffic_%s_%s.json" % (k, w))).write_text(json.dumps(rec))
    assert profiling.load_traffic(str(tmp_path), k, w) is None
    assert profiling.load_traffic(str(tmp_path), k, "other") is None
