"""CPU checks of the benchmark's algorithmic work accounting: the per-step
roofline amounts add up to the layer's flops, and the 7B-shape totals are
the closed forms of the layer's matrix shapes (QKV 3 d^2 at MHA, o_proj d^2,
gate/up and down 3 d f weights per token, causal attention 4 dh H T(T+1)/2)."""
import bench
import synth


def test_step_flops_add_up_to_the_layer():
    for name in ("llama7b_prefill", "llama13b_prefill", "llama70b_gqa", "llama70b_tp8_shard"):
        wl = synth.WORKLOADS[name]
        B, T = wl.batch, wl.seq
        one_ms = {k: 1.0 for k in ("rmsnorm_attn", "qkv_rope_cache", "attention", "o_proj_residual",
                                   "rmsnorm_mlp", "gate_up_swiglu", "down_residual")}
        r = bench.step_rooflines(wl, B, T, one_ms)
        # at 1 ms per step, TFLOP/s x 1e9 is the step's flops
        total = sum(v["achieved"] * 1e9 for v in r.values() if v["unit"] == "TFLOP/s")
        assert round(total) == bench.prefill_flops(wl, T, B)


def test_7b_closed_forms():
    wl = synth.WORKLOADS["llama7b_prefill"]
    d, f, T = 4096, 11008, 2048
    lin = 2 * T * (4 * d * d + 3 * d * f)
    attn = 4 * 128 * 32 * T * (T + 1) // 2
    assert bench.prefill_flops(wl, T, 1) == lin + attn == 863305203712
    wd = synth.WORKLOADS["llama7b_decode"]
    kv = 2 * 32 * 2 * 32 * 128 * 4095          # bf16 K and V of 32 sequences, 4095 prior slots
    assert bench.decode_bytes(wd, 32, 4095) == 2 * (4 * d * d + 3 * d * f + 2 * d) + kv + 2 * 32 * 2 * 32 * 128 + 2 * 2 * 32 * d


def test_decode_step_bytes():
    wd = synth.WORKLOADS["llama7b_decode"]
    one_ms = {"qkv_rope_cache": 1.0, "attention": 1.0, "o_proj_residual": 1.0, "gate_up_swiglu": 1.0,
              "down_residual": 1.0}
    r = bench.step_rooflines(wd, 32, 1, one_ms, pos=4095)
    by = {k: v["achieved"] * 1e6 for k, v in r.items()}  # GB/s x 1 ms = bytes / 1e6
    d, f = 4096, 11008
    assert round(by["qkv_rope_cache"]) == 2 * 3 * d * d
    assert round(by["o_proj_residual"]) == 2 * d * d
    assert round(by["gate_up_swiglu"]) == 2 * 2 * f * d
    assert round(by["down_residual"]) == 2 * d * f
    assert round(by["attention"]) == 2 * 32 * 2 * 32 * 128 * 4096  # prior slots and the appended one


def test_int8_decode_bytes():
    """The int8 cache's step moves each cached row as 128 one-byte codes and a
    4-byte scale instead of 128 bf16 values: 124 bytes less per row."""
    wd = synth.WORKLOADS["llama7b_decode"]
    rows = 32 * 2 * 32 * 4096  # sequences x (K, V) x kv heads x (4095 prior slots + the appended one)
    assert bench.decode_int8_bytes(wd, 32, 4095) == bench.decode_bytes(wd, 32, 4095) - rows * (2 * 128 - 128 - 4)
