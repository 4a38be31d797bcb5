"""Workload shapes for the MoE FFN layer (one GPU's expert slice).

Each workload is a dataclass of integers and format tags; it carries no arithmetic of the method.

Shape sources (pages):
  * Qwen3-235B: 128 experts, top-8 (Hosting Qwen on Blackwell, section "Prefillers");
    EP=4 prefill sharding gives 32 experts per rank (same section).
  * Qwen3.5-397B: 512 experts, intermediate 1024, top-10 plus one always-active shared expert
    ("How we served a 397B MoE ... on TPU v7", section on the architectural constraints);
    512 / 8 = 64 experts per chip (section on attention DP + expert EP).
  * DeepSeek-V3 with 4-bit MoE weights and 4-bit dispatch ("Driving vLLM WideEP ... on Blackwell
    (Part I)", section on lower-precision operations); block scaling as used for DeepSeek
    (Hosting Qwen on Blackwell, section "Quantization").
  * The Qwen3-235B slice in MXFP8, the format the Qwen deployment uses for its MoE GEMMs (Hosting
    Qwen on Blackwell, section "Quantization").
  * The DeepSeek-V3 slice in NVFP4, the 4-bit format with FP8 per-group scales over 16 elements of
    the DeepSeek deployment ("Driving vLLM WideEP ... (Part I)", lower-precision operations;
    "CuTeDSL at Perplexity", section "Blackwell").
"""
from dataclasses import dataclass, replace

# scoring
SOFTMAX = 0
SIGMOID = 1

# number formats of the expert path (weights and the activations fed to the expert GEMMs)
FMT_F32 = 0      # fp32 values (tiny config)
FMT_BF16 = 1     # bf16 values
FMT_FP8 = 2      # OCP e4m3 codes with fp32 scales per 128x128 block (weights, x) / 1x128 (h)
FMT_MX4 = 3      # OCP e2m1 codes, two per byte, with one E8M0 scale per 32 elements along K
FMT_MX8 = 4      # OCP e4m3 codes with one E8M0 scale per 32 elements along K (MXFP8)
FMT_NV4 = 5      # NVFP4: OCP e2m1 codes with one e4m3 scale per 16 along K and an fp32 scale per row


@dataclass(frozen=True)
class Workload:
    name: str
    T: int            # tokens
    H: int            # hidden
    E: int            # experts in the model
    e0: int           # first local expert
    E_loc: int        # local experts on this GPU
    I: int            # expert intermediate
    k: int            # top-k
    I_s: int          # shared expert intermediate (0 = none)
    scoring: int
    renormalize: int
    io_fmt: int       # FMT_F32 or FMT_BF16: x, router weight, output
    fmt: int          # expert path format
    zipf_s: float     # Zipf exponent of the per-expert router bias (0 = no bias)
    seed: int = 0
    gated: int = 0    # 1: the shared expert is scaled by a per-token logistic gate

    @property
    def desc(self):
        return dict(T=self.T, H=self.H, E=self.E, e0=self.e0, E_loc=self.E_loc, I=self.I,
                    k=self.k, I_s=self.I_s, scoring=self.scoring, renormalize=self.renormalize,
                    io_fmt=self.io_fmt, fmt=self.fmt)

    def with_tokens(self, T):
        return replace(self, T=T, name=f"{self.name.split('@')[0]}@T{T}")


WORKLOADS = {
    # tiny fp32 layer, 8 experts, top-2, softmax, no shared expert, seed 0
    "C1": Workload("C1", 64, 256, 8, 0, 8, 128, 2, 0, SOFTMAX, 1, FMT_F32, FMT_F32, 0.0),
    # Qwen3-235B-shaped, EP=4 slice (experts 0..31 of 128), bf16, Zipf(1.1) router bias
    "C2p": Workload("C2p", 16384, 4096, 128, 0, 32, 1536, 8, 0, SOFTMAX, 1, FMT_BF16, FMT_BF16, 1.1),
    "C2d": Workload("C2d", 64, 4096, 128, 0, 32, 1536, 8, 0, SOFTMAX, 1, FMT_BF16, FMT_BF16, 1.1),
    # Qwen3.5-397B-shaped, EP=8 slice (64 of 512), top-10, shared expert, bf16
    "C3a": Workload("C3a", 1024, 4096, 512, 0, 64, 1024, 10, 1024, SOFTMAX, 1, FMT_BF16, FMT_BF16, 0.0),
    "C3b": Workload("C3b", 8192, 4096, 512, 0, 64, 1024, 10, 1024, SOFTMAX, 1, FMT_BF16, FMT_BF16, 0.0),
    # the same slices with the shared expert behind its per-token logistic gate
    "C3a_g": Workload("C3a_g", 1024, 4096, 512, 0, 64, 1024, 10, 1024, SOFTMAX, 1, FMT_BF16, FMT_BF16,
                      0.0, gated=1),
    "C3b_g": Workload("C3b_g", 8192, 4096, 512, 0, 64, 1024, 10, 1024, SOFTMAX, 1, FMT_BF16, FMT_BF16,
                      0.0, gated=1),
    # DeepSeek-V3-shaped slice (32 of 256), fp8 e4m3 with 128x128 fp32 block scales, sigmoid
    "C4p": Workload("C4p", 4096, 7168, 256, 0, 32, 2048, 8, 2048, SIGMOID, 1, FMT_BF16, FMT_FP8, 0.0),
    "C4d": Workload("C4d", 256, 7168, 256, 0, 32, 2048, 8, 2048, SIGMOID, 1, FMT_BF16, FMT_FP8, 0.0),
    # same shape, MXFP4 experts and activations
    "C5p": Workload("C5p", 16384, 7168, 256, 0, 32, 2048, 8, 2048, SIGMOID, 1, FMT_BF16, FMT_MX4, 1.2),
    "C5d": Workload("C5d", 64, 7168, 256, 0, 32, 2048, 8, 2048, SIGMOID, 1, FMT_BF16, FMT_MX4, 0.0),
    # the Qwen3-235B-shaped slice with MXFP8 experts and activations (x and h in MXFP8)
    "C2p_mx8": Workload("C2p_mx8", 16384, 4096, 128, 0, 32, 1536, 8, 0, SOFTMAX, 1, FMT_BF16, FMT_MX8, 1.1),
    "C2d_mx8": Workload("C2d_mx8", 64, 4096, 128, 0, 32, 1536, 8, 0, SOFTMAX, 1, FMT_BF16, FMT_MX8, 1.1),
    # the DeepSeek-V3-shaped slice with NVFP4 experts and activations (h in bf16)
    "C5p_nv4": Workload("C5p_nv4", 16384, 7168, 256, 0, 32, 2048, 8, 2048, SIGMOID, 1, FMT_BF16, FMT_NV4,
                        1.2),
    "C5d_nv4": Workload("C5d_nv4", 64, 7168, 256, 0, 32, 2048, 8, 2048, SIGMOID, 1, FMT_BF16, FMT_NV4, 0.0),
}
