"""Dense GEMM rate of the vendor library (torch.matmul, hipBLASLt on ROCm) at
the shapes of the layer's two products when the +-1 factors are stored
expanded to fp16 / bf16: a calibration point for the MFMA path, which reads
the packed bits instead.  Not part of the library.

    python3 bit_adapters_amd/probe/vendor_gemm.py

Each shape is T x K times K x N (the weight stored N x K, as a Linear
weight), timed with events over 30 calls that rotate three input copies.
"""
import torch

SHAPES = [
    # (name, T, K, N)
    ("8192^2 R 6144, 4096 tokens, first product", 4096, 8192, 6144),
    ("8192^2 R 6144, 4096 tokens, second product", 4096, 6144, 8192),
    ("11008x4096 R 2048 x3 terms, 256 tokens, first products", 256, 4096, 6144),
    ("11008x4096 R 2048 x3 terms, 256 tokens, second products", 256, 6144, 11008),
    ("two 4096^2 boolean kernels, 256 tokens", 256, 8192, 4096),
]


def main() -> None:
    dev = "cuda"
    print("device", torch.cuda.get_device_name(0))
    for dt in (torch.float16, torch.bfloat16):
        for name, T, K, N in SHAPES:
            a = [torch.randn(T, K, device=dev, dtype=dt) for _ in range(3)]
            b = [torch.randn(N, K, device=dev, dtype=dt) for _ in range(3)]
            for i in range(5):
                torch.matmul(a[i % 3], b[i % 3].t())
            torch.cuda.synchronize()
            n = 30
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(n):
                torch.matmul(a[i % 3], b[i % 3].t())
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1000.0 / n
            tf = 2.0 * T * K * N / us / 1e6
            print("%-9s %-58s T %5d K %5d N %5d  %8.1f us  %6.0f TFLOP/s  %4.1f%% of 2.5 PFLOP/s"
                  % (str(dt)[6:], name, T, K, N, us, tf, tf / 25.0), flush=True)


if __name__ == "__main__":
    main()
