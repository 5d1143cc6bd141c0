"""Plain device copy of a known size, used to calibrate HBM byte counters.

Copies 1 GiB (2^28 float32) once after a warm-up, so that the FETCH_SIZE and
WRITE_SIZE counters of the copy kernel can be compared with the 1 GiB read
and 1 GiB written it must move.
"""
import torch

N = 1 << 28


def main():
    src = torch.ones(N, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)  # warm-up (also a counted dispatch; the log names both)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {N * 4} bytes twice", flush=True)


if __name__ == "__main__":
    main()
