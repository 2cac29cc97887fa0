"""A plain device-to-device copy of known size, profiled beside the CSA kernels to
calibrate the FETCH_SIZE / WRITE_SIZE hardware counters (bytes read and written by a
copy are known exactly)."""
import torch

N_BYTES = 1 << 30


def main():
    src = torch.empty(N_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {N_BYTES} bytes x3")


if __name__ == "__main__":
    main()
