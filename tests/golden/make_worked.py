"""Writes ``worked_k64.json``: two tiny hand-worked products (one 4-bit, one 8-bit).

The expected outputs are derived by hand below. They come from neither the
oracle nor the GPU library. The script only lays out the inputs those
derivations describe.

The operand formats are from "MLX CUDA Cleanup Plan", Target Architecture §1:
BF16 activations, U32-packed affine codes, BF16 scales and biases. Bit widths
and group size are from Refactor Plan, Phase 3: 4-bit and 8-bit, group 64.
The affine map is w = scale*q + bias, and codes are packed low-first
(element k at bit offset bits*(k % (32/bits)) of word k // (32/bits)).

4-bit case (K = 64, one group, N = 2 rows, M = 2 activation rows):
  row 0: q_k = k mod 16, scale 0.5, bias -1  -> w_k = 0.5*(k mod 16) - 1
  row 1: q_k = 15 - (k mod 16), scale 0.25, bias 0.5
  x0 = all ones, x1 = (+1, -1, +1, -1, ...)
  y[x0,row0] = 0.5*4*120 - 64 = 176
  y[x0,row1] = 0.25*4*120 + 32 = 152
  y[x1,row0]: each (even, odd) pair of k gives (0.5e-1) - (0.5(e+1)-1) = -0.5,
              over 32 pairs -> -16
  y[x1,row1]: each pair gives +0.25 -> 8
  A = sum |x*w|: row 0 per 16 columns: 1 + 0.5 + 0 + sum_{j=3..15}(0.5j-1) = 47,
  times 4 -> 188 (both x). Row 1 has every w > 0 -> 152 (both x).
  Packed words: row 0 = 0x76543210, 0xFEDCBA98 repeated; row 1 = 0x89ABCDEF,
  0x01234567 repeated.

8-bit case (K = 64, N = 1):
  q_k = 4k, scale 0.25, bias -8 -> w_k = k - 8
  y[x0] = sum(k) - 512 = 2016 - 512 = 1504
  y[x1]: each pair gives (2i-8) - (2i+1-8) = -1 -> -32
  A = sum_{k<=8}(8-k) + sum_{k>8}(k-8) = 36 + 1540 = 1576
"""
import json
import os

ONE, NEG_ONE, HALF, QUARTER, NEG_EIGHT = 0x3F80, 0xBF80, 0x3F00, 0x3E80, 0xC100


def main():
    x0 = [ONE] * 64
    x1 = [ONE if k % 2 == 0 else NEG_ONE for k in range(64)]
    four = {
        "bits": 4, "group_size": 64, "N": 2, "K": 64,
        "x_bf16": [x0, x1],
        "w_u32": [[0x76543210, 0xFEDCBA98] * 4, [0x89ABCDEF, 0x01234567] * 4],
        "scales_bf16": [[HALF], [QUARTER]],
        "biases_bf16": [[NEG_ONE], [HALF]],
        "y": [[176.0, 152.0], [-16.0, 8.0]],
        "A": [[188.0, 152.0], [188.0, 152.0]],
    }
    words8 = []
    for i in range(16):
        b = [4 * (4 * i + j) for j in range(4)]
        words8.append(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24))
    eight = {
        "bits": 8, "group_size": 64, "N": 1, "K": 64,
        "x_bf16": [x0, x1],
        "w_u32": [words8],
        "scales_bf16": [[QUARTER]],
        "biases_bf16": [[NEG_EIGHT]],
        "y": [[1504.0], [-32.0]],
        "A": [[1576.0], [1576.0]],
    }
    doc = {
        "citation": ("Operand formats: 'MLX CUDA Cleanup Plan', Target Architecture section 1 and "
                     "Refactor Plan Phase 3 (BF16 x, U32-packed 4/8-bit affine codes, BF16 scales/biases, "
                     "group 64). Affine map w = scale*q + bias, low-first packing (reading). "
                     "Expected values derived by hand in make_worked.py."),
        "cases": [four, eight],
    }
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "worked_k64.json")
    with open(out, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
