// Expert records between the two codes layouts ("One GPU, three storage
// tiers": MXFP4 experts of 17,547,264 bytes; the byte layout is this
// library's).  A record is W_gate [f x d], W_up [f x d], W_down [d x f], each a
// codes plane then a scales plane.  In row order block kb (32 elements) of row
// `row` of a plane with K columns sits at row*K/2 + kb*16; in tile order at
// ((row/16)*(K/32) + kb)*256 + (row%16)*16, so the 16 rows of a tile store each
// block's 16-byte pieces side by side.  Scales and padding keep their place.
#include "common.h"
#include "launch.h"

#include <algorithm>

namespace moe {

// one thread per 16-byte piece of a record, grid-stride over all records
__global__ void pack_kernel(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int64_t n_records,
                            int64_t stride, int d, int f, int to_tiles) {
  const int64_t pieces = stride / 16, total = n_records * pieces;
  const int64_t plane_c = (int64_t)f * d / 2, plane_s = (int64_t)f * d / 32;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t rec = i / pieces, off = (i - rec * pieces) * 16;
    int64_t plane = -1, K = 0;
    if (off < plane_c) {
      plane = 0, K = d;
    } else if (off >= plane_c + plane_s && off < 2 * plane_c + plane_s) {
      plane = plane_c + plane_s, K = d;
    } else if (off >= 2 * (plane_c + plane_s) && off < 3 * plane_c + 2 * plane_s) {
      plane = 2 * (plane_c + plane_s), K = f;
    }
    int64_t doff = off;
    if (plane >= 0) {
      const int64_t nb = K / 32, local = (off - plane) / 16;  // piece index inside the plane
      if (to_tiles) {  // local = row * nb + kb
        const int64_t row = local / nb, kb = local - row * nb;
        doff = plane + (((row >> 4) * nb + kb) * 16 + (row & 15)) * 16;
      } else {  // local = ((row/16) * nb + kb) * 16 + row % 16
        const int64_t tile = local / (nb * 16), rem = local - tile * nb * 16;
        const int64_t kb = rem / 16, row = tile * 16 + (rem & 15);
        doff = plane + (row * nb + kb) * 16;
      }
    }
    *(u32x4 *)(dst + rec * stride + doff) = *(const u32x4 *)(src + rec * stride + off);
  }
}

int pack_launch(const uint8_t *src, uint8_t *dst, int64_t n_records, int64_t stride, int d, int f, int to_tiles,
                hipStream_t stream) {
  const int64_t total = n_records * (stride / 16);
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 256 * 64);
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, src, dst, n_records, stride, d, f,
                     to_tiles);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Q8_0 int8 plane [N x K] (N % 16 == 0): block b (32 bytes) of row n at
// n*K + 32b in row order and at ((n/16)*(K/32) + b)*512 + (n%16)*32 in tile
// order.  One thread per 16-byte piece.
__global__ void q8_0_pack_kernel(const int8_t *__restrict__ src, int8_t *__restrict__ dst, int N, int K,
                                 int to_tiles) {
  const int64_t per_row = K / 16, total = (int64_t)N * per_row, nb = K / 32;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = i / per_row, c = i - n * per_row;  // row-order piece: row n, piece c
    const int64_t rows_off = n * K + c * 16;
    const int64_t tiles_off = ((n >> 4) * nb + (c >> 1)) * 512 + (n & 15) * 32 + (c & 1) * 16;
    const int64_t so = to_tiles ? rows_off : tiles_off, dof = to_tiles ? tiles_off : rows_off;
    *(u32x4 *)(dst + dof) = *(const u32x4 *)(src + so);
  }
}

int q8_0_pack_launch(const int8_t *src, int8_t *dst, int N, int K, int to_tiles, hipStream_t stream) {
  const int64_t total = (int64_t)N * (K / 16);
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 256 * 64);
  hipLaunchKernelGGL(q8_0_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, src, dst, N, K, to_tiles);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace moe
