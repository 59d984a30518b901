// Layout of the per-head device tables, shared by the host uploader and the
// kernels.  One contiguous device blob holds every head's tables; a DevHead
// record per head gives byte offsets into it.
#pragma once
#include <stdint.h>

namespace sq {

// Per-coordinate descriptor: bit offset of the code field in the record, its
// width, and the start of its threshold / centroid runs in the head's tables.
struct DevCoord {
  int32_t bit_off;
  int32_t width;
  int32_t thr_base;
  int32_t cent_base;
};

struct DevHead {
  int32_t d, d_eff, m, W;
  int32_t code_bits, n_thr, n_cent, has_gamma;
  float qjl_scale;      // sqrt(pi/2) / m  (0 when m == 0)
  int32_t n_cent_sig;   // centroids of the signal coordinates (the first d_eff)
  int32_t pad1, pad2;
  int64_t off_R;        // float [d][d], row i = eigenvector i (y = R x)
  int64_t off_Rfrag;    // bf16 [3][d/32][d/16][64][8]: hi/mid/lo split of R in
                        // MFMA 32x32x16 A-operand order (see compress kernel)
  int64_t off_coord;    // DevCoord [d]
  int64_t off_thr;      // float [n_cent]  thresholds * sigma_i of coordinate i in
                        // breadth-first (Eytzinger) order at [cent_base_i + 1,
                        // cent_base_i + 2^b_i): node n has children 2n, 2n+1
  int64_t off_cent;     // float [n_cent]  centroids * sigma_i
  int64_t off_S;        // float [m][d_eff] QJL sketch
  int64_t off_wstart;   // int32 [W]: first coordinate reaching into word k | count << 16
  int64_t off_desc;     // uint32 [d]: bit offset | width << 12 | centroid base << 16
  int64_t off_lutp;     // uint32 [n_cent]: each centroid as bf16 hi | bf16 lo << 16
                        // (hi + lo reproduces the fp32 centroid to ~2^-17)
  int64_t off_chunks;   // int32 [d/32][4 + d] per wave of the compress kernel:
                        //   [0] number of chunks, [1] first bit | end bit << 16 of
                        //   the wave's contiguous code range, [2] first | end of
                        //   the shared record words this wave stores, [3] unused,
                        //   then chunks (start | count << 10 | width << 20) of <= 8
                        //   equal-width coordinates in coordinate order
};

static_assert(sizeof(DevCoord) == 16, "DevCoord layout");
static_assert(sizeof(DevHead) == 128, "DevHead layout");

}  // namespace sq
