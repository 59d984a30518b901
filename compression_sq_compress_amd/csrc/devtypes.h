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

// Compress work plan.  The kernel's d/16 waves each own a contiguous range of
// eigen-coordinates; a range is cut into chunks of 1, 2, 4 or 8 coordinates
// of equal width (runs of zero-width coordinates outside the signal range
// need no chunk).  Wave header w (16 words): [0] chunks, [1] first bit | end
// bit << 16 of the wave's code range, [2] first | end of the shared record
// words the wave stores, [3] first | end of the words it stores straight from
// its bit window, [4] index of its first chunk.  Chunk (16 words): [0..7]
// root threshold of each coordinate (fp32 bits), [8] tree base, [9] first
// coordinate, [10] count n, [11] width b, [12] number of signal coordinates
// (residual needed), [13] signal-centroid base, [14] log2 n.  Coordinate c's
// threshold tree holds node k (1 <= k < 2^b, children 2k, 2k+1) at tree base
// + c * 2^b + k - 1, and its signal centroids at signal base + c * 2^b + code.
constexpr int PLAN_WORDS = 16;

// Score schedule (sq_scores).  Coordinates are taken in order as "halves":
// two adjacent coordinates whose widths sum to at most 8 bits form one half
// (their codes are adjacent in the record, so one bit field of the summed
// width indexes a joint table), any other coordinate is a half of its own.
// Two halves make a quad = the 4 k-slots of one v_mfma_f32_4x4x4_16b_bf16.
// Quad (SCHED_WORDS): [0], [1] bit position | summed width << 16 of its two
// halves, [2], [3] their first entry in the joint table, [4] k-slot
// coordinates 0 | 1 << 16, [5] k-slots 2 | 3 << 16 (0xFFFF = empty slot).
// Joint table entry v of a half (a, b): C_a[v & (2^w_a - 1)] and C_b[v >> w_a]
// as bf16 hi pair (hi_a | hi_b << 16) and bf16 lo pair (lo_a | lo_b << 16),
// stored (lo pair, hi pair) for the first half of a quad and (hi pair, lo
// pair) for the second, so that the two entries of a quad read into four
// consecutive registers (lo_ab, hi_ab, hi_cd, lo_cd) give the MFMA B
// operands hi|lo of ab, hi|lo of cd and the four hi parts.
constexpr int SCHED_WORDS = 8;

struct DevHead {
  int32_t d, d_eff, m, W;
  int32_t code_bits, n_tree, n_cent, has_gamma;
  float qjl_scale;      // sqrt(pi/2) / m  (0 when m == 0)
  int32_t n_csig;       // floats in the signal-centroid table of the plan
  int32_t n_chunks;
  int32_t n_quads;      // score schedule quads
  int32_t n_plut;       // joint-table entries (the last one is all zero)
  int32_t n_fgroups;    // fused decode schedule: groups (code groups, then QJL groups)
  int32_t n_fent;       // fused decode schedule: table entries over all groups
  int32_t n_fqjl;       // of the groups, the trailing QJL groups
  int64_t off_R;        // float [d][d], row i = eigenvector i (y = R x)
  int64_t off_RT;       // float [d][d], R transposed
  int64_t off_Rfrag;    // bf16 [3][d/16][d/32][64][8]: hi/mid/lo split of R in
                        // MFMA 16x16x32 A-operand order (see compress kernel)
  int64_t off_coord;    // DevCoord [d]
  int64_t off_tree;     // float [n_tree]  thresholds * sigma_i, per chunk of the
                        // compress plan, breadth-first (see PLAN_WORDS)
  int64_t off_cent;     // float [n_cent]  centroids * sigma_i
  int64_t off_S;        // float [m][d_eff] QJL sketch
  int64_t off_plan;     // uint32 [d/16 + n_chunks + 1][PLAN_WORDS] compress plan
  int64_t off_sched;    // uint32 [n_quads][SCHED_WORDS] score schedule
  int64_t off_plut;     // uint32 [n_plut][2] joint tables (hi pair, lo pair)
  int64_t off_lutp;     // uint32 [n_cent]: each centroid as bf16 hi | bf16 lo << 16
                        // (hi + lo reproduces the fp32 centroid to ~2^-17)
  int64_t off_csig;     // float [n_csig]  signal centroids * sigma_i per plan chunk
  // register-quantising compress plan (P2_* layout below); n_p2 = 0: not available
  int32_t n_p2, n_tree2, n_csig2;
  int32_t normalized;   // records carry the vector norm nu (half): bits [32W-32, 32W-16)
                        // if m > 0, else [32W-16, 32W); the unit vector was quantised
  int64_t off_p2;       // uint32 [d/16][P2_WAVE]
  int64_t off_tree2;    // float [n_tree2] per-coordinate padded trees (see P2_WAVE)
  int64_t off_csig2;    // float [n_csig2] signal centroids * sigma_i, padded per coordinate
  int64_t off_Rfrag2;   // bf16 [3][d/16][d/32][64][8] like off_Rfrag, rows permuted (see P2_WAVE)
  int64_t off_fsched;   // uint32 fused decode schedule (FS_* layout below)
  // grid quantiser of the register compress plan (GRID_* layout below);
  // n_gcells = 0: not available for this head
  int32_t n_gcells, n_gcsig;
  int64_t off_gcoord;   // uint32 [d][GRID_COORD_WORDS]
  int64_t off_gcells;   // uint32 [n_gcells][2]
  int64_t off_gcsig;    // float [n_gcsig] signal centroids * sigma_i, per coordinate
  int64_t off_Rfrag_u;  // bf16 [3][d/16][d/32][64][8] like off_Rfrag with row i scaled by the
                        // grid quantiser's a_i (its MFMA gives u = a_i y_i + b_i when the
                        // accumulator starts at b_i); grid heads only
};

// Grid quantiser.  A coordinate's thresholds are sigma_i times the thresholds
// t_0 < .. < t_{n-1} of its region (regime, width); each region gets a
// uniform grid of cells of width h < min(t_{j+1} - t_j) starting at o, so a
// cell holds at most one threshold, and o, h are chosen so that every
// threshold sits at least 1/512 of a cell away from the cell edges.  With
// u = (y / sigma_i - o) / h = y * a_i + b_i and cell = clamp(trunc(u), 0,
// C - 1), the code is code_lo(cell) + [u > t_cell(cell)], where code_lo
// counts the thresholds left of the cell and t_cell is the cell's threshold
// in cell units (+inf when it has none).  A rounding of u that moves a value
// across a cell edge cannot change the code: no threshold lies that close to
// an edge.  Cell 0 of the table is (+inf, 0), used by zero-width coordinates
// (a_i = b_i = 0).  Per coordinate c (natural order; MFMA row 4s + r of wave
// w is coordinate 16w + 4s + r): [0] a_i (fp32 bits), [1] b_i, [2] byte offset
// of its region's cells, [3] C - 1, [4] signal-centroid base (floats) or
// 0xFFFFFFFF, [5] bit offset of its field within the fields of coordinates
// 4k .. 4k + 3 (k = c / 4), [6] that run's record word | bit shift << 8.
// Cells: (t_cell as fp32 bits, code_lo).
constexpr int GRID_COORD_WORDS = 8;
constexpr int GRID_MAX_CELLS = 6144;

// Register-quantising compress plan.  Coordinates are taken in groups of 4
// (equal widths where possible, spread over different record words; depth =
// the group's largest width); each wave gets 4 groups, one per MFMA
// accumulator register r, chosen to balance the waves' total depth and
// ordered by decreasing depth.  Row 4s + r of wave w's 16 MFMA rows holds
// coordinate s of group g(w, r), so lane l (s = l / 16) finds in register r
// the value of that coordinate for tokens l % 16 + 16 j.  Wave header
// (P2_WAVE): [r] depth of register r's group, [4 + 4r + s] tree base
// (floats) of its coordinate, [20 + 4r + s] signal-centroid base or
// 0xFFFFFFFF (not a signal coordinate), [36 + 4r + s] the coordinate.  A
// tree holds the coordinate's sorted thresholds padded with +inf to
// 2^depth - 1 entries in breadth-first order (node k = 1 .. 2^depth - 1 at
// base + k - 1); the four trees of a register start at 16 s (mod 64).
constexpr int P2_WAVE = 64;

static_assert(sizeof(DevCoord) == 16, "DevCoord layout");
// Fused decode schedule of a key head (sq_decode).  The record's code fields
// are cut, in bit order, into groups of adjacent fields of at most FG_BITS
// bits together (a wider field is a group of its own; zero-width coordinates
// have no field), then the m QJL bits into groups of at most FG_BITS.  At run
// time each group gets a table of 2^width entries per query head: for a code
// group entry v = sum over its coordinates of q~_i C_i[the field of i in v],
// for a QJL group entry v = sqrt(pi/2)/m sum over its bits j of
// w_j (2 v_j - 1), w = S q~[0:d_eff]; a token's score is then one table
// read per group (QJL groups scaled by gamma).  Tables are placed largest
// first, so each starts at a multiple of its own size; one zero entry follows
// them.  Layout (uint32), n = n_fgroups, nq = n_fqjl:
//   [2n]   per group: width (bits 0-3) | QJL group (bit 4) | first table entry
//          << 8; first coordinate or QJL bit (bits 0-11) | count << 12;
//   [nq]   per QJL group: bit position relative to word qb (bits 0-7) |
//          width << 8 | first table entry << 12, qb = W - 2, or W - 3 when
//          normalised (the QJL bits then lie in words qb, qb + 1: m <= 16);
//   (padded to 16 words)
//   [3][W + 1][FS_SLOTS][2]  for table entries of 4, 8 and 16 bytes (E = 2,
//          3, 4) and each window j (record words j - 1, j; word -1 is zero):
//          FS_SLOTS slots of (window shift | table byte offset << 5, field
//          mask << E), the code groups whose field, read from bit
//          (pos + 32 - E) % 32 of word j - 1, lands at bit E of the window; unused
//          slots read the zero entry (the used slots come first);
//   [3][W + 1]  the number of used slots of each window, per entry size.
constexpr int FS_SLOTS = 8;
constexpr int FG_BITS = 6;

static_assert(sizeof(DevHead) == 256, "DevHead layout");

}  // namespace sq
