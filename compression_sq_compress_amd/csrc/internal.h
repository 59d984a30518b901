// Internal host-side structures of libsq (not part of the C ABI).
#pragma once
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/sq.h"
#include "devtypes.h"

namespace sq {

// One calibrated head, host copy (double where the calibration computes in
// double; float where the device consumes float).
struct HeadCal {
  int d = 0, d_eff = 0, m = 0, W = 0, code_bits = 0;
  int n_thr = 0, n_cent = 0, n_regions = 0, unconverged = 0;
  double pr = 0.0, kappa = 0.0;
  bool normalized = false;        // records carry the vector norm; unit vectors quantised
  std::vector<double> lam;        // [d] descending
  std::vector<double> R;          // [d*d] row i = eigenvector i
  std::vector<int32_t> widths;    // [d]
  std::vector<int32_t> bit_off;   // [d]
  std::vector<int32_t> thr_base;  // [d]
  std::vector<int32_t> cent_base; // [d]
  std::vector<float> thr;         // [n_thr]
  std::vector<float> cent;        // [n_cent]
  std::vector<float> S;           // [m*d_eff]
};

}  // namespace sq

struct sq_calib {
  sq_calib_opts opts{};
  std::vector<sq::HeadCal> heads;
  int W_max = 0;
  // device side (filled by sq_calib_upload)
  int device = -1;
  void *dev_blob = nullptr;       // all tables
  sq::DevHead *dev_heads = nullptr;  // [n_heads] descriptors (device)
  std::vector<sq::DevHead> host_desc;  // same descriptors, host copy
  size_t dev_bytes = 0;
};

namespace sq {

// error reporting (thread-local message)
sq_status fail(sq_status st, const std::string &msg);
void clear_error();

// calibration of one head (calib.cpp)
sq_status calibrate_head(const float *x, int64_t n, int d, const sq_calib_opts &o,
                         const float *gauss, HeadCal &out, std::string &err);
void finish_layout(HeadCal &h);
sq_status calibrate_head_tq(const float *rotation, int d, const sq_calib_opts &o, const float *gauss,
                            HeadCal &out, std::string &err);

// device entry points (kernels.hip)
sq_status upload_tables(sq_calib *c, void *stream);
void release_tables(sq_calib *c);

}  // namespace sq
