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
// eigenpairs of a Jacobi result (diag(a), columns of V) in descending order,
// clamped at zero, each vector signed so its largest-magnitude entry is positive
void order_eigenpairs(const std::vector<double> &a, const std::vector<double> &V, int d,
                      std::vector<double> &lam, std::vector<double> &R);
// d_eff: rounded participation ratio (cumvar == 0) or the cumulative-variance rule
int deff_from_spectrum(const std::vector<double> &lam, double cumvar);
// steps 3-6 of a calibration from the ordered eigenpairs and the rotated
// samples Y [n][d] (of the unit samples in the normalised variant)
sq_status finish_head_from_eigen(const std::vector<double> &lam, const std::vector<double> &R, const double *Y,
                                 int64_t n, int d, const sq_calib_opts &o, const float *gauss, HeadCal &h,
                                 std::string &err);
sq_status check_calib_opts(const sq_calib_opts *o);
sq_status calibrate_head_tq(const float *rotation, int d, const sq_calib_opts &o, const float *gauss,
                            HeadCal &out, std::string &err);

// device entry points (kernels.hip)
sq_status upload_tables(sq_calib *c, void *stream);
void release_tables(sq_calib *c);

}  // namespace sq
