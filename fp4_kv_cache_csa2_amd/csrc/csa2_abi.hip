// csa2_abi.hip -- version, status strings and the host-side RoPE table of libcsa2.
#include <math.h>

#include "csa2_device.hpp"

extern "C" int csa2_abi_version(void) { return CSA2_ABI_VERSION; }

extern "C" const char* csa2_status_string(int status) {
  switch (status) {
    case CSA2_OK: return "ok";
    case CSA2_ERR_INVALID_ARG: return "invalid argument";
    case CSA2_ERR_UNSUPPORTED: return "unsupported configuration";
    case CSA2_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA2_ERR_HIP: return "HIP runtime error at launch";
    case CSA2_ERR_SCRATCH: return "problem larger than the fixed scratch array of the allocation-free call";
    default: return "unknown status";
  }
}

// cos/sin of p * theta^(-2i/64) for the compressed-entry RoPE ([ZB] "把 KV Cache 压缩推到极致"
// §1.2 model table, compress_rope_theta), evaluated in double on the host.
extern "C" int csa2_rope_table(const int64_t* pos, int64_t n, double theta, float* out) {
  if (n < 0 || (n > 0 && (!pos || !out))) return CSA2_ERR_INVALID_ARG;
  for (int64_t j = 0; j < n; j++) {
    for (int i = 0; i < csa2::kDRope / 2; i++) {
      const double inv_freq = pow(theta, -(double)(2 * i) / (double)csa2::kDRope);
      const double ang = (double)pos[j] * inv_freq;
      out[j * csa2::kDRope + i] = (float)cos(ang);
      out[j * csa2::kDRope + csa2::kDRope / 2 + i] = (float)sin(ang);
    }
  }
  return CSA2_OK;
}
