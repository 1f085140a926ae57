// version.hip -- status strings and version of the C ABI.
#include "idx_common.hpp"

extern "C" const char* idx_status_string(idx_status s) {
  switch (s) {
    case IDX_OK: return "IDX_OK";
    case IDX_EINVAL: return "IDX_EINVAL: invalid pointer, size or shape";
    case IDX_EUNSUPPORTED: return "IDX_EUNSUPPORTED: valid but not implemented";
    case IDX_EHIP: return "IDX_EHIP: a HIP launch failed";
  }
  return "unknown idx_status";
}

extern "C" const char* idx_version(void) { return "idx-gfx950 0.1"; }
