// Status strings and version of the CSA2 library.
#include "csa2_common.h"

extern "C" const char* csa2_status_string(int32_t status) {
  switch (status) {
    case CSA2_OK: return "CSA2_OK";
    case CSA2_ERR_INVALID_ARG: return "CSA2_ERR_INVALID_ARG";
    case CSA2_ERR_UNSUPPORTED: return "CSA2_ERR_UNSUPPORTED";
    case CSA2_ERR_WORKSPACE: return "CSA2_ERR_WORKSPACE";
    case CSA2_ERR_LAUNCH: return "CSA2_ERR_LAUNCH";
    default: return "CSA2_ERR_UNKNOWN";
  }
}

extern "C" const char* csa2_version(void) { return "csa2-mi355x 0.1 gfx950"; }
