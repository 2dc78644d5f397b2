// Library-wide entry points of libsdv: version and status text.
#include "sdv_common.h"

extern "C" int sd_abi_version(void) { return SDV_ABI_VERSION; }

extern "C" const char* sd_status_string(int code) {
  switch (code) {
    case SD_OK: return "ok";
    case SD_EINVAL: return "invalid argument";
    case SD_ERANGE: return "table or workspace too small for the sizes given";
    case SD_EUNSUPPORTED: return "sizes beyond this build's limits";
    case SD_ELAUNCH: return "kernel launch failed";
    case SD_ST_BAD_TOKEN: return "token id outside [0, V)";
    case SD_ST_NONFINITE: return "logit row holds NaN or +inf";
    case SD_ST_ZERO_Z: return "logit row is entirely -inf";
    case SD_ST_ZERO_RESIDUAL: return "rejection with empty residual: drawn from the target";
    case SD_ST_ZERO_Q: return "draft probability of the tested token is zero";
    default: return "unknown status";
  }
}
