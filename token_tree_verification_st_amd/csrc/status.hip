// Text for return codes and device status bits (host only).
#include "st_internal.h"

extern "C" const char* st_status_str(int code) {
  switch (code) {
    case ST_OK: return "ok";
    case ST_E_INVALID: return "invalid argument (null pointer or out-of-range scalar)";
    case ST_E_UNSUPPORTED: return "unsupported size or layout";
    case ST_E_WORKSPACE: return "workspace too small";
    case ST_E_LAUNCH: return "kernel launch failed";
    case ST_STATUS_BAD_PARENT: return "bad parent array";
    case ST_STATUS_BAD_TOKEN: return "draft token out of range";
    case ST_STATUS_NONFINITE: return "non-finite logit";
    case ST_STATUS_PATH_OVERFLOW: return "accepted path longer than max_depth";
    case ST_STATUS_BAD_PREFIX: return "bad prefix length";
    case ST_STATUS_BAD_BLOCK: return "block-table entry out of range";
    default: return "unknown code";
  }
}
