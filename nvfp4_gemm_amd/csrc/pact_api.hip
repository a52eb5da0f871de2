// pact_api.hip -- version and status strings of the libpact C ABI.
#include "pact_host.h"

extern "C" int pact_version(void) { return PACT_VERSION; }

extern "C" const char *pact_status_string(pact_status s) {
    switch (s) {
        case PACT_OK: return "PACT_OK";
        case PACT_ERR_INVALID_ARG: return "PACT_ERR_INVALID_ARG";
        case PACT_ERR_UNSUPPORTED_SHAPE: return "PACT_ERR_UNSUPPORTED_SHAPE";
        case PACT_ERR_MISALIGNED: return "PACT_ERR_MISALIGNED";
        case PACT_ERR_WORKSPACE: return "PACT_ERR_WORKSPACE";
        case PACT_ERR_HIP: return "PACT_ERR_HIP";
    }
    return "PACT_ERR_UNKNOWN";
}
