// Library identity and status strings.
#include "moeq8_host.hpp"

extern "C" const char* moeq8_status_string(int status) {
    switch (status) {
        case MOEQ8_OK: return "MOEQ8_OK";
        case MOEQ8_EINVAL: return "MOEQ8_EINVAL: invalid argument (null pointer, shape, K % 64, ncols, topk)";
        case MOEQ8_EALIGN: return "MOEQ8_EALIGN: pointer, stride or block-offset alignment";
        case MOEQ8_EUNSUPPORTED: return "MOEQ8_EUNSUPPORTED: valid request outside what the library implements";
        case MOEQ8_EHIP: return "MOEQ8_EHIP: HIP launch failed";
        default: return "MOEQ8: unknown status";
    }
}

extern "C" int moeq8_abi_version(void) { return MOEQ8_ABI_VERSION; }
