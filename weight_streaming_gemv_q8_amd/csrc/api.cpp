// Status strings and version of the wsgemv C ABI.
#include "wsgemv.h"

extern "C" {

const char* wsg_status_str(int status) {
    switch (status) {
        case WSG_OK: return "ok";
        case WSG_ERR_NULL: return "a required pointer is NULL";
        case WSG_ERR_SHAPE: return "n or k out of range (negative, >= 2^31, not a multiple of the block, or above the path's maximum k)";
        case WSG_ERR_ALIGN: return "a pointer is not aligned (16 bytes for weights and activations, 4 for outputs)";
        case WSG_ERR_MODE: return "unknown activation format, weight type or op (or a mode the call does not support)";
        case WSG_ERR_WORKSPACE: return "workspace too small";
        case WSG_ERR_HIP: return "the HIP runtime rejected a launch or graph call";
        default: return "unknown status";
    }
}

const char* wsg_version(void) { return "0.1.0"; }

}  // extern "C"
