#include "common.h"
namespace sa {
hipError_t launch_mla_decode(const DecodeParams& p, hipStream_t s) { (void)p; (void)s; return hipErrorNotSupported; }
}
