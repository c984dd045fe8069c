#include "common.h"
namespace sa {
hipError_t launch_union(const UnionParams& p, hipStream_t s) { (void)p; (void)s; return hipErrorNotSupported; }
hipError_t launch_prefill(const PrefillParams& p, hipStream_t s) { (void)p; (void)s; return hipErrorNotSupported; }
}
