#include "attn_internal.h"
namespace attn {
hipError_t launch_decode_mla(const DecodeMlaArgs &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_prefill(const PrefillArgs &, hipStream_t) { return hipErrorNotSupported; }
}
