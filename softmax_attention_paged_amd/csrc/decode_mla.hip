// placeholder until the latent-decode kernel lands
#include "attn_internal.h"
namespace attn {
hipError_t launch_decode_mla(const DecodeMlaArgs &, hipStream_t) { return hipErrorNotSupported; }
}
