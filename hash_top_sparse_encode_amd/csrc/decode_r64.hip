// The decode-step kernel for 64-bit codes (see decode_fused.h).
#include "decode_fused.h"

namespace hata {
template hipError_t launch_fused<64>(int, FusedArgs &, hipStream_t);
}  // namespace hata
