// The decode-step kernel for 128-bit codes (see decode_fused.h).
#include "decode_fused.h"

namespace hata {
template hipError_t launch_fused<128>(int, FusedArgs &, hipStream_t);
}  // namespace hata
