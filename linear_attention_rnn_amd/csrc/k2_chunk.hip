// Chunked-prefill kernel (placeholder until the chunked kernel lands).
#include "internal.h"

namespace wkv7 {

hipError_t launch_chunked(const SeqArgs&, int32_t, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace wkv7
