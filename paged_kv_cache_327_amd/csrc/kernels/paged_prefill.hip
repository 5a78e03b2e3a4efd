// Chunked-prefill attention over a paged KV cache (MFMA bf16) -- not built yet.
#include "../internal.hpp"
#include "common.hpp"

namespace pa {

int launch_paged_prefill(const PrefillArgs&, void*) { return (int)hipErrorNotSupported; }

}  // namespace pa
