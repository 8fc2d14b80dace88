// Decode attention for group size 4 on MFMA (placeholder until the kernel lands).
#include "dqk_internal.h"

namespace dqk {

bool use_mfma_decode(int hq, int hkv) {
    (void)hq;
    (void)hkv;
    return false;
}

int decode_splits_mfma(int batch, int hkv, int max_pages) { return decode_splits_generic(batch, hkv, max_pages); }

hipError_t launch_decode_mfma(const DecodeArgs &a, hipStream_t s) { return launch_decode_generic(a, s); }

}  // namespace dqk
