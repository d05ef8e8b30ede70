// Placeholder: bf16 MFMA fused forward/backward (not yet enabled).
#include "ttt_internal.h"
namespace ttt {
bool mfma_full_supported(const Problem&) { return false; }
int mfma_full_splits(const Problem&, int) { return 1; }
void launch_mfma_full_grad(const Problem&, const bf16*, int, int, int, float*, hipStream_t) {}
bool mfma_query_supported(const Problem&) { return false; }
void launch_mfma_query(const Problem&, const bf16*, long long, int, int, hipStream_t) {}
}  // namespace ttt
